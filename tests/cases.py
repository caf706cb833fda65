"""Small seeded cases with ragged lengths, unaligned forks and partial pages."""
from __future__ import annotations

import numpy as np

from workloads import bf16_bits_from_f32


def encode(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return x.copy() if dtype == "f32" else bf16_bits_from_f32(x)


def random_ops(rng, n_agents, P=16, max_prefix=40, max_suffix=24):
    """Root with a ragged prefix; agents fork at (often unaligned) points and append."""
    L0 = int(rng.integers(1, max_prefix + 1))
    ops = [("create", "root", 0), ("append", "root", L0)]
    agents = []
    for j in range(n_agents):
        alias = int(rng.integers(0, L0 + 1))
        ops.append(("fork", "root", alias, f"a{j}"))
        agents.append(f"a{j}")
    for a in agents:
        n = int(rng.integers(1, max_suffix + 1))
        ops.append(("append", a, n))
    return ops, agents


def freeze_ops(rng, n_agents, P=16, max_prefix=40, max_suffix=24):
    """Frozen tails (fork mode 1 = freeze): a root of unaligned length whose tail every agent
    shares read-only; agents then append, the root continues past its frozen tail, and the
    last agent is a grandchild frozen again at its parent's (unaligned) end."""
    L0 = int(rng.integers(1, max_prefix // P)) * P + int(rng.integers(1, P))
    ops = [("create", "root", 0), ("append", "root", L0)]
    agents = []
    for j in range(n_agents - 1):
        ops.append(("fork", "root", L0, f"a{j}", 1, 0))
        agents.append(f"a{j}")
    ops.append(("append", "root", int(rng.integers(1, P))))
    for a in agents:
        n = int(rng.integers(1, max_suffix + 1))
        if n % P == 0:
            n += 1
        ops.append(("append", a, n))
    ops.append(("fork", agents[0], None, f"a{n_agents - 1}", 1, 0))  # at a0's end
    agents.append(f"a{n_agents - 1}")
    ops.append(("append", agents[-1], int(rng.integers(1, max_suffix + 1))))
    return ops, agents


def resolve_ops(ops):
    """Fill fork points given as None (the parent's current length) by tracking lengths."""
    lens, out = {}, []
    for op in ops:
        if op[0] == "create":
            lens[op[1]] = 0
        elif op[0] == "append":
            lens[op[1]] += op[2]
        else:
            alias = lens[op[1]] if op[2] is None else op[2]
            op = (op[0], op[1], alias) + tuple(op[3:])
            lens[op[3]] = alias
        out.append(op)
    return out


def tiny_case(seed, dtype="f32", Hq=4, Hkv=2, d=8, r=3, n_agents=3, P=16, max_prefix=40,
              max_suffix=24, b_std=0.3, num_pages=64, chunk=0, freeze=False):
    rng = np.random.default_rng(seed)
    if freeze:
        ops, agents = freeze_ops(rng, n_agents, P, max_prefix, max_suffix)
        ops = resolve_ops(ops)
    else:
        ops, agents = random_ops(rng, n_agents, P, max_prefix, max_suffix)
    perm_b = rng.permutation(num_pages).astype(np.int32)
    perm_r = rng.permutation(num_pages).astype(np.int32)
    case = dict(
        P=P, Hq=Hq, Hkv=Hkv, d=d, r=r, dtype=dtype, ops=ops, agents=agents,
        perm_b=perm_b, perm_r=perm_r, num_bpages=num_pages, num_rpages=num_pages,
        bpool=encode(rng.standard_normal((num_pages, 2, Hkv, P * d)), dtype),
        rpool=encode(rng.standard_normal((num_pages, 2, P * r)), dtype),
        Bk=encode(b_std * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
        Bv=encode(b_std * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
        lora_scale=float(rng.choice([0.5, 1.0, 2.0])), theta=float(rng.choice([1e4, 5e5])),
    )
    case["sm_scale"] = 1.0 / np.sqrt(d)
    if chunk:
        case["q"] = encode(rng.standard_normal((n_agents, chunk, Hq, d)), dtype)
        case["k_new"] = encode(rng.standard_normal((n_agents, chunk, Hkv, d)), dtype)
        case["v_new"] = encode(rng.standard_normal((n_agents, chunk, Hkv, d)), dtype)
        case["rk_new"] = encode(rng.standard_normal((n_agents, chunk, r)), dtype)
        case["rv_new"] = encode(rng.standard_normal((n_agents, chunk, r)), dtype)
    else:
        case["q"] = encode(rng.standard_normal((n_agents, Hq, d)), dtype)
    return case
