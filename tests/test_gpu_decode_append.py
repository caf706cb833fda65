"""Decode with append on the GPU, through the C ABI, against the fp64 oracle.

Each agent's new token is reserved on the host (after unaligned forks, whose tails were
packed into private pages by an n_valid-row device copy), stored by the call at position
len - 1 and attended to in the same call (write, then attend).  The new row's slot holds
NaN before the call, so an attention that read it before the write could not pass.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from lora_shared_prefix_amd import forkkv as fk  # noqa: E402
from lora_shared_prefix_amd.session import DeviceBatch, to_device, workload_geom  # noqa: E402
from oracle.attention import Geometry, apply_chunk_write, decode_attention  # noqa: E402
from tests.cases import encode  # noqa: E402
from tests.gpu_common import (apply_cows_host, assert_close, gpu_values,  # noqa: E402
                              model_tables, poison_unused, used_rows)
from workloads import config_by_name, draw_inputs, pool_ops  # noqa: E402


def _fork_ops(rng, n_agents, L0):
    """Root of L0 rows; agents fork at unaligned, aligned and full-length points and append
    nothing themselves, so the appended token lands in a freshly packed tail page (or
    opens a new page)."""
    ops = [("create", "root", 0), ("append", "root", L0)]
    points = [L0, (L0 // 16) * 16, max(1, L0 - 5), int(rng.integers(1, L0 + 1))]
    agents = []
    for j in range(n_agents):
        ops.append(("fork", "root", points[j % len(points)], f"a{j}"))
        agents.append(f"a{j}")
    return ops, agents


CASES = [  # seed, dtype, kernel, d, r, Hq, Hkv
    (0, "f32", fk.KERNEL_GENERIC, 16, 4, 8, 2),
    (1, "bf16", fk.KERNEL_GENERIC, 32, 8, 8, 2),
    (2, "bf16", fk.KERNEL_MFMA, 128, 16, 8, 2),
    (3, "bf16", fk.KERNEL_MFMA, 128, 16, 16, 2),
]


@pytest.mark.parametrize("seed,dtype,kernel,d,r,Hq,Hkv", CASES)
def test_decode_append_tiny(seed, dtype, kernel, d, r, Hq, Hkv):
    rng = np.random.default_rng(900 + seed)
    n_agents, num_pages = 5, 64
    L0 = int(rng.integers(20, 120))
    ops, agents = _fork_ops(rng, n_agents, L0)
    perm_b = rng.permutation(num_pages).astype(np.int32)
    perm_r = rng.permutation(num_pages).astype(np.int32)
    bpool = encode(rng.standard_normal((num_pages, 2, Hkv, 16 * d)), dtype)
    rpool = encode(rng.standard_normal((num_pages, 2, 16 * r)), dtype)
    Bk = encode(0.3 * rng.standard_normal((n_agents, r, Hkv * d)), dtype)
    Bv = encode(0.3 * rng.standard_normal((n_agents, r, Hkv * d)), dtype)
    q = encode(rng.standard_normal((n_agents, Hq, d)), dtype)
    rows = dict(k_new=encode(rng.standard_normal((n_agents, Hkv, d)), dtype),
                v_new=encode(rng.standard_normal((n_agents, Hkv, d)), dtype),
                rk_new=encode(rng.standard_normal((n_agents, r)), dtype),
                rv_new=encode(rng.standard_normal((n_agents, r)), dtype))
    lora_scale, theta, sm = 2.0, 5e5, 1.0 / np.sqrt(d)

    # every slot the batch does not read before the append -- the new rows included -- is NaN
    _, _, bt0, rt0, lens0 = model_tables(num_pages, num_pages, perm_b, perm_r, ops, agents, 16)
    from oracle import PoolModel
    pm = PoolModel(num_pages, num_pages, 16, perm_b, perm_r)
    names, cows = {}, []
    for op in ops:
        if op[0] == "create":
            names[op[1]] = pm.create(bool(op[2]))
        elif op[0] == "append":
            c = pm.append(names[op[1]], op[2])[2]
            cows += [c] if c else []
        else:
            names[op[3]], c = pm.fork(names[op[1]], op[2])
            cows += [c] if c else []
    ub, ur = used_rows(bt0, rt0, lens0)
    for src, dst, n in cows:
        ub |= {(src, row) for row in range(n)}
    bpool, rpool = poison_unused(bpool, rpool, ub, ur, dtype, d, r)

    geom = dict(num_bpages=num_pages, num_rpages=num_pages, num_kv_heads=Hkv, num_q_heads=Hq,
                head_dim=d, rank=r, dtype=dtype)
    b = DeviceBatch(geom, dict(bpool=bpool, rpool=rpool, q=q, Bk=Bk, Bv=Bv), ops, agents,
                    perm_b, perm_r, plan=False)
    assert b.cows == cows
    start = b.reserve_chunk(1)  # host bookkeeping of the new token, tables re-uploaded
    assert start == list(lens0)
    # the library's bookkeeping of the append matches the model bit for bit (no copy is
    # needed: the fork already packed every unaligned tail into a private page)
    for a in agents:
        assert pm.append(names[a], 1)[2] is None
    bt_m, rt_m, lens_m = pm.tables([names[a] for a in agents], b.max_pages)
    assert np.array_equal(np.array(bt_m, dtype=np.int32).reshape(b.btab_host.shape), b.btab_host)
    assert np.array_equal(np.array(rt_m, dtype=np.int32).reshape(b.rtab_host.shape), b.rtab_host)
    b.make_plan(kernel)
    assert b.plan.info["kernel"] == kernel
    dev_rows = {k: to_device(v) for k, v in rows.items()}
    b.out.fill_(float("nan") if dtype == "f32" else 0x7FC0)
    out = b.decode_append(dev_rows, lora_scale, sm, theta)
    torch.cuda.synchronize()

    # oracle: the pools after the fork packing and the row write, then decode over len + 1
    geo = Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rank=r,
                   dtype=dtype)
    bt, rt, lens = b.btab_host, b.rtab_host, np.array(b.lens)
    assert list(lens) == [L + 1 for L in lens0]
    host_b = apply_cows_host(bpool, cows, Hkv, d)
    exp_b, exp_r = apply_chunk_write(geo, host_b, rpool, bt, rt, lens0,
                                     rows["k_new"][:, None], rows["v_new"][:, None],
                                     rows["rk_new"][:, None], rows["rv_new"][:, None])
    got_b = b.bcache.cpu().numpy()
    got_r = b.rcache.cpu().numpy()
    if dtype == "bf16":
        got_b, got_r = got_b.view(np.uint16), got_r.view(np.uint16)
    assert np.array_equal(got_b.view(np.uint8), exp_b.view(np.uint8)), "pool bytes (base)"
    assert np.array_equal(got_r.view(np.uint8), exp_r.view(np.uint8)), "pool bytes (residual)"
    ref = decode_attention(geo, exp_b, exp_r, bt, rt, lens, q, Bk, Bv, lora_scale, sm, theta)
    g = gpu_values(out, dtype)
    assert_close(g, ref, f"append seed={seed} {dtype} kernel={kernel}", scale_abs=True)


STEP_CASES = [(fk.KERNEL_MFMA, False, False), (fk.KERNEL_MFMA, True, False),
              (fk.KERNEL_GENERIC, True, False), (fk.KERNEL_MFMA, False, True),
              (fk.KERNEL_MFMA, True, True), (fk.KERNEL_GENERIC, False, True)]


@pytest.mark.parametrize("kernel,freeze,graph", STEP_CASES)
def test_decode_append_steps(kernel, freeze, graph):
    """A serving loop: 40 decode-with-append steps in a row on one plan, so the new tokens
    cross page boundaries (and, after unaligned packed forks, first fill the packed tail
    pages); with ``freeze`` the agents share the root's frozen unaligned tail (the slot map
    is in use).  The plan's device lengths advance inside each call; between steps the host
    reserves the next tokens in one batched call and only at a page crossing updates the
    tables in place and rebuilds and re-uploads the plan.  With ``graph`` one captured call
    is replayed for every step (with new query and row values copied in), which must stay
    valid across the rebuilds.  Every step's output, and the pools at the end, are checked
    against the oracle replaying the same writes."""
    from oracle.attention import apply_rows_write
    rng = np.random.default_rng(4321 + int(freeze) + 2 * int(graph))
    dtype, d, r, Hq, Hkv = "bf16", 128, 16, 8, 2
    if kernel == fk.KERNEL_GENERIC:
        dtype, d, r = "f32", 32, 8
    n_agents, num_pages, L0, steps = 3, 96, 37, 40
    ops = [("create", "root", 0), ("append", "root", L0)]
    points = [L0, 32, 21]
    for j in range(n_agents):
        ops.append(("fork", "root", L0, f"a{j}", fk.FORK_FREEZE, 0) if freeze
                   else ("fork", "root", points[j], f"a{j}"))
    agents = [f"a{j}" for j in range(n_agents)]
    perm_b = rng.permutation(num_pages).astype(np.int32)
    perm_r = rng.permutation(num_pages).astype(np.int32)
    bpool = encode(rng.standard_normal((num_pages, 2, Hkv, 16 * d)), dtype)
    rpool = encode(rng.standard_normal((num_pages, 2, 16 * r)), dtype)
    Bk = encode(0.3 * rng.standard_normal((n_agents, r, Hkv * d)), dtype)
    Bv = encode(0.3 * rng.standard_normal((n_agents, r, Hkv * d)), dtype)
    q0 = encode(rng.standard_normal((n_agents, Hq, d)), dtype)
    geom = dict(num_bpages=num_pages, num_rpages=num_pages, num_kv_heads=Hkv, num_q_heads=Hq,
                head_dim=d, rank=r, dtype=dtype)
    b = DeviceBatch(geom, dict(bpool=bpool, rpool=rpool, q=q0, Bk=Bk, Bv=Bv), ops, agents,
                    perm_b, perm_r, plan=False)
    geo = Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rank=r,
                   dtype=dtype)
    host_b, host_r = apply_cows_host(bpool, b.cows, Hkv, d), rpool.copy()
    lora_scale, theta, sm = 2.0, 5e5, 1.0 / np.sqrt(d)
    # the first token: reserved, tables with room for the loop's pages, one plan
    _, cows, _, _ = b.pool.append_batch(b.handles, 1)
    if cows:
        b.pool.cow_copy(cows)
        host_b = apply_cows_host(host_b, cows, Hkv, d)
    b.refresh_tables(extra_pages=steps // 16 + 2)
    b.make_plan(kernel)
    assert b.plan.info["kernel"] == kernel and (b.pstart is not None) == freeze
    dev_rows = {k: to_device(np.zeros(shape, dtype=np.float32 if dtype == "f32" else np.uint16))
                for k, shape in (("k_new", (n_agents, Hkv, d)), ("v_new", (n_agents, Hkv, d)),
                                 ("rk_new", (n_agents, r)), ("rv_new", (n_agents, r)))}
    g = None
    rebuilds = 0
    for step in range(steps):
        if step > 0:
            before = [b.pool.length(h) for h in b.handles]
            n_bpages = b.pool.stats()["live_bpages"]
            same, cows = b.next_step()
            if cows:
                host_b = apply_cows_host(host_b, cows, Hkv, d)
            rebuilds += int(b.pool.stats()["live_bpages"] != n_bpages)
            assert [b.pool.length(h) for h in b.handles] == [n + 1 for n in before]
            # the tables next_step patched equal a fresh export, and so do the device tables
            bt, rt, lens = b.pool.tables(b.handles, b.max_pages)
            assert np.array_equal(np.array(bt).reshape(b.btab_host.shape), b.btab_host)
            assert np.array_equal(np.array(rt).reshape(b.rtab_host.shape), b.rtab_host)
            assert list(lens) == list(b.lens)
            assert np.array_equal(b.btab.cpu().numpy(), b.btab_host)
            if freeze:
                st, _ = b.pool.starts(b.handles, b.max_pages)
                assert np.array_equal(np.array(st).reshape(b.pstart_host.shape), b.pstart_host)
                assert np.array_equal(b.pstart.cpu().numpy(), b.pstart_host)
            assert same or not graph
        q = encode(rng.standard_normal((n_agents, Hq, d)), dtype)
        rows = dict(k_new=encode(rng.standard_normal((n_agents, Hkv, d)), dtype),
                    v_new=encode(rng.standard_normal((n_agents, Hkv, d)), dtype),
                    rk_new=encode(rng.standard_normal((n_agents, r)), dtype),
                    rv_new=encode(rng.standard_normal((n_agents, r)), dtype))
        b.q.copy_(to_device(q))
        for k, v in rows.items():
            dev_rows[k].copy_(to_device(v))
        b.out.fill_(float("nan") if dtype == "f32" else 0x7FC0)
        if graph and g is not None:
            g.replay()
        else:
            b.decode_append(dev_rows, lora_scale, sm, theta)
            if graph:  # capture the call once, after the eager first step
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    b.decode_append(dev_rows, lora_scale, sm, theta)
        torch.cuda.synchronize()
        # the copy-on-write copies the library reported are mirrored on the oracle's pools
        lens = [b.pool.length(h) for h in b.handles]
        starts = b.pstart_host if freeze else None
        host_b, host_r = apply_rows_write(geo, host_b, host_r, b.btab_host, b.rtab_host,
                                          [[t - 1] for t in lens], rows["k_new"][:, None],
                                          rows["v_new"][:, None], rows["rk_new"][:, None],
                                          rows["rv_new"][:, None], starts=starts)
        ref = decode_attention(geo, host_b, host_r, b.btab_host, b.rtab_host, np.array(lens),
                               q, Bk, Bv, lora_scale, sm, theta, starts=starts)
        assert_close(gpu_values(b.out, dtype), ref,
                     f"append step {step} kernel={kernel} freeze={freeze} graph={graph}",
                     scale_abs=True)
    assert rebuilds >= 2  # the loop crossed pages
    got_b = b.bcache.cpu().numpy().view(np.uint16 if dtype == "bf16" else np.float32)
    got_r = b.rcache.cpu().numpy().view(np.uint16 if dtype == "bf16" else np.float32)
    assert np.array_equal(got_b.view(np.uint8), host_b.view(np.uint8)), "pool bytes (base)"
    assert np.array_equal(got_r.view(np.uint8), host_r.view(np.uint8)), "pool bytes (residual)"


def test_decode_append_llama3_react_shape():
    """The Llama3-8B ReAct workload (4 agents, 8192 shared + 512 private tokens):
    one appended token per agent at position 8704, MFMA kernel, sampled heads."""
    cfg = config_by_name("llama3_8b_react_decode")
    print(f"[gpu-append] drawing inputs of {cfg.name}", flush=True)
    x = draw_inputs(cfg)
    ops, agents = pool_ops(cfg)
    rng = np.random.default_rng(77)
    N, Hkv, d, r = cfg.n_agents, cfg.num_kv_heads, cfg.head_dim, cfg.rank
    rows = dict(k_new=encode(rng.standard_normal((N, Hkv, d)), "bf16"),
                v_new=encode(rng.standard_normal((N, Hkv, d)), "bf16"),
                rk_new=encode(rng.standard_normal((N, r)), "bf16"),
                rv_new=encode(rng.standard_normal((N, r)), "bf16"))
    b = DeviceBatch(workload_geom(cfg), x, ops, agents, x["perm_b"], x["perm_r"], plan=False)
    lens0 = b.reserve_chunk(1)
    b.make_plan(fk.KERNEL_MFMA)
    b.out.fill_(0x7FC0)
    out = b.decode_append({k: to_device(v) for k, v in rows.items()}, cfg.lora_scale,
                          1.0 / np.sqrt(d), cfg.rope_theta)
    torch.cuda.synchronize()
    geo = Geometry.of(cfg)
    bt, rt, lens = b.btab_host, b.rtab_host, np.array(b.lens)
    exp_b, exp_r = apply_chunk_write(geo, x["bpool"], x["rpool"], bt, rt, lens0,
                                     rows["k_new"][:, None], rows["v_new"][:, None],
                                     rows["rk_new"][:, None], rows["rv_new"][:, None])
    ref = decode_attention(geo, exp_b, exp_r, bt, rt, lens, x["q"], x["Bk"], x["Bv"],
                           cfg.lora_scale, 1.0 / np.sqrt(d), cfg.rope_theta, agents=[0, 3],
                           kv_heads=[0, 5])
    g = gpu_values(out, "bf16")
    mask = ~np.isnan(ref[..., 0])
    assert_close(g[mask], ref[mask], "append llama3 react shape")
    # the stored rows: every agent's new token at position 8704, bit for bit
    got_b = b.bcache.cpu().numpy().view(np.uint16)
    for a in range(N):
        t = lens0[a]
        pg = bt[a][t // 16]
        assert np.array_equal(got_b[pg], exp_b[pg]), f"agent {a} page {pg}"


def test_decode_append_errors():
    """Plan lengths below 1 and null row pointers are rejected before any launch."""
    geom = dict(num_bpages=8, num_rpages=8, num_kv_heads=1, num_q_heads=2, head_dim=16, rank=4,
                dtype="f32")
    rng = np.random.default_rng(3)
    arrays = dict(bpool=rng.standard_normal((8, 2, 1, 256)).astype(np.float32),
                  rpool=rng.standard_normal((8, 2, 64)).astype(np.float32),
                  q=rng.standard_normal((2, 2, 16)).astype(np.float32),
                  Bk=rng.standard_normal((2, 4, 16)).astype(np.float32),
                  Bv=rng.standard_normal((2, 4, 16)).astype(np.float32))
    ops = [("create", "root", 0), ("append", "root", 20), ("fork", "root", 0, "a0"),
           ("fork", "root", 16, "a1")]
    b = DeviceBatch(geom, arrays, ops, ["a0", "a1"])  # a0 has no keys: length 0
    rows = {k: torch.zeros(s, dtype=torch.float32, device="cuda")
            for k, s in (("k_new", (2, 1, 16)), ("v_new", (2, 1, 16)), ("rk_new", (2, 4)),
                         ("rv_new", (2, 4)))}
    with pytest.raises(fk.ForkKVError) as e:
        b.decode_append(rows, 1.0, 0.25, 1e4)
    assert e.value.code == fk.EINVAL


@pytest.mark.parametrize("kernel,dtype,d,r", [(fk.KERNEL_GENERIC, "f32", 16, 4),
                                              (fk.KERNEL_MFMA, "bf16", 128, 16)])
def test_decode_append_graph_replay_matches_eager(kernel, dtype, d, r):
    """Decode with append advances the plan's device lengths, so one captured call replayed
    step after step is a serving loop.  Two identical batches run 20 steps: one calls eagerly
    every step, the other replays a graph captured after its first eager step; between steps
    both reserve the next tokens (rebuilding and re-uploading the plan at page crossings).
    Outputs and pools agree bit for bit after every step."""
    rng = np.random.default_rng(990 + d)
    n_agents, num_pages, Hq, Hkv = 5, 96, 8, 2
    ops, agents = _fork_ops(rng, n_agents, int(rng.integers(20, 120)))
    perm_b = rng.permutation(num_pages).astype(np.int32)
    perm_r = rng.permutation(num_pages).astype(np.int32)
    arrays = dict(bpool=encode(rng.standard_normal((num_pages, 2, Hkv, 16 * d)), dtype),
                  rpool=encode(rng.standard_normal((num_pages, 2, 16 * r)), dtype),
                  q=encode(rng.standard_normal((n_agents, Hq, d)), dtype),
                  Bk=encode(0.3 * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
                  Bv=encode(0.3 * rng.standard_normal((n_agents, r, Hkv * d)), dtype))
    rows = {k: to_device(encode(rng.standard_normal(shape), dtype)) for k, shape in
            (("k_new", (n_agents, Hkv, d)), ("v_new", (n_agents, Hkv, d)),
             ("rk_new", (n_agents, r)), ("rv_new", (n_agents, r)))}
    geom = dict(num_bpages=num_pages, num_rpages=num_pages, num_kv_heads=Hkv, num_q_heads=Hq,
                head_dim=d, rank=r, dtype=dtype)
    steps = 20
    batches = []
    for _ in range(2):
        b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, plan=False)
        b.reserve_chunk(1)
        b.refresh_tables(extra_pages=3)
        b.make_plan(kernel)
        assert b.plan.info["kernel"] == kernel
        batches.append(b)
    eager_b, graph_b = batches
    args = (2.0, 1.0 / np.sqrt(d), 5e5)
    graph = None
    for step in range(steps):
        if step > 0:
            for b in batches:
                same, _ = b.next_step()
                assert same
        eager_b.decode_append(rows, *args)
        if graph is None:
            graph_b.decode_append(rows, *args)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                graph_b.decode_append(rows, *args)
        else:
            graph_b.out.fill_(step + 1)
            torch.cuda.synchronize()
            graph.replay()
        torch.cuda.synchronize()
        same = (torch.equal(eager_b.out, graph_b.out) and torch.equal(eager_b.bcache, graph_b.bcache)
                and torch.equal(eager_b.rcache, graph_b.rcache))
        print(f"[parity] decode-append graph step {step} kernel={kernel}: bitwise equal={same}",
              flush=True)
        assert same
