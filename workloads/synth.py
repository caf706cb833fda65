"""Seeded draws and pool-operation scripts for the workloads.

Everything here is input preparation: random numbers in the storage encoding,
and the list of pool operations (create / append / fork) that builds each
workload's sharing topology.  Both the oracle's bookkeeping model and the HIP
library replay the same operation list with their own code.

Storage layout of the two page pools (the pages are silent on it; the library
fixes it, and both sides read the same bytes): a base page is
``bpool[page][plane][Hkv][P*d]`` (plane 0 = post-RoPE keys, plane 1 = values)
and a residual page ``rpool[page][plane][P*r]`` (plane 0 = key residual,
plane 1 = value residual); inside each tile the elements are in the order the
matrix cores consume them (see ``include/forkkv.h``).  The draws below fill whole
pools with i.i.d. values, so the tile order does not affect them.

Draw recipe (seeded ``numpy.random.default_rng(seed)``, PCG64), in this order:
base-page permutation, residual-page permutation, the whole base pool, the whole
residual pool, q, B_k, B_v, then (prefill only) the chunk rows k_new, v_new,
rk_new, rv_new.  Every value is a float32 standard normal (scaled by ``b_std``
for B_k and B_v) rounded to the storage type with round-to-nearest-even.  The
stored base keys are drawn directly: a rotation of an isotropic Gaussian pair is
again isotropic, so drawing post-RoPE keys from N(0,1) gives the same
distribution as drawing pre-RoPE keys and rotating them.
"""
from __future__ import annotations

import numpy as np

from .configs import WorkloadConfig

_CHUNK_VALUES = 1 << 24


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def _encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f32(x32)
    raise ValueError(dtype)


def _storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def _draw(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Draw N(0, scale^2) in chunks (identical to one large draw) and encode."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=_storage_dtype(dtype))
    pos = 0
    while pos < total:
        n = min(_CHUNK_VALUES, total - pos)
        v = rng.standard_normal(n, dtype=np.float32)
        if scale != 1.0:
            v = (v.astype(np.float64) * scale).astype(np.float32)
        out[pos:pos + n] = _encode(v, dtype)
        pos += n
    return out.reshape(shape)


def pool_value_shapes(cfg: WorkloadConfig) -> dict:
    P, d, r, hkv = cfg.page_size, cfg.head_dim, cfg.rank, cfg.num_kv_heads
    n = cfg.n_agents
    shapes = {
        "bpool": (cfg.num_bpages, 2, hkv, P * d),
        "rpool": (cfg.num_rpages, 2, P * r),
        "Bk": (n, r, hkv * d),
        "Bv": (n, r, hkv * d),
    }
    if cfg.kind == "decode":
        shapes["q"] = (n, cfg.num_q_heads, d)
    else:
        C = cfg.chunk_len
        shapes["q"] = (n, C, cfg.num_q_heads, d)
        shapes["k_new"] = (n, C, hkv, d)
        shapes["v_new"] = (n, C, hkv, d)
        shapes["rk_new"] = (n, C, r)
        shapes["rv_new"] = (n, C, r)
    return shapes


def draw_inputs(cfg: WorkloadConfig, seed: int | None = None) -> dict:
    """All seeded tensors of one workload, in storage encoding (uint16 bf16 bits or float32)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    shapes = pool_value_shapes(cfg)
    out = {
        "perm_b": rng.permutation(cfg.num_bpages).astype(np.int32),
        "perm_r": rng.permutation(cfg.num_rpages).astype(np.int32),
    }
    out["bpool"] = _draw(rng, shapes["bpool"], cfg.dtype)
    out["rpool"] = _draw(rng, shapes["rpool"], cfg.dtype)
    out["q"] = _draw(rng, shapes["q"], cfg.dtype)
    out["Bk"] = _draw(rng, shapes["Bk"], cfg.dtype, cfg.b_std)
    out["Bv"] = _draw(rng, shapes["Bv"], cfg.dtype, cfg.b_std)
    if cfg.kind == "prefill":
        for key in ("k_new", "v_new", "rk_new", "rv_new"):
            out[key] = _draw(rng, shapes[key], cfg.dtype)
    return out


def pool_ops(cfg: WorkloadConfig):
    """Operation script that builds the workload's sequences.

    Returns ``(ops, agents)``.  Each op is one of
    ``("create", name, with_residual)``, ``("append", name, n_tokens)`` or
    ``("fork", parent, alias_len, child)``.  ``agents`` lists the sequences
    that take part in the attention call, in batch order.
    """
    ops, agents = [], []
    for s in range(cfg.sessions):
        root = f"s{s}"
        ops.append(("create", root, 0))
        ops.append(("append", root, cfg.prefix_len))
        names = [f"s{s}a{j}" for j in range(cfg.agents_per_session)]
        for a in names:
            ops.append(("fork", root, cfg.prefix_len, a))
        if cfg.suffix_len:
            for a in names:
                ops.append(("append", a, cfg.suffix_len))
        agents.extend(names)
    return ops, agents


def chunk_ops(cfg: WorkloadConfig, agents):
    """Appends that reserve the prefill chunk rows, one per agent, in batch order."""
    return [("append", a, cfg.chunk_len) for a in agents] if cfg.chunk_len else []
