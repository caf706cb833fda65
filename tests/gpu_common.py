"""Helpers of the GPU parity tests: tolerance checks and oracle-side batch builders."""
from __future__ import annotations

import numpy as np

from oracle import PoolModel
from oracle.storage import (decode_values, key_offset, res_key_offset, res_value_offset,
                            value_offset)

# Tolerance (bf16 inputs, fp32 accumulation): max-abs error <= 1e-2 and the largest
# absolute error relative to the largest reference magnitude (a normwise relative
# error) <= 2e-2, per output tensor.  Element-wise relative error is ill-posed here:
# attention outputs over thousands of keys have many entries near zero.
MAX_ABS = 1e-2
MAX_REL = 2e-2


def errors(g, r):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    diff = np.abs(g - r)
    max_abs = float(diff.max()) if diff.size else 0.0
    scale = float(np.abs(r).max()) if r.size else 0.0
    rel = max_abs / scale if scale > 0 else max_abs
    return max_abs, rel


def assert_close(g, r, what="", max_abs=MAX_ABS, max_rel=MAX_REL, scale_abs=False):
    """scale_abs: synthetic cases whose outputs exceed 1 in magnitude -- bf16 rounding of
    the output alone is |o| * 2^-9 there -- scale the absolute bar by max(1, max|r|)."""
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    a, rel = errors(g, r)
    if scale_abs:
        max_abs = max_abs * max(1.0, float(np.abs(np.asarray(r)).max()))
    print(f"[parity] {what}: max_abs={a:.3e} normwise_rel={rel:.3e}", flush=True)
    assert a <= max_abs and rel <= max_rel, f"{what}: max_abs={a:.3e} rel={rel:.3e}"


def gpu_values(t, dtype):
    a = t.detach().cpu().numpy()
    if dtype == "bf16":
        a = a.view(np.uint16)
    return decode_values(a, dtype)


def model_tables(num_bpages, num_rpages, perm_b, perm_r, ops, agents, max_pages):
    pm = PoolModel(num_bpages, num_rpages, 16, perm_b, perm_r)
    names = pm.replay(ops)
    hs = [names[a] for a in agents]
    bt, rt, lens = pm.tables(hs, max_pages)
    return pm, hs, np.array(bt, dtype=np.int32), np.array(rt, dtype=np.int32), np.array(lens)


def apply_cows_host(bpool, cows, Hkv, d):
    """Row copies of fork packing applied to a host pool (the first n rows, K and V)."""
    out = bpool.copy()
    dims = np.arange(d)
    for src, dst, n in cows:
        for h in range(Hkv):
            for plane, off in ((0, key_offset), (1, value_offset)):
                for row in range(n):
                    idx = off(row, dims)
                    out[dst, plane, h, idx] = out[src, plane, h, idx]
    return out


def used_rows(bt, rt, lens, starts=None):
    """Sets of (page, row) slots read by the batch (``starts``: the slot map, if any)."""
    b, r = set(), set()
    for a in range(len(lens)):
        for t in range(int(lens[a])):
            if starts is None:
                j, row = t // 16, t % 16
            else:
                j = max(i for i, s in enumerate(starts[a]) if 0 <= s <= t)
                row = t - int(starts[a][j])
            b.add((int(bt[a][j]), row))
            r.add((int(rt[a][j]), row))
    return b, r


def poison_unused(bpool, rpool, used_b, used_r, dtype, d, r):
    """Fill every slot the batch never reads with NaN (bit pattern for bf16)."""
    nan = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
    bp, rp = bpool.copy(), rpool.copy()
    dims, ranks = np.arange(d), np.arange(r)
    for page in range(bp.shape[0]):
        for row in range(16):
            if (page, row) not in used_b:
                for h in range(bp.shape[2]):
                    bp[page, 0, h, key_offset(row, dims)] = nan
                    bp[page, 1, h, value_offset(row, dims)] = nan
    for page in range(rp.shape[0]):
        for row in range(16):
            if (page, row) not in used_r:
                rp[page, 0, res_key_offset(row, ranks)] = nan
                rp[page, 1, res_value_offset(row, ranks, r)] = nan
    return bp, rp


def model_replay(num_bpages, num_rpages, perm_b, perm_r, ops):
    """Replay a pool script on the oracle's model; returns (model, names, cow row copies)."""
    pm = PoolModel(num_bpages, num_rpages, 16, perm_b, perm_r)
    names, cows = {}, []
    for op in ops:
        if op[0] == "create":
            names[op[1]] = pm.create(bool(op[2]))
        elif op[0] == "append":
            c = pm.append(names[op[1]], op[2])[2]
            cows += [c] if c else []
        else:
            names[op[3]], c = pm.fork(names[op[1]], op[2], *op[4:])
            cows += [c] if c else []
    return pm, names, cows
