"""ResidualAttention by its plain definition, fp64 (oracle side; test infrastructure).

ForkKV study note, "2. Q1 / Q2 / Q3" (Q2) and the "Reconstruction" equation of
"4. 作者证明": the cached projection of agent i is the shared base ``xW`` plus
the agent's residual ``xA_i`` times ``B_i``.  For keys the base is stored after
RoPE and the residual before it ("3. 架构 / 方法图", Figure 8), so the agent's
key is ``RoPE(xW_k + s * xA_k B_k)`` where ``xW_k`` is the stored base key with
its rotation undone.  Values carry no RoPE: ``V = xW_v + s * xA_v B_v``.
Attention is ``softmax(sm_scale * q K^T) V`` over every cached key of the
agent; query head g reads KV head ``g // (Hq / Hkv)``.

The oracle builds these merged K and V explicitly -- the eager form that the
note's reproduction check 4 compares the fused kernel against -- and applies a
textbook softmax.  No blocking, no online softmax, no split-K.
"""
from __future__ import annotations

import numpy as np

from .rope import rope_rotate, rope_unrotate
from .storage import (base_key_rows, base_value_rows, decode_values, key_offset,
                      res_key_offset, res_key_rows, res_value_offset, res_value_rows,
                      table_pages, value_offset)


class Geometry:
    def __init__(self, *, page_size, num_q_heads, num_kv_heads, head_dim, rank, dtype):
        self.P, self.Hq, self.Hkv = page_size, num_q_heads, num_kv_heads
        self.d, self.r, self.dtype = head_dim, rank, dtype
        self.G = num_q_heads // num_kv_heads

    @classmethod
    def of(cls, cfg):
        return cls(page_size=cfg.page_size, num_q_heads=cfg.num_q_heads,
                   num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim, rank=cfg.rank,
                   dtype=cfg.dtype)


def _cached_rows(geo, bpool, rpool, btab, rtab, a, h, positions, starts=None):
    """Stored rows of agent a, KV head h at the given positions, and which positions are keys.

    Missing pages (table entry -1; ForkKV study note, "Error / eviction recovery"): a
    position whose base page was evicted holds no key until it is refilled, so it takes no
    part in attention (``present`` is False there); a position without a residual page (a
    sequence that has none, such as a base-only snapshot) has a zero residual.
    """
    st = None if starts is None else starts[a]
    bk = base_key_rows(bpool, btab[a], positions, h, geo.P, geo.d, geo.dtype, st)
    bv = base_value_rows(bpool, btab[a], positions, h, geo.P, geo.d, geo.dtype, st)
    rk = res_key_rows(rpool, rtab[a], positions, geo.P, geo.r, geo.dtype, st)
    rv = res_value_rows(rpool, rtab[a], positions, geo.P, geo.r, geo.dtype, st)
    present = table_pages(btab[a], positions, geo.P, st) >= 0
    no_res = table_pages(rtab[a], positions, geo.P, st) < 0
    rk[no_res] = 0.0
    rv[no_res] = 0.0
    return bk, bv, rk, rv, present


def merged_kv(geo, bk, bv, rk, rv, Bk_a, Bv_a, h, positions, lora_scale, theta):
    """Merged key and value rows of one agent and KV head.

    bk: stored post-RoPE base keys [L, d]; bv: base values [L, d];
    rk, rv: rank-r residuals [L, r]; Bk_a, Bv_a: the agent's up-projections
    [r, Hkv*d] (fp64).  Returns (K, V), each [L, d].
    """
    cols = slice(h * geo.d, (h + 1) * geo.d)
    xw_k = rope_unrotate(bk, positions, theta)
    k = rope_rotate(xw_k + lora_scale * (rk @ Bk_a[:, cols]), positions, theta)
    v = bv + lora_scale * (rv @ Bv_a[:, cols])
    return k, v


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def decode_attention(geo, bpool, rpool, btab, rtab, seq_lens, q, Bk, Bv, lora_scale,
                     sm_scale, theta, agents=None, kv_heads=None, starts=None):
    """One decode query per agent over its cached keys 0 .. seq_len-1.

    q: [N, Hq, d] (post-RoPE, stored encoding).  Returns fp64 [N, Hq, d]; rows
    not requested through ``agents`` / ``kv_heads`` are NaN.  An agent with no
    cached keys gets a zero output.  ``starts`` ([N][max_pages] page start
    positions, -1 padded) is the slot map of sequences holding a frozen tail
    (ForkServe README, "Design vs APC"); None means page lp starts at lp * P.
    """
    N = q.shape[0]
    qv = decode_values(q, geo.dtype)
    Bkv = decode_values(Bk, geo.dtype)
    Bvv = decode_values(Bv, geo.dtype)
    out = np.full((N, geo.Hq, geo.d), np.nan)
    for a in (range(N) if agents is None else agents):
        L = int(seq_lens[a])
        pos = np.arange(L, dtype=np.int64)
        for h in (range(geo.Hkv) if kv_heads is None else kv_heads):
            gs = range(h * geo.G, (h + 1) * geo.G)
            if L == 0:
                out[a, list(gs)] = 0.0
                continue
            bk, bv, rk, rv, present = _cached_rows(geo, bpool, rpool, btab, rtab, a, h, pos,
                                                   starts)
            k, v = merged_kv(geo, bk, bv, rk, rv, Bkv[a], Bvv[a], h, pos, lora_scale, theta)
            k, v = k[present], v[present]
            for g in gs:
                if len(k) == 0:
                    out[a, g] = 0.0
                    continue
                p = _softmax_rows(sm_scale * (k @ qv[a, g]))
                out[a, g] = p @ v
    return out


def _slot(geo, starts, a, t):
    """(logical page, row) of position t of agent a, under the slot map if given."""
    if starts is None:
        return t // geo.P, t % geo.P
    st = [s for s in starts[a] if s >= 0]
    j = max(i for i, s in enumerate(st) if s <= t)
    return j, t - st[j]


def apply_rows_write(geo, bpool, rpool, btab, rtab, positions, k_new, v_new, rk_new, rv_new,
                     starts=None):
    """Pool contents after rows are stored (copies; inputs untouched).

    Row i of agent a goes to position ``positions[a][i]``: page ``table[a][pos // P]``,
    row ``pos % P`` (under a slot map: the page whose start is the last one <= pos, row
    pos - start), laid out as the pool layout says.  With ``rk_new`` None only the base
    pool is written.  A row whose page is missing (table entry -1) is not stored.
    """
    bp, rp = bpool.copy(), rpool.copy()
    N, C = k_new.shape[0], k_new.shape[1]
    d, r = geo.d, geo.r
    dims, ranks = np.arange(d), np.arange(r)
    for a in range(N):
        for i in range(C):
            t = int(positions[a][i])
            lp, row = _slot(geo, starts, a, t)
            page = int(btab[a][lp])
            for h in range(geo.Hkv if page >= 0 else 0):
                bp[page, 0, h, key_offset(row, dims)] = k_new[a, i, h]
                bp[page, 1, h, value_offset(row, dims)] = v_new[a, i, h]
            page = int(rtab[a][lp]) if rk_new is not None else -1
            if page >= 0:
                rp[page, 0, res_key_offset(row, ranks)] = rk_new[a, i]
                rp[page, 1, res_value_offset(row, ranks, r)] = rv_new[a, i]
    return bp, rp


def apply_chunk_write(geo, bpool, rpool, btab, rtab, start_pos, k_new, v_new, rk_new, rv_new):
    """Pool contents after the prefill chunk rows are stored: row i of agent a at position
    ``start_pos[a] + i`` (copies; inputs untouched)."""
    C = k_new.shape[1]
    positions = [[int(start_pos[a]) + i for i in range(C)] for a in range(k_new.shape[0])]
    return apply_rows_write(geo, bpool, rpool, btab, rtab, positions, k_new, v_new, rk_new,
                            rv_new)


def prefill_attention(geo, bpool, rpool, btab, rtab, start_pos, q, k_new, v_new, rk_new,
                      rv_new, Bk, Bv, lora_scale, sm_scale, theta, samples=None):
    """Chunked prefill: the chunk rows are written first, then every query attends causally.

    ``bpool``/``rpool`` are the pools *before* the write; keys at positions below
    ``start_pos[a]`` come from them and the chunk's own keys from
    ``k_new``/``v_new``/``rk_new``/``rv_new`` -- the same as reading the pools
    after the write (Penelope review, 部件二: each layer writes the batch's K/V,
    then attends).  Query i of agent a sits at position ``start_pos[a] + i`` and
    sees keys ``0 .. start_pos[a] + i`` (self included).

    Returns fp64 [N, C, Hq, d]; with ``samples`` (a list of (a, i, g)) only those
    rows are computed and the rest are NaN.
    """
    N, C = q.shape[0], q.shape[1]
    qv = decode_values(q, geo.dtype)
    Bkv, Bvv = decode_values(Bk, geo.dtype), decode_values(Bv, geo.dtype)
    out = np.full((N, C, geo.Hq, geo.d), np.nan)
    want = {}
    if samples is None:
        for a in range(N):
            for g in range(geo.Hq):
                want.setdefault((a, g // geo.G), []).extend((i, g) for i in range(C))
    else:
        for a, i, g in samples:
            want.setdefault((int(a), int(g) // geo.G), []).append((int(i), int(g)))
    for (a, h), rows in sorted(want.items()):
        start = int(start_pos[a])
        last = start + max(i for i, _ in rows)
        pos = np.arange(last + 1, dtype=np.int64)
        old = pos[pos < start]
        bk, bv, rk, rv, present = _cached_rows(geo, bpool, rpool, btab, rtab, a, h, old)
        n_new = last + 1 - start
        present = np.concatenate([present, table_pages(btab[a], pos[start:], geo.P) >= 0])
        no_res = np.concatenate([np.zeros(len(old), bool),
                                 table_pages(rtab[a], pos[start:], geo.P) < 0])
        bk = np.concatenate([bk, decode_values(k_new[a, :n_new, h], geo.dtype)])
        bv = np.concatenate([bv, decode_values(v_new[a, :n_new, h], geo.dtype)])
        rk = np.concatenate([rk, decode_values(rk_new[a, :n_new], geo.dtype)])
        rv = np.concatenate([rv, decode_values(rv_new[a, :n_new], geo.dtype)])
        rk[no_res] = 0.0  # a chunk row without a residual page has no residual to store
        rv[no_res] = 0.0
        k, v = merged_kv(geo, bk, bv, rk, rv, Bkv[a], Bvv[a], h, pos, lora_scale, theta)
        for i, g in rows:
            sel = present[:start + i + 1]
            p = _softmax_rows(sm_scale * (k[:start + i + 1][sel] @ qv[a, i, g]))
            out[a, i, g] = p @ v[:start + i + 1][sel]
    return out


def prefill_attention_at(geo, bpool, rpool, btab, rtab, positions, q, k_new, v_new, rk_new,
                         rv_new, Bk, Bv, lora_scale, sm_scale, theta, samples=None, starts=None):
    """Prefill over an arbitrary list of positions: row i of agent a sits at position
    ``positions[a][i]`` (e.g. a hole in the middle of the history followed by the real
    request's tail -- Penelope review, 部件二: the phantom request and the real request keep
    their original positions and run in one batch).  All rows are written first; then query
    i attends to keys ``0 .. positions[a][i]`` of the written pools (self included).

    Returns fp64 [N, C, Hq, d]; with ``samples`` (a list of (a, i, g)) only those rows are
    computed and the rest are NaN.  ``starts`` is the slot map, as for ``decode_attention``.
    """
    N, C = q.shape[0], q.shape[1]
    bp, rp = apply_rows_write(geo, bpool, rpool, btab, rtab, positions, k_new, v_new, rk_new,
                              rv_new, starts)
    qv = decode_values(q, geo.dtype)
    Bkv, Bvv = decode_values(Bk, geo.dtype), decode_values(Bv, geo.dtype)
    out = np.full((N, C, geo.Hq, geo.d), np.nan)
    want = {}
    if samples is None:
        for a in range(N):
            for g in range(geo.Hq):
                want.setdefault((a, g // geo.G), []).extend((i, g) for i in range(C))
    else:
        for a, i, g in samples:
            want.setdefault((int(a), int(g) // geo.G), []).append((int(i), int(g)))
    for (a, h), rows in sorted(want.items()):
        last = max(int(positions[a][i]) for i, _ in rows)
        pos = np.arange(last + 1, dtype=np.int64)
        bk, bv, rk, rv, present = _cached_rows(geo, bp, rp, btab, rtab, a, h, pos, starts)
        k, v = merged_kv(geo, bk, bv, rk, rv, Bkv[a], Bvv[a], h, pos, lora_scale, theta)
        for i, g in rows:
            n_keys = int(positions[a][i]) + 1
            sel = present[:n_keys]
            p = _softmax_rows(sm_scale * (k[:n_keys][sel] @ qv[a, i, g]))
            out[a, i, g] = p @ v[:n_keys][sel]
    return out
