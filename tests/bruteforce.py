"""Pure-Python scalar brute force of ResidualAttention (independent of ``oracle/``).

Written from the ForkKV study note's definitions with plain loops and the
``math`` module only: read the stored bytes, undo the base key's rotation,
add the up-projected residual, rotate again, and take a softmax-weighted sum of
base value + up-projected value residual.  Used on tiny inputs only.
"""
from __future__ import annotations

import math
import struct


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _val(x, dtype):
    return float(x) if dtype == "f32" else _bf16(x)


def _lists(a):
    return a.tolist() if hasattr(a, "tolist") else a


def _slot_of(P, starts_a, t):
    """(logical page, row) of position t: page t // P, or under a slot map the last page
    whose start is <= t (linear scan)."""
    if starts_a is None:
        return divmod(t, P)
    j = 0
    for i, st in enumerate(starts_a):
        if 0 <= st <= t:
            j = i
    return j, t - starts_a[j]


def _key_value(P, d, r, dtype, bpool, rpool, btab_a, rtab_a, Bk_a, Bv_a, h, t, s, theta,
               row_override=None, starts_a=None):
    """Merged key and value of one agent/head at position t (lists of d floats), or None
    when the position's base page is missing (-1: evicted, so no key there).  A missing
    residual page contributes nothing (zero residual rows)."""
    lp, row = _slot_of(P, starts_a, t)
    if btab_a[lp] < 0:
        return None
    if row_override is not None:
        bk, bv, rk, rv = row_override
        if rtab_a[lp] < 0:  # the row's residual cannot be stored: zero residual
            rk, rv = [0.0] * r, [0.0] * r
    else:
        bp, rp = btab_a[lp], rtab_a[lp]
        # tiles are stored in matrix-core operand order (see include/forkkv.h)
        bk = [_val(bpool[bp][0][h][(j // 8) * 128 + row * 8 + j % 8], dtype) for j in range(d)]
        bv = [_val(bpool[bp][1][h][((j // 16) * 4 + row // 4) * 64 + (j % 16) * 4 + row % 4],
                   dtype) for j in range(d)]
        if rp < 0:
            rk, rv = [0.0] * r, [0.0] * r
        else:
            rk = [_val(rpool[rp][0][(k // 4) * 64 + row * 4 + k % 4], dtype) for k in range(r)]
            rv = [_val(rpool[rp][1][(row // 4) * 4 * r + k * 4 + row % 4], dtype)
                  for k in range(r)]
    half = d // 2
    key = [0.0] * d
    for j in range(half):
        w = theta ** (-(2.0 * j) / d)
        c, sn = math.cos(t * w), math.sin(t * w)
        # pre-RoPE base: rotate back by -t*w
        x1 = bk[j] * c + bk[j + half] * sn
        x2 = bk[j + half] * c - bk[j] * sn
        u1 = s * sum(rk[k] * _val(Bk_a[k][h * d + j], dtype) for k in range(r))
        u2 = s * sum(rk[k] * _val(Bk_a[k][h * d + j + half], dtype) for k in range(r))
        y1, y2 = x1 + u1, x2 + u2
        key[j] = y1 * c - y2 * sn
        key[j + half] = y2 * c + y1 * sn
    val = [bv[j] + s * sum(rv[k] * _val(Bv_a[k][h * d + j], dtype) for k in range(r))
           for j in range(d)]
    return key, val


def _attend(qrow, kv, sm_scale, d):
    kv = [x for x in kv if x is not None]
    if not kv:
        return [0.0] * d
    scores = [sm_scale * sum(qrow[j] * k[j] for j in range(d)) for k, _ in kv]
    m = max(scores)
    e = [math.exp(x - m) for x in scores]
    z = math.fsum(e)
    return [math.fsum(e[t] * kv[t][1][j] for t in range(len(kv))) / z for j in range(d)]


def brute_decode(P, Hq, Hkv, d, r, dtype, bpool, rpool, btab, rtab, seq_lens, q, Bk, Bv,
                 s, sm_scale, theta, starts=None):
    bpool, rpool, btab, rtab = map(_lists, (bpool, rpool, btab, rtab))
    starts = None if starts is None else _lists(starts)
    q, Bk, Bv = map(_lists, (q, Bk, Bv))
    G = Hq // Hkv
    out = []
    for a in range(len(q)):
        rows = []
        for g in range(Hq):
            h = g // G
            kv = [_key_value(P, d, r, dtype, bpool, rpool, btab[a], rtab[a], Bk[a], Bv[a], h, t,
                             s, theta, starts_a=None if starts is None else starts[a])
                  for t in range(int(seq_lens[a]))]
            qrow = [_val(x, dtype) for x in q[a][g]]
            rows.append(_attend(qrow, kv, sm_scale, d))
        out.append(rows)
    return out


def brute_prefill(P, Hq, Hkv, d, r, dtype, bpool, rpool, btab, rtab, start_pos, q, k_new,
                  v_new, rk_new, rv_new, Bk, Bv, s, sm_scale, theta):
    """Chunk rows are written at start_pos[a] + i, then query i attends to keys 0..start+i."""
    bpool, rpool, btab, rtab = map(_lists, (bpool, rpool, btab, rtab))
    q, k_new, v_new, rk_new, rv_new, Bk, Bv = map(_lists, (q, k_new, v_new, rk_new, rv_new, Bk, Bv))
    G = Hq // Hkv
    out = []
    for a in range(len(q)):
        start = int(start_pos[a])
        C = len(q[a])
        per_q = []
        for i in range(C):
            rows = []
            for g in range(Hq):
                h = g // G
                kv = []
                for t in range(start + i + 1):
                    ov = None
                    if t >= start:
                        j = t - start
                        ov = ([_val(x, dtype) for x in k_new[a][j][h]],
                              [_val(x, dtype) for x in v_new[a][j][h]],
                              [_val(x, dtype) for x in rk_new[a][j]],
                              [_val(x, dtype) for x in rv_new[a][j]])
                    kv.append(_key_value(P, d, r, dtype, bpool, rpool, btab[a], rtab[a], Bk[a],
                                         Bv[a], h, t, s, theta, row_override=ov))
                qrow = [_val(x, dtype) for x in q[a][i][g]]
                rows.append(_attend(qrow, kv, sm_scale, d))
            per_q.append(rows)
        out.append(per_q)
    return out


def brute_prefill_at(P, Hq, Hkv, d, r, dtype, bpool, rpool, btab, rtab, positions, q, k_new,
                     v_new, rk_new, rv_new, Bk, Bv, s, sm_scale, theta):
    """Rows are written at positions[a][i] (all of them first), then query i attends to keys
    0 .. positions[a][i]; positions strictly increase per agent."""
    bpool, rpool, btab, rtab = map(_lists, (bpool, rpool, btab, rtab))
    q, k_new, v_new, rk_new, rv_new, Bk, Bv = map(_lists, (q, k_new, v_new, rk_new, rv_new, Bk, Bv))
    G = Hq // Hkv
    out = []
    for a in range(len(q)):
        written = {int(t): j for j, t in enumerate(positions[a])}
        per_q = []
        for i in range(len(q[a])):
            rows = []
            for g in range(Hq):
                h = g // G
                kv = []
                for t in range(int(positions[a][i]) + 1):
                    ov = None
                    if t in written:
                        j = written[t]
                        ov = ([_val(x, dtype) for x in k_new[a][j][h]],
                              [_val(x, dtype) for x in v_new[a][j][h]],
                              [_val(x, dtype) for x in rk_new[a][j]],
                              [_val(x, dtype) for x in rv_new[a][j]])
                    kv.append(_key_value(P, d, r, dtype, bpool, rpool, btab[a], rtab[a], Bk[a],
                                         Bv[a], h, t, s, theta, row_override=ov))
                qrow = [_val(x, dtype) for x in q[a][i][g]]
                rows.append(_attend(qrow, kv, sm_scale, d))
            per_q.append(rows)
        out.append(per_q)
    return out
