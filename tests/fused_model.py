"""CPU model of the fused ResidualAttention form (a diagnostic, not the oracle).

It restates, in numpy, the kernel-side algorithm the ForkKV study note describes
("7. 实现 cross-reference", core barrier (1)/(2); reproduction checks 3, 4 and 6
of "4. 作者证明"): keys are rebuilt page by page as base + RoPE(s * rK B_k);
scores go through an online softmax whose running max rescales *both* the base
accumulator ``acc`` and the residual accumulator ``acc_r``; B_v is applied once,
after the loop.  Pages are cut into arbitrary split-K partitions whose partial
results are merged with a log-sum-exp rule.  Tests check that this equals the
plain-definition oracle for every partition, and that skipping the ``acc_r``
rescale (``rescale_residual=False``) does not.
"""
from __future__ import annotations

import numpy as np

from oracle.rope import rope_rotate
from oracle.storage import (base_key_rows, base_value_rows, decode_values, res_key_rows,
                            res_value_rows)


def _partial(geo, bpool, rpool, btab_a, rtab_a, Bk_ah, qg, lp_range, L, s, sm_scale, theta,
             rescale_residual):
    m, l = -np.inf, 0.0
    acc = np.zeros(geo.d)
    acc_r = np.zeros(geo.r)
    for lp in lp_range:
        pos = np.arange(lp * geo.P, min((lp + 1) * geo.P, L))
        bk = base_key_rows(bpool, btab_a, pos, qg[1], geo.P, geo.d, geo.dtype)
        bv = base_value_rows(bpool, btab_a, pos, qg[1], geo.P, geo.d, geo.dtype)
        rk = res_key_rows(rpool, rtab_a, pos, geo.P, geo.r, geo.dtype)
        rv = res_value_rows(rpool, rtab_a, pos, geo.P, geo.r, geo.dtype)
        k = bk + rope_rotate(s * (rk @ Bk_ah), pos, theta)      # deferred RoPE
        sc = sm_scale * (k @ qg[0])
        m_new = max(m, float(sc.max()))
        alpha = np.exp(m - m_new) if np.isfinite(m) else 0.0
        p = np.exp(sc - m_new)
        l = alpha * l + p.sum()
        acc = alpha * acc + p @ bv
        acc_r = (alpha * acc_r if rescale_residual else acc_r) + p @ rv
        m = m_new
    return m, l, acc, acc_r


def fused_decode(geo, bpool, rpool, btab, rtab, seq_lens, q, Bk, Bv, s, sm_scale, theta,
                 splits, rescale_residual=True):
    """splits(a, n_pages) -> list of page-index ranges covering 0..n_pages-1."""
    qv = decode_values(q, geo.dtype)
    Bkv, Bvv = decode_values(Bk, geo.dtype), decode_values(Bv, geo.dtype)
    N = q.shape[0]
    out = np.zeros((N, geo.Hq, geo.d))
    for a in range(N):
        L = int(seq_lens[a])
        n_pages = -(-L // geo.P)
        parts = splits(a, n_pages)
        for g in range(geo.Hq):
            h = g // geo.G
            cols = slice(h * geo.d, (h + 1) * geo.d)
            res = [_partial(geo, bpool, rpool, btab[a], rtab[a], Bkv[a][:, cols], (qv[a, g], h),
                            rng, L, s, sm_scale, theta, rescale_residual) for rng in parts]
            res = [x for x in res if x[1] > 0]
            if not res:
                continue
            M = max(x[0] for x in res)
            w = [np.exp(x[0] - M) for x in res]
            Lsum = sum(wi * x[1] for wi, x in zip(w, res))
            A = sum(wi * x[2] for wi, x in zip(w, res))
            Ar = sum(wi * x[3] for wi, x in zip(w, res))
            out[a, g] = (A + s * (Ar @ Bvv[a][:, cols])) / Lsum   # B_v applied once
    return out
