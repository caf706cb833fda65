"""Reading stored pool bytes as fp64 values (oracle side; test infrastructure).

Pool layout (fixed by this library; the pages leave it open).  A base page is
``[plane][kv_head][P*d]`` elements, a residual page ``[plane][P*r]``, with P = 16.
Inside a tile the elements sit in the order the gfx950 matrix cores consume them:

* base key   (row t, dim x):  ``(x // 8) * (16 * 8) + t * 8 + x % 8``
* base value (row t, dim x):  ``((x // 16) * 4 + t // 4) * 64 + (x % 16) * 4 + t % 4``
* key residual   (row t, rank k): ``(k // 4) * (16 * 4) + t * 4 + k % 4``
* value residual (row t, rank k): ``(t // 4) * (4 * r) + k * 4 + t % 4``

so d must be a multiple of 16 and r a multiple of 4.
"""
from __future__ import annotations

import numpy as np

P = 16


def decode_values(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored elements -> float64.  bf16 is stored as its 16-bit pattern."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(arr).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def key_offset(t, x):
    return (x // 8) * (P * 8) + t * 8 + x % 8


def value_offset(t, x):
    return ((x // 16) * 4 + t // 4) * 64 + (x % 16) * 4 + t % 4


def res_key_offset(t, k):
    return (k // 4) * (P * 4) + t * 4 + k % 4


def res_value_offset(t, k, r):
    return (t // 4) * (4 * r) + k * 4 + t % 4


def _pages_rows(tab_row: np.ndarray, positions: np.ndarray, P_: int, starts_row=None):
    """Physical page and row of each position.  Without a slot map page lp holds positions
    lp*P .. lp*P + P-1; with one (``starts_row``: start position of each logical page, -1
    padded) page lp holds the positions from its start up to the next page's start."""
    positions = np.asarray(positions, dtype=np.int64)
    if starts_row is None:
        lp = positions // P_
        return np.asarray(tab_row)[lp].astype(np.int64), (positions % P_).astype(np.int64)
    st = np.asarray([s for s in starts_row if s >= 0], dtype=np.int64)
    lp = np.searchsorted(st, positions, side="right") - 1
    return np.asarray(tab_row)[lp].astype(np.int64), (positions - st[lp]).astype(np.int64)


def table_pages(tab_row, positions, P_, starts_row=None):
    """Table entry (physical page, or -1 for a missing page) of each position."""
    return _pages_rows(tab_row, positions, P_, starts_row)[0]


def _readable(pages_rows):
    """Missing pages (-1) are read as page 0 here; callers discard or zero those rows."""
    pages, rows = pages_rows
    return np.maximum(pages, 0), rows


def base_key_rows(bpool, btab_row, positions, head, P_, d, dtype, starts_row=None):
    """Stored (post-RoPE) base keys of one KV head at the given positions -> [L, d]."""
    pages, rows = _readable(_pages_rows(btab_row, positions, P_, starts_row))
    idx = key_offset(rows[:, None], np.arange(d)[None, :])
    return decode_values(bpool[:, 0, head, :][pages[:, None], idx], dtype)


def base_value_rows(bpool, btab_row, positions, head, P_, d, dtype, starts_row=None):
    """Base values of one KV head at the given positions -> [L, d]."""
    pages, rows = _readable(_pages_rows(btab_row, positions, P_, starts_row))
    idx = value_offset(rows[:, None], np.arange(d)[None, :])
    return decode_values(bpool[:, 1, head, :][pages[:, None], idx], dtype)


def res_key_rows(rpool, rtab_row, positions, P_, r, dtype, starts_row=None):
    """Rank-r key residuals (no RoPE) at the given positions -> [L, r]."""
    pages, rows = _readable(_pages_rows(rtab_row, positions, P_, starts_row))
    idx = res_key_offset(rows[:, None], np.arange(r)[None, :])
    return decode_values(rpool[:, 0, :][pages[:, None], idx], dtype)


def res_value_rows(rpool, rtab_row, positions, P_, r, dtype, starts_row=None):
    """Rank-r value residuals at the given positions -> [L, r]."""
    pages, rows = _readable(_pages_rows(rtab_row, positions, P_, starts_row))
    idx = res_value_offset(rows[:, None], np.arange(r)[None, :], r)
    return decode_values(rpool[:, 1, :][pages[:, None], idx], dtype)
