"""Reading stored pool bytes as fp64 values (oracle side; test infrastructure).

Layout of the pools (fixed by this library; the pages leave it open):
base pool ``[page][plane][kv_head][P*d]`` with plane 0 = key tile ``[row][dim]``
and plane 1 = value tile ``[dim][row]``; residual pool ``[page][plane][P*r]``
with plane 0 = key residual ``[row][k]`` and plane 1 = value residual ``[k][row]``.
"""
from __future__ import annotations

import numpy as np


def decode_values(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored elements -> float64.  bf16 is stored as its 16-bit pattern."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(arr).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def _pages_rows(tab_row: np.ndarray, positions: np.ndarray, P: int):
    lp = positions // P
    return tab_row[lp].astype(np.int64), (positions % P).astype(np.int64)


def base_key_rows(bpool, btab_row, positions, head, P, d, dtype):
    """Stored (post-RoPE) base keys of one KV head at the given positions -> [L, d]."""
    pages, rows = _pages_rows(btab_row, positions, P)
    tiles = bpool[:, 0, head, :]
    idx = rows[:, None] * d + np.arange(d)[None, :]
    return decode_values(tiles[pages[:, None], idx], dtype)


def base_value_rows(bpool, btab_row, positions, head, P, d, dtype):
    """Base values of one KV head at the given positions -> [L, d]."""
    pages, rows = _pages_rows(btab_row, positions, P)
    tiles = bpool[:, 1, head, :]
    idx = np.arange(d)[None, :] * P + rows[:, None]
    return decode_values(tiles[pages[:, None], idx], dtype)


def res_key_rows(rpool, rtab_row, positions, P, r, dtype):
    """Rank-r key residuals (no RoPE) at the given positions -> [L, r]."""
    pages, rows = _pages_rows(rtab_row, positions, P)
    tiles = rpool[:, 0, :]
    idx = rows[:, None] * r + np.arange(r)[None, :]
    return decode_values(tiles[pages[:, None], idx], dtype)


def res_value_rows(rpool, rtab_row, positions, P, r, dtype):
    """Rank-r value residuals at the given positions -> [L, r]."""
    pages, rows = _pages_rows(rtab_row, positions, P)
    tiles = rpool[:, 1, :]
    idx = np.arange(r)[None, :] * P + rows[:, None]
    return decode_values(tiles[pages[:, None], idx], dtype)
