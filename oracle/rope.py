"""Rotary position embedding in fp64 (oracle side; test infrastructure).

The pages never spell RoPE out; the ForkKV note only says that RoPE is applied
to the base cache and must be deferred for the residual until after the
up-projection (section "3. 架构 / 方法图", reproduction check 3 in "4. 作者证明").
Reading taken: the rotate-half form used by the Llama and Qwen attention layers
the workloads are shaped after -- dimension j is paired with j + d/2 and rotated
by the angle ``t * theta**(-2j/d)``.
"""
from __future__ import annotations

import numpy as np


def inv_freq(d: int, theta: float) -> np.ndarray:
    j = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / d)


def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Apply R_t to each row of x ([..., L, d]) at positions t ([L])."""
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq(d, theta)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_unrotate(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Apply R_t^T (= R_{-t}) to each row: recovers the pre-RoPE vector."""
    return rope_rotate(x, -np.asarray(positions, dtype=np.float64), theta)
