"""Operation scripts for the ForkServe README's fan-out scenarios (shared by CPU tests)."""
from __future__ import annotations

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def read_kv(name):
    out = {}
    for k, v in read_table(name):
        out[k] = int(v)
    return out


def fanout_ops(L, k, ell, mode=None, hint=0):
    """Snapshot the trunk (base-only), fork k children at L, each writes ell tokens.
    ``mode`` (pool_model.PACK / FREEZE / AUTO, with ``hint``) selects the unaligned-tail
    treatment; None is the default (pack)."""
    ops = [("create", "trunk", 0), ("append", "trunk", L)]
    for j in range(k):
        ops.append(("fork", "trunk", L, f"c{j}") + (() if mode is None else (mode, hint)))
    for j in range(k):
        ops.append(("append", f"c{j}", ell))
    return ops


def clone_ops(L, k, ell):
    """Every child holds its own copy of trunk + residual (no sharing)."""
    ops = []
    for j in range(k):
        ops.append(("create", f"c{j}", 0))
        ops.append(("append", f"c{j}", L + ell))
    return ops
