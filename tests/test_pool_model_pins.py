"""Pins of the oracle's bookkeeping model (CPU only).

* ForkServe README, "Results" table: live frame counts for six fan-out
  scenarios, with sharing (FS) and with per-child clones (APC), P = 16.
* ForkServe README, "Design vs APC" / "Methods": M_CoW = b(L + sum l_i) versus
  M_clone = b(kL + sum l_i); the ``pages_pack`` formula for unaligned tails.
* ForkKV study note, "4. 作者证明": M_R = 1/N + r/n and reproduction checks 1-2.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

from oracle import PoolError, PoolModel
from tests.pool_scenarios import clone_ops, fanout_ops, read_kv, read_table

TABLE = read_table("forkserve_results_table.txt")


@pytest.mark.parametrize("row", TABLE, ids=[r[0] for r in TABLE])
def test_forkserve_results_table(row):
    name, L, k, ell, apc, fs, save, apc_gib, fs_gib = row
    L, k, ell, apc, fs = map(int, (L, k, ell, apc, fs))
    pm = PoolModel(1 << 16, 1 << 17)
    pm.replay(fanout_ops(L, k, ell))
    assert pm.stats()["live_bpages"] == fs
    cl = PoolModel(1 << 16, 1)
    cl.replay(clone_ops(L, k, ell))
    assert cl.stats()["live_bpages"] == apc
    # derived columns, as printed
    assert f"{100 * (1 - fs / apc):.1f}" == save
    gib = lambda blk: blk * 16 * 128 * 1024 / 2 ** 30
    assert f"{gib(apc):.2f}" == apc_gib and f"{gib(fs):.2f}" == fs_gib


@pytest.mark.parametrize("L,k,ell", [(2050, 4, 48), (37, 3, 5), (100, 2, 60)])
def test_pack_formula_for_unaligned_tail(L, k, ell):
    """pages_pack = k * ceil((L mod P + l) / P) private pages; the trunk keeps its pages."""
    P = 16
    pm = PoolModel(4096, 8192)
    pm.replay(fanout_ops(L, k, ell))
    trunk = -(-L // P)
    assert pm.stats()["live_bpages"] == trunk + k * (-(-((L % P) + ell) // P))


@pytest.mark.parametrize("L,k,ells", [(2048, 4, [64, 16, 32, 128]), (512, 3, [16, 0, 48])])
def test_cow_vs_clone_live_tokens(L, k, ells):
    """Aligned sizes: live capacity is exactly L + sum(l_i) (CoW) vs kL + sum(l_i) (clone)."""
    pm = PoolModel(4096, 8192)
    names = pm.replay([("create", "t", 0), ("append", "t", L)])
    kids = [pm.fork(names["t"], L)[0] for _ in range(k)]
    for h, e in zip(kids, ells):
        pm.append(h, e)
    assert pm.stats()["live_bpages"] * 16 == L + sum(ells)
    cl = PoolModel(4096, 1)
    for e in ells:
        h = cl.create(False)
        cl.append(h, L + e)
    assert cl.stats()["live_bpages"] * 16 == k * L + sum(ells)


def test_memory_ratio_equation_and_example():
    """M_R = (s n + N s r) / (N s n) = 1/N + r/n, in integer bytes from the model's page counts."""
    ex = read_kv("forkkv_memory_example.txt")
    N, s, n, r, layers, e = (ex["agents"], ex["tokens"], ex["n"], ex["r"], ex["layers"],
                             ex["elem_bytes"])
    pm = PoolModel(s // 16 + 8, N * s // 16 + 8)
    names = pm.replay([("create", "root", 0), ("append", "root", s)] +
                      [("fork", "root", s, f"a{j}") for j in range(N)])
    st = pm.stats()
    base_bytes = st["live_bpages"] * 16 * 2 * n * e * layers
    res_bytes = st["live_rpages"] * 16 * 2 * r * e * layers
    unified = N * s * 2 * n * e * layers
    ratio = Fraction(base_bytes + res_bytes, unified)
    assert ratio == Fraction(1, N) + Fraction(r, n)
    assert unified == ex["unified_gib"] * 2 ** 30
    assert base_bytes + res_bytes == ex["disaggregated_gib"] * 2 ** 30
    assert base_bytes == ex["bcache_gib"] * 2 ** 30
    assert res_bytes // N == ex["rcache_mib"] * 2 ** 20
    assert Fraction(base_bytes, res_bytes // N) == ex["size_ratio"] == n // r
    # check 1: decreasing in N, increasing in r
    mr = lambda N_, r_: Fraction(1, N_) + Fraction(r_, n)
    assert mr(2, 16) > mr(4, 16) > mr(16, 16) and mr(16, 8) < mr(16, 16) < mr(16, 32)


def _invariants(pm: PoolModel):
    live = [s for s in pm.seqs if s.alive]
    refs_b = [0] * pm.nb
    refs_r = [0] * pm.nr
    for s in live:
        for p in s.bpages:
            refs_b[p] += 1
        for p in s.rpages:
            refs_r[p] += 1
        assert len(s.bpages) == -(-s.length // pm.P)
        assert len(s.rpages) == (len(s.bpages) if s.has_res else 0)
    assert refs_b == pm.ref_b and refs_r == pm.ref_r
    assert len(set(pm.free_b)) == len(pm.free_b) and len(set(pm.free_r)) == len(pm.free_r)
    assert all(pm.ref_b[p] == 0 for p in pm.free_b) and all(pm.ref_r[p] == 0 for p in pm.free_r)
    assert len(pm.free_b) + sum(1 for c in pm.ref_b if c) == pm.nb
    assert len(pm.free_r) + sum(1 for c in pm.ref_r if c) == pm.nr


@pytest.mark.parametrize("seed", range(8))
def test_random_operations_keep_invariants(seed):
    rng = np.random.default_rng(seed)
    pm = PoolModel(48, 64, 16, rng.permutation(48), rng.permutation(64))
    live = []
    for _ in range(300):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                live.append(pm.create(bool(rng.integers(0, 2))))
            elif op == 1:
                h = live[rng.integers(len(live))]
                pm.append(h, int(rng.integers(0, 40)))
            elif op == 2:
                h = live[rng.integers(len(live))]
                c, _ = pm.fork(h, int(rng.integers(0, pm.length(h) + 1)))
                live.append(c)
            else:
                h = live.pop(rng.integers(len(live)))
                pm.free(h)
        except PoolError as e:
            assert e.kind == "ENOMEM"
        _invariants(pm)


def test_failures_leave_state_unchanged():
    pm = PoolModel(4, 4)
    h = pm.create(True)
    pm.append(h, 40)                    # 3 pages of 4
    before = (list(pm.free_b), list(pm.free_r), list(pm.ref_b), list(pm.ref_r))
    with pytest.raises(PoolError) as e:
        pm.append(h, 30)                # needs 2 more
    assert e.value.kind == "ENOMEM"
    with pytest.raises(PoolError) as e:
        pm.fork(h, 40)                  # needs 3 residual pages, 1 free
    assert e.value.kind == "ENOMEM"
    with pytest.raises(PoolError) as e:
        pm.fork(h, 41)
    assert e.value.kind == "EINVAL"
    assert before == (list(pm.free_b), list(pm.free_r), list(pm.ref_b), list(pm.ref_r))
    pm.free(h)
    with pytest.raises(PoolError):
        pm.free(h)


def test_free_parent_keeps_trunk_and_order():
    """ForkServe "Status": freeing the parent does not drop the trunk the children alias."""
    pm = PoolModel(16, 32)
    t = pm.create(False)
    pm.append(t, 64)
    c, _ = pm.fork(t, 64)
    pm.free(t)
    assert pm.stats()["live_bpages"] == 4 and list(pm.free_b) == list(range(4, 16))
    pm.free(c)
    assert list(pm.free_b)[-4:] == [0, 1, 2, 3]
