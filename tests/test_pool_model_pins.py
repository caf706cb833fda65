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
from oracle.pool_model import AUTO, FREEZE, PACK
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


# ---- freeze-tail (ForkServe README, "Design vs APC": the adaptive unaligned tail) ---------

@pytest.mark.parametrize("L,k,ell", [(2050, 4, 48), (37, 3, 5), (100, 2, 60), (31, 5, 1),
                                     (4097, 8, 128)])
def test_freeze_formula_for_unaligned_tail(L, k, ell):
    """pages_freeze = 1 + k * ceil(l / P): one read-only tail shared by the trunk and every
    child, plus each child's own pages; the trunk's full pages are aliased as before."""
    P = 16
    pm = PoolModel(4096, 8192)
    names = pm.replay(fanout_ops(L, k, ell, FREEZE))
    assert pm.stats()["live_bpages"] == L // P + 1 + k * (-(-ell // P))
    # the frozen tail is one page, mapped by the trunk and all k children
    tail_page = pm.tables([names["trunk"]], -(-L // P))[0][0][L // P]
    assert pm.ref_b[tail_page] == k + 1
    # the same fan-out packed costs pages_pack instead (the printed scenario row: 145)
    pk = PoolModel(4096, 8192)
    pk.replay(fanout_ops(L, k, ell, PACK))
    assert pk.stats()["live_bpages"] == -(-L // P) + k * (-(-((L % P) + ell) // P))
    if (L, k, ell) == (2050, 4, 48):
        assert pk.stats()["live_bpages"] == 145


@pytest.mark.parametrize("L,k,ell", [(2050, 4, 10), (2050, 4, 14), (2050, 4, 15), (2061, 3, 6),
                                     (2061, 3, 40), (2063, 6, 2)])
def test_adaptive_tail_rule(L, k, ell):
    """AUTO packs when the trunk tail and the child's suffix fit in one page (r + l <= P),
    else freezes: the live page count follows the matching formula."""
    P, r = 16, L % 16
    pm = PoolModel(4096, 8192)
    pm.replay(fanout_ops(L, k, ell, AUTO, ell))
    # pack: the trunk keeps its partial page and each child copies r rows into its own;
    # freeze: that partial page is the one shared read-only tail
    want = (1 + k * (-(-(r + ell) // P)) if r + ell <= P else 1 + k * (-(-ell // P)))
    assert pm.stats()["live_bpages"] == L // P + want


def test_freeze_slot_map_covers_each_position_once():
    """After a freeze fork, positions 0 .. len-1 of every sequence map one to one onto
    (page, row) slots: the frozen tail holds r rows, later pages start at r-shifted
    positions, and no slot is used by two positions of one sequence."""
    P = 16
    pm = PoolModel(256, 512)
    names = pm.replay(fanout_ops(37, 3, 21, FREEZE))
    names["gc"], _ = pm.fork(names["c1"], 37 + 21)  # a grandchild at the child's end (aligned? no)
    pm.append(names["gc"], 9)
    pm.append(names["trunk"], 5)  # the trunk continues after its own frozen tail
    for nm in ("trunk", "c0", "c1", "c2", "gc"):
        h = names[nm]
        s = pm.seqs[h]
        starts = pm.starts_table([h], 8)[0]
        L = pm.length(h)
        slots = set()
        for t in range(L):
            j = max(i for i, st in enumerate(starts) if 0 <= st <= t)
            row = t - starts[j]
            assert 0 <= row < s.rows(j) <= P
            slots.add((s.bpages[j], row))
        assert len(slots) == L
        assert starts[:3] == [0, 16, 32]
        if nm != "gc" and L > 37:
            assert starts[3] == 37  # the row after the frozen 5-row tail opens a page
    # the trunk's tail page is read-only: its own append opened a page at position 37
    assert pm.seqs[names["trunk"]].rows(2) == 5


def test_freeze_only_at_the_parents_end():
    pm = PoolModel(64, 64)
    names = pm.replay([("create", "t", 0), ("append", "t", 40)])
    with pytest.raises(PoolError) as e:
        pm.fork(names["t"], 37, FREEZE)
    assert e.value.kind == "EINVAL"
    c, cow = pm.fork(names["t"], 37, AUTO, 40)  # AUTO cannot freeze there: it packs
    assert cow == (pm.seqs[names["t"]].bpages[2], pm.seqs[c].bpages[2], 5)


# ---- decoupled eviction (ForkKV study note: "Error / eviction recovery", trick 1) --------

def test_base_eviction_keeps_residuals_and_refill_restores_sharing():
    """Evicting the trunk's base pages leaves every agent's residual pages live (the two
    pools are evicted independently); the agents hold -1 there, cannot append or fork
    until refilled, and a refill maps one fresh page per logical page into all of them."""
    P = 16
    pm = PoolModel(64, 128)
    names = pm.replay(fanout_ops(64, 3, 20))
    kids = [names[f"c{j}"] for j in range(3)]
    before = pm.stats()
    bt0, rt0, lens0 = pm.tables(kids, 8)
    victims = bt0[0][1:3]  # two shared trunk pages
    pm.evict_base(victims)
    st = pm.stats()
    assert st["live_rpages"] == before["live_rpages"] and st["rpage_refs"] == before["rpage_refs"]
    assert st["live_bpages"] == before["live_bpages"] - 2
    assert list(pm.free_b)[-2:] == list(victims)
    bt1, rt1, lens1 = pm.tables(kids, 8)
    assert rt1 == rt0 and lens1 == lens0
    for row in bt1:
        assert row[1:3] == [-1, -1]
    for h in kids:
        with pytest.raises(PoolError) as e:
            pm.append(h, 1)
        assert e.value.kind == "ESTATE"
    with pytest.raises(PoolError) as e:
        pm.fork(kids[0], 40)
    assert e.value.kind == "ESTATE"
    pm.fork(kids[0], 16)  # below the evicted range: fine
    # the trunk (base-only snapshot) lost them too; refill the three agents and the trunk
    new = pm.refill_base(kids + [names["trunk"]], 1, 3)
    assert len(new) == 2 and all(pm.ref_b[pg] == 4 for pg in new)
    bt2, _, _ = pm.tables(kids, 8)
    for row, row0 in zip(bt2, bt0):
        assert row[:1] + row[3:] == row0[:1] + row0[3:] and row[1:3] == new
    pm.append(kids[1], 3)


def test_eviction_errors():
    pm = PoolModel(32, 32)
    names = pm.replay(fanout_ops(32, 2, 4))
    kids = [names["c0"], names["c1"]]
    with pytest.raises(PoolError):
        pm.evict_base([31 if pm.ref_b[31] == 0 else 30])  # a free page
    pg = pm.tables([kids[0]], 4)[0][0][0]
    with pytest.raises(PoolError):
        pm.evict_base([pg, pg])
    with pytest.raises(PoolError):
        pm.refill_base(kids, 0, 1)  # nothing evicted there
    pm.evict_base([pg])
    with pytest.raises(PoolError):
        pm.refill_base(kids, 0, 2)  # page 1 is still mapped
    st = pm.stats()
    assert pm.refill_base(kids, 0, 1) and pm.stats()["live_bpages"] == st["live_bpages"] + 1
