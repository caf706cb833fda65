"""libforkkv's host bookkeeping against the oracle's pool model, bit for bit (CPU only).

Tables, reference counts, free-list order, slots, copy-on-write row copies and
error behaviour must be identical; the plan's work list must cover every
(agent, page) exactly once with agents that really share the page.
"""
from __future__ import annotations

import numpy as np
import pytest

from lora_shared_prefix_amd import forkkv as fk
from oracle import PoolError, PoolModel
from tests.pool_scenarios import fanout_ops, read_table
from workloads import CONFIGS, chunk_ops, config_by_name, pool_ops

ITEM_INTS = 20   # lp0, pages, agents, unused, 8 agent ids, 8 slot ids


def _pair(nb, nr, perm_b=None, perm_r=None, Hkv=1, d=16, r=4):
    lib_pool = fk.Pool(nb, nr, Hkv, d, r, "f32", perm_b, perm_r)
    model = PoolModel(nb, nr, 16, perm_b, perm_r)
    return lib_pool, model


def _same_state(lp: fk.Pool, pm: PoolModel, handles):
    assert lp.free_list(0) == list(pm.free_b)
    assert lp.free_list(1) == list(pm.free_r)
    assert lp.refcounts(0) == pm.ref_b
    assert lp.refcounts(1) == pm.ref_r
    st = lp.stats()
    ms = pm.stats()
    for k, v in ms.items():
        assert st[k] == v, k
    if handles:
        mp = max(1, max(len(pm.seqs[h].bpages) for h in handles))
        assert lp.tables(handles, mp) == tuple(map(list, pm.tables(handles, mp)))


def _replay_both(lp, pm, ops):
    names_l, cows_l = lp.replay(ops)
    names_m, cows_m = {}, []
    for op in ops:
        if op[0] == "create":
            names_m[op[1]] = pm.create(bool(op[2]))
        elif op[0] == "append":
            _, _, c = pm.append(names_m[op[1]], op[2])
            if c:
                cows_m.append(c)
        else:
            names_m[op[3]], c = pm.fork(names_m[op[1]], op[2])
            if c:
                cows_m.append(c)
    assert names_l == names_m and cows_l == cows_m
    return names_l


@pytest.mark.parametrize("name", [c.name for c in CONFIGS])
def test_workload_topologies_match_model(name):
    cfg = config_by_name(name)
    rng = np.random.default_rng(cfg.seed)
    pb = rng.permutation(cfg.num_bpages)
    pr = rng.permutation(cfg.num_rpages)
    lp, pm = _pair(cfg.num_bpages, cfg.num_rpages, pb, pr)
    ops, agents = pool_ops(cfg)
    names = _replay_both(lp, pm, ops + chunk_ops(cfg, agents))
    _same_state(lp, pm, [names[a] for a in agents])


@pytest.mark.parametrize("row", read_table("forkserve_results_table.txt"), ids=lambda r: r[0])
def test_forkserve_scenarios_match_model(row):
    L, k, ell, fs = int(row[1]), int(row[2]), int(row[3]), int(row[5])
    lp, pm = _pair(1 << 15, 1 << 16)
    names = _replay_both(lp, pm, fanout_ops(L, k, ell))
    _same_state(lp, pm, list(names.values()))
    assert lp.stats()["live_bpages"] == fs


@pytest.mark.parametrize("seed", range(10))
def test_random_operations_match_model(seed):
    rng = np.random.default_rng(1000 + seed)
    nb, nr = 40, 56
    lp, pm = _pair(nb, nr, rng.permutation(nb), rng.permutation(nr))
    live = []
    for step in range(250):
        op = int(rng.integers(0, 5))
        if op == 0 or not live:
            res = bool(rng.integers(0, 2))
            h = lp.create(res)
            assert h == pm.create(res)
            live.append(h)
        elif op in (1, 2):
            h = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, 37))
            try:
                exp = pm.append(h, n)
            except PoolError as e:
                with pytest.raises(fk.ForkKVError) as ei:
                    lp.append(h, n)
                assert ei.value.code == fk.ENOMEM and e.kind == "ENOMEM"
            else:
                got = lp.append(h, n)
                assert (got[0], got[1], got[2]) == (exp[0], exp[1], exp[2])
        elif op == 3:
            h = live[int(rng.integers(len(live)))]
            alias = int(rng.integers(0, pm.length(h) + 1))
            try:
                exp = pm.fork(h, alias)
            except PoolError as e:
                with pytest.raises(fk.ForkKVError) as ei:
                    lp.fork(h, alias)
                assert ei.value.code == fk.ENOMEM and e.kind == "ENOMEM"
            else:
                assert lp.fork(h, alias) == exp
                live.append(exp[0])
        else:
            h = live.pop(int(rng.integers(len(live))))
            lp.free(h)
            pm.free(h)
        _same_state(lp, pm, live)


def test_error_codes():
    lp = fk.Pool(4, 4, 1, 16, 4, "f32")
    h = lp.create(True)
    lp.append(h, 40)
    with pytest.raises(fk.ForkKVError) as e:
        lp.append(h, 30)
    assert e.value.code == fk.ENOMEM
    with pytest.raises(fk.ForkKVError) as e:
        lp.fork(h, 41)
    assert e.value.code == fk.EINVAL
    with pytest.raises(fk.ForkKVError) as e:
        lp.append(h, -1)
    assert e.value.code == fk.EINVAL
    lp.free(h)
    with pytest.raises(fk.ForkKVError) as e:
        lp.free(h)
    assert e.value.code == fk.EINVAL
    with pytest.raises(fk.ForkKVError) as e:
        fk.Pool(4, 4, 1, 16, 4, "f32", bpage_order=[0, 1, 1, 2])
    assert e.value.code == fk.EINVAL
    for d, r in [(7, 4), (24, 4), (16, 6), (16, 0), (272, 4)]:
        with pytest.raises(fk.ForkKVError):   # d % 16, r % 4 and ranges
            fk.Pool(4, 4, 1, d, r, "f32")
    # device call on a host-only pool
    with pytest.raises(fk.ForkKVError) as e:
        lp.cow_copy([(0, 1, 3)], stream=type("S", (), {"cuda_stream": 0})())
    assert e.value.code == fk.ESTATE


# ---- decode plan validity ------------------------------------------------------------------

def _check_plan(lp: fk.Pool, pm_tables, handles, plan: fk.Plan, group_cap):
    blob = plan.blob()
    n_agents, n_items, n_slots = blob[1], blob[2], blob[3]
    off_items, off_lens, off_ptr, off_list = blob[6], blob[7], blob[8], blob[9]
    bt, rt, lens = pm_tables
    assert n_agents == len(handles)
    assert blob[off_lens:off_lens + n_agents] == list(lens)
    covered = {}
    slots_seen = set()
    per_agent = {a: [] for a in range(n_agents)}
    for i in range(n_items):
        it = blob[off_items + i * ITEM_INTS: off_items + (i + 1) * ITEM_INTS]
        lp0, npg, na = it[:3]
        agents = it[4:4 + na]
        slots = it[12:12 + na]
        assert 1 <= na <= group_cap and npg >= 1 and agents == sorted(agents)
        for a, sl in zip(agents, slots):
            assert sl not in slots_seen
            slots_seen.add(sl)
            per_agent[a].append(sl)
        for lpg in range(lp0, lp0 + npg):
            pages = {bt[a][lpg] for a in agents}
            assert len(pages) == 1 and -1 not in pages
            for a in agents:
                assert (a, lpg) not in covered
                covered[(a, lpg)] = i
    want = {(a, lpg) for a in range(n_agents) for lpg in range(-(-lens[a] // 16))}
    assert set(covered) == want
    # read once: a physical base page held by n agents of the batch is streamed by exactly
    # ceil(n / cap) items (one per chunk of at most cap agents), per KV head -- a planner that
    # split the agents sharing a page any further would pass the coverage checks above and
    # show only as extra HBM traffic
    cap = blob[11]
    assert 1 <= cap <= group_cap
    holders, items_of = {}, {}
    for (a, lpg), i in covered.items():
        page = bt[a][lpg]
        holders.setdefault(page, set()).add(a)
        items_of.setdefault(page, set()).add(i)
    for page, hs_ in holders.items():
        assert len(items_of[page]) == -(-len(hs_) // cap), (page, len(hs_), cap)
    # decode with append: the last-page section holds each agent's last logical page (the
    # kernels store the new token there, at row length - 1 - page start); word 3 of an item
    # flags the items that hold one of their agents' last pages (only those store)
    off_last = blob[12]
    for i in range(n_items):
        it = blob[off_items + i * ITEM_INTS: off_items + (i + 1) * ITEM_INTS]
        lp0, npg, na = it[:3]
        holds = any(lp0 <= -(-lens[a] // 16) - 1 < lp0 + npg for a in it[4:4 + na] if lens[a] > 0)
        assert it[3] == int(holds), (i, it[:4])
    for a in range(n_agents):
        assert blob[off_last + a] == (-(-lens[a] // 16) - 1 if lens[a] > 0 else -1)
    # capacities: the items section has room for item_capacity items, zero past n_items
    item_cap, slot_cap = blob[13], blob[14]
    assert item_cap >= n_items and slot_cap >= n_slots
    assert off_lens == off_items + item_cap * ITEM_INTS
    assert all(v == 0 for v in blob[off_items + n_items * ITEM_INTS:off_lens])
    # the partial slots of each agent are exactly the range slot_ptr[a] .. slot_ptr[a+1]
    assert blob[off_ptr] == 0 and off_list == off_ptr + n_agents + 1
    for a in range(n_agents):
        ptr0, ptr1 = blob[off_ptr + a], blob[off_ptr + a + 1]
        assert sorted(per_agent[a]) == list(range(ptr0, ptr1))
    assert slots_seen == set(range(n_slots))


@pytest.mark.parametrize("name,kernel", [("tiny_f32", fk.KERNEL_GENERIC), ("llama3_8b_react_decode", fk.KERNEL_GENERIC),
                                         ("llama3_8b_mapreduce_decode", fk.KERNEL_GENERIC),
                                         ("qwen25_14b_batched_decode", fk.KERNEL_GENERIC), ("llama3_8b_react_decode", fk.KERNEL_MFMA),
                                         ("llama3_8b_mapreduce_decode", fk.KERNEL_MFMA), ("qwen25_14b_batched_decode", fk.KERNEL_MFMA)])
def test_plan_covers_workloads(name, kernel):
    cfg = config_by_name(name)
    lp = fk.Pool(cfg.num_bpages, cfg.num_rpages, cfg.num_kv_heads, cfg.head_dim, cfg.rank,
                 cfg.dtype)
    ops, agents = pool_ops(cfg)
    names, _ = lp.replay(ops)
    hs = [names[a] for a in agents]
    plan = fk.Plan(lp, hs, cfg.num_q_heads, kernel=kernel)
    mp = -(-cfg.seq_len // 16)
    # shared pages are read once per agent chunk, not once per agent
    blob = plan.blob()
    items = [blob[16 + i * ITEM_INTS: 16 + (i + 1) * ITEM_INTS] for i in range(blob[2])]
    cap = 8
    if kernel == fk.KERNEL_MFMA:
        # the largest item whose agent groups (A agents each) split four waves evenly
        A = min(4, 16 // cfg.group)
        cap = max(k * A for k in (1, 2, 4) if k * A <= 8)
    assert blob[11] == cap
    _check_plan(lp, lp.tables(hs, mp), hs, plan, cap)
    assert max(it[2] for it in items) == min(cfg.agents_per_session, cap)
    if kernel == fk.KERNEL_MFMA:
        # four waves per item: agents in groups of A = min(4, 16 // G), pages split over the
        # remaining waves; no wave may get more than 64 pages, and the grid fits one round
        A = min(4, 16 // cfg.group)
        waves = 0
        for it in items:
            n_sub = 4 // (-(-it[2] // A))
            assert -(-it[1] // n_sub) <= 64
            waves += 4
        assert waves * cfg.num_kv_heads <= 2048 or cfg.name.startswith("qwen25")


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("cap,ppi", [(0, 0), (2, 1), (3, 5)])
def test_plan_random_topologies(seed, cap, ppi):
    from tests.cases import random_ops
    rng = np.random.default_rng(2000 + seed)
    ops, agents = random_ops(rng, 5, max_prefix=90, max_suffix=50)
    lp = fk.Pool(128, 128, 2, 16, 4, "f32", rng.permutation(128), rng.permutation(128))
    names, _ = lp.replay(ops)
    hs = [names[a] for a in agents]
    plan = fk.Plan(lp, hs, 4, kernel=fk.KERNEL_GENERIC, max_agents_per_item=cap, pages_per_item=ppi)
    _check_plan(lp, lp.tables(hs, 16), hs, plan, cap if cap else 8)


def test_plan_rejects_base_only_and_bad_heads():
    lp = fk.Pool(8, 8, 2, 16, 4, "f32")
    root = lp.create(False)
    lp.append(root, 20)
    with pytest.raises(fk.ForkKVError):
        fk.Plan(lp, [root], 4)
    c, _ = lp.fork(root, 20)
    with pytest.raises(fk.ForkKVError):
        fk.Plan(lp, [c], 3)
    p = fk.Plan(lp, [], 4)
    assert p.info["n_items"] == 0


# ---- freeze-tail forks, the slot map, base eviction and refill --------------------------

_KIND = {"EINVAL": fk.EINVAL, "ENOMEM": fk.ENOMEM, "ESTATE": fk.ESTATE}


def _both(lp_call, pm_call):
    """Run the same operation on the library and the model: same result or same error."""
    try:
        exp = pm_call()
    except PoolError as e:
        with pytest.raises(fk.ForkKVError) as ei:
            lp_call()
        assert ei.value.code == _KIND[e.kind], (e.kind, ei.value.code)
        return None, False
    got = lp_call()
    return (got, exp), True


def _same_starts(lp, pm, handles):
    if handles:
        mp = max(1, max(len(pm.seqs[h].bpages) for h in handles))
        got, aligned = lp.starts(handles, mp)
        exp = pm.starts_table(handles, mp)
        assert got == exp
        assert aligned == all(row[j] == 16 * j for row in exp for j in range(mp) if row[j] >= 0)


@pytest.mark.parametrize("seed", range(12))
def test_random_freeze_evict_refill_match_model(seed):
    """Random scripts mixing pack / freeze / auto forks, appends, frees, base evictions and
    refills: the library's free lists, reference counts, tables, slot maps, copies and
    error codes equal the model's after every step."""
    rng = np.random.default_rng(7000 + seed)
    nb, nr = 48, 64
    lp, pm = _pair(nb, nr, rng.permutation(nb), rng.permutation(nr))
    live = []
    for step in range(300):
        op = int(rng.integers(0, 8))
        if op == 0 or not live:
            res = bool(rng.integers(0, 2))
            assert lp.create(res) == pm.create(res)
            live.append(pm.seqs.__len__() - 1)
        elif op in (1, 2):
            h = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, 30))
            r, ok = _both(lambda: lp.append(h, n), lambda: pm.append(h, n))
            if ok:
                assert r[0] == r[1]
        elif op in (3, 4):
            h = live[int(rng.integers(len(live)))]
            L = pm.length(h)
            alias = L if rng.integers(0, 2) else int(rng.integers(0, L + 1))
            mode = int(rng.integers(0, 3))
            hint = int(rng.integers(0, 24))
            r, ok = _both(lambda: lp.fork(h, alias, mode, hint), lambda: pm.fork(h, alias, mode, hint))
            if ok:
                assert r[0] == r[1]
                live.append(r[1][0])
        elif op == 5:
            h = live.pop(int(rng.integers(len(live))))
            lp.free(h)
            pm.free(h)
        elif op == 6:  # evict one or two live base pages (or an invalid list)
            pages = [p for p in range(nb) if pm.ref_b[p] > 0]
            if rng.integers(0, 4) == 0 or not pages:
                pages = [int(rng.integers(0, nb))] * 2
            else:
                pages = [int(x) for x in rng.choice(pages, size=min(2, len(pages)), replace=False)]
            _both(lambda: lp.evict_base(pages), lambda: pm.evict_base(pages))
        else:  # refill a missing run for every live sequence that misses it
            miss = [(h, j) for h in live for j, pg in enumerate(pm.seqs[h].bpages) if pg < 0]
            if miss:
                h0, j0 = miss[int(rng.integers(len(miss)))]
                hs = [h for h in live if j0 < len(pm.seqs[h].bpages) and pm.seqs[h].bpages[j0] < 0
                      and pm.seqs[h].starts[:j0 + 1] == pm.seqs[h0].starts[:j0 + 1]]
                r, ok = _both(lambda: lp.refill_base(hs, j0, j0 + 1),
                              lambda: pm.refill_base(hs, j0, j0 + 1))
                if ok:
                    assert r[0] == r[1]
        _same_state(lp, pm, live)
        _same_starts(lp, pm, live)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_freeze_scenarios_match_model(mode):
    """The six printed fan-out scenarios under each tail mode (hint = the child's suffix)."""
    for row in read_table("forkserve_results_table.txt"):
        L, k, ell = int(row[1]), int(row[2]), int(row[3])
        lp, pm = _pair(1 << 15, 1 << 16)
        names = _replay_both_modes(lp, pm, fanout_ops(L, k, ell, mode, ell))
        _same_state(lp, pm, list(names.values()))
        _same_starts(lp, pm, list(names.values()))


def _replay_both_modes(lp, pm, ops):
    names_l, cows_l = lp.replay(ops)
    names_m = pm.replay(ops)
    assert names_l == names_m
    return names_l


def test_plan_rejects_partial_hit_and_flags_frozen_tail():
    """A plan over a sequence with an evicted base page fails with FORKKV_ESTATE; a batch
    holding a frozen tail needs the slot map (checked at decode time, see the GPU tests)."""
    lp = fk.Pool(64, 64, 1, 16, 4, "f32")
    names, _ = lp.replay([("create", "t", 0), ("append", "t", 37),
                          ("fork", "t", 37, "a", fk.FORK_FREEZE, 0),
                          ("fork", "t", 37, "b", fk.FORK_FREEZE, 0),
                          ("append", "a", 5), ("append", "b", 20)])
    hs = [names["a"], names["b"]]
    st, aligned = lp.starts(hs, 5)
    assert not aligned and st[0] == [0, 16, 32, 37, -1] and st[1] == [0, 16, 32, 37, 53]
    fk.Plan(lp, hs, 2, kernel=fk.KERNEL_GENERIC)
    bt, _, _ = lp.tables(hs, 5)
    lp.evict_base([bt[0][1]])
    with pytest.raises(fk.ForkKVError) as e:
        fk.Plan(lp, hs, 2, kernel=fk.KERNEL_GENERIC)
    assert e.value.code == fk.ESTATE
    new = lp.refill_base(hs + [names["t"]], 1, 2)
    assert lp.tables(hs, 5)[0][0][1] == new[0]
    fk.Plan(lp, hs, 2, kernel=fk.KERNEL_GENERIC)


# ---- step-stable plans: batched append, in-place rebuild ---------------------------------

def _state(lp, hs, max_pages=64):
    bt, rt, lens = lp.tables(hs, max_pages)
    return bt, rt, lens, lp.free_list(0), lp.free_list(1), lp.refcounts(0), lp.refcounts(1)


@pytest.mark.parametrize("seed", range(8))
def test_append_batch_equals_one_by_one(seed):
    """forkkv_seq_append_batch reserves what forkkv_seq_append would, sequence by sequence,
    with the same copy-on-write reports, and counts the base pages it took."""
    from tests.cases import freeze_ops, random_ops, resolve_ops
    rng = np.random.default_rng(3100 + seed)
    if seed % 2:
        ops, agents = freeze_ops(rng, 4, 16, 70, 40)
        ops = resolve_ops(ops)
    else:
        ops, agents = random_ops(rng, 5, max_prefix=70, max_suffix=40)
    pb, pr = rng.permutation(128), rng.permutation(128)
    one, many = (fk.Pool(128, 128, 2, 16, 4, "f32", pb, pr) for _ in range(2))
    n1, _ = one.replay(ops)
    n2, _ = many.replay(ops)
    h1, h2 = [n1[a] for a in agents], [n2[a] for a in agents]
    for rows in (1, 1, 3, 16, 1, 17):
        live = many.stats()["live_bpages"]
        cows1, slots1 = [], []
        for h in h1:
            bs, rs, cow = one.append(h, rows)
            slots1 += bs
            cows1 += [cow] if cow else []
        pages, cows2, slots2, _ = many.append_batch(h2, rows, want_slots=True)
        assert cows2 == cows1 and slots2 == slots1
        assert pages == many.stats()["live_bpages"] - live
        assert _state(one, h1) == _state(many, h2)


def test_append_batch_is_all_or_nothing():
    lp = fk.Pool(8, 16, 1, 16, 4, "f32")
    root = lp.create(False)
    lp.append(root, 16)
    a, _ = lp.fork(root, 16)
    b, _ = lp.fork(root, 16)
    before = _state(lp, [a, b])
    with pytest.raises(fk.ForkKVError) as e:  # 2 x 4 fresh pages > 7 free
        lp.append_batch([a, b], 64)
    assert e.value.code == fk.ENOMEM and _state(lp, [a, b]) == before
    with pytest.raises(fk.ForkKVError) as e:  # a sequence listed twice
        lp.append_batch([a, a], 1)
    assert e.value.code == fk.EINVAL and _state(lp, [a, b]) == before


@pytest.mark.parametrize("kernel", [fk.KERNEL_GENERIC, fk.KERNEL_MFMA])
def test_plan_rebuild_equals_fresh_plan(kernel):
    """After decode steps that cross pages, a rebuilt plan has exactly the items, lengths,
    slots and last pages of a plan built afresh, keeps its capacities (so a captured launch
    stays valid) and passes the validity checks."""
    cfg = config_by_name("llama3_8b_react_decode")
    lp = fk.Pool(cfg.num_bpages, cfg.num_rpages, cfg.num_kv_heads, cfg.head_dim, cfg.rank,
                 cfg.dtype)
    ops, agents = pool_ops(cfg)
    names, _ = lp.replay(ops)
    hs = [names[a] for a in agents]
    lp.append_batch(hs, 1)
    plan = fk.Plan(lp, hs, cfg.num_q_heads, kernel=kernel)
    cap0 = plan.info["item_capacity"], plan.info["slot_capacity"], plan.info["plan_bytes"]
    for step in range(40):
        pages, _, _, _ = lp.append_batch(hs, 1)
        if not pages:
            continue
        same = plan.rebuild(hs)
        fresh = fk.Plan(lp, hs, cfg.num_q_heads, kernel=kernel)
        b1, b2 = plan.blob(), fresh.blob()
        assert b1[2] == b2[2] and b1[3] == b2[3]  # items, slots
        n = len(hs)
        for off_word, size in ((6, b1[2] * ITEM_INTS), (7, n), (8, n + 1), (12, n)):
            assert b1[b1[off_word]:b1[off_word] + size] == b2[b2[off_word]:b2[off_word] + size]
        assert same and (plan.info["item_capacity"], plan.info["slot_capacity"],
                         plan.info["plan_bytes"]) == cap0
        _check_plan(lp, lp.tables(hs, -(-lp.length(hs[0]) // 16)), hs, plan, 8)
