"""Decoupled eviction and partial-hit refill on the GPU, through the C ABI.

ForkKV study note, "Error / eviction recovery" and implementation detail 1: the base and the
residual caches are evicted independently.  Base pages shared by every agent are evicted (the
residual pages survive), the plan refuses the partial hit, fresh base pages are mapped back
into every sequence that lost them, and only the base rows (xW, recomputed by the caller --
here the original rows stand in for them) are stored through the row-write call without
residual rows.  The residual pool is untouched, and the decode afterwards equals the decode
before the eviction bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from lora_shared_prefix_amd import forkkv as fk  # noqa: E402
from lora_shared_prefix_amd.session import DeviceBatch, to_device  # noqa: E402
from oracle.attention import (Geometry, apply_chunk_write, decode_attention,  # noqa: E402
                              prefill_attention)
from oracle.storage import key_offset, value_offset  # noqa: E402
from tests.cases import encode  # noqa: E402
from tests.gpu_common import (apply_cows_host, assert_close, gpu_values,  # noqa: E402
                              model_replay)


def _rows_of(bpool, pages, Hkv, d):
    """Rows of whole base pages as row-major [rows][Hkv][d] (K and V), bit exact."""
    dims = np.arange(d)
    k = np.stack([np.stack([bpool[pg, 0, h, key_offset(t, dims)] for h in range(Hkv)])
                  for pg in pages for t in range(16)])
    v = np.stack([np.stack([bpool[pg, 1, h, value_offset(t, dims)] for h in range(Hkv)])
                  for pg in pages for t in range(16)])
    return k, v


@pytest.mark.parametrize("kernel,dtype,d,r,Hq,Hkv", [
    (fk.KERNEL_MFMA, "bf16", 128, 16, 16, 4),
    (fk.KERNEL_GENERIC, "f32", 32, 8, 4, 2),
])
def test_evict_refill_restores_decode(kernel, dtype, d, r, Hq, Hkv):
    rng = np.random.default_rng(61)
    L0, n_agents, npg, nrp = 16 * 40, 4, 160, 256
    agents = [f"a{j}" for j in range(n_agents)]
    ops = [("create", "t", 0), ("append", "t", L0)]
    ops += [("fork", "t", L0, a) for a in agents]
    ops += [("append", a, int(rng.integers(20, 90))) for a in agents]
    perm_b = rng.permutation(npg).astype(np.int32)
    perm_r = rng.permutation(nrp).astype(np.int32)
    arrays = dict(bpool=encode(rng.standard_normal((npg, 2, Hkv, 16 * d)), dtype),
                  rpool=encode(rng.standard_normal((nrp, 2, 16 * r)), dtype),
                  Bk=encode(0.3 * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
                  Bv=encode(0.3 * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
                  q=encode(rng.standard_normal((n_agents, Hq, d)), dtype))
    geom = dict(num_bpages=npg, num_rpages=nrp, num_kv_heads=Hkv, num_q_heads=Hq,
                head_dim=d, rank=r, dtype=dtype)
    print(f"[gpu-evict] kernel={kernel} {dtype} d={d}", flush=True)
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, kernel=kernel)
    sm = 1.0 / np.sqrt(d)
    before = b.decode(2.0, sm, 5e5).clone()
    torch.cuda.synchronize()
    bt0 = b.btab_host.copy()
    rt0 = b.rtab_host.copy()
    rcache0 = b.rcache.clone()
    lp0, lp1 = 7, 19  # twelve shared trunk pages
    victims = [int(x) for x in bt0[0][lp0:lp1]]
    host_b = b.bcache.cpu().numpy()
    host_b = host_b.view(np.uint16) if dtype == "bf16" else host_b
    k_rows, v_rows = _rows_of(host_b, victims, Hkv, d)

    b.pool.evict_base(victims)
    b.refresh_tables()
    assert (b.btab_host[:, lp0:lp1] == -1).all()
    assert np.array_equal(b.rtab_host, rt0)  # the residual pages survive
    with pytest.raises(fk.ForkKVError) as e:
        b.make_plan(kernel)
    assert e.value.code == fk.ESTATE
    # the trunk snapshot lost the pages too; refill all five sequences
    new = b.pool.refill_base(b.handles + [b.names["t"]], lp0, lp1)
    assert set(new).isdisjoint(victims)  # fresh pages from the head of the free list
    b.refresh_tables()
    b.make_plan(kernel)
    # store the recomputed base rows once, through one sequence's tables, base pool only
    n = (lp1 - lp0) * 16
    pos = np.arange(lp0 * 16, lp1 * 16, dtype=np.int32)[None, :]
    fk.write_rows(b.pool, b.btab[:1].contiguous(), None, torch.from_numpy(pos).cuda(),
                  pos.tolist(), to_device(k_rows[None]), to_device(v_rows[None]))
    torch.cuda.synchronize()
    assert torch.equal(b.rcache, rcache0), "the residual pool must be untouched"
    after_b = b.bcache.cpu().numpy()
    after_b = after_b.view(np.uint16) if dtype == "bf16" else after_b
    for old, pg in zip(victims, new):
        assert np.array_equal(after_b[pg], host_b[old])
    after = b.decode(2.0, sm, 5e5)
    torch.cuda.synchronize()
    assert torch.equal(after.view(torch.int32 if dtype == "f32" else torch.int16),
                       before.view(torch.int32 if dtype == "f32" else torch.int16))
    geo = Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rank=r,
                   dtype=dtype)
    ref = decode_attention(geo, after_b, arrays["rpool"], b.btab_host, b.rtab_host,
                           np.array(b.lens), arrays["q"], arrays["Bk"], arrays["Bv"], 2.0, sm,
                           5e5)
    assert_close(gpu_values(after, dtype), ref, f"decode after refill k={kernel}",
                 scale_abs=True)
    assert n == k_rows.shape[0]


def test_write_rows_errors():
    geom = dict(num_bpages=8, num_rpages=8, num_kv_heads=1, num_q_heads=2, head_dim=16,
                rank=4, dtype="f32")
    rng = np.random.default_rng(2)
    arrays = dict(bpool=rng.standard_normal((8, 2, 1, 256)).astype(np.float32),
                  rpool=rng.standard_normal((8, 2, 64)).astype(np.float32),
                  q=rng.standard_normal((1, 2, 16)).astype(np.float32),
                  Bk=rng.standard_normal((1, 4, 16)).astype(np.float32),
                  Bv=rng.standard_normal((1, 4, 16)).astype(np.float32))
    b = DeviceBatch(geom, arrays, [("create", "a", 1), ("append", "a", 20)], ["a"])
    k = torch.zeros((1, 2, 1, 16), device="cuda")
    for pos in ([[3, 3]], [[5, 40]], [[-1, 2]]):
        with pytest.raises(fk.ForkKVError) as e:
            fk.write_rows(b.pool, b.btab, b.rtab, torch.tensor(pos, dtype=torch.int32).cuda(),
                          pos, k, k)
        assert e.value.code == fk.EINVAL
    with pytest.raises(fk.ForkKVError) as e:  # only one of the residual rows
        fk.write_rows(b.pool, b.btab, b.rtab, torch.tensor([[1, 2]], dtype=torch.int32).cuda(),
                      [[1, 2]], k, k, rk_new=torch.zeros((1, 2, 4), device="cuda"))
    assert e.value.code == fk.EINVAL


@pytest.mark.parametrize("kernel", [fk.KERNEL_MFMA, fk.KERNEL_GENERIC])
def test_prefill_over_missing_pages(kernel):
    """Prefill over a partial hit: one shared trunk page evicted from every holder (no key
    there until a refill), and the base-only trunk itself in the batch (no residual pages: a
    zero residual, its chunk's residual rows not stored).  Both prefill kernels follow the
    oracle's rule, each against the oracle, every output row."""
    rng = np.random.default_rng(71)
    d, r, Hq, Hkv, C = 128, 16, 8, 2, 40
    L0, npg, nrp = 16 * 30 + 5, 96, 128
    agents = ["a0", "a1", "t"]
    ops = [("create", "t", 0), ("append", "t", L0), ("fork", "t", 16 * 30, "a0"),
           ("fork", "t", L0, "a1"), ("append", "a0", 7)]
    perm_b = rng.permutation(npg).astype(np.int32)
    perm_r = rng.permutation(nrp).astype(np.int32)
    N = len(agents)
    arrays = dict(bpool=encode(rng.standard_normal((npg, 2, Hkv, 16 * d)), "bf16"),
                  rpool=encode(rng.standard_normal((nrp, 2, 16 * r)), "bf16"),
                  Bk=encode(0.3 * rng.standard_normal((N, r, Hkv * d)), "bf16"),
                  Bv=encode(0.3 * rng.standard_normal((N, r, Hkv * d)), "bf16"),
                  q=encode(rng.standard_normal((N, C, Hq, d)), "bf16"),
                  k_new=encode(rng.standard_normal((N, C, Hkv, d)), "bf16"),
                  v_new=encode(rng.standard_normal((N, C, Hkv, d)), "bf16"),
                  rk_new=encode(rng.standard_normal((N, C, r)), "bf16"),
                  rv_new=encode(rng.standard_normal((N, C, r)), "bf16"))
    geom = dict(num_bpages=npg, num_rpages=nrp, num_kv_heads=Hkv, num_q_heads=Hq, head_dim=d,
                rank=r, dtype="bf16")
    print(f"[gpu-evict] prefill over missing pages kernel={kernel}", flush=True)
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, plan=False)
    start = b.reserve_chunk(C)
    # evict the trunk's page 3 (shared by a0, a1 and the trunk), then re-export the tables
    victim = int(b.btab_host[2][3])
    b.pool.evict_base([victim])
    b.refresh_tables()
    assert b.btab_host[0][3] == -1 and b.btab_host[1][3] == -1 and b.btab_host[2][3] == -1
    assert np.all(b.rtab_host[2] == -1)
    chunk = {k: to_device(arrays[k]) for k in ("q", "k_new", "v_new", "rk_new", "rv_new")}
    out = b.prefill(chunk, 2.0, 1 / np.sqrt(d), 1e6, kernel=kernel)
    torch.cuda.synchronize()
    # oracle side: the model's tables after the same script, chunk appends and eviction
    pm, names, cows = model_replay(npg, nrp, perm_b, perm_r,
                                   ops + [("append", a, C) for a in agents])
    pm.evict_base([victim])
    hs = [names[a] for a in agents]
    bt, rt, _ = (np.array(x) for x in pm.tables(hs, b.max_pages))
    assert np.array_equal(bt, b.btab_host) and np.array_equal(rt, b.rtab_host)
    host_b = apply_cows_host(arrays["bpool"], cows, Hkv, d)
    g = Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rank=r,
                 dtype="bf16")
    ref = prefill_attention(g, host_b, arrays["rpool"], bt, rt, np.array(start), arrays["q"],
                            arrays["k_new"], arrays["v_new"], arrays["rk_new"], arrays["rv_new"],
                            arrays["Bk"], arrays["Bv"], 2.0, 1 / np.sqrt(d), 1e6)
    assert_close(gpu_values(out, "bf16"), ref, f"prefill over missing pages kernel={kernel}",
                 scale_abs=True)
    # rows on the evicted page are absent; the pool's other bytes are as the write leaves them
    exp_b, exp_r = apply_chunk_write(g, host_b, arrays["rpool"], bt, rt, start, arrays["k_new"],
                                     arrays["v_new"], arrays["rk_new"], arrays["rv_new"])
    assert np.array_equal(b.bcache.cpu().numpy().view(np.uint16), exp_b)
    assert np.array_equal(b.rcache.cpu().numpy().view(np.uint16), exp_r)


@pytest.mark.parametrize("kernel,dtype,d,r,Hq,Hkv", [
    (fk.KERNEL_MFMA, "bf16", 128, 16, 16, 4),
    (fk.KERNEL_GENERIC, "f32", 32, 8, 4, 2),
])
def test_decode_reads_tables_at_launch(kernel, dtype, d, r, Hq, Hkv):
    """Decode takes page ids from the tables at launch, not from the plan: entries changed
    after the plan was built -- a page evicted from every holder, an id outside its pool, a
    residual page dropped -- follow the missing-page rule of the ForkKV study note ("Error /
    eviction recovery"): no key on a missing base page, a zero residual without a residual
    page.  Against the oracle on the same tables with those entries -1; with every base entry
    gone each output is zero (no keys); the original tables give the original output again,
    bit for bit.  On the MFMA kernel this is the masked page loop without a slot map."""
    rng = np.random.default_rng(83)
    L0, n_agents, npg, nrp = 16 * 40, 4, 160, 256
    agents = [f"a{j}" for j in range(n_agents)]
    ops = [("create", "t", 0), ("append", "t", L0)]
    ops += [("fork", "t", L0, a) for a in agents]
    ops += [("append", a, int(rng.integers(20, 90))) for a in agents]
    perm_b = rng.permutation(npg).astype(np.int32)
    perm_r = rng.permutation(nrp).astype(np.int32)
    arrays = dict(bpool=encode(rng.standard_normal((npg, 2, Hkv, 16 * d)), dtype),
                  rpool=encode(rng.standard_normal((nrp, 2, 16 * r)), dtype),
                  Bk=encode(0.3 * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
                  Bv=encode(0.3 * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
                  q=encode(rng.standard_normal((n_agents, Hq, d)), dtype))
    geom = dict(num_bpages=npg, num_rpages=nrp, num_kv_heads=Hkv, num_q_heads=Hq,
                head_dim=d, rank=r, dtype=dtype)
    print(f"[gpu-evict] tables at launch kernel={kernel} {dtype} d={d}", flush=True)
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, kernel=kernel)
    sm = 1.0 / np.sqrt(d)
    as_int = torch.int32 if dtype == "f32" else torch.int16
    before = b.decode(2.0, sm, 5e5).clone()
    torch.cuda.synchronize()
    bt0, rt0 = b.btab_host.copy(), b.rtab_host.copy()
    # oracle side: pool bytes from the inputs and the model's fork packing, not the device
    _, _, cows = model_replay(npg, nrp, perm_b, perm_r, ops)
    host_b = apply_cows_host(arrays["bpool"], cows, Hkv, d)
    geo = Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rank=r,
                   dtype=dtype)

    bt, rt = bt0.copy(), rt0.copy()
    assert (bt0[:, 9] == bt0[0, 9]).all() and (bt0[:, 22] == bt0[0, 22]).all()
    assert (bt0[:, 41] >= 0).all() and (rt0[:, 40] >= 0).all() and rt0[2, 3] >= 0
    bt[:, 9] = npg + 5   # a trunk page, outside the pool in every holder's table
    bt[:, 22] = -1       # a trunk page evicted from every holder
    bt[1, 41] = -1       # a private page
    rt[2, 3] = nrp + 1   # a residual page outside the pool
    rt[3, 40] = -1       # a residual page dropped
    b.btab.copy_(torch.from_numpy(bt))
    b.rtab.copy_(torch.from_numpy(rt))
    got = b.decode(2.0, sm, 5e5).clone()
    torch.cuda.synchronize()
    bt_ref, rt_ref = bt.copy(), rt.copy()
    bt_ref[bt_ref >= npg] = -1
    rt_ref[rt_ref >= nrp] = -1
    ref = decode_attention(geo, host_b, arrays["rpool"], bt_ref, rt_ref, np.array(b.lens),
                           arrays["q"], arrays["Bk"], arrays["Bv"], 2.0, sm, 5e5)
    assert_close(gpu_values(got, dtype), ref, f"decode over changed tables k={kernel}",
                 scale_abs=True)
    full = decode_attention(geo, host_b, arrays["rpool"], bt0, rt0, np.array(b.lens),
                            arrays["q"], arrays["Bk"], arrays["Bv"], 2.0, sm, 5e5)
    assert np.abs(ref - full).max() > 1e-2, "the changed entries must change the output"

    b.btab.fill_(-1)  # every base page gone: no keys anywhere
    none = b.decode(2.0, sm, 5e5).clone()
    torch.cuda.synchronize()
    assert torch.equal(none.view(as_int), torch.zeros_like(none).view(as_int))

    b.btab.copy_(torch.from_numpy(bt0))
    b.rtab.copy_(torch.from_numpy(rt0))
    again = b.decode(2.0, sm, 5e5)
    torch.cuda.synchronize()
    assert torch.equal(again.view(as_int), before.view(as_int))
