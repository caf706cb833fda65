"""Frozen tails on the GPU (the fork-aware slot map), through the C ABI, against the oracle.

A freeze fork (ForkServe README, "Design vs APC": pages_freeze = 1 + k * ceil(l / P)) leaves
one read-only partial page shared by the trunk and its children; later rows start fresh
pages, so pages no longer start at multiples of P and the kernels take the page start table.
Every slot the batch does not read -- the rows of a frozen page past its valid rows included
-- holds NaN, so a kernel that read past a frozen tail could not pass.
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
from oracle import PoolModel  # noqa: E402
from oracle.attention import (Geometry, apply_rows_write, decode_attention,  # noqa: E402
                              prefill_attention_at)
from tests.cases import encode, freeze_ops, resolve_ops  # noqa: E402
from tests.gpu_common import (assert_close, gpu_values, poison_unused,  # noqa: E402
                              used_rows)


def _setup(seed, dtype, d, r, Hq, Hkv, n_agents, num_pages=200, max_prefix=40, max_suffix=24,
           b_std=0.3, extra=None):
    rng = np.random.default_rng(seed)
    ops, agents = freeze_ops(rng, n_agents, 16, max_prefix, max_suffix)
    ops = resolve_ops(ops)
    if extra:
        ops = ops + extra(agents)
    perm_b = rng.permutation(num_pages).astype(np.int32)
    perm_r = rng.permutation(num_pages).astype(np.int32)
    pm = PoolModel(num_pages, num_pages, 16, perm_b, perm_r)
    names = pm.replay(ops)
    hs = [names[a] for a in agents]
    mp = max(len(pm.seqs[h].bpages) for h in hs)
    bt, rt, lens = (np.array(x) for x in pm.tables(hs, mp))
    st = np.array(pm.starts_table(hs, mp))
    bpool = encode(rng.standard_normal((num_pages, 2, Hkv, 16 * d)), dtype)
    rpool = encode(rng.standard_normal((num_pages, 2, 16 * r)), dtype)
    ub, ur = used_rows(bt, rt, lens, st)
    bpool, rpool = poison_unused(bpool, rpool, ub, ur, dtype, d, r)
    arrays = dict(bpool=bpool, rpool=rpool,
                  Bk=encode(b_std * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
                  Bv=encode(b_std * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
                  q=encode(rng.standard_normal((n_agents, Hq, d)), dtype))
    geom = dict(num_bpages=num_pages, num_rpages=num_pages, num_kv_heads=Hkv, num_q_heads=Hq,
                head_dim=d, rank=r, dtype=dtype)
    return rng, ops, agents, perm_b, perm_r, arrays, geom, (bt, rt, lens, st)


CASES = [  # seed, dtype, kernel, d, r, Hq, Hkv
    (0, "f32", fk.KERNEL_GENERIC, 16, 4, 8, 2),
    (1, "bf16", fk.KERNEL_GENERIC, 32, 8, 8, 2),
    (2, "bf16", fk.KERNEL_MFMA, 128, 16, 8, 2),
    (3, "bf16", fk.KERNEL_MFMA, 128, 16, 16, 2),
    (4, "bf16", fk.KERNEL_MFMA, 128, 16, 8, 2),
]


@pytest.mark.parametrize("seed,dtype,kernel,d,r,Hq,Hkv", CASES)
def test_freeze_decode_tiny(seed, dtype, kernel, d, r, Hq, Hkv):
    """Decode over a root's frozen tail shared by every agent (and a grandchild's second
    frozen tail): library tables and slot map equal the model's, output matches the oracle."""
    n_agents = 5
    print(f"[gpu-freeze] seed={seed} {dtype} kernel={kernel} d={d} r={r} Hq={Hq}", flush=True)
    rng, ops, agents, perm_b, perm_r, arrays, geom, (bt, rt, lens, st) = _setup(
        800 + seed, dtype, d, r, Hq, Hkv, n_agents, max_prefix=[40, 40, 80, 200, 600][seed],
        max_suffix=[24, 24, 40, 90, 300][seed])
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, kernel=kernel)
    assert b.plan.info["kernel"] == kernel
    assert np.array_equal(b.btab_host, bt) and np.array_equal(b.pstart_host, st)
    assert b.pstart is not None  # the batch holds a frozen tail
    b.out.fill_(float("nan") if dtype == "f32" else 0x7FC0)
    out = b.decode(2.0, 1.0 / np.sqrt(d), 5e5)
    torch.cuda.synchronize()
    geo = Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rank=r,
                   dtype=dtype)
    ref = decode_attention(geo, arrays["bpool"], arrays["rpool"], bt, rt, lens, arrays["q"],
                           arrays["Bk"], arrays["Bv"], 2.0, 1.0 / np.sqrt(d), 5e5, starts=st)
    assert_close(gpu_values(out, dtype), ref, f"freeze decode seed={seed} {dtype} k={kernel}",
                 scale_abs=True)


def test_freeze_decode_llama3_shape():
    """Llama3-8B attention shape (32 q / 8 KV heads, d = 128, r = 16, MFMA): a trunk of
    8192 + 7 tokens frozen at its end, 6 agents with 300-700 private tokens each, the trunk
    continuing by 40 tokens; sampled heads against the oracle."""
    rng = np.random.default_rng(31)
    L0 = 8192 + 7
    ops = [("create", "t", 0), ("append", "t", L0)]
    agents = [f"a{j}" for j in range(6)]
    ops += [("fork", "t", L0, a, fk.FORK_FREEZE, 0) for a in agents]
    ops += [("append", "t", 40)]
    ops += [("append", a, int(rng.integers(300, 700))) for a in agents]
    npg, nrp = 1200, 4096  # every agent owns residual pages for its whole history
    perm_b = rng.permutation(npg).astype(np.int32)
    perm_r = rng.permutation(nrp).astype(np.int32)
    Hq, Hkv, d, r = 32, 8, 128, 16
    arrays = dict(bpool=encode(rng.standard_normal((npg, 2, Hkv, 16 * d)), "bf16"),
                  rpool=encode(rng.standard_normal((nrp, 2, 16 * r)), "bf16"),
                  Bk=encode(0.02 * rng.standard_normal((6, r, Hkv * d)), "bf16"),
                  Bv=encode(0.02 * rng.standard_normal((6, r, Hkv * d)), "bf16"),
                  q=encode(rng.standard_normal((6, Hq, d)), "bf16"))
    geom = dict(num_bpages=npg, num_rpages=nrp, num_kv_heads=Hkv, num_q_heads=Hq, head_dim=d,
                rank=r, dtype="bf16")
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, kernel=fk.KERNEL_MFMA)
    b.out.fill_(0x7FC0)
    out = b.decode(2.0, 1.0 / np.sqrt(d), 5e5)
    torch.cuda.synchronize()
    geo = Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rank=r,
                   dtype="bf16")
    ref = decode_attention(geo, arrays["bpool"], arrays["rpool"], b.btab_host, b.rtab_host,
                           np.array(b.lens), arrays["q"], arrays["Bk"], arrays["Bv"], 2.0,
                           1.0 / np.sqrt(d), 5e5, agents=[0, 5], kv_heads=[0, 7],
                           starts=b.pstart_host)
    g = gpu_values(out, "bf16")
    mask = ~np.isnan(ref[..., 0])
    assert_close(g[mask], ref[mask], "freeze decode llama3 shape")


@pytest.mark.parametrize("kernel", [fk.KERNEL_GENERIC, fk.KERNEL_MFMA])
def test_freeze_prefill_then_decode_append(kernel):
    """Agents right after a freeze fork: a chunk prefill of their own rows (they start a
    fresh page at the frozen tail's end position), then one decode-with-append step; the
    stored rows land on the slots the pool reports, outputs match the oracle."""
    rng = np.random.default_rng(41)
    Hq, Hkv, d, r = 8, 2, 128, 16
    L0 = 53
    agents = ["a0", "a1", "a2"]
    ops = [("create", "t", 0), ("append", "t", L0)]
    ops += [("fork", "t", L0, a, fk.FORK_FREEZE, 0) for a in agents]
    npg = 64
    perm_b = rng.permutation(npg).astype(np.int32)
    perm_r = rng.permutation(npg).astype(np.int32)
    arrays = dict(bpool=encode(rng.standard_normal((npg, 2, Hkv, 16 * d)), "bf16"),
                  rpool=encode(rng.standard_normal((npg, 2, 16 * r)), "bf16"),
                  Bk=encode(0.3 * rng.standard_normal((3, r, Hkv * d)), "bf16"),
                  Bv=encode(0.3 * rng.standard_normal((3, r, Hkv * d)), "bf16"),
                  q=encode(rng.standard_normal((3, Hq, d)), "bf16"))
    geom = dict(num_bpages=npg, num_rpages=npg, num_kv_heads=Hkv, num_q_heads=Hq, head_dim=d,
                rank=r, dtype="bf16")
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, plan=False)
    C = 37
    start = b.reserve_chunk(C)
    assert start == [L0] * 3 and b.pstart is not None
    assert list(b.pstart_host[0][:5]) == [0, 16, 32, 48, 53]
    chunk = {k: encode(rng.standard_normal(s), "bf16") for k, s in
             (("q", (3, C, Hq, d)), ("k_new", (3, C, Hkv, d)), ("v_new", (3, C, Hkv, d)),
              ("rk_new", (3, C, r)), ("rv_new", (3, C, r)))}
    dev = {k: to_device(v) for k, v in chunk.items()}
    out = b.prefill(dev, 2.0, 1.0 / np.sqrt(d), 5e5)
    torch.cuda.synchronize()
    geo = Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rank=r,
                   dtype="bf16")
    pos = np.array([[L0 + i for i in range(C)]] * 3)
    exp_b, exp_r = apply_rows_write(geo, arrays["bpool"], arrays["rpool"], b.btab_host,
                                    b.rtab_host, pos, chunk["k_new"], chunk["v_new"],
                                    chunk["rk_new"], chunk["rv_new"], starts=b.pstart_host)
    assert np.array_equal(b.bcache.cpu().numpy().view(np.uint16), exp_b)
    assert np.array_equal(b.rcache.cpu().numpy().view(np.uint16), exp_r)
    ref = prefill_attention_at(geo, arrays["bpool"], arrays["rpool"], b.btab_host, b.rtab_host,
                               pos, chunk["q"], chunk["k_new"], chunk["v_new"], chunk["rk_new"],
                               chunk["rv_new"], arrays["Bk"], arrays["Bv"], 2.0,
                               1.0 / np.sqrt(d), 5e5, starts=b.pstart_host)
    assert_close(gpu_values(out, "bf16"), ref, "freeze prefill", scale_abs=True)

    # one decode step with append on top
    lens0 = b.reserve_chunk(1)
    b.make_plan(kernel)
    rows = {k: encode(rng.standard_normal(s), "bf16") for k, s in
            (("k_new", (3, Hkv, d)), ("v_new", (3, Hkv, d)), ("rk_new", (3, r)),
             ("rv_new", (3, r)))}
    b.out.fill_(0x7FC0)
    o2 = b.decode_append({k: to_device(v) for k, v in rows.items()}, 2.0, 1.0 / np.sqrt(d), 5e5)
    torch.cuda.synchronize()
    pos1 = np.array([[L] for L in lens0])
    exp_b, exp_r = apply_rows_write(geo, exp_b, exp_r, b.btab_host, b.rtab_host, pos1,
                                    rows["k_new"][:, None], rows["v_new"][:, None],
                                    rows["rk_new"][:, None], rows["rv_new"][:, None],
                                    starts=b.pstart_host)
    assert np.array_equal(b.bcache.cpu().numpy().view(np.uint16), exp_b)
    ref2 = decode_attention(geo, exp_b, exp_r, b.btab_host, b.rtab_host, np.array(b.lens),
                            arrays["q"], arrays["Bk"], arrays["Bv"], 2.0, 1.0 / np.sqrt(d), 5e5,
                            starts=b.pstart_host)
    assert_close(gpu_values(o2, "bf16"), ref2, f"freeze decode append k={kernel}",
                 scale_abs=True)


def test_freeze_decode_needs_the_slot_map():
    """A plan over a frozen tail refuses a decode call without the start table."""
    rng, ops, agents, perm_b, perm_r, arrays, geom, _ = _setup(9, "f32", 16, 4, 4, 2, 3)
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, kernel=fk.KERNEL_GENERIC)
    with pytest.raises(fk.ForkKVError) as e:
        fk.residual_attn_decode(b.pool, b.plan, b.q, b.Bk, b.Bv, b.btab, b.rtab, b.out,
                                b.workspace, 1.0, 0.25, 1e4)
    assert e.value.code == fk.EINVAL


@pytest.mark.parametrize("L0,nested", [(16 * 40 + 7, False), (7, False), (16 * 70 + 11, True)])
def test_freeze_prefill_both_kernels(L0, nested):
    """Chunk prefill over frozen tails on both kernels (the MFMA kernel's slot-map
    instantiation and the generic kernel), each against the oracle on every row, with a
    material adapter: a trunk frozen at an unaligned end (at 7 rows: the first page itself is
    the frozen tail), agents whose chunks start fresh pages there, and with ``nested`` a
    grandchild frozen again at its parent's unaligned end (two frozen tails in its history).
    The stored rows are compared bit for bit."""
    rng = np.random.default_rng(L0)
    Hq, Hkv, d, r, C = 8, 2, 128, 16, 70
    agents = ["a0", "a1"]
    ops = [("create", "t", 0), ("append", "t", L0)]
    ops += [("fork", "t", L0, a, fk.FORK_FREEZE, 0) for a in agents]
    if nested:
        ops += [("append", "a0", 21), ("fork", "a0", L0 + 21, "g", fk.FORK_FREEZE, 0)]
        agents = ["a1", "g"]
    npg = (L0 + 16 * 8 + 2 * C) // 16 + 24
    perm_b = rng.permutation(npg).astype(np.int32)
    perm_r = rng.permutation(3 * npg).astype(np.int32)
    N = len(agents)
    arrays = dict(bpool=encode(rng.standard_normal((npg, 2, Hkv, 16 * d)), "bf16"),
                  rpool=encode(rng.standard_normal((3 * npg, 2, 16 * r)), "bf16"),
                  Bk=encode(0.3 * rng.standard_normal((N, r, Hkv * d)), "bf16"),
                  Bv=encode(0.3 * rng.standard_normal((N, r, Hkv * d)), "bf16"),
                  q=encode(rng.standard_normal((N, Hq, d)), "bf16"))
    chunk = {k: encode(rng.standard_normal(s), "bf16") for k, s in
             (("q", (N, C, Hq, d)), ("k_new", (N, C, Hkv, d)), ("v_new", (N, C, Hkv, d)),
              ("rk_new", (N, C, r)), ("rv_new", (N, C, r)))}
    geom = dict(num_bpages=npg, num_rpages=3 * npg, num_kv_heads=Hkv, num_q_heads=Hq,
                head_dim=d, rank=r, dtype="bf16")
    geo = Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rank=r,
                   dtype="bf16")
    outs = {}
    for kernel in (fk.KERNEL_MFMA, fk.KERNEL_GENERIC):
        print(f"[gpu-freeze] prefill L0={L0} nested={nested} kernel={kernel}", flush=True)
        b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, plan=False)
        start = b.reserve_chunk(C)
        assert b.pstart is not None
        pos = np.array([[s0 + i for i in range(C)] for s0 in start])
        dev = {k: to_device(v) for k, v in chunk.items()}
        out = b.prefill(dev, 2.0, 1.0 / np.sqrt(d), 1e6, kernel=kernel)
        torch.cuda.synchronize()
        exp_b, exp_r = apply_rows_write(geo, arrays["bpool"], arrays["rpool"], b.btab_host,
                                        b.rtab_host, pos, chunk["k_new"], chunk["v_new"],
                                        chunk["rk_new"], chunk["rv_new"], starts=b.pstart_host)
        assert np.array_equal(b.bcache.cpu().numpy().view(np.uint16), exp_b)
        assert np.array_equal(b.rcache.cpu().numpy().view(np.uint16), exp_r)
        ref = prefill_attention_at(geo, arrays["bpool"], arrays["rpool"], b.btab_host,
                                   b.rtab_host, pos, chunk["q"], chunk["k_new"], chunk["v_new"],
                                   chunk["rk_new"], chunk["rv_new"], arrays["Bk"], arrays["Bv"],
                                   2.0, 1.0 / np.sqrt(d), 1e6, starts=b.pstart_host)
        outs[kernel] = gpu_values(out, "bf16")
        assert_close(outs[kernel], ref, f"freeze prefill L0={L0} nested={nested} k={kernel}",
                     scale_abs=True)
