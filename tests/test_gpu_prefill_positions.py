"""Prefill over a position list on the GPU (a hole inside the history refilled by a
prefill-only request, followed by the real request's appended tail, in one launch), through
the C ABI, against the fp64 oracle; the stored rows bit-exact."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from lora_shared_prefix_amd import forkkv as fk  # noqa: E402
from lora_shared_prefix_amd.session import DeviceBatch, to_device  # noqa: E402
from oracle.attention import Geometry, apply_rows_write, prefill_attention_at  # noqa: E402
from tests.cases import encode  # noqa: E402
from tests.gpu_common import assert_close, gpu_values  # noqa: E402


def _host(t, dtype):
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if dtype == "bf16" else a


def _case(seed, dtype, d, r, Hq, Hkv, n_agents, fork_at, own, hole, tail, num_pages,
          b_std=0.3):
    """A root forked at `fork_at` (page-aligned) by every agent, each of which then holds
    `own` private rows of history; per agent: a hole of `hole` rows inside its private
    history (holes in aliased pages would have several agents store into one slot), then
    `tail` appended rows."""
    rng = np.random.default_rng(seed)
    ops = [("create", "root", 0), ("append", "root", fork_at + 5)]
    agents = []
    for j in range(n_agents):
        ops.append(("fork", "root", fork_at, f"a{j}"))
        ops.append(("append", f"a{j}", own + int(rng.integers(0, 20))))
        agents.append(f"a{j}")
    perm_b = rng.permutation(num_pages).astype(np.int32)
    perm_r = rng.permutation(num_pages).astype(np.int32)
    arrays = dict(
        bpool=encode(rng.standard_normal((num_pages, 2, Hkv, 16 * d)), dtype),
        rpool=encode(rng.standard_normal((num_pages, 2, 16 * r)), dtype),
        Bk=encode(b_std * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
        Bv=encode(b_std * rng.standard_normal((n_agents, r, Hkv * d)), dtype),
        q=encode(rng.standard_normal((n_agents, Hq, d)), dtype))
    geom = dict(num_bpages=num_pages, num_rpages=num_pages, num_kv_heads=Hkv, num_q_heads=Hq,
                head_dim=d, rank=r, dtype=dtype)
    C = hole + tail
    rows = dict(q=encode(rng.standard_normal((n_agents, C, Hq, d)), dtype),
                k_new=encode(rng.standard_normal((n_agents, C, Hkv, d)), dtype),
                v_new=encode(rng.standard_normal((n_agents, C, Hkv, d)), dtype),
                rk_new=encode(rng.standard_normal((n_agents, C, r)), dtype),
                rv_new=encode(rng.standard_normal((n_agents, C, r)), dtype))
    return rng, ops, agents, perm_b, perm_r, arrays, geom, rows


def _run(seed, dtype, d, r, Hq, Hkv, n_agents, fork_at, own, hole, tail, num_pages,
         samples=None, b_std=0.3):
    rng, ops, agents, perm_b, perm_r, arrays, geom, rows = _case(
        seed, dtype, d, r, Hq, Hkv, n_agents, fork_at, own, hole, tail, num_pages, b_std)
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, plan=False)
    lens = [b.pool.length(h) for h in b.handles]
    positions = []
    for L in lens:
        h0 = int(rng.integers(fork_at, L - hole + 1))
        positions.append(list(range(h0, h0 + hole)) + list(range(L, L + tail)))
    for h in b.handles:  # the tail rows are new; the hole rows exist already
        _, _, cow = b.pool.append(h, tail, want_slots=False)
        assert cow is None
    b.refresh_tables()
    positions = np.array(positions, dtype=np.int32)
    dev = {k: to_device(v) for k, v in rows.items()}
    out = torch.empty_like(dev["q"])
    out.fill_(float("nan") if dtype == "f32" else 0x7FC0)
    fk.residual_attn_prefill(b.pool, dev["q"], dev["k_new"], dev["v_new"], dev["rk_new"],
                             dev["rv_new"], b.Bk, b.Bv, b.btab, b.rtab, None, None, out,
                             2.0, 1.0 / np.sqrt(d), 5e5,
                             positions=torch.from_numpy(positions).cuda(),
                             positions_host=positions.tolist())
    torch.cuda.synchronize()
    geo = Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rank=r,
                   dtype=dtype)
    bt, rt = b.btab_host, b.rtab_host
    exp_b, exp_r = apply_rows_write(geo, arrays["bpool"], arrays["rpool"], bt, rt, positions,
                                    rows["k_new"], rows["v_new"], rows["rk_new"],
                                    rows["rv_new"])
    assert np.array_equal(_host(b.bcache, dtype).view(np.uint8), exp_b.view(np.uint8))
    assert np.array_equal(_host(b.rcache, dtype).view(np.uint8), exp_r.view(np.uint8))
    ref = prefill_attention_at(geo, arrays["bpool"], arrays["rpool"], bt, rt, positions,
                               rows["q"], rows["k_new"], rows["v_new"], rows["rk_new"],
                               rows["rv_new"], arrays["Bk"], arrays["Bv"], 2.0,
                               1.0 / np.sqrt(d), 5e5, samples=samples)
    return gpu_values(out, dtype), ref


@pytest.mark.parametrize("seed,dtype,d,r", [(0, "f32", 16, 4), (1, "bf16", 32, 8),
                                            (2, "bf16", 128, 16), (3, "bf16", 128, 16)])
def test_prefill_positions_tiny(seed, dtype, d, r):
    hole, tail = [(3, 4), (5, 11), (7, 9), (16, 16)][seed]
    g, ref = _run(500 + seed, dtype, d, r, Hq=8, Hkv=2, n_agents=3, fork_at=16, own=40,
                  hole=hole, tail=tail, num_pages=64)
    assert_close(g, ref, f"positions prefill seed={seed} {dtype}", scale_abs=True)


def test_prefill_positions_qwen3_shape():
    """Qwen3-8B attention shape (32 q / 8 KV heads, d = 128, r = 16, MFMA kernel): 2 agents
    sharing a 1024-token prefix with about 3000 private tokens each, a 96-row hole in the
    private history plus a 160-row tail in one launch; the workloads' value distributions
    (B ~ N(0, 0.02^2)); sampled rows against the oracle."""
    rng = np.random.default_rng(5)
    C = 256
    samples = [(int(a), int(i), int(g)) for a, i, g in
               zip(rng.integers(0, 2, 24), rng.integers(0, C, 24), rng.integers(0, 32, 24))]
    samples += [(0, 0, 0), (1, 95, 31), (0, 96, 5), (1, C - 1, 7)]  # hole ends, tail ends
    g, ref = _run(77, "bf16", 128, 16, Hq=32, Hkv=8, n_agents=2, fork_at=1024, own=3000,
                  hole=96, tail=160, num_pages=1024, samples=samples, b_std=0.02)
    mask = ~np.isnan(ref[..., 0])
    assert_close(g[mask], ref[mask], "positions prefill qwen3 shape")


def test_prefill_positions_errors():
    """Non-increasing positions, positions outside the tables and a softmax scale that is
    not positive are rejected."""
    rng, ops, agents, perm_b, perm_r, arrays, geom, rows = _case(9, "f32", 16, 4, 4, 2, 2, 16,
                                                                 20, 2, 2, 32)
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, plan=False)
    dev = {k: to_device(v) for k, v in rows.items()}
    out = torch.empty_like(dev["q"])
    for bad in ([[3, 3, 4, 5], [1, 2, 3, 4]], [[1, 2, 3, 2000], [1, 2, 3, 4]],
                [[-1, 2, 3, 4], [1, 2, 3, 4]]):
        with pytest.raises(fk.ForkKVError) as e:
            fk.residual_attn_prefill(b.pool, dev["q"], dev["k_new"], dev["v_new"],
                                     dev["rk_new"], dev["rv_new"], b.Bk, b.Bv, b.btab, b.rtab,
                                     None, None, out, 1.0, 0.25, 1e4,
                                     positions=torch.tensor(bad, dtype=torch.int32).cuda(),
                                     positions_host=bad)
        assert e.value.code == fk.EINVAL
    # a softmax scale that is not positive (valid positions)
    good = [[1, 2, 3, 4], [1, 2, 3, 4]]
    for sm in (-0.25, 0.0):
        with pytest.raises(fk.ForkKVError) as e:
            fk.residual_attn_prefill(b.pool, dev["q"], dev["k_new"], dev["v_new"],
                                     dev["rk_new"], dev["rv_new"], b.Bk, b.Bv, b.btab, b.rtab,
                                     None, None, out, 1.0, sm, 1e4,
                                     positions=torch.tensor(good, dtype=torch.int32).cuda(),
                                     positions_host=good)
        assert e.value.code == fk.EINVAL
