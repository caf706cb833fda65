"""The allocation-free decode entry point (for callers that cannot allocate), through the C ABI.

forkkv_residual_attn_decode_noalloc runs the same kernels as forkkv_residual_attn_decode with
the library's static split-K scratch in place of the caller's workspace.  Two calls in a row
on one GPU -- the Llama3-8B ReAct decode workload, then a smaller batch (and a generic-kernel
fp32 batch) -- must each give the bytes of the existing entry point; the second call reuses
the scratch the first one left behind.  A plan whose workspace exceeds the scratch is
refused before any device work.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from lora_shared_prefix_amd import forkkv as fk  # noqa: E402
from lora_shared_prefix_amd.session import DeviceBatch, workload_geom  # noqa: E402
from oracle.attention import Geometry, decode_attention  # noqa: E402
from tests.cases import tiny_case  # noqa: E402
from tests.gpu_common import apply_cows_host, assert_close, gpu_values, model_replay  # noqa: E402
from workloads import config_by_name, draw_inputs, pool_ops  # noqa: E402


def _both(b, s, sm, theta):
    """Output of the existing entry point and of the allocation-free one, same batch."""
    ref = b.decode(s, sm, theta).clone()
    out = torch.empty_like(ref)
    if out.dtype == torch.float32:
        out.fill_(float("nan"))
    else:
        out.fill_(0x7FC0)  # bf16 storage: the NaN bit pattern
    fk.residual_attn_decode_noalloc(b.pool, b.plan, b.q, b.Bk, b.Bv, b.btab, b.rtab, out, s, sm,
                                    theta, pstart=b.pstart)
    torch.cuda.synchronize()
    return ref, out


def _tiny(seed, dtype, kernel, d, r):
    case = tiny_case(seed, dtype, Hq=8, Hkv=2, d=d, r=r, n_agents=4, max_prefix=120,
                     max_suffix=40, num_pages=64)
    geom = dict(num_bpages=64, num_rpages=64, num_kv_heads=2, num_q_heads=8, head_dim=d, rank=r,
                dtype=dtype)
    b = DeviceBatch(geom, case, case["ops"], case["agents"], case["perm_b"], case["perm_r"],
                    kernel=kernel)
    return case, b


def test_noalloc_decode_matches_workspace_decode():
    cfg = config_by_name("llama3_8b_react_decode")
    print(f"[no-alloc] {cfg.name}", flush=True)
    x = draw_inputs(cfg)
    ops, agents = pool_ops(cfg)
    b = DeviceBatch(workload_geom(cfg), x, ops, agents, x["perm_b"], x["perm_r"])
    assert 0 < b.plan.info["workspace_bytes"] <= fk.NOALLOC_SCRATCH_BYTES
    sm = 1.0 / np.sqrt(cfg.head_dim)
    ref, out = _both(b, cfg.lora_scale, sm, cfg.rope_theta)
    same = torch.equal(ref.view(torch.int16), out.view(torch.int16))
    print(f"[no-alloc] {cfg.name}: bitwise equal={same}", flush=True)
    assert same
    del b
    # second call, smaller batch, on the scratch the first call left behind
    for seed, dtype, kernel, d, r in ((3, "bf16", fk.KERNEL_MFMA, 128, 16),
                                      (4, "f32", fk.KERNEL_GENERIC, 32, 8)):
        print(f"[no-alloc] tiny seed={seed} {dtype} kernel={kernel}", flush=True)
        case, b = _tiny(seed, dtype, kernel, d, r)
        assert b.plan.info["kernel"] == kernel
        ref, out = _both(b, case["lora_scale"], case["sm_scale"], case["theta"])
        view = torch.int16 if dtype == "bf16" else torch.int32
        same = torch.equal(ref.view(view), out.view(view))
        print(f"[no-alloc] tiny {dtype}: bitwise equal={same}", flush=True)
        assert same
        # and the oracle, on the model's tables and the packed-tail copies
        pm, names, cows = model_replay(64, 64, case["perm_b"], case["perm_r"], case["ops"])
        hs = [names[a] for a in case["agents"]]
        bt, rt, lens = (np.array(v) for v in pm.tables(hs, b.max_pages))
        host_b = apply_cows_host(case["bpool"], cows, 2, d)
        geo = Geometry(page_size=16, num_q_heads=8, num_kv_heads=2, head_dim=d, rank=r,
                       dtype=dtype)
        o = decode_attention(geo, host_b, case["rpool"], bt, rt, lens, case["q"], case["Bk"],
                             case["Bv"], case["lora_scale"], case["sm_scale"], case["theta"])
        assert_close(gpu_values(out, dtype), o, f"no-alloc tiny {dtype}", scale_abs=True)


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    """The Qwen2.5-14B batch planned for the generic kernel needs 188 MiB of partials: the
    call returns FORKKV_ETOOBIG before touching the device (the pool has no storage)."""
    cfg = config_by_name("qwen25_14b_batched_decode")
    pool = fk.Pool(cfg.num_bpages, cfg.num_rpages, cfg.num_kv_heads, cfg.head_dim, cfg.rank,
                   cfg.dtype)
    ops, agents = pool_ops(cfg)
    names, _ = pool.replay(ops)
    plan = fk.Plan(pool, [names[a] for a in agents], cfg.num_q_heads, kernel=fk.KERNEL_GENERIC)
    assert plan.info["workspace_bytes"] > fk.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(16, dtype=torch.int32, device="cuda").view(1, 16)
    with pytest.raises(fk.ForkKVError) as e:
        fk.residual_attn_decode_noalloc(pool, plan, t, t, t, t, t, t, 1.0, 0.1, 1e4)
    assert e.value.code == fk.ETOOBIG
