"""Chunked-prefill parity on the GPU: rows written bit-exactly, attention vs the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from lora_shared_prefix_amd.session import DeviceBatch, to_device, workload_geom  # noqa: E402
from oracle.attention import Geometry, apply_chunk_write, prefill_attention  # noqa: E402
from tests.cases import encode, tiny_case  # noqa: E402
from tests.gpu_common import assert_close, errors, gpu_values, model_tables  # noqa: E402
from workloads import chunk_ops, config_by_name, draw_inputs, pool_ops  # noqa: E402


def _host(t, dtype):
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if dtype == "bf16" else a


def _run(geom, arrays, ops, agents, perm_b, perm_r, C, s, sm, theta, samples=None,
         keep=None):
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, plan=False)
    pool_before = (arrays["bpool"], arrays["rpool"])
    start = b.reserve_chunk(C)
    chunk = {k: to_device(arrays[k]) for k in ("q", "k_new", "v_new", "rk_new", "rv_new")}
    if keep is not None:
        keep["chunk"] = chunk
    out = b.prefill(chunk, s, sm, theta)
    torch.cuda.synchronize()
    dtype = geom["dtype"]
    g = Geometry(page_size=16, num_q_heads=geom["num_q_heads"], num_kv_heads=geom["num_kv_heads"],
                 head_dim=geom["head_dim"], rank=geom["rank"], dtype=dtype)
    # oracle-side bookkeeping, then the expected pool contents after the write
    pm, hs, _, _, _ = model_tables(geom["num_bpages"], geom["num_rpages"], perm_b, perm_r, ops,
                                   agents, b.max_pages)
    for h in hs:
        pm.append(h, C)
    bt, rt, _ = pm.tables(hs, b.max_pages)
    bt, rt = np.array(bt, dtype=np.int32), np.array(rt, dtype=np.int32)
    assert np.array_equal(bt, b.btab_host) and np.array_equal(rt, b.rtab_host)
    ref = prefill_attention(g, pool_before[0], pool_before[1], bt, rt, np.array(start),
                            arrays["q"], arrays["k_new"], arrays["v_new"], arrays["rk_new"],
                            arrays["rv_new"], arrays["Bk"], arrays["Bv"], s, sm, theta,
                            samples=samples)
    return b, out, ref, bt, rt, start, g


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_tiny_prefill(seed, dtype):
    C = [5, 16, 23][seed]
    d, r = [(16, 4), (64, 8), (128, 16)][seed]
    case = tiny_case(900 + seed, dtype, Hq=8, Hkv=2, d=d, r=r, n_agents=3, chunk=C,
                     max_prefix=60, max_suffix=20)
    case["ops"] = [op if op[0] != "fork" else (op[0], op[1], (op[2] // 16) * 16, op[3])
                   for op in case["ops"]]
    geom = dict(num_bpages=64, num_rpages=64, num_kv_heads=2, num_q_heads=8, head_dim=d, rank=r,
                dtype=dtype)
    print(f"[gpu-prefill] tiny seed={seed} {dtype} C={C} d={d} r={r}", flush=True)
    b, out, ref, bt, rt, start, g = _run(geom, case, case["ops"], case["agents"], case["perm_b"],
                                         case["perm_r"], C, case["lora_scale"], case["sm_scale"],
                                         case["theta"])
    exp_b, exp_r = apply_chunk_write(g, case["bpool"], case["rpool"], bt, rt, start,
                                     case["k_new"], case["v_new"], case["rk_new"], case["rv_new"])
    # written rows are bit-exact and no other pool byte changed
    assert np.array_equal(_host(b.bcache, dtype).view(np.uint8), exp_b.view(np.uint8))
    assert np.array_equal(_host(b.rcache, dtype).view(np.uint8), exp_r.view(np.uint8))
    gv = gpu_values(out, dtype)
    assert_close(gv, ref, f"prefill tiny seed={seed} {dtype}", scale_abs=True)
    if dtype == "f32":
        assert errors(gv, ref)[1] < 1e-5


@pytest.mark.parametrize("G", [1, 3, 16])
def test_mfma_prefill_gqa_group_sizes(G):
    """The MFMA prefill kernel flattens (query, head of the group) into rows of 256-row
    blocks: G = 1 (one block), 3 (a block ends inside a query's heads) and 16 (seven blocks),
    over a 101-query chunk, so the last block is ragged."""
    C = 101
    case = tiny_case(930 + G, "bf16", Hq=2 * G, Hkv=2, d=128, r=16, n_agents=2, chunk=C,
                     max_prefix=70, max_suffix=20, num_pages=64)
    case["ops"] = [op if op[0] != "fork" else (op[0], op[1], (op[2] // 16) * 16, op[3])
                   for op in case["ops"]]
    geom = dict(num_bpages=64, num_rpages=64, num_kv_heads=2, num_q_heads=2 * G, head_dim=128,
                rank=16, dtype="bf16")
    print(f"[gpu-prefill] mfma G={G} C={C}", flush=True)
    b, out, ref, bt, rt, start, g = _run(geom, case, case["ops"], case["agents"], case["perm_b"],
                                         case["perm_r"], C, case["lora_scale"], case["sm_scale"],
                                         case["theta"])
    exp_b, exp_r = apply_chunk_write(g, case["bpool"], case["rpool"], bt, rt, start,
                                     case["k_new"], case["v_new"], case["rk_new"], case["rv_new"])
    assert np.array_equal(_host(b.bcache, "bf16").view(np.uint8), exp_b.view(np.uint8))
    assert np.array_equal(_host(b.rcache, "bf16").view(np.uint8), exp_r.view(np.uint8))
    assert_close(gpu_values(out, "bf16"), ref, f"prefill mfma G={G}", scale_abs=True)


def test_qwen3_shape_scaled_prefill():
    """Qwen3-8B attention shape (32/8 heads, d=128, r=16, theta 1e6) at a reduced prefix."""
    rng = np.random.default_rng(44)
    N, L, C = 3, 1000, 77
    nb, nr = 512, 512
    geom = dict(num_bpages=nb, num_rpages=nr, num_kv_heads=8, num_q_heads=32, head_dim=128,
                rank=16, dtype="bf16")
    arrays = dict(bpool=encode(rng.standard_normal((nb, 2, 8, 2048)), "bf16"),
                  rpool=encode(rng.standard_normal((nr, 2, 256)), "bf16"),
                  q=encode(rng.standard_normal((N, C, 32, 128)), "bf16"),
                  k_new=encode(rng.standard_normal((N, C, 8, 128)), "bf16"),
                  v_new=encode(rng.standard_normal((N, C, 8, 128)), "bf16"),
                  rk_new=encode(rng.standard_normal((N, C, 16)), "bf16"),
                  rv_new=encode(rng.standard_normal((N, C, 16)), "bf16"),
                  Bk=encode(0.02 * rng.standard_normal((N, 16, 1024)), "bf16"),
                  Bv=encode(0.02 * rng.standard_normal((N, 16, 1024)), "bf16"))
    ops = [("create", "root", 0), ("append", "root", L)]
    ops += [("fork", "root", 992, f"a{j}") for j in range(N)]
    ops += [("append", f"a{j}", 8 * j) for j in range(N)]
    agents = [f"a{j}" for j in range(N)]
    samples = [(a, i, g) for a in range(N) for i in (0, 1, 40, C - 1) for g in (0, 13, 31)]
    b, out, ref, *_ = _run(geom, arrays, ops, agents, rng.permutation(nb), rng.permutation(nr),
                           C, 2.0, 1 / np.sqrt(128), 1e6, samples=samples)
    gv = gpu_values(out, "bf16")
    idx = tuple(np.array(samples).T)
    assert np.all(np.isfinite(gv))
    assert_close(gv[idx], ref[idx], "qwen3-shape scaled prefill")


def test_qwen3_8b_chunked_prefill_workload():
    """The Qwen3-8B prefill workload at full size: 8 agents x 512-token chunks over a
    131072-token shared prefix.

    Written rows are checked bit for bit at sampled slots; attention is checked on sampled
    (agent, query, head) rows the oracle computes one by one, and so is the adapter's own
    contribution: a second call on the same batch with B = 0 (it stores the same rows again),
    (output with B) - (output with B = 0) against the oracle's difference, normwise <= 5e-2.
    """
    cfg = config_by_name("qwen3_8b_chunked_prefill")
    print(f"[gpu-prefill] drawing inputs of {cfg.name}", flush=True)
    x = draw_inputs(cfg)
    ops, agents = pool_ops(cfg)
    samples = [(a, i, g) for a in (0, 3, 7) for i in (0, 1, 255, 511) for g in (0, 17, 31)]
    keep = {}
    sm = 1 / np.sqrt(cfg.head_dim)
    b, out, ref, bt, rt, start, g = _run(workload_geom(cfg), x, ops, agents, x["perm_b"],
                                          x["perm_r"], cfg.chunk_len, cfg.lora_scale, sm,
                                          cfg.rope_theta, samples=samples, keep=keep)
    gv = gpu_values(out, "bf16")
    assert np.all(np.isfinite(gv))
    idx = tuple(np.array(samples).T)
    assert_close(gv[idx], ref[idx], "qwen3-8b chunked prefill (sampled rows)")
    # a sample of the written rows, bit for bit
    from oracle.storage import key_offset, res_key_offset, res_value_offset, value_offset
    bpool = _host(b.bcache, "bf16")
    rpool = _host(b.rcache, "bf16")
    dims, ranks = np.arange(128), np.arange(16)
    for a in (0, 5):
        for i in (0, 17, 511):
            t = start[a] + i
            page, row = bt[a][t // 16], t % 16
            for h in (0, 7):
                assert np.array_equal(bpool[page, 0, h, key_offset(row, dims)], x["k_new"][a, i, h])
                assert np.array_equal(bpool[page, 1, h, value_offset(row, dims)], x["v_new"][a, i, h])
            rpage = rt[a][t // 16]
            assert np.array_equal(rpool[rpage, 0, res_key_offset(row, ranks)], x["rk_new"][a, i])
            assert np.array_equal(rpool[rpage, 1, res_value_offset(row, ranks, 16)], x["rv_new"][a, i])
    # the adapter's contribution
    zB = np.zeros_like(x["Bk"])
    b.Bk, b.Bv = to_device(zB), to_device(zB)
    out0 = b.prefill(keep["chunk"], cfg.lora_scale, sm, cfg.rope_theta)
    torch.cuda.synchronize()
    g0 = gpu_values(out0, "bf16")[idx]
    r0 = prefill_attention(g, x["bpool"], x["rpool"], bt, rt, np.array(start), x["q"],
                           x["k_new"], x["v_new"], x["rk_new"], x["rv_new"], zB, zB,
                           cfg.lora_scale, sm, cfg.rope_theta, samples=samples)[idx]
    assert_close(g0, r0, "qwen3-8b chunked prefill, B = 0 (sampled rows)")
    dg, dr = gv[idx] - g0, ref[idx] - r0
    rel = np.linalg.norm(dg - dr) / np.linalg.norm(dr)
    print(f"[parity] qwen3-8b prefill residual delta rel={rel:.3e}", flush=True)
    assert rel <= 5e-2


@pytest.mark.parametrize("dtype,d,r,Hkv,G", [("bf16", 128, 16, 2, 4), ("f32", 256, 64, 1, 2)])
def test_prefill_graph_replay_matches_eager(dtype, d, r, Hkv, G):
    """A prefill call captured in a HIP graph (row write, then attention: the MFMA kernel, or
    at d = 256 the generic kernel with more than 64 KiB of LDS) gives the eager call's output
    and pool bytes on every replay (three replays, eager work on the output between them)."""
    C = 29
    case = tiny_case(960 + d, dtype, Hq=G * Hkv, Hkv=Hkv, d=d, r=r, n_agents=2, chunk=C,
                     max_prefix=50, max_suffix=20, num_pages=48)
    case["ops"] = [op if op[0] != "fork" else (op[0], op[1], (op[2] // 16) * 16, op[3])
                   for op in case["ops"]]
    geom = dict(num_bpages=48, num_rpages=48, num_kv_heads=Hkv, num_q_heads=G * Hkv,
                head_dim=d, rank=r, dtype=dtype)
    print(f"[gpu-prefill] graph replay {dtype} d={d} r={r} G={G}", flush=True)
    b = DeviceBatch(geom, case, case["ops"], case["agents"], case["perm_b"], case["perm_r"],
                    plan=False)
    b.reserve_chunk(C)
    chunk = {k: to_device(case[k]) for k in ("q", "k_new", "v_new", "rk_new", "rv_new")}
    args = (case["lora_scale"], case["sm_scale"], case["theta"])
    out = torch.empty_like(chunk["q"])
    b.prefill(chunk, *args, out=out)
    torch.cuda.synchronize()
    eager, pool_b, pool_r = out.clone(), b.bcache.clone(), b.rcache.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        b.prefill(chunk, *args, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(rep + 1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = (torch.equal(out, eager) and torch.equal(b.bcache, pool_b)
                and torch.equal(b.rcache, pool_r))
        print(f"[parity] prefill graph replay {rep}: bitwise equal={same}", flush=True)
        assert same
