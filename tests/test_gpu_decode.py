"""Decode parity on the GPU: the HIP path (through the C ABI) against the fp64 oracle."""
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
from tests.cases import encode, tiny_case  # noqa: E402
from tests.gpu_common import (apply_cows_host, assert_close, errors, gpu_values,  # noqa: E402
                              model_tables, poison_unused, used_rows)
from workloads import config_by_name, draw_inputs, pool_ops  # noqa: E402

KERNELS = [fk.KERNEL_GENERIC, fk.KERNEL_MFMA]


def _kernel_available(cfg_like_dtype, d, r, G, kernel):
    if kernel == fk.KERNEL_GENERIC:
        return True
    return fk.lib() is not None and _mfma_ok(cfg_like_dtype, d, r, G)


def _mfma_ok(dtype, d, r, G):
    # ask the library by planning a one-agent batch
    p = fk.Pool(4, 4, 1, d, r, dtype)
    root = p.create(False)
    p.append(root, 1)
    c, _ = p.fork(root, 1)
    try:
        fk.Plan(p, [c], G, kernel=fk.KERNEL_MFMA)
        return True
    except fk.ForkKVError:
        return False


_CACHE = {}


def _poison(t):
    """Fill an output tensor with NaN (fp32) or the bf16 NaN bit pattern (16-bit storage)."""
    if t.dtype == torch.float32:
        t.fill_(float("nan"))
    else:
        t.fill_(0x7FC0)


def _workload(name):
    if name not in _CACHE:
        cfg = config_by_name(name)
        print(f"[gpu-decode] drawing inputs of {cfg.name}", flush=True)
        _CACHE.clear()
        _CACHE[name] = (cfg, draw_inputs(cfg))
    return _CACHE[name]


def _run_workload(name, kernel, sample_agents=None, sample_heads=None, arrays=None):
    cfg, x = _workload(name)
    if arrays is not None:
        x = dict(x, **arrays)
    ops, agents = pool_ops(cfg)
    print(f"[gpu-decode] {cfg.name} kernel={kernel}", flush=True)
    b = DeviceBatch(workload_geom(cfg), x, ops, agents, x["perm_b"], x["perm_r"], kernel=kernel)
    # bookkeeping on the real run is bit-exact against the model
    _, _, bt, rt, lens = model_tables(cfg.num_bpages, cfg.num_rpages, x["perm_b"], x["perm_r"],
                                      ops, agents, b.max_pages)
    assert np.array_equal(bt, b.btab_host) and np.array_equal(rt, b.rtab_host)
    assert list(lens) == list(b.lens)
    sm = 1.0 / np.sqrt(cfg.head_dim)
    _poison(b.out)  # every output row must be written by the call
    out = b.decode(cfg.lora_scale, sm, cfg.rope_theta)
    torch.cuda.synchronize()
    g = gpu_values(out, cfg.dtype)
    ref = decode_attention(Geometry.of(cfg), x["bpool"], x["rpool"], bt, rt, lens, x["q"], x["Bk"],
                           x["Bv"], cfg.lora_scale, sm, cfg.rope_theta, agents=sample_agents,
                           kv_heads=sample_heads)
    mask = ~np.isnan(ref[..., 0])
    return cfg, g, ref, mask


@pytest.mark.parametrize("kernel", KERNELS)
def test_tiny_fp32_workload(kernel):
    cfg = config_by_name("tiny_f32")
    if not _kernel_available(cfg.dtype, cfg.head_dim, cfg.rank, cfg.group, kernel):
        pytest.skip("kernel does not cover this shape")
    cfg, g, ref, mask = _run_workload("tiny_f32", kernel)
    assert_close(g, ref, "tiny fp32")
    a, rel = errors(g, ref)
    assert rel < 1e-5  # fp32 throughout


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name,agents,heads", [
    ("llama3_8b_react_decode", None, None),
    ("llama3_8b_mapreduce_decode", None, [0, 3, 7]),
    ("qwen25_14b_batched_decode", [0, 9, 18, 31], [0, 5]),
])
def test_bf16_workloads(kernel, name, agents, heads):
    cfg = config_by_name(name)
    if not _kernel_available(cfg.dtype, cfg.head_dim, cfg.rank, cfg.group, kernel):
        pytest.skip("kernel does not cover this shape")
    cfg, g, ref, mask = _run_workload(name, kernel, agents, heads)
    assert np.all(np.isfinite(g))
    assert_close(g[mask], ref[mask], cfg.name)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name,agents,heads", [
    ("llama3_8b_react_decode", None, None),
    ("llama3_8b_mapreduce_decode", None, [0, 3, 7]),
    ("qwen25_14b_batched_decode", [0, 9, 18, 31], [0, 5]),
])
def test_residual_delta(kernel, name, agents, heads):
    """The adapter's contribution itself must match, not only the (base-dominated) output:
    (output with B) - (output with B = 0) against the oracle's same difference, normwise
    within 5e-2, on every decode workload (sampled agents and heads as above)."""
    cfg = config_by_name(name)
    if not _kernel_available(cfg.dtype, cfg.head_dim, cfg.rank, cfg.group, kernel):
        pytest.skip("kernel does not cover this shape")
    _, gB, rB, mask = _run_workload(name, kernel, agents, heads)
    x = _CACHE[name][1]
    zero = {"Bk": np.zeros_like(x["Bk"]), "Bv": np.zeros_like(x["Bv"])}
    _, g0, r0, _ = _run_workload(name, kernel, agents, heads, arrays=zero)
    dg, dr = (gB - g0)[mask], (rB - r0)[mask]
    rel = np.linalg.norm(dg - dr) / np.linalg.norm(dr)
    print(f"[parity] {name} residual delta rel={rel:.3e}", flush=True)
    assert rel <= 5e-2


def _tiny_batch(seed, dtype, kernel, poison=True, **kw):
    case = tiny_case(seed, dtype, **kw)
    geom = dict(num_bpages=case["num_bpages"], num_rpages=case["num_rpages"],
                num_kv_heads=case["Hkv"], num_q_heads=case["Hq"], head_dim=case["d"],
                rank=case["r"], dtype=dtype)
    pm, hs, bt, rt, lens = model_tables(case["num_bpages"], case["num_rpages"], case["perm_b"],
                                        case["perm_r"], case["ops"], case["agents"], 32)
    # the fork packs of unaligned tails copy rows on the device; mirror them on the host
    cows = []
    pm2 = type(pm)(case["num_bpages"], case["num_rpages"], 16, case["perm_b"], case["perm_r"])
    names = {}
    for op in case["ops"]:
        if op[0] == "create":
            names[op[1]] = pm2.create(bool(op[2]))
        elif op[0] == "append":
            c = pm2.append(names[op[1]], op[2])[2]
            cows += [c] if c else []
        else:
            names[op[3]], c = pm2.fork(names[op[1]], op[2])
            cows += [c] if c else []
    arrays = dict(case)
    if poison:
        ub, ur = used_rows(bt, rt, lens)
        # rows read by the copies must stay finite too
        for src, dst, n in cows:
            ub |= {(src, row) for row in range(n)}
        arrays["bpool"], arrays["rpool"] = poison_unused(case["bpool"], case["rpool"], ub, ur,
                                                         dtype, case["d"], case["r"])
    b = DeviceBatch(geom, arrays, case["ops"], case["agents"], case["perm_b"], case["perm_r"],
                    kernel=kernel)
    assert b.cows == cows
    host_after = apply_cows_host(arrays["bpool"], cows, case["Hkv"], case["d"])
    return case, arrays, host_after, b, bt, rt, lens


RAGGED = [(0, "f32", fk.KERNEL_GENERIC), (1, "f32", fk.KERNEL_GENERIC),
          (2, "f32", fk.KERNEL_GENERIC), (3, "f32", fk.KERNEL_GENERIC),
          (0, "bf16", fk.KERNEL_GENERIC), (1, "bf16", fk.KERNEL_GENERIC),
          (2, "bf16", fk.KERNEL_GENERIC), (3, "bf16", fk.KERNEL_GENERIC),
          (2, "bf16", fk.KERNEL_MFMA), (4, "bf16", fk.KERNEL_MFMA), (5, "bf16", fk.KERNEL_MFMA),
          (6, "bf16", fk.KERNEL_MFMA)]


@pytest.mark.parametrize("seed,dtype,kernel", RAGGED)
def test_ragged_tiny_batches(seed, dtype, kernel):
    """Odd lengths, unaligned forks (device row copy), NaN in every unread slot."""
    d, r = [(16, 4), (64, 8), (128, 16), (32, 12), (128, 16), (128, 16), (128, 16)][seed]
    Hq = [8, 8, 8, 8, 8, 20, 16][seed]  # G = 4, 10 (one agent per group), 8
    case, arrays, host_after, b, bt, rt, lens = _tiny_batch(
        700 + seed, dtype, kernel, Hq=Hq, Hkv=2, d=d, r=r, n_agents=[5, 5, 5, 5, 7, 3, 6][seed],
        max_prefix=[70, 70, 70, 70, 300, 90, 200][seed], max_suffix=40, num_pages=128)
    assert b.plan.info["kernel"] == kernel
    # the copy-on-write rows landed bit-exactly
    got_pool = b.bcache.cpu().numpy()
    got_pool = got_pool.view(np.uint16) if dtype == "bf16" else got_pool
    assert np.array_equal(got_pool.view(np.uint8), host_after.view(np.uint8))
    _poison(b.out)  # every output row must be written by the call
    out = b.decode(case["lora_scale"], case["sm_scale"], case["theta"])
    torch.cuda.synchronize()
    ref = decode_attention(Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=2, head_dim=d,
                                    rank=r, dtype=dtype), host_after, arrays["rpool"], bt, rt,
                           lens, case["q"], case["Bk"], case["Bv"], case["lora_scale"],
                           case["sm_scale"], case["theta"])
    g = gpu_values(out, dtype)
    assert_close(g, ref, f"ragged seed={seed} {dtype} kernel={kernel}", scale_abs=True)
    if dtype == "f32":
        assert errors(g, ref)[1] < 1e-5


@pytest.mark.parametrize("G", [1, 2, 3, 16])
def test_mfma_gqa_group_sizes(G):
    """GQA groups the other tests leave out: G = 1 (one query head per KV head, four columns
    of a wave's 16 used), 2, 3 (columns not a power of two) and 16 (one agent per wave, every
    column used); ragged lengths and unaligned forks as above."""
    case, arrays, host_after, b, bt, rt, lens = _tiny_batch(
        760 + G, "bf16", fk.KERNEL_MFMA, Hq=2 * G, Hkv=2, d=128, r=16, n_agents=6,
        max_prefix=200, max_suffix=40, num_pages=128)
    assert b.plan.info["kernel"] == fk.KERNEL_MFMA
    print(f"[gpu-decode] G={G} lens={list(lens)}", flush=True)
    _poison(b.out)
    out = b.decode(case["lora_scale"], case["sm_scale"], case["theta"])
    torch.cuda.synchronize()
    ref = decode_attention(Geometry(page_size=16, num_q_heads=2 * G, num_kv_heads=2,
                                    head_dim=128, rank=16, dtype="bf16"), host_after,
                           arrays["rpool"], bt, rt, lens, case["q"], case["Bk"], case["Bv"],
                           case["lora_scale"], case["sm_scale"], case["theta"])
    assert_close(gpu_values(out, "bf16"), ref, f"mfma G={G}", scale_abs=True)


def test_placement_invariance_bitwise():
    """The same logical caches at other physical pages give bit-identical outputs."""
    case = tiny_case(801, "bf16", Hq=8, Hkv=2, d=128, r=16, n_agents=4, max_prefix=90,
                     max_suffix=40, num_pages=64)
    case["ops"] = [op if op[0] != "fork" else (op[0], op[1], (op[2] // 16) * 16, op[3])
                   for op in case["ops"]]  # aligned forks: no device copies needed
    outs = []
    for perm_seed in (0, 1):
        rng = np.random.default_rng(perm_seed)
        pb, pr = rng.permutation(64).astype(np.int32), rng.permutation(64).astype(np.int32)
        _, _, bt, rt, lens = model_tables(64, 64, pb, pr, case["ops"], case["agents"], 8)
        if perm_seed == 0:
            base = (case["bpool"], case["rpool"], bt, rt)
            bp, rp = case["bpool"], case["rpool"]
        else:
            bp, rp = case["bpool"].copy(), case["rpool"].copy()
            for a in range(len(lens)):
                for lp_ in range(-(-int(lens[a]) // 16)):
                    bp[bt[a][lp_]] = base[0][base[2][a][lp_]]
                    rp[rt[a][lp_]] = base[1][base[3][a][lp_]]
        geom = dict(num_bpages=64, num_rpages=64, num_kv_heads=2, num_q_heads=8, head_dim=128,
                    rank=16, dtype="bf16")
        b = DeviceBatch(geom, dict(case, bpool=bp, rpool=rp), case["ops"], case["agents"], pb, pr)
        outs.append(b.decode(case["lora_scale"], case["sm_scale"], case["theta"]).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_sharing_invariance():
    """Duplicating the shared prefix per agent (no aliasing) gives the same outputs."""
    cfg = config_by_name("llama3_8b_react_decode")
    cfg_small = dict(num_bpages=2048, num_rpages=4096, num_kv_heads=8, num_q_heads=32,
                     head_dim=128, rank=16, dtype="bf16")
    rng = np.random.default_rng(5)
    from tests.cases import encode
    L, ell, N = 512, 48, 3
    bp = encode(rng.standard_normal((2048, 2, 8, 2048)), "bf16")
    rp = encode(rng.standard_normal((4096, 2, 256)), "bf16")
    arrays = dict(bpool=bp, rpool=rp, q=encode(rng.standard_normal((N, 32, 128)), "bf16"),
                  Bk=encode(0.02 * rng.standard_normal((N, 16, 1024)), "bf16"),
                  Bv=encode(0.02 * rng.standard_normal((N, 16, 1024)), "bf16"))
    shared_ops = [("create", "root", 0), ("append", "root", L)]
    shared_ops += [("fork", "root", L, f"a{j}") for j in range(N)]
    shared_ops += [("append", f"a{j}", ell) for j in range(N)]
    agents = [f"a{j}" for j in range(N)]
    b1 = DeviceBatch(cfg_small, arrays, shared_ops, agents)
    o1 = b1.decode(2.0, 1 / np.sqrt(128), cfg.rope_theta)
    # private copies: each agent gets its own root and copies the shared pages' bytes
    priv_ops = []
    for j in range(N):
        priv_ops += [("create", f"r{j}", 0), ("append", f"r{j}", L), ("fork", f"r{j}", L, f"a{j}")]
    priv_ops += [("append", f"a{j}", ell) for j in range(N)]
    # logical content must match: copy pages so that each private prefix equals the shared one
    _, _, bt1, rt1, lens1 = model_tables(2048, 4096, None, None, shared_ops, agents, 40)
    _, _, bt2, rt2, lens2 = model_tables(2048, 4096, None, None, priv_ops, agents, 40)
    bp2, rp2 = bp.copy(), rp.copy()
    for a in range(N):
        for lp_ in range(-(-int(lens1[a]) // 16)):
            bp2[bt2[a][lp_]] = bp[bt1[a][lp_]]
            rp2[rt2[a][lp_]] = rp[rt1[a][lp_]]
    b2 = DeviceBatch(cfg_small, dict(arrays, bpool=bp2, rpool=rp2), priv_ops, agents)
    o2 = b2.decode(2.0, 1 / np.sqrt(128), cfg.rope_theta)
    torch.cuda.synchronize()
    assert_close(gpu_values(o1, "bf16"), gpu_values(o2, "bf16"), "sharing invariance",
                 max_abs=2e-3, max_rel=5e-3)


@pytest.mark.parametrize("kernel", KERNELS)
def test_graph_replay_matches_eager(kernel):
    """A decode call captured in a HIP graph gives the eager call's bytes on every replay
    (three replays, with eager work on the output between them)."""
    cfg, x = _workload("llama3_8b_react_decode")
    ops, agents = pool_ops(cfg)
    b = DeviceBatch(workload_geom(cfg), x, ops, agents, x["perm_b"], x["perm_r"], kernel=kernel)
    sm = 1.0 / np.sqrt(cfg.head_dim)
    eager = b.decode(cfg.lora_scale, sm, cfg.rope_theta).clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        b.decode(cfg.lora_scale, sm, cfg.rope_theta)
    torch.cuda.synchronize()
    for rep in range(3):
        b.out.fill_(float(rep + 1))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(b.out.view(torch.int16), eager.view(torch.int16))
        print(f"[parity] graph replay {rep} kernel={kernel}: bitwise equal={same}", flush=True)
        assert same


@pytest.mark.parametrize("kernel", KERNELS)
def test_many_partials_per_agent(kernel):
    """One page per split item: every agent's row merges well over 64 split-K partials, so
    the combine takes several chunks per row (the Llama3-8B ReAct workload, heads 0 and 5
    checked)."""
    cfg, x = _workload("llama3_8b_react_decode")
    ops, agents = pool_ops(cfg)
    b = DeviceBatch(workload_geom(cfg), x, ops, agents, x["perm_b"], x["perm_r"], kernel=kernel,
                    pages_per_item=1)
    assert b.plan.info["n_slots"] > 64 * len(agents)
    sm = 1.0 / np.sqrt(cfg.head_dim)
    _poison(b.out)
    out = b.decode(cfg.lora_scale, sm, cfg.rope_theta)
    torch.cuda.synchronize()
    _, _, bt, rt, lens = model_tables(cfg.num_bpages, cfg.num_rpages, x["perm_b"], x["perm_r"],
                                      ops, agents, b.max_pages)
    ref = decode_attention(Geometry.of(cfg), x["bpool"], x["rpool"], bt, rt, lens, x["q"], x["Bk"],
                           x["Bv"], cfg.lora_scale, sm, cfg.rope_theta, kv_heads=[0, 5])
    mask = ~np.isnan(ref[..., 0])
    g = gpu_values(out, cfg.dtype)
    assert_close(g[mask], ref[mask], f"{cfg.name} one page per item kernel={kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_empty_agent_bf16_d128(kernel):
    """An agent with no keys next to short ones at the bf16, d = 128, r = 16 shape: its
    output is exactly zero, the others match the oracle."""
    rng = np.random.default_rng(11)
    Hkv, Hq, d, r, npg = 2, 8, 128, 16, 32
    geom = dict(num_bpages=npg, num_rpages=npg, num_kv_heads=Hkv, num_q_heads=Hq, head_dim=d,
                rank=r, dtype="bf16")
    arrays = dict(bpool=encode(rng.standard_normal((npg, 2, Hkv, 16 * d)), "bf16"),
                  rpool=encode(rng.standard_normal((npg, 2, 16 * r)), "bf16"),
                  q=encode(rng.standard_normal((3, Hq, d)), "bf16"),
                  Bk=encode(0.02 * rng.standard_normal((3, r, Hkv * d)), "bf16"),
                  Bv=encode(0.02 * rng.standard_normal((3, r, Hkv * d)), "bf16"))
    ops = [("create", "root", 0), ("append", "root", 37), ("fork", "root", 0, "a0"),
           ("fork", "root", 16, "a1"), ("append", "a1", 5), ("fork", "root", 37, "a2"),
           ("append", "a2", 40)]
    agents = ["a0", "a1", "a2"]
    b = DeviceBatch(geom, arrays, ops, agents, kernel=kernel)
    assert b.plan.info["kernel"] == kernel
    _poison(b.out)
    out = b.decode(2.0, 1.0 / np.sqrt(d), 5e5)
    torch.cuda.synchronize()
    g = gpu_values(out, "bf16")
    assert np.all(g[0] == 0.0)
    _, _, bt, rt, lens = model_tables(npg, npg, None, None, ops, agents, b.max_pages)
    host = apply_cows_host(arrays["bpool"], b.cows, Hkv, d)
    ref = decode_attention(Geometry(page_size=16, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                                    rank=r, dtype="bf16"), host, arrays["rpool"], bt, rt, lens,
                           arrays["q"], arrays["Bk"], arrays["Bv"], 2.0, 1.0 / np.sqrt(d), 5e5)
    assert_close(g[1:], ref[1:], f"empty agent bf16 d=128 kernel={kernel}", scale_abs=True)


def test_empty_agent_and_errors():
    geom = dict(num_bpages=16, num_rpages=16, num_kv_heads=1, num_q_heads=2, head_dim=16, rank=4,
                dtype="f32")
    rng = np.random.default_rng(0)
    arrays = dict(bpool=rng.standard_normal((16, 2, 1, 256)).astype(np.float32),
                  rpool=rng.standard_normal((16, 2, 64)).astype(np.float32),
                  q=rng.standard_normal((2, 2, 16)).astype(np.float32),
                  Bk=rng.standard_normal((2, 4, 16)).astype(np.float32),
                  Bv=rng.standard_normal((2, 4, 16)).astype(np.float32))
    ops = [("create", "root", 0), ("append", "root", 20), ("fork", "root", 0, "a0"),
           ("fork", "root", 16, "a1")]
    b = DeviceBatch(geom, arrays, ops, ["a0", "a1"])
    out = b.decode(1.0, 0.3, 1e4)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy()[0] == 0.0)      # no keys -> zeros
    assert np.all(np.isfinite(out.cpu().numpy()[1]))
    # workspace too small, tables too narrow
    with pytest.raises(fk.ForkKVError) as e:
        fk.residual_attn_decode(b.pool, b.plan, b.q, b.Bk, b.Bv, b.btab, b.rtab, b.out,
                                b.workspace[:1], 1.0, 0.3, 1e4)
    assert e.value.code == fk.EINVAL
    with pytest.raises(fk.ForkKVError) as e:
        fk.residual_attn_decode(b.pool, b.plan, b.q, b.Bk, b.Bv, b.btab[:, :0].contiguous(),
                                b.rtab, b.out, b.workspace, 1.0, 0.3, 1e4)
    assert e.value.code == fk.EINVAL
    # a softmax scale that is not positive and finite, theta <= 0
    for sm, theta in ((-0.3, 1e4), (0.0, 1e4), (float("nan"), 1e4), (0.3, 0.0)):
        with pytest.raises(fk.ForkKVError) as e:
            fk.residual_attn_decode(b.pool, b.plan, b.q, b.Bk, b.Bv, b.btab, b.rtab, b.out,
                                    b.workspace, 1.0, sm, theta)
        assert e.value.code == fk.EINVAL
    # device buffers off a 16-byte boundary
    qm = torch.empty(b.q.numel() + 1, dtype=b.q.dtype, device="cuda")[1:].view_as(b.q)
    with pytest.raises(fk.ForkKVError) as e:
        fk.residual_attn_decode(b.pool, b.plan, qm, b.Bk, b.Bv, b.btab, b.rtab, b.out,
                                b.workspace, 1.0, 0.3, 1e4)
    assert e.value.code == fk.EINVAL
    bm = torch.empty(b.bcache.numel() + 1, dtype=b.bcache.dtype, device="cuda")[1:]
    with pytest.raises(fk.ForkKVError) as e:
        fk.Pool(16, 16, 1, 16, 4, "f32", bcache=bm, rcache=b.rcache)
    assert e.value.code == fk.EINVAL
    # plan not uploaded
    p2 = fk.Plan(b.pool, b.handles, 2)
    with pytest.raises(fk.ForkKVError) as e:
        fk.residual_attn_decode(b.pool, p2, b.q, b.Bk, b.Bv, b.btab, b.rtab, b.out, b.workspace,
                                1.0, 0.3, 1e4)
    assert e.value.code == fk.ESTATE
