"""Seeded random shapes through the C ABI against the fp64 oracle.  Each case draws the dtype,
head dim, rank, KV heads, GQA group, agent count, prefix and suffix lengths and fork points
(decode: unaligned forks, so the device tail copies run too; prefill: page-aligned forks and
a chunk of 1 to 80 rows); the library picks the kernel (MFMA for bf16, d = 128, r = 16,
groups up to 16 -- drawn for half the cases -- else the generic one)."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from lora_shared_prefix_amd import forkkv as fk  # noqa: E402
from oracle.attention import Geometry, apply_chunk_write, decode_attention  # noqa: E402
from tests.cases import tiny_case  # noqa: E402
from tests.gpu_common import assert_close, errors, gpu_values  # noqa: E402
from tests.test_gpu_decode import _poison, _tiny_batch  # noqa: E402
from tests.test_gpu_prefill import _host, _run  # noqa: E402


def _supported(dtype, d, r, Hkv, G):
    """Whether the library plans a one-agent batch of this shape (a kernel covers it)."""
    pool = fk.Pool(4, 4, Hkv, d, r, dtype)
    root = pool.create(False)
    pool.append(root, 1)
    child, _ = pool.fork(root, 1)
    try:
        fk.Plan(pool, [child], G * Hkv)
        return True
    except fk.ForkKVError as e:
        if e.code != fk.EUNSUPPORTED:
            raise
        return False


def _draw(rng):
    while True:
        if rng.random() < 0.5:
            dtype, d, r = "bf16", 128, 16
        else:
            dtype = str(rng.choice(["f32", "bf16"]))
            d = int(rng.choice([16, 32, 64, 128]))
            r = int(rng.choice([4, 8, 12, 16]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        if _supported(dtype, d, r, Hkv, G):
            return dtype, d, r, Hkv, G


def _check(g, ref, dtype, what):
    assert_close(g, ref, what, scale_abs=True)
    if dtype == "f32":
        assert errors(g, ref)[1] < 1e-5, what


@pytest.mark.parametrize("seed", range(16))
def test_random_decode(seed):
    rng = np.random.default_rng(4200 + seed)
    dtype, d, r, Hkv, G = _draw(rng)
    n_agents = int(rng.integers(1, 9))
    max_prefix, max_suffix = int(rng.integers(1, 300)), int(rng.integers(1, 60))
    what = (f"random decode seed={seed} {dtype} d={d} r={r} Hkv={Hkv} G={G} N={n_agents} "
            f"prefix<={max_prefix} suffix<={max_suffix}")
    print(f"[gpu-random] {what}", flush=True)
    case, arrays, host_after, b, bt, rt, lens = _tiny_batch(
        4300 + seed, dtype, fk.KERNEL_AUTO, Hq=G * Hkv, Hkv=Hkv, d=d, r=r, n_agents=n_agents,
        max_prefix=max_prefix, max_suffix=max_suffix, num_pages=160)
    _poison(b.out)
    out = b.decode(case["lora_scale"], case["sm_scale"], case["theta"])
    torch.cuda.synchronize()
    ref = decode_attention(Geometry(page_size=16, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                                    head_dim=d, rank=r, dtype=dtype), host_after,
                           arrays["rpool"], bt, rt, lens, case["q"], case["Bk"], case["Bv"],
                           case["lora_scale"], case["sm_scale"], case["theta"])
    _check(gpu_values(out, dtype), ref, dtype, f"{what} kernel={b.plan.info['kernel']}")


@pytest.mark.parametrize("seed", range(8))
def test_random_prefill(seed):
    rng = np.random.default_rng(5200 + seed)
    dtype, d, r, Hkv, G = _draw(rng)
    n_agents = int(rng.integers(1, 5))
    C = int(rng.integers(1, 81))
    max_prefix, max_suffix = int(rng.integers(1, 120)), int(rng.integers(1, 40))
    what = (f"random prefill seed={seed} {dtype} d={d} r={r} Hkv={Hkv} G={G} N={n_agents} "
            f"C={C}")
    print(f"[gpu-random] {what}", flush=True)
    case = tiny_case(5300 + seed, dtype, Hq=G * Hkv, Hkv=Hkv, d=d, r=r, n_agents=n_agents,
                     chunk=C, max_prefix=max_prefix, max_suffix=max_suffix, num_pages=96)
    case["ops"] = [op if op[0] != "fork" else (op[0], op[1], (op[2] // 16) * 16, op[3])
                   for op in case["ops"]]
    geom = dict(num_bpages=96, num_rpages=96, num_kv_heads=Hkv, num_q_heads=G * Hkv,
                head_dim=d, rank=r, dtype=dtype)
    b, out, ref, bt, rt, start, g = _run(geom, case, case["ops"], case["agents"], case["perm_b"],
                                         case["perm_r"], C, case["lora_scale"], case["sm_scale"],
                                         case["theta"])
    exp_b, exp_r = apply_chunk_write(g, case["bpool"], case["rpool"], bt, rt, start,
                                     case["k_new"], case["v_new"], case["rk_new"], case["rv_new"])
    assert np.array_equal(_host(b.bcache, dtype).view(np.uint8), exp_b.view(np.uint8)), what
    assert np.array_equal(_host(b.rcache, dtype).view(np.uint8), exp_r.view(np.uint8)), what
    _check(gpu_values(out, dtype), ref, dtype, what)


# The largest shapes the pools accept: d = 256 and r = 64 (the generic kernel, whose LDS plan
# then exceeds the default 64 KiB), and the largest GQA group at each size.
MAX_SHAPES = [("f32", 256, 64, 2, 1), ("bf16", 256, 64, 1, 4), ("f32", 256, 16, 1, 32),
              ("bf16", 224, 64, 2, 8), ("bf16", 128, 16, 1, 64)]


@pytest.mark.parametrize("dtype,d,r,Hkv,G", MAX_SHAPES)
def test_max_shapes_decode(dtype, d, r, Hkv, G):
    what = f"max-shape decode {dtype} d={d} r={r} Hkv={Hkv} G={G}"
    print(f"[gpu-random] {what}", flush=True)
    case, arrays, host_after, b, bt, rt, lens = _tiny_batch(
        4400 + d + r + G, dtype, fk.KERNEL_AUTO, Hq=G * Hkv, Hkv=Hkv, d=d, r=r, n_agents=5,
        max_prefix=150, max_suffix=40, num_pages=96)
    _poison(b.out)
    out = b.decode(case["lora_scale"], case["sm_scale"], case["theta"])
    torch.cuda.synchronize()
    ref = decode_attention(Geometry(page_size=16, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                                    head_dim=d, rank=r, dtype=dtype), host_after,
                           arrays["rpool"], bt, rt, lens, case["q"], case["Bk"], case["Bv"],
                           case["lora_scale"], case["sm_scale"], case["theta"])
    _check(gpu_values(out, dtype), ref, dtype, f"{what} kernel={b.plan.info['kernel']}")


@pytest.mark.parametrize("dtype,d,r,Hkv,G", MAX_SHAPES)
def test_max_shapes_prefill(dtype, d, r, Hkv, G):
    C = 37
    what = f"max-shape prefill {dtype} d={d} r={r} Hkv={Hkv} G={G} C={C}"
    print(f"[gpu-random] {what}", flush=True)
    case = tiny_case(5400 + d + r + G, dtype, Hq=G * Hkv, Hkv=Hkv, d=d, r=r, n_agents=2,
                     chunk=C, max_prefix=60, max_suffix=20, num_pages=48)
    case["ops"] = [op if op[0] != "fork" else (op[0], op[1], (op[2] // 16) * 16, op[3])
                   for op in case["ops"]]
    geom = dict(num_bpages=48, num_rpages=48, num_kv_heads=Hkv, num_q_heads=G * Hkv,
                head_dim=d, rank=r, dtype=dtype)
    b, out, ref, bt, rt, start, g = _run(geom, case, case["ops"], case["agents"], case["perm_b"],
                                         case["perm_r"], C, case["lora_scale"], case["sm_scale"],
                                         case["theta"])
    exp_b, exp_r = apply_chunk_write(g, case["bpool"], case["rpool"], bt, rt, start,
                                     case["k_new"], case["v_new"], case["rk_new"], case["rv_new"])
    assert np.array_equal(_host(b.bcache, dtype).view(np.uint8), exp_b.view(np.uint8)), what
    assert np.array_equal(_host(b.rcache, dtype).view(np.uint8), exp_r.view(np.uint8)), what
    _check(gpu_values(out, dtype), ref, dtype, what)
