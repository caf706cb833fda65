"""The device-ceiling microbenchmarks the bench reports (read-only stream, bf16 MFMA loop,
SIMD pipe probes) compute what they claim: each result is checked against its closed form,
so a timing figure never comes from a kernel that skipped its work."""
from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bench  # noqa: E402


def _lib():
    return bench._microbench_lib()


def test_stream_read_sums_every_word():
    L = _lib()
    sp = torch.cuda.current_stream().cuda_stream
    n_bytes = 64 << 20
    buf = torch.arange(n_bytes // 4, dtype=torch.int32, device="cuda")
    expect = (n_bytes // 4) * (n_bytes // 4 - 1) // 2
    for variant in (0, 1, 2):
        part = torch.zeros(512, dtype=torch.int64, device="cuda")
        assert L.mb_stream_read(buf.data_ptr(), n_bytes, part.data_ptr(), 512, variant, sp) == 0
        torch.cuda.synchronize()
        assert int(part.sum().item()) == expect, f"variant {variant}"
    part = torch.zeros(8, dtype=torch.int64, device="cuda")
    assert L.mb_stream_read(buf.data_ptr(), n_bytes, part.data_ptr(), 8, 3, sp) != 0


def test_mfma_loop_accumulates_exactly():
    L = _lib()
    sp = torch.cuda.current_stream().cuda_stream
    ops = torch.tensor([0x3F80] * 8 + [0x3D00] * 8, dtype=torch.int16, device="cuda")
    blocks, iters = 64, 100
    out = torch.zeros(blocks * 4, dtype=torch.float32, device="cuda")
    assert L.mb_mfma_bf16(ops.data_ptr(), iters, out.data_ptr(), blocks, sp) == 0
    torch.cuda.synchronize()
    # A = 1, B = 1/32: each MFMA adds 32 * (1/32) = 1 to every element; 4 elements summed
    assert bool(torch.all(out == float(4 * L.mb_mfma_chains() * iters)))


@pytest.mark.parametrize("chains", [1, 2, 4, 16])
def test_pipe_probe_mfma_waves_do_their_work(chains):
    L = _lib()
    sp = torch.cuda.current_stream().cuda_stream
    ops = torch.tensor([0x3F80] * 8 + [0x3D00] * 8, dtype=torch.int16, device="cuda")
    blocks, iters = 32, 50
    out = torch.full((blocks * 8,), -1.0, dtype=torch.float32, device="cuda")
    assert L.mb_pipe_probe(0, 1, chains, ops.data_ptr(), iters, out.data_ptr(), blocks, sp) == 0
    torch.cuda.synchronize()
    o = out.view(blocks, 8).cpu()
    # waves 0-3: element 0 of every chain's accumulator, each chain 16 / chains MFMAs a trip
    assert bool(torch.all(o[:, :4] == float(16 * iters)))
    assert bool(torch.all(torch.isfinite(o[:, 4:])))


def test_pipe_probe_rejects_unknown_combinations():
    L = _lib()
    sp = torch.cuda.current_stream().cuda_stream
    ops = torch.zeros(16, dtype=torch.int16, device="cuda")
    out = torch.zeros(8, dtype=torch.float32, device="cuda")
    for mode, mfma, chains in ((4, 1, 4), (0, 0, 4), (1, 1, 3), (0, 2, 4)):
        assert L.mb_pipe_probe(mode, mfma, chains, ops.data_ptr(), 1, out.data_ptr(), 1, sp) != 0
