"""Deferred RoPE where an error in it would show: a material adapter at long positions.

ForkKV study note, "4. 作者证明" (reproduction checks 3 and 6) and "7. 实现 cross-reference"
(core barrier 1): the residual key is up-projected first and rotated afterwards, at the
key's own position.  With B ~ N(0, 0.02^2) the residual key is a sixth of the base key and a
rotation error of a few hundredths of a radian hides under the output tolerance; here
B ~ N(0, 0.3^2) and s = 2 make the residual key about 2.4x the base key, and the keys reach
positions of about 131K (theta = 1e6), where every rotation angle is far from its reduced
value.  Covered:

* MFMA decode with the planner's split and with 64-page wave sub-ranges (the longest run of
  the per-page rotation recurrence), after unaligned (packed) forks;
* MFMA decode over a frozen tail (the slot-map instantiation re-anchors the rotation);
* MFMA prefill whose keys cross several fp64 re-anchors of its rotation recurrence, at a
  short and at a long prefix;
* the adapter's own contribution (output with B minus output with B = 0) against the
  oracle's, for each decode case and the short prefill.
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
from oracle.attention import Geometry, decode_attention, prefill_attention  # noqa: E402
from tests.cases import encode  # noqa: E402
from tests.gpu_common import (apply_cows_host, assert_close, gpu_values,  # noqa: E402
                              model_replay)

B_STD = 0.3
S = 2.0
THETA = 1e6
HQ, HKV, D, R = 8, 2, 128, 16
SM = 1.0 / np.sqrt(D)
GEO = Geometry(page_size=16, num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, rank=R, dtype="bf16")
RESIDUAL_DELTA = 5e-2


def _residual_delta(gB, g0, rB, r0, what):
    dg, dr = gB - g0, rB - r0
    rel = float(np.linalg.norm(dg - dr) / np.linalg.norm(dr))
    print(f"[parity] {what}: residual delta rel={rel:.3e} (|dr|/|r|="
          f"{np.linalg.norm(dr) / np.linalg.norm(rB):.2f})", flush=True)
    assert rel <= RESIDUAL_DELTA


_DECODE = {}


def _decode_inputs(freeze):
    """4 agents over a 130,053-token root (forks at its unaligned end) with 1 - 1019 private
    rows each: keys at positions up to 131,071."""
    if freeze in _DECODE:
        return _DECODE[freeze]
    _DECODE.clear()
    rng = np.random.default_rng(4100 + int(freeze))
    L0, suffix = 130_053, [900, 1019, 517, 1]
    nb, nr = 8448, 33024
    ops = [("create", "root", 0), ("append", "root", L0)]
    for j in range(4):
        ops.append(("fork", "root", L0, f"a{j}") + ((fk.FORK_FREEZE, 0) if freeze else ()))
    ops += [("append", f"a{j}", n) for j, n in enumerate(suffix)]
    agents = [f"a{j}" for j in range(4)]
    print(f"[gpu-rope] drawing decode inputs (freeze={freeze})", flush=True)
    arrays = dict(bpool=encode(rng.standard_normal((nb, 2, HKV, 16 * D), dtype=np.float32), "bf16"),
                  rpool=encode(rng.standard_normal((nr, 2, 16 * R), dtype=np.float32), "bf16"),
                  q=encode(rng.standard_normal((4, HQ, D)), "bf16"),
                  Bk=encode(B_STD * rng.standard_normal((4, R, HKV * D)), "bf16"),
                  Bv=encode(B_STD * rng.standard_normal((4, R, HKV * D)), "bf16"))
    perm_b = rng.permutation(nb).astype(np.int32)
    perm_r = rng.permutation(nr).astype(np.int32)
    geom = dict(num_bpages=nb, num_rpages=nr, num_kv_heads=HKV, num_q_heads=HQ, head_dim=D,
                rank=R, dtype="bf16")
    # oracle-side tables, slot map and packed-tail row copies from the pool model (the
    # library must agree bit for bit)
    pm, names, cows = model_replay(nb, nr, perm_b, perm_r, ops)
    hs = [names[a] for a in agents]
    mp = max(len(pm.seqs[h].bpages) for h in hs)
    bt, rt, lens = (np.array(x) for x in pm.tables(hs, mp))
    st = np.array(pm.starts_table(hs, mp)) if freeze else None
    host_b = apply_cows_host(arrays["bpool"], cows, HKV, D)
    _DECODE[freeze] = (geom, arrays, ops, agents, perm_b, perm_r, bt, rt, lens, st, host_b)
    return _DECODE[freeze]


@pytest.mark.parametrize("freeze,pages_per_wave", [(False, 0), (False, 64), (True, 0)])
def test_decode_strong_adapter_long_positions(freeze, pages_per_wave):
    geom, arrays, ops, agents, perm_b, perm_r, bt, rt, lens, st, bpool = _decode_inputs(freeze)
    print(f"[gpu-rope] decode freeze={freeze} pages/wave={pages_per_wave or 'planner'} "
          f"lens={list(lens)}", flush=True)
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, kernel=fk.KERNEL_MFMA,
                    pages_per_item=pages_per_wave)
    assert b.plan.info["kernel"] == fk.KERNEL_MFMA
    assert np.array_equal(b.btab_host[:, :bt.shape[1]], bt) and list(b.lens) == list(lens)
    assert (b.pstart is not None) == freeze
    assert np.array_equal(b.bcache.cpu().numpy().view(np.uint16), bpool)  # the row copies
    outs = {}
    for tag, Bk, Bv in (("B", arrays["Bk"], arrays["Bv"]),
                        ("0", np.zeros_like(arrays["Bk"]), np.zeros_like(arrays["Bv"]))):
        b.Bk, b.Bv = to_device(Bk), to_device(Bv)
        b.out.fill_(0x7FC0)
        out = b.decode(S, SM, THETA)
        torch.cuda.synchronize()
        ref = decode_attention(GEO, bpool, arrays["rpool"], bt, rt, lens, arrays["q"], Bk, Bv,
                               S, SM, THETA, starts=st)
        g = gpu_values(out, "bf16")
        assert_close(g, ref, f"decode long strong adapter freeze={freeze} B={tag}",
                     scale_abs=True)
        outs[tag] = (g, ref)
    _residual_delta(outs["B"][0], outs["0"][0], outs["B"][1], outs["0"][1],
                    f"decode long freeze={freeze} ppw={pages_per_wave}")


def _prefill_case(seed, L0, fork_at, C, samples):
    rng = np.random.default_rng(seed)
    n_ag = 2
    nb = (L0 + 16) // 16 + n_ag * ((C + 31) // 16) + 8
    nr = n_ag * ((L0 + C) // 16 + 4)
    arrays = dict(bpool=encode(rng.standard_normal((nb, 2, HKV, 16 * D), dtype=np.float32), "bf16"),
                  rpool=encode(rng.standard_normal((nr, 2, 16 * R), dtype=np.float32), "bf16"),
                  q=encode(rng.standard_normal((n_ag, C, HQ, D)), "bf16"),
                  k_new=encode(rng.standard_normal((n_ag, C, HKV, D)), "bf16"),
                  v_new=encode(rng.standard_normal((n_ag, C, HKV, D)), "bf16"),
                  rk_new=encode(rng.standard_normal((n_ag, C, R)), "bf16"),
                  rv_new=encode(rng.standard_normal((n_ag, C, R)), "bf16"),
                  Bk=encode(B_STD * rng.standard_normal((n_ag, R, HKV * D)), "bf16"),
                  Bv=encode(B_STD * rng.standard_normal((n_ag, R, HKV * D)), "bf16"))
    ops = [("create", "root", 0), ("append", "root", L0)]
    ops += [("fork", "root", fork_at[j], f"a{j}") for j in range(n_ag)]
    agents = [f"a{j}" for j in range(n_ag)]
    geom = dict(num_bpages=nb, num_rpages=nr, num_kv_heads=HKV, num_q_heads=HQ, head_dim=D,
                rank=R, dtype="bf16")
    perm_b, perm_r = rng.permutation(nb).astype(np.int32), rng.permutation(nr).astype(np.int32)
    b = DeviceBatch(geom, arrays, ops, agents, perm_b, perm_r, plan=False)
    start = b.reserve_chunk(C)
    # the model's view: packed-tail copies of the forks, then the chunk reservation
    pm, names, cows = model_replay(nb, nr, perm_b, perm_r,
                                   ops + [("append", a, C) for a in agents])
    hs = [names[a] for a in agents]
    bt, rt, _ = (np.array(x) for x in pm.tables(hs, b.max_pages))
    assert np.array_equal(bt, b.btab_host) and np.array_equal(rt, b.rtab_host)
    assert [pm.length(h) - C for h in hs] == list(start)
    pool_b = apply_cows_host(arrays["bpool"], cows, HKV, D)
    chunk = {k: to_device(arrays[k]) for k in ("q", "k_new", "v_new", "rk_new", "rv_new")}
    outs = {}
    for tag, Bk, Bv in (("B", arrays["Bk"], arrays["Bv"]),
                        ("0", np.zeros_like(arrays["Bk"]), np.zeros_like(arrays["Bv"]))):
        b.Bk, b.Bv = to_device(Bk), to_device(Bv)
        # the second call stores the same rows again, then attends with B = 0
        out = b.prefill(chunk, S, SM, THETA)
        torch.cuda.synchronize()
        ref = prefill_attention(GEO, pool_b, arrays["rpool"], bt, rt, np.array(start),
                                arrays["q"], arrays["k_new"], arrays["v_new"], arrays["rk_new"],
                                arrays["rv_new"], Bk, Bv, S, SM, THETA, samples=samples)
        g = gpu_values(out, "bf16")
        if samples is not None:
            idx = tuple(np.array(samples).T)
            g, ref = g[idx], ref[idx]
        outs[tag] = (g, ref)
    return start, outs


def test_prefill_strong_adapter_crosses_reanchors():
    """MFMA prefill, keys 0 .. ~4140: the rotation recurrence (two pages per iteration) is
    re-anchored in fp64 every 1024 positions, four times here; every output row checked."""
    start, outs = _prefill_case(4200, 4000, [3990, 3997], 150, None)
    print(f"[gpu-rope] prefill starts={start}", flush=True)
    for tag in ("B", "0"):
        assert_close(*outs[tag], f"prefill strong adapter B={tag}", scale_abs=True)
    _residual_delta(outs["B"][0], outs["0"][0], outs["B"][1], outs["0"][1], "prefill 4K")


def test_prefill_strong_adapter_long_prefix():
    """MFMA prefill at positions about 98K (a 98,000-token root, two agents, 64-row chunks):
    96 re-anchors before the chunk; sampled rows."""
    C = 64
    samples = [(a, i, g) for a in (0, 1) for i in (0, 1, 33, C - 1) for g in (0, 3, 5, 7)]
    start, outs = _prefill_case(4300, 98_000, [97_990, 98_000], C, samples)
    print(f"[gpu-rope] prefill starts={start}", flush=True)
    for tag in ("B", "0"):
        assert_close(*outs[tag], f"prefill long prefix B={tag}", scale_abs=True)
    _residual_delta(outs["B"][0], outs["0"][0], outs["B"][1], outs["0"][1], "prefill 98K")
