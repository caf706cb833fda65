"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names the passage it follows.  Together they are chosen so that a
plausible slip in the oracle (a sign in RoPE, a dropped scale or residual, a
wrong GQA map, an unrotated base key, a transposed operand, an off-by-one
position) fails at least one of them -- ``test_planted_mistakes_are_caught``
checks exactly that.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oatt
from oracle import PoolModel
from oracle.attention import (Geometry, apply_rows_write, decode_attention, merged_kv,
                              prefill_attention, prefill_attention_at)
from oracle.rope import inv_freq, rope_rotate, rope_unrotate
from oracle.storage import base_key_rows, base_value_rows, decode_values
from tests.bruteforce import brute_decode, brute_prefill, brute_prefill_at
from tests.cases import tiny_case
from tests.fused_model import fused_decode
from workloads import config_by_name, draw_inputs, pool_ops


def _nrel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _build(case, extra_appends=()):
    pm = PoolModel(case["num_bpages"], case["num_rpages"], case["P"], case["perm_b"],
                   case["perm_r"])
    names = pm.replay(case["ops"])
    hs = [names[a] for a in case["agents"]]
    for a, n in extra_appends:
        pm.append(names[a], n)
    bt, rt, lens = pm.tables(hs, 64)
    return np.array(bt, dtype=np.int32), np.array(rt, dtype=np.int32), np.array(lens), pm, hs


def _geo(case):
    return Geometry(page_size=case["P"], num_q_heads=case["Hq"], num_kv_heads=case["Hkv"],
                    head_dim=case["d"], rank=case["r"], dtype=case["dtype"])


def _oracle_decode(case, bt, rt, lens, **kw):
    return decode_attention(_geo(case), case["bpool"], case["rpool"], bt, rt, lens, case["q"],
                            case["Bk"], case["Bv"], case["lora_scale"], case["sm_scale"],
                            case["theta"], **kw)


def _brute(case, bt, rt, lens):
    return np.array(brute_decode(case["P"], case["Hq"], case["Hkv"], case["d"], case["r"],
                                 case["dtype"], case["bpool"], case["rpool"], bt, rt, lens,
                                 case["q"], case["Bk"], case["Bv"], case["lora_scale"],
                                 case["sm_scale"], case["theta"]))


# ---- C2: brute force on tiny inputs ---------------------------------------------------------

def test_tiny_config_matches_brute_force():
    """The tiny fp32 workload in full against the pure-Python scalar brute force."""
    cfg = config_by_name("tiny_f32")
    x = draw_inputs(cfg)
    pm = PoolModel(cfg.num_bpages, cfg.num_rpages, cfg.page_size, x["perm_b"], x["perm_r"])
    ops, agents = pool_ops(cfg)
    names = pm.replay(ops)
    bt, rt, lens = pm.tables([names[a] for a in agents], 8)
    bt, rt = np.array(bt), np.array(rt)
    geo = Geometry.of(cfg)
    sm = 1.0 / np.sqrt(cfg.head_dim)
    o = decode_attention(geo, x["bpool"], x["rpool"], bt, rt, lens, x["q"], x["Bk"], x["Bv"],
                         cfg.lora_scale, sm, cfg.rope_theta)
    b = brute_decode(16, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.rank, "f32",
                     x["bpool"], x["rpool"], bt, rt, lens, x["q"], x["Bk"], x["Bv"],
                     cfg.lora_scale, sm, cfg.rope_theta)
    assert _nrel(o, b) < 1e-12


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_random_tiny_decode_matches_brute_force(seed, dtype):
    """Odd lengths, unaligned forks, partial pages, d in {16, 32}, r in {4, 8, 12}."""
    d = [16, 32][seed % 2]
    r = [4, 8, 12][seed % 3]
    case = tiny_case(100 + seed, dtype, Hq=4, Hkv=2, d=d, r=r, n_agents=3)
    bt, rt, lens, _, _ = _build(case)
    assert _nrel(_oracle_decode(case, bt, rt, lens), _brute(case, bt, rt, lens)) < 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_random_tiny_prefill_matches_brute_force(seed):
    """Chunked prefill: write-then-attend with a causal mask that includes the query itself."""
    C = 5
    case = tiny_case(200 + seed, "f32", Hq=2, Hkv=1, d=16, r=4, n_agents=2, chunk=C)
    pm = PoolModel(64, 64, 16, case["perm_b"], case["perm_r"])
    names = pm.replay(case["ops"])
    hs = [names[a] for a in case["agents"]]
    start = np.array([pm.length(h) for h in hs])
    for h in hs:
        pm.append(h, C)
    bt, rt, _ = pm.tables(hs, 64)
    bt, rt = np.array(bt), np.array(rt)
    geo = _geo(case)
    args = (case["bpool"], case["rpool"], bt, rt, start, case["q"], case["k_new"], case["v_new"],
            case["rk_new"], case["rv_new"], case["Bk"], case["Bv"], case["lora_scale"],
            case["sm_scale"], case["theta"])
    o = prefill_attention(geo, *args)
    b = np.array(brute_prefill(16, 2, 1, 16, 4, "f32", *args))
    assert _nrel(o, b) < 1e-12
    # sampled rows equal the full computation bit for bit
    samples = [(1, 3, 0), (0, 0, 1), (0, 4, 0)]
    os_ = prefill_attention(geo, *args, samples=samples)
    for a, i, g in samples:
        assert np.array_equal(os_[a, i, g], o[a, i, g])


def _hole_case(seed, dtype="f32", Hq=2, Hkv=1, d=16, r=4):
    """Agents with a history; a hole inside it is refilled and a tail is appended: rows at
    strictly increasing positions [hole ..., tail ...] (Penelope review, 部件二)."""
    rng = np.random.default_rng(seed)
    case = tiny_case(seed, dtype, Hq=Hq, Hkv=Hkv, d=d, r=r, n_agents=2, max_prefix=60,
                     max_suffix=30)
    pm = PoolModel(64, 64, 16, case["perm_b"], case["perm_r"])
    names = pm.replay(case["ops"])
    hs = [names[a] for a in case["agents"]]
    lens = [pm.length(h) for h in hs]
    tail = 3
    hole = 2 if min(lens) >= 2 else 1
    positions = []
    for h, L in zip(hs, lens):
        h0 = int(rng.integers(0, L - hole + 1))
        positions.append(list(range(h0, h0 + hole)) + list(range(L, L + tail)))
        pm.append(h, tail)
    C = hole + tail
    bt, rt, _ = pm.tables(hs, 64)
    from tests.cases import encode
    n = len(hs)
    rows = dict(q=encode(rng.standard_normal((n, C, Hq, d)), dtype),
                k_new=encode(rng.standard_normal((n, C, Hkv, d)), dtype),
                v_new=encode(rng.standard_normal((n, C, Hkv, d)), dtype),
                rk_new=encode(rng.standard_normal((n, C, r)), dtype),
                rv_new=encode(rng.standard_normal((n, C, r)), dtype))
    return case, np.array(bt), np.array(rt), np.array(positions), rows


@pytest.mark.parametrize("seed", range(3))
def test_positions_prefill_matches_brute_force(seed):
    """Rows at arbitrary increasing positions (a refilled hole + an appended tail): all rows
    written first, each query attends to keys 0 .. its position."""
    case, bt, rt, positions, rows = _hole_case(300 + seed)
    assert all(p_[0] >= 0 for p_ in positions)
    geo = _geo(case)
    args = (case["bpool"], case["rpool"], bt, rt, positions, rows["q"], rows["k_new"],
            rows["v_new"], rows["rk_new"], rows["rv_new"], case["Bk"], case["Bv"],
            case["lora_scale"], case["sm_scale"], case["theta"])
    o = prefill_attention_at(geo, *args)
    b = np.array(brute_prefill_at(16, 2, 1, 16, 4, "f32", *args))
    assert _nrel(o, b) < 1e-12


def test_positions_prefill_is_decode_over_written_pools():
    """Each query equals one decode query over the pools after the write, with its own
    position + 1 keys (the plain definition, through the decode path of the oracle)."""
    case, bt, rt, positions, rows = _hole_case(311, Hq=4, Hkv=2)
    geo = _geo(case)
    o = prefill_attention_at(geo, case["bpool"], case["rpool"], bt, rt, positions, rows["q"],
                             rows["k_new"], rows["v_new"], rows["rk_new"], rows["rv_new"],
                             case["Bk"], case["Bv"], case["lora_scale"], case["sm_scale"],
                             case["theta"])
    bp, rp = apply_rows_write(geo, case["bpool"], case["rpool"], bt, rt, positions,
                              rows["k_new"], rows["v_new"], rows["rk_new"], rows["rv_new"])
    for a in range(positions.shape[0]):
        for i in range(positions.shape[1]):
            lens = np.zeros(positions.shape[0], dtype=np.int64)
            lens[a] = positions[a, i] + 1
            qa = np.zeros_like(rows["q"][:, 0])
            qa[a] = rows["q"][a, i]
            d_ = decode_attention(geo, bp, rp, bt, rt, lens, qa, case["Bk"], case["Bv"],
                                  case["lora_scale"], case["sm_scale"], case["theta"],
                                  agents=[a])
            assert _nrel(o[a, i], d_[a]) < 1e-12


def test_positions_prefill_contiguous_equals_chunked_prefill():
    """Contiguous positions start .. start + C - 1 reproduce the chunked prefill, which
    concatenates the chunk rows instead of reading the written pools."""
    C = 4
    case = tiny_case(321, "f32", Hq=2, Hkv=1, d=16, r=4, n_agents=2, chunk=C)
    pm = PoolModel(64, 64, 16, case["perm_b"], case["perm_r"])
    names = pm.replay(case["ops"])
    hs = [names[a] for a in case["agents"]]
    start = np.array([pm.length(h) for h in hs])
    for h in hs:
        pm.append(h, C)
    bt, rt, _ = pm.tables(hs, 64)
    bt, rt = np.array(bt), np.array(rt)
    geo = _geo(case)
    tail = (case["q"], case["k_new"], case["v_new"], case["rk_new"], case["rv_new"], case["Bk"],
            case["Bv"], case["lora_scale"], case["sm_scale"], case["theta"])
    o1 = prefill_attention(geo, case["bpool"], case["rpool"], bt, rt, start, *tail)
    positions = np.array([[int(s0) + i for i in range(C)] for s0 in start])
    o2 = prefill_attention_at(geo, case["bpool"], case["rpool"], bt, rt, positions, *tail)
    assert _nrel(o1, o2) < 1e-12


# ---- C1: zero adapter reduces to plain attention (library routine) --------------------------

@pytest.mark.parametrize("variant", ["zero_B", "zero_scale"])
def test_zero_adapter_equals_sdpa(variant):
    case = tiny_case(7, "f32", Hq=6, Hkv=2, d=16, r=4, n_agents=3)
    if variant == "zero_B":
        case["Bk"] = np.zeros_like(case["Bk"])
        case["Bv"] = np.zeros_like(case["Bv"])
    else:
        case["lora_scale"] = 0.0
    bt, rt, lens, _, _ = _build(case)
    o = _oracle_decode(case, bt, rt, lens)
    geo = _geo(case)
    for a in range(3):
        pos = np.arange(lens[a])
        K = np.stack([base_key_rows(case["bpool"], bt[a], pos, h, 16, 16, "f32") for h in range(2)])
        V = np.stack([base_value_rows(case["bpool"], bt[a], pos, h, 16, 16, "f32") for h in range(2)])
        K = torch.from_numpy(np.repeat(K, geo.G, axis=0))[None]
        V = torch.from_numpy(np.repeat(V, geo.G, axis=0))[None]
        q = torch.from_numpy(decode_values(case["q"][a], "f32"))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=case["sm_scale"])
        assert _nrel(o[a], ref[0, :, 0].numpy()) < 1e-12


# ---- missing pages (ForkKV study note, "Error / eviction recovery") -------------------------
# A base page evicted from every holder leaves table entries of -1 until it is refilled: its
# positions hold no key.  A sequence without residual pages has table entries of -1 there and
# a zero residual.

def _knock_out(bt, rt, lens, rng):
    """Mark one inner base page of each agent with keys as missing, and one residual page."""
    bt, rt = bt.copy(), rt.copy()
    for a in range(len(lens)):
        n = -(-int(lens[a]) // 16)
        if n >= 2:
            bt[a, int(rng.integers(0, n - 1))] = -1
        if n >= 1:
            rt[a, int(rng.integers(0, n))] = -1
    return bt, rt


@pytest.mark.parametrize("seed", range(3))
def test_missing_pages_decode_matches_brute_force(seed):
    case = tiny_case(150 + seed, "f32", Hq=4, Hkv=2, d=16, r=4, n_agents=3, max_prefix=60)
    bt, rt, lens, _, _ = _build(case)
    bt, rt = _knock_out(bt, rt, lens, np.random.default_rng(seed))
    assert (bt < 0).any() and (rt < 0).any()
    assert _nrel(_oracle_decode(case, bt, rt, lens), _brute(case, bt, rt, lens)) < 1e-12


def test_missing_pages_prefill_matches_brute_force():
    C = 5
    case = tiny_case(160, "f32", Hq=2, Hkv=1, d=16, r=4, n_agents=2, chunk=C, max_prefix=60)
    pm = PoolModel(64, 64, 16, case["perm_b"], case["perm_r"])
    names = pm.replay(case["ops"])
    hs = [names[a] for a in case["agents"]]
    start = np.array([pm.length(h) for h in hs])
    for h in hs:
        pm.append(h, C)
    bt, rt, lens = (np.array(x) for x in pm.tables(hs, 64))
    # base pages go missing only wholly before the chunk (the chunk's own rows are stored);
    # a residual page anywhere, the chunk's last page included
    bt2, rt2 = _knock_out(bt, rt, np.minimum(lens, start // 16 * 16 + 1),
                          np.random.default_rng(7))
    rt2[1, (int(lens[1]) - 1) // 16] = -1
    args = (case["bpool"], case["rpool"], bt2, rt2, start, case["q"], case["k_new"],
            case["v_new"], case["rk_new"], case["rv_new"], case["Bk"], case["Bv"],
            case["lora_scale"], case["sm_scale"], case["theta"])
    o = prefill_attention(_geo(case), *args)
    b = np.array(brute_prefill(16, 2, 1, 16, 4, "f32", *args))
    assert _nrel(o, b) < 1e-12


def test_missing_base_page_zero_adapter_equals_masked_sdpa():
    """With B = 0, attention over a sequence with a missing base page is the library routine
    with those keys masked out (and a missing residual page changes nothing)."""
    case = tiny_case(170, "f32", Hq=6, Hkv=2, d=16, r=4, n_agents=3, max_prefix=70)
    case["Bk"] = np.zeros_like(case["Bk"])
    case["Bv"] = np.zeros_like(case["Bv"])
    bt, rt, lens, _, _ = _build(case)
    bt2, rt2 = _knock_out(bt, rt, lens, np.random.default_rng(3))
    o = _oracle_decode(case, bt2, rt2, lens)
    geo = _geo(case)
    for a in range(3):
        pos = np.arange(lens[a])
        K = np.stack([base_key_rows(case["bpool"], bt[a], pos, h, 16, 16, "f32") for h in range(2)])
        V = np.stack([base_value_rows(case["bpool"], bt[a], pos, h, 16, 16, "f32") for h in range(2)])
        K = torch.from_numpy(np.repeat(K, geo.G, axis=0))[None]
        V = torch.from_numpy(np.repeat(V, geo.G, axis=0))[None]
        keep = torch.from_numpy(bt2[a][pos // 16] >= 0)[None, None, None, :]
        q = torch.from_numpy(decode_values(case["q"][a], "f32"))[None, :, None, :]
        if not bool(keep.any()):
            assert np.all(o[a] == 0.0)
            continue
        ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=keep,
                                                               scale=case["sm_scale"])
        assert _nrel(o[a], ref[0, :, 0].numpy()) < 1e-12


# ---- C3: RoPE invariants ------------------------------------------------------------------

def test_rope_invariants():
    rng = np.random.default_rng(3)
    d, theta = 16, 1e4
    pos = np.array([0, 1, 7, 1000, 131583], dtype=np.int64)
    a, b = rng.standard_normal((5, d)), rng.standard_normal((5, d))
    # linearity and orthogonality
    assert np.allclose(rope_rotate(a + 2.5 * b, pos, theta),
                       rope_rotate(a, pos, theta) + 2.5 * rope_rotate(b, pos, theta), atol=1e-12)
    assert np.allclose(np.linalg.norm(rope_rotate(a, pos, theta), axis=1),
                       np.linalg.norm(a, axis=1), atol=1e-12)
    # identity at position 0; inverse
    assert np.array_equal(rope_rotate(a[:1], np.array([0]), theta), a[:1])
    assert np.allclose(rope_unrotate(rope_rotate(a, pos, theta), pos, theta), a, atol=1e-9)
    # relative position: <R_m q, R_n k> = <q, R_{n-m} k>
    for m, n in [(3, 11), (500, 17), (131000, 131583)]:
        lhs = rope_rotate(a[:1], np.array([m]), theta) @ rope_rotate(b[:1], np.array([n]), theta).T
        rhs = a[:1] @ rope_rotate(b[:1], np.array([n - m]), theta).T
        assert abs(lhs - rhs).max() < 1e-9
    # d = 2 is a rotation by t radians (theta**0 = 1), counter-clockwise
    t = 0.75
    assert np.allclose(rope_rotate(np.array([[1.0, 0.0]]), np.array([t]), theta),
                       [[np.cos(t), np.sin(t)]], atol=1e-15)
    # pairing of dimension j with j + d/2 at frequency theta**(-2j/d)
    e = np.zeros((1, 8))
    e[0, 1] = 1.0
    w = theta ** (-2.0 / 8)
    assert np.allclose(rope_rotate(e, np.array([5]), theta)[0],
                       [0, np.cos(5 * w), 0, 0, 0, np.sin(5 * w), 0, 0], atol=1e-15)
    assert np.allclose(inv_freq(8, theta), theta ** (-np.arange(4) * 2.0 / 8), rtol=1e-15)


# ---- C4 / C5: deferred RoPE and associativity (reproduction checks 3 and 4) ------------------

def test_deferred_rope_and_associativity():
    case = tiny_case(11, "f32", Hq=4, Hkv=2, d=16, r=4, n_agents=2)
    bt, rt, lens, _, _ = _build(case)
    geo = _geo(case)
    s = case["lora_scale"]
    for a in range(2):
        pos = np.arange(lens[a])
        rk = oracle.res_key_rows(case["rpool"], rt[a], pos, 16, 4, "f32")
        rv = oracle.res_value_rows(case["rpool"], rt[a], pos, 16, 4, "f32")
        Bk = decode_values(case["Bk"][a], "f32")
        Bv = decode_values(case["Bv"][a], "f32")
        for h in range(2):
            bk = base_key_rows(case["bpool"], bt[a], pos, h, 16, 16, "f32")
            bv = base_value_rows(case["bpool"], bt[a], pos, h, 16, 16, "f32")
            K, V = merged_kv(geo, bk, bv, rk, rv, Bk, Bv, h, pos, s, case["theta"])
            cols = slice(16 * h, 16 * h + 16)
            # RoPE(xW + s xA B) = stored base + RoPE(s xA B)
            assert np.abs(K - (bk + rope_rotate(s * (rk @ Bk[:, cols]), pos, case["theta"]))).max() < 1e-12
            # Eq.(4): P (V_b + s V_r B_v) = P V_b + s (P V_r) B_v
            qv = decode_values(case["q"][a, 2 * h], "f32")
            p = np.exp(case["sm_scale"] * K @ qv)
            p /= p.sum()
            assert np.abs(p @ V - (p @ bv + s * (p @ rv) @ Bv[:, cols])).max() < 1e-12


# ---- C6: online softmax with split-K merge; the acc_r rescale matters (check 6) ------------

@pytest.mark.parametrize("seed", range(4))
def test_fused_split_k_form_equals_oracle(seed):
    case = tiny_case(300 + seed, "f32", Hq=4, Hkv=2, d=16, r=4, n_agents=3, max_prefix=70,
                     max_suffix=40)
    bt, rt, lens, _, _ = _build(case)
    rng = np.random.default_rng(seed)

    def splits(a, n):
        cuts = sorted(set(rng.integers(1, max(n, 2), size=3).tolist()) - {n})
        edges = [0] + [c for c in cuts if 0 < c < n] + [n]
        return [range(edges[i], edges[i + 1]) for i in range(len(edges) - 1)]

    args = (_geo(case), case["bpool"], case["rpool"], bt, rt, lens, case["q"], case["Bk"],
            case["Bv"], case["lora_scale"], case["sm_scale"], case["theta"])
    ref = decode_attention(*args)
    assert _nrel(fused_decode(*args, splits), ref) < 1e-12


def test_skipping_residual_rescale_is_detected():
    """The note's check 6: acc_r must be rescaled like acc, else B_v's term is misweighted."""
    case = tiny_case(400, "f32", Hq=4, Hkv=2, d=16, r=4, n_agents=2, max_prefix=70, max_suffix=40)
    case["Bv"] = (np.asarray(case["Bv"]) * 5).astype(np.float32)
    bt, rt, lens, _, _ = _build(case)
    args = (_geo(case), case["bpool"], case["rpool"], bt, rt, lens, case["q"], case["Bk"],
            case["Bv"], case["lora_scale"], case["sm_scale"], case["theta"])
    ref = decode_attention(*args)
    one = lambda a, n: [range(0, n)]
    assert _nrel(fused_decode(*args, one), ref) < 1e-12
    assert _nrel(fused_decode(*args, one, rescale_residual=False), ref) > 1e-3


# ---- the pins catch plausible mistakes planted in the oracle -------------------------------

def _mut_rope_sign(x, positions, theta):
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq(d, theta)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)


def _mut_rope_adjacent_pairs(x, positions, theta):
    d = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq(d, theta)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * c - x2 * s
    out[..., 1::2] = x2 * c + x1 * s
    return out


def _merged_variant(kind):
    def fn(geo, bk, bv, rk, rv, Bk_a, Bv_a, h, positions, lora_scale, theta):
        cols = slice(h * geo.d, (h + 1) * geo.d)
        xw = bk if kind == "no_unrotate" else rope_unrotate(bk, positions, theta)
        sk = 1.0 if kind == "drop_scale" else lora_scale
        Bkc = Bk_a[:, cols] if kind != "wrong_head_cols" else Bk_a[:, :geo.d]
        pos = positions + 1 if kind == "pos_off_by_one" else positions
        k = rope_rotate(xw + sk * (rk @ Bkc), pos, theta)
        v = bv if kind == "drop_v_residual" else bv + lora_scale * (rv @ Bv_a[:, cols])
        return k, v
    return fn


@pytest.mark.parametrize("mutation", ["rope_sign", "rope_pairs", "no_unrotate", "drop_scale",
                                      "wrong_head_cols", "pos_off_by_one", "drop_v_residual",
                                      "gqa_map"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    case = tiny_case(500, "f32", Hq=4, Hkv=2, d=16, r=4, n_agents=2)
    case["lora_scale"] = 2.0
    bt, rt, lens, _, _ = _build(case)
    if mutation == "rope_sign":
        monkeypatch.setattr(oatt, "rope_rotate", _mut_rope_sign)
        monkeypatch.setattr(oatt, "rope_unrotate",
                            lambda x, p, t: _mut_rope_sign(x, -np.asarray(p, dtype=np.float64), t))
    elif mutation == "rope_pairs":
        monkeypatch.setattr(oatt, "rope_rotate", _mut_rope_adjacent_pairs)
        monkeypatch.setattr(oatt, "rope_unrotate", lambda x, p, t: _mut_rope_adjacent_pairs(
            x, -np.asarray(p, dtype=np.float64), t))
    elif mutation == "gqa_map":
        real = oatt.Geometry.__init__

        def init(self, **kw):
            real(self, **kw)
            self.G = 1  # q head g would read KV head g // 1
        monkeypatch.setattr(oatt.Geometry, "__init__", init)
        case["Hq"], case["Hkv"] = 4, 2
    else:
        monkeypatch.setattr(oatt, "merged_kv", _merged_variant(mutation))
    brute = _brute(case, bt, rt, lens)
    try:
        o = _oracle_decode(case, bt, rt, lens)
    except (IndexError, ValueError):
        return  # the mistake crashed the oracle: caught
    assert not (_nrel(o, brute) < 1e-9), f"mutation {mutation} not detected"


# ---- storage layout: the documented tile orders are bijections with lane-linear reads ------

def test_tile_orders_are_permutations_with_lane_linear_operands():
    from oracle.storage import key_offset, res_key_offset, res_value_offset, value_offset
    t = np.arange(16)[:, None]
    for d in (16, 64, 128, 256):
        x = np.arange(d)[None, :]
        assert sorted(key_offset(t, x).ravel()) == list(range(16 * d))
        assert sorted(value_offset(t, x).ravel()) == list(range(16 * d))
    for r in (4, 8, 16, 64):
        k = np.arange(r)[None, :]
        assert sorted(res_key_offset(t, k).ravel()) == list(range(16 * r))
        assert sorted(res_value_offset(t, k, r).ravel()) == list(range(16 * r))
    # MFMA lane l (col = l % 16, g = l // 16): the piece it supplies is contiguous at l*size
    for l in range(64):
        col, g = l % 16, l // 16
        for c in range(4):      # key tile, 16x16x32 A operand: row col, dims 32c + 8g + e
            assert [key_offset(col, 32 * c + 8 * g + e) for e in range(8)] == \
                [512 * c + 8 * l + e for e in range(8)]
        for T in range(8):      # value tile, 16x16x16 A operand: dim 16T + col, rows 4g + e
            assert [value_offset(4 * g + e, 16 * T + col) for e in range(4)] == \
                [256 * T + 4 * l + e for e in range(4)]
        # residuals, r = 16: key as B operand (ranks 4g + e of row col), value as A operand
        assert [res_key_offset(col, 4 * g + e) for e in range(4)] == [4 * l + e for e in range(4)]
        assert [res_value_offset(4 * g + e, col, 16) for e in range(4)] == [4 * l + e for e in range(4)]


# ---- the slot map of frozen tails (ForkServe README, "Design vs APC") ----------------------

def _build_freeze(case):
    pm = PoolModel(case["num_bpages"], case["num_rpages"], case["P"], case["perm_b"],
                   case["perm_r"])
    names = pm.replay(case["ops"])
    hs = [names[a] for a in case["agents"]]
    bt, rt, lens = pm.tables(hs, 16)
    st = pm.starts_table(hs, 16)
    return np.array(bt), np.array(rt), np.array(lens), np.array(st), pm, hs


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_frozen_tail_decode_matches_brute_force(seed, dtype):
    """Decode over sequences holding frozen tails: the oracle's slot-map reading against the
    scalar brute force, which finds each position's page by a linear scan of the starts."""
    case = tiny_case(300 + seed, dtype, Hq=4, Hkv=2, d=16, r=4, n_agents=4, freeze=True)
    bt, rt, lens, st, _, _ = _build_freeze(case)
    assert (st[:, 1:] - st[:, :-1] < 16).any()  # there is a frozen tail somewhere
    o = _oracle_decode(case, bt, rt, lens, starts=st)
    b = np.array(brute_decode(case["P"], case["Hq"], case["Hkv"], case["d"], case["r"], dtype,
                              case["bpool"], case["rpool"], bt, rt, lens, case["q"], case["Bk"],
                              case["Bv"], case["lora_scale"], case["sm_scale"], case["theta"],
                              starts=st))
    assert _nrel(o, b) < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_frozen_tail_decode_equals_aligned_relayout(seed):
    """Moving every position's stored row into a fresh, aligned layout (page t // P, row
    t % P) leaves the decode unchanged: the slot map only relocates rows."""
    case = tiny_case(320 + seed, "f32", Hq=4, Hkv=2, d=16, r=4, n_agents=4, freeze=True)
    bt, rt, lens, st, _, _ = _build_freeze(case)
    geo = _geo(case)
    N, P = len(lens), 16
    n_pg = -(-int(lens.max()) // P)
    nb = N * n_pg
    bp2 = np.zeros((nb, 2, case["Hkv"], P * case["d"]), dtype=case["bpool"].dtype)
    rp2 = np.zeros((nb, 2, P * case["r"]), dtype=case["rpool"].dtype)
    bt2 = np.arange(nb).reshape(N, n_pg)
    from oracle.storage import _pages_rows
    for a in range(N):
        pos = np.arange(int(lens[a]))
        sp, sr = _pages_rows(bt[a], pos, P, st[a])
        rpg, _ = _pages_rows(rt[a], pos, P, st[a])
        dp, dr = bt2[a][pos // P], pos % P
        for h in range(case["Hkv"]):
            for x in range(case["d"]):
                ko = (x // 8) * 128 + x % 8
                bp2[dp, 0, h, ko + dr * 8] = case["bpool"][sp, 0, h, ko + sr * 8]
                vo = (x // 16) * 256 + (x % 16) * 4
                bp2[dp, 1, h, vo + (dr // 4) * 64 + dr % 4] = \
                    case["bpool"][sp, 1, h, vo + (sr // 4) * 64 + sr % 4]
        for k in range(case["r"]):
            ko = (k // 4) * 64 + k % 4
            rp2[dp, 0, ko + dr * 4] = case["rpool"][rpg, 0, ko + sr * 4]
            rp2[dp, 1, (dr // 4) * 4 * case["r"] + k * 4 + dr % 4] = \
                case["rpool"][rpg, 1, (sr // 4) * 4 * case["r"] + k * 4 + sr % 4]
    o = _oracle_decode(case, bt, rt, lens, starts=st)
    o2 = decode_attention(geo, bp2, rp2, bt2, bt2, lens, case["q"], case["Bk"], case["Bv"],
                          case["lora_scale"], case["sm_scale"], case["theta"])
    assert np.array_equal(o, o2)


def test_slot_map_write_lands_on_the_models_slots():
    """apply_rows_write under the slot map stores each appended row in the slot the pool
    model's append reported for it (page * P + row)."""
    rng = np.random.default_rng(5)
    case = tiny_case(340, "f32", Hq=2, Hkv=1, d=16, r=4, n_agents=3, freeze=True)
    pm = PoolModel(64, 64, 16, case["perm_b"], case["perm_r"])
    names = pm.replay(case["ops"])
    hs = [names[a] for a in case["agents"]]
    lens0 = [pm.length(h) for h in hs]
    n = 21
    slots = [pm.append(h, n) for h in hs]
    bt, rt, _ = pm.tables(hs, 16)
    st = pm.starts_table(hs, 16)
    pos = np.array([[L + i for i in range(n)] for L in lens0])
    kn = rng.standard_normal((3, n, 1, 16)).astype(np.float32)
    vn = rng.standard_normal((3, n, 1, 16)).astype(np.float32)
    rkn = rng.standard_normal((3, n, 4)).astype(np.float32)
    rvn = rng.standard_normal((3, n, 4)).astype(np.float32)
    geo = _geo(case)
    bp, rp = apply_rows_write(geo, case["bpool"], case["rpool"], bt, rt, pos, kn, vn, rkn, rvn,
                              starts=st)
    for a in range(3):
        for i in range(n):
            page, row = divmod(slots[a][0][i], 16)
            rpage, rrow = divmod(slots[a][1][i], 16)
            assert rrow == row
            got = [bp[page, 0, 0, (x // 8) * 128 + row * 8 + x % 8] for x in range(16)]
            assert np.array_equal(np.array(got), kn[a, i, 0])
            got = [rp[rpage, 0, (k // 4) * 64 + row * 4 + k % 4] for k in range(4)]
            assert np.array_equal(np.array(got), rkn[a, i])
