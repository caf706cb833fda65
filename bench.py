"""Benchmark: ResidualAttention decode on one MI355X.

Workload: Llama3-8B attention shape (32 q heads, 8 KV heads, d=128, LoRA rank 16, bf16),
8 agents sharing a 32768-token prefix with 1024 private tokens each (MapReduce fan-out),
one decode query per agent.  A step is one decode call (split-K kernel + LSE/B_v
combine) over the whole batch; inputs are resident in HBM.  Input copies are rotated
so the step streams from HBM rather than the 256 MB Infinity Cache.  The step time comes
from the K calls captured as one HIP graph and replayed (no host launch cost inside); the
split kernel's launch duration (for the roofline figure) from a further pass of K eager
calls with per-launch events recorded by the library on the launch stream.

Also reported (skippable): the other two decode workloads, decode with append, decode over
a frozen tail, eviction / refill / base-only row write (`next_rows`), chunked prefill on the
Qwen3-8B workload with a hole-refill variant, and the fp64 oracle timed on the host.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# the timed decode workload, the two other decode shapes reported beside it, and the
# prefill workload
DECODE_WORKLOAD = "llama3_8b_mapreduce_decode"
OTHER_DECODE_WORKLOADS = ("llama3_8b_react_decode", "qwen25_14b_batched_decode")
PREFILL_WORKLOAD = "qwen3_8b_chunked_prefill"
PMC_FILE = os.path.join(ROOT, "profiles", "decode_split_pmc_llama3_8b_mapreduce.json")
KERNEL_SOURCES = {
    "generic": "lora_shared_prefix_amd/csrc/kernels_generic.hip",
    "mfma": "lora_shared_prefix_amd/csrc/kernels_mfma.hip",
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, n_unique_tokens):
    """Unique base-cache bytes once + per-agent residual, q, o and B bytes."""
    e = cfg.elem_bytes
    n = cfg.kv_width
    N = cfg.n_agents
    base = n_unique_tokens * n * 2 * e
    res = N * cfg.seq_len * 2 * cfg.rank * e
    q = N * cfg.num_q_heads * cfg.head_dim * e
    bk = N * cfg.rank * n * e
    split = base + res + q + bk          # what the split kernel must read
    step = split + q + bk                # + o written and B_v read by the combine
    return split, step


def source_sha(kernel):
    with open(os.path.join(ROOT, KERNEL_SOURCES[kernel]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel):
    """Counter-measured HBM bytes per launch, if taken on the current kernel source."""
    try:
        with open(PMC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, x, ops, agents, n_sample):
    """The fp64 oracle, as it is, on a sample of the agents (all heads)."""
    import numpy as np
    from oracle import PoolModel
    from oracle.attention import Geometry, decode_attention
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    pm = PoolModel(cfg.num_bpages, cfg.num_rpages, 16, x["perm_b"], x["perm_r"])
    names = pm.replay(ops)
    bt, rt, lens = pm.tables([names[a] for a in agents], -(-cfg.seq_len // 16))
    n_sample = min(n_sample, cfg.n_agents)
    sample = list(range(n_sample))
    t0 = time.perf_counter()
    decode_attention(Geometry.of(cfg), x["bpool"], x["rpool"], np.array(bt), np.array(rt), lens,
                     x["q"], x["Bk"], x["Bv"], cfg.lora_scale, 1 / np.sqrt(cfg.head_dim),
                     cfg.rope_theta, agents=sample)
    dt = time.perf_counter() - t0
    return {"value": n_sample / dt, "unit": "agent-tokens/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{n_sample} of {cfg.n_agents} agents, all {cfg.num_q_heads} q heads, "
                      f"fp64 numpy, {dt:.1f} s; host cpus={len(os.sched_getaffinity(0))}"}


MFMA_PEAK_BF16_TFLOPS = 2500.0


def prefill_flops(cfg):
    """Dense attention flops of one prefill call: QK^T and PV over keys 0..pos, plus the
    rank-r value accumulator, per (agent, chunk query, q head)."""
    total = 0
    for i in range(cfg.chunk_len):
        keys = cfg.prefix_len + i + 1
        total += keys
    per_key = 2 * cfg.head_dim * 2 + 2 * cfg.rank
    return cfg.n_agents * cfg.num_q_heads * total * per_key


def bench_prefill(steps, warmup):
    """Chunk tokens/s of the prefill call (row write + causal attention) on the Qwen3-8B
    workload: 8 agents, one 512-row chunk each, after a shared 131072-token prefix."""
    import numpy as np
    import torch
    from lora_shared_prefix_amd.session import DeviceBatch, to_device, workload_geom
    from workloads import config_by_name, draw_inputs, pool_ops
    cfg = config_by_name(PREFILL_WORKLOAD)
    log(f"drawing inputs of {cfg.name}")
    x = draw_inputs(cfg)
    ops, agents = pool_ops(cfg)
    b = DeviceBatch(workload_geom(cfg), x, ops, agents, x["perm_b"], x["perm_r"], plan=False)
    b.reserve_chunk(cfg.chunk_len)
    chunk = {k: to_device(x[k]) for k in ("q", "k_new", "v_new", "rk_new", "rv_new")}
    out = torch.empty_like(chunk["q"])
    sm = 1.0 / np.sqrt(cfg.head_dim)
    n = max(3, steps // 10)
    for _ in range(max(1, warmup // 5)):
        b.prefill(chunk, cfg.lora_scale, sm, cfg.rope_theta, out=out)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(n):
        b.prefill(chunk, cfg.lora_scale, sm, cfg.rope_theta, out=out)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n
    fl = prefill_flops(cfg)
    tflops = fl / (ms * 1e-3) / 1e12
    log(f"prefill {ms:.3f} ms per call, {tflops:.1f} TFLOP/s")
    res = {"workload": cfg.name, "calls": n, "ms_per_call": ms,
           "chunk_tokens_per_s": cfg.n_agents * cfg.chunk_len / (ms * 1e-3),
           "dense_flops_per_call": fl, "tflops": tflops,
           "mfma_frac": tflops / MFMA_PEAK_BF16_TFLOPS, "peak_tflops": MFMA_PEAK_BF16_TFLOPS}

    # Hole refill with a position list, same shape: every agent refills 256 rows inside its
    # private rows (positions prefix + 128 .. prefix + 383) and appends a 256-row tail, in
    # one call of the same 512 rows.
    from lora_shared_prefix_amd import forkkv as fk
    half = cfg.chunk_len // 2
    lens = [b.pool.length(h) for h in b.handles]
    for h in b.handles:
        b.pool.append(h, half, want_slots=False)
    b.refresh_tables()
    h0 = cfg.prefix_len + cfg.chunk_len // 4
    pos = [list(range(h0, h0 + half)) + list(range(L, L + half)) for L in lens]
    pos_dev = torch.tensor(pos, dtype=torch.int32, device="cuda")

    def refill():
        fk.residual_attn_prefill(b.pool, chunk["q"], chunk["k_new"], chunk["v_new"],
                                 chunk["rk_new"], chunk["rv_new"], b.Bk, b.Bv, b.btab, b.rtab,
                                 None, None, out, cfg.lora_scale, sm, cfg.rope_theta,
                                 positions=pos_dev, positions_host=pos)
    refill()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(n):
        refill()
    t1.record()
    torch.cuda.synchronize()
    ms_r = t0.elapsed_time(t1) / n
    per_key = 2 * cfg.head_dim * 2 + 2 * cfg.rank
    fl_r = cfg.num_q_heads * per_key * sum(p + 1 for row in pos for p in row)
    log(f"hole-refill prefill {ms_r:.3f} ms per call, {fl_r / (ms_r * 1e-3) / 1e12:.1f} TFLOP/s")
    res["hole_refill"] = {
        "rows_per_agent": f"{half} refilled at {h0}..{h0 + half - 1} + {half} appended",
        "ms_per_call": ms_r, "dense_flops_per_call": fl_r,
        "tflops": fl_r / (ms_r * 1e-3) / 1e12}
    return res


def bench_decode(name, steps, warmup, kernel, pages_per_item, copies_arg):
    """Decode step time (graph replay), split/combine launch times (events) on the named
    decode workload."""
    import numpy as np
    import torch

    from lora_shared_prefix_amd import forkkv as fk
    from lora_shared_prefix_amd.session import DeviceBatch, workload_geom
    from workloads import config_by_name, draw_inputs, pool_ops

    cfg = config_by_name(name)
    assert cfg.kind == "decode"
    log(f"drawing inputs of {cfg.name}")
    x = draw_inputs(cfg)
    ops, agents = pool_ops(cfg)
    geom = workload_geom(cfg)
    sm = 1.0 / np.sqrt(cfg.head_dim)
    unique = cfg.sessions * cfg.prefix_len + cfg.n_agents * cfg.suffix_len
    split_bytes, step_bytes = algorithmic_bytes(cfg, unique)
    ws_mb = step_bytes / 1e6
    copies = copies_arg or max(1, int(np.ceil(3 * 256e6 / (split_bytes))))
    log(f"uploading {copies} input copies (working set {ws_mb:.1f} MB each)")
    first = DeviceBatch(geom, x, ops, agents, x["perm_b"], x["perm_r"], kernel=kernel,
                        pages_per_item=pages_per_item)
    batches = [first]
    for _ in range(copies - 1):
        b = DeviceBatch.__new__(DeviceBatch)
        b.__dict__.update(first.__dict__)
        b.bcache = first.bcache.clone()
        b.rcache = first.rcache.clone()
        b.q, b.Bk, b.Bv = first.q.clone(), first.Bk.clone(), first.Bv.clone()
        b.out = torch.empty_like(first.out)
        b.pool = fk.Pool(cfg.num_bpages, cfg.num_rpages, cfg.num_kv_heads, cfg.head_dim,
                         cfg.rank, cfg.dtype, x["perm_b"], x["perm_r"], b.bcache, b.rcache)
        b.pool.replay(ops)
        batches.append(b)
    plan = first.plan
    kname = "mfma" if plan.info["kernel"] == fk.KERNEL_MFMA else "generic"
    log(f"plan: kernel={kname} items={plan.info['n_items']} slots={plan.info['n_slots']} "
        f"workspace={plan.info['workspace_bytes'] / 1e6:.1f} MB")

    def step(i):
        b = batches[i % copies]
        fk.residual_attn_decode(b.pool, plan, b.q, b.Bk, b.Bv, first.btab, first.rtab, b.out,
                                first.workspace, cfg.lora_scale, sm, cfg.rope_theta)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # eager calls, for context: each call also pays the host-side (Python) launch cost
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    eager_ms_step = t0.elapsed_time(t1) / steps
    # 1) the timed region: the K steps captured once as a HIP graph (K decode calls, the
    #    input copies in rotation), replayed once untimed, then once timed, bracketed by
    #    events on the replay stream; no per-call events or host launches inside
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    t0.record()
    graph.replay()
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / steps
    # 2) the same K steps again with HIP events recorded by the library around each kernel
    #    launch (on the launch stream): average launch duration of the split and combine
    plan.timing()  # drop anything recorded so far
    plan.set_timing(True)
    split_ms = comb_ms = 0.0
    launches = 0
    split_samples = []
    for i in range(steps):
        step(i)
        if (i + 1) % copies == 0 or i + 1 == steps:  # read the events of this rotation
            torch.cuda.synchronize()
            sm_, cm_, n_ = plan.timing()
            split_ms, comb_ms, launches = split_ms + sm_, comb_ms + cm_, launches + n_
            split_samples.append(sm_ / max(n_, 1))
    plan.set_timing(False)
    split_avg = split_ms / max(launches, 1)
    comb_avg = comb_ms / max(launches, 1)
    log(f"step {ms_step * 1e3:.1f} us (eager {eager_ms_step * 1e3:.1f} us); split "
        f"{split_avg * 1e3:.1f} us, combine {comb_avg * 1e3:.1f} us")

    # warm (cache-resident) figure for context: the same copy every step
    plan.set_timing(True)
    for _ in range(steps):
        fk.residual_attn_decode(first.pool, plan, first.q, first.Bk, first.Bv, first.btab,
                                first.rtab, first.out, first.workspace, cfg.lora_scale, sm,
                                cfg.rope_theta)
    torch.cuda.synchronize()
    plan.set_timing(False)
    wsplit, _, wl = plan.timing()

    achieved = split_bytes / (split_avg * 1e-3) / 1e9
    traffic = load_traffic(kname) if name == DECODE_WORKLOAD else None
    pct = np.percentile(np.array(split_samples) * 1e3, [10, 50, 90]).tolist()
    return {
        "_cfg": cfg, "_x": x, "_ops": ops, "_agents": agents,
        "agent_tokens_per_s": cfg.n_agents / (ms_step * 1e-3),
        "ms_per_step": ms_step,
        "config": {"workload": cfg.name, "agents": cfg.n_agents, "sessions": cfg.sessions,
                   "shared_prefix": cfg.prefix_len, "private_suffix": cfg.suffix_len,
                   "q_heads": cfg.num_q_heads, "kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "rank": cfg.rank, "page_size": 16, "kernel": kname,
                   "input_copies_rotated": copies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": f"residual_attn_{kname} (split-K decode)",
                     "algorithmic_bytes_per_launch": split_bytes,
                     "avg_launch_us": split_avg * 1e3},
        "step_hbm_gbs": step_bytes / (ms_step * 1e-3) / 1e9,
        "split_us_p10_p50_p90": pct,
        "combine_avg_us": comb_avg * 1e3,
        "eager_ms_per_step": eager_ms_step,
        "warm_split_avg_us": wsplit / max(wl, 1) * 1e3,
    }


def _graph_ms(fn, steps):
    """Per-call ms of `steps` calls of fn captured as one HIP graph (after one untimed replay)."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def _split_us(plan, fn, steps):
    """Average split-kernel and combine launch durations (library events), in us."""
    import torch
    plan.timing()
    plan.set_timing(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    plan.set_timing(False)
    s, c, n = plan.timing()
    return s / max(n, 1) * 1e3, c / max(n, 1) * 1e3


def bench_next_rows(cfg, x, ops, agents, steps):
    """Decode with append, decode over a frozen tail (the slot map), and eviction / refill /
    base-only row write, at the decode workload's shape with ONE input copy: its 185 MB
    working set fits the 256 MB Infinity Cache, so every figure stands beside plain decode
    timed the same way on the same box, not beside the rotated-copy headline."""
    import numpy as np
    import torch

    from lora_shared_prefix_amd import forkkv as fk
    from lora_shared_prefix_amd.session import DeviceBatch, workload_geom

    geom = workload_geom(cfg)
    sm = 1.0 / np.sqrt(cfg.head_dim)
    N, Hkv, d, r = cfg.n_agents, cfg.num_kv_heads, cfg.head_dim, cfg.rank
    out = {}

    # plain decode, the reference for this section
    ab = DeviceBatch(geom, x, ops, agents, x["perm_b"], x["perm_r"])
    dec = lambda: ab.decode(cfg.lora_scale, sm, cfg.rope_theta)
    plain_ms = _graph_ms(dec, steps)
    plain_split, _ = _split_us(ab.plan, dec, steps)
    out["plain_decode"] = {"ms_per_call": plain_ms, "split_avg_us": plain_split}

    # decode with append: every agent's new token is stored, then attended (one call)
    pb = DeviceBatch(geom, x, ops, agents, x["perm_b"], x["perm_r"], plan=False)
    pb.reserve_chunk(1)
    pb.make_plan()
    bf = torch.bfloat16
    rows = {"k_new": torch.randn(N, Hkv, d, dtype=bf, device="cuda"),
            "v_new": torch.randn(N, Hkv, d, dtype=bf, device="cuda"),
            "rk_new": torch.randn(N, r, dtype=bf, device="cuda"),
            "rv_new": torch.randn(N, r, dtype=bf, device="cuda")}
    app = lambda: pb.decode_append(rows, cfg.lora_scale, sm, cfg.rope_theta)
    app_ms = _graph_ms(app, steps)
    out["decode_append"] = {"ms_per_call": app_ms, "agent_tokens_per_s": N / (app_ms * 1e-3),
                            "over_plain_decode_us": (app_ms - plain_ms) * 1e3}
    del pb

    # decode over a frozen tail: the trunk ends 7 rows into a page that every agent shares
    # read-only (fork mode freeze); the agents' own rows start on fresh pages
    L0 = cfg.prefix_len + 7
    fops = [("create", "root", 0), ("append", "root", L0)]
    for a in agents:
        fops += [("fork", "root", L0, a, fk.FORK_FREEZE, 0), ("append", a, cfg.suffix_len)]
    fb = DeviceBatch(geom, x, fops, agents, x["perm_b"], x["perm_r"])
    assert fb.pstart is not None
    fdec = lambda: fb.decode(cfg.lora_scale, sm, cfg.rope_theta)
    f_ms = _graph_ms(fdec, steps)
    f_split, _ = _split_us(fb.plan, fdec, steps)
    f_bytes, _ = algorithmic_bytes(cfg, L0 + N * cfg.suffix_len)
    out["frozen_tail_decode"] = {
        "ms_per_call": f_ms, "split_avg_us": f_split,
        "split_hbm_gbs": f_bytes / (f_split * 1e-6) / 1e9,
        "trunk": f"{L0} tokens, the last 7 in a shared read-only page"}
    del fb

    # decoupled eviction: 64 shared trunk pages leave every holder, fresh pages are mapped
    # back into the agents (host bookkeeping), and the recomputed base rows are stored
    # through one holder (base pool only; the residual pages never left)
    lp0, lp1 = 1000, 1064
    pages = [int(v) for v in ab.btab_host[0][lp0:lp1]]
    t = time.perf_counter()
    ab.pool.evict_base(pages)
    ab.pool.refill_base(ab.handles, lp0, lp1)
    host_us = (time.perf_counter() - t) * 1e6
    ab.refresh_tables()
    n_rows = (lp1 - lp0) * 16
    wpos = [list(range(lp0 * 16, lp1 * 16))]
    wpos_dev = torch.tensor(wpos, dtype=torch.int32, device="cuda")
    kw = torch.randn(1, n_rows, Hkv, d, dtype=bf, device="cuda")
    vw = torch.randn(1, n_rows, Hkv, d, dtype=bf, device="cuda")
    btab0 = ab.btab[:1].contiguous()
    wr = lambda: fk.write_rows(ab.pool, btab0, None, wpos_dev, wpos, kw, vw)
    w_ms = _graph_ms(wr, steps)
    w_bytes = n_rows * Hkv * d * 2 * cfg.elem_bytes
    out["evict_refill"] = {"pages": lp1 - lp0, "holders": len(ab.handles) + 1,
                           "evict_refill_host_us": host_us, "write_rows_us": w_ms * 1e3,
                           "write_rows_bytes": w_bytes,
                           "write_rows_gbs": 2 * w_bytes / (w_ms * 1e-3) / 1e9}
    log("next rows: " + json.dumps(out))
    return out


def copy_bandwidth_gbs():
    """Read + write bytes per second of a plain 1 GiB device-to-device copy (practical ceiling)."""
    import torch
    n = 2 ** 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(10):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / 10
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DECODE_WORKLOAD, help="name of the decode workload")
    ap.add_argument("--kernel", choices=["auto", "generic", "mfma"], default="auto")
    ap.add_argument("--pages-per-item", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated (0 = auto)")
    ap.add_argument("--cpu-sample", type=int, default=8,
                    help="agents timed on the oracle (0 = skip; 8 = the whole batch, about 10 s)")
    ap.add_argument("--no-more-workloads", action="store_true",
                    help="skip the extra decode figures of the ReAct and batched workloads")
    ap.add_argument("--no-next", action="store_true",
                    help="skip decode-with-append, frozen-tail decode and eviction/refill timing")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip timing chunked prefill on the Qwen3-8B 131072-prefix workload")
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    help="only run a plain device copy of this many MiB (PMC scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from lora_shared_prefix_amd import forkkv as fk
    from lora_shared_prefix_amd.session import DeviceBatch, workload_geom
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration > 0:
        n = int(args.copy_calibration * 2 ** 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy calibration: {n * 4} bytes read and written per copy, 3 copies")
        return

    kernel = {"auto": fk.KERNEL_AUTO, "generic": fk.KERNEL_GENERIC, "mfma": fk.KERNEL_MFMA}[args.kernel]
    d = bench_decode(args.workload, args.steps, args.warmup, kernel, args.pages_per_item,
                     args.copies)
    cfg, x, ops, agents = d.pop("_cfg"), d.pop("_x"), d.pop("_ops"), d.pop("_agents")
    ceiling = copy_bandwidth_gbs()
    log(f"device copy bandwidth {ceiling:.0f} GB/s (read + write bytes / time, 1 GiB copy)")
    result = {
        "metric": "ResidualAttention decode agent-tokens/s + achieved HBM GB/s (% roofline), 1 GPU",
        "value": d["agent_tokens_per_s"],
        "unit": "agent-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": d["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) caches and queries, B ~ N(0, 0.02^2))",
        "config": d["config"],
        "roofline": d["roofline"],
        "step_hbm_gbs": d["step_hbm_gbs"],
        "split_us_p10_p50_p90": d["split_us_p10_p50_p90"],
        "combine_avg_us": d["combine_avg_us"],
        "eager_ms_per_step": d["eager_ms_per_step"],
        "warm_split_avg_us": d["warm_split_avg_us"],
        "copy_bandwidth_gbs": ceiling,
        "split_frac_of_copy_bandwidth": d["roofline"]["achieved"] / ceiling,
    }
    if not args.no_more_workloads and args.workload == DECODE_WORKLOAD:
        others = {}
        for name in OTHER_DECODE_WORKLOADS:
            torch.cuda.empty_cache()
            o = bench_decode(name, max(10, args.steps // 2), max(2, args.warmup // 2), kernel, 0, 0)
            for k in ("_cfg", "_x", "_ops", "_agents"):
                o.pop(k)
            others[o["config"]["workload"]] = {
                "agent_tokens_per_s": o["agent_tokens_per_s"], "ms_per_step": o["ms_per_step"],
                "split_avg_us": o["roofline"]["avg_launch_us"],
                "split_hbm_gbs": o["roofline"]["achieved"], "split_frac": o["roofline"]["frac"],
                "algorithmic_bytes_per_launch": o["roofline"]["algorithmic_bytes_per_launch"],
                "combine_avg_us": o["combine_avg_us"], "config": o["config"]}
        result["other_decode_workloads"] = others
    if not args.no_next and args.workload == DECODE_WORKLOAD:
        torch.cuda.empty_cache()
        result["next_rows"] = bench_next_rows(cfg, x, ops, agents, max(10, args.steps // 2))
    if not args.no_prefill:
        torch.cuda.empty_cache()  # the decode inputs are freed by now
        result["prefill"] = bench_prefill(args.steps, args.warmup)
    if args.cpu_sample > 0:
        log("timing the fp64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(cfg, x, ops, agents, args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
