"""Benchmark: ResidualAttention decode on one MI355X.

Workload: Llama3-8B attention shape (32 q heads, 8 KV heads, d=128, LoRA rank 16, bf16),
8 agents sharing a 32768-token prefix with 1024 private tokens each (MapReduce fan-out),
one decode query per agent.  A step is one decode call (split-K kernel + LSE/B_v
combine) over the whole batch; inputs are resident in HBM.  Input copies are rotated
so the step streams from HBM rather than the 256 MB Infinity Cache.  The step time comes
from the K calls captured as one HIP graph and replayed (no host launch cost inside); the
split kernel's time (for the roofline figure) from the same K calls captured the same way
with the plan in split-only mode (the split kernel launched alone), so both come from one
kind of timing and the split time is the smaller.  The roofline is reported against the
8 TB/s spec peak and against the box's measured read-only streaming ceiling; the GPU
clocks and power cap are read while the step graph replays.

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
# the sources of each split kernel (its counters are valid while these are unchanged)
KERNEL_SOURCES = {
    "generic": ("lora_shared_prefix_amd/csrc/kernels_generic.hip",),
    "mfma": ("lora_shared_prefix_amd/csrc/kernels_mfma_decode.hip",
             "lora_shared_prefix_amd/csrc/kernels_mfma_common.h"),
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
    h = hashlib.sha256()
    for path in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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
                      f"fp64 numpy, {dt:.1f} s; host cpus={len(os.sched_getaffinity(0))} "
                      f"(os.cpu_count()={os.cpu_count()}), BLAS threads={blas_threads}"}


MFMA_PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 (spec)


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
    del b

    # Frozen tail, same shape: the prefix ends 7 rows into a page that every agent shares
    # read-only (fork mode freeze), so each agent's chunk starts on a fresh page and the
    # page start table (the slot map) is in use.
    L0 = cfg.prefix_len + 7
    fops = [("create", "root", 0), ("append", "root", L0)]
    for a in agents:
        fops += [("fork", "root", L0, a, fk.FORK_FREEZE, 0)]
    fb = DeviceBatch(workload_geom(cfg), x, fops, agents, x["perm_b"], x["perm_r"],
                     plan=False)
    fb.reserve_chunk(cfg.chunk_len)  # the chunk's first page starts 7 rows past a page edge
    assert fb.pstart is not None
    fl_f = cfg.n_agents * cfg.num_q_heads * per_key * sum(
        L0 + i + 1 for i in range(cfg.chunk_len))
    frozen = {"prefix": f"{L0} tokens, the last 7 in a shared read-only page",
              "dense_flops_per_call": fl_f}
    for name, kern in (("mfma", fk.KERNEL_MFMA),):
        run = lambda: fb.prefill(chunk, cfg.lora_scale, sm, cfg.rope_theta, out=out,
                                 kernel=kern)
        run()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(n):
            run()
        t1.record()
        torch.cuda.synchronize()
        ms_f = t0.elapsed_time(t1) / n
        log(f"frozen-tail prefill ({name}) {ms_f:.3f} ms per call, "
            f"{fl_f / (ms_f * 1e-3) / 1e12:.1f} TFLOP/s")
        frozen[name] = {"ms_per_call": ms_f, "tflops": fl_f / (ms_f * 1e-3) / 1e12}
    res["frozen_tail"] = frozen
    del fb
    return res


def bench_decode(name, steps, warmup, kernel, pages_per_item, copies_arg, clocks=None):
    """Decode step time and split-kernel time (both from graph replays) on the named decode
    workload; ``clocks`` (a dict) receives the GPU clocks and power read while the step
    graph replays."""
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
    graph = _capture(lambda: [step(i) for i in range(steps)])
    ms_step = _replay_ms(graph, steps)
    # 2) the split kernel alone, timed the same way: the same K calls (same rotation) with
    #    the plan in split-only mode, captured as a graph of K split launches
    plan.set_timing(fk.TIMING_SPLIT_ONLY)
    split_graph = _capture(lambda: [step(i) for i in range(steps)])
    plan.set_timing(fk.TIMING_OFF)
    split_avg = _replay_ms(split_graph, steps)
    # spread over further timed replays of both graphs (per-call ms of each replay)
    reps = [_replay_ms(split_graph, steps, warm=False) for _ in range(5)]
    step_reps = [_replay_ms(graph, steps) for _ in range(1)]
    step_reps += [_replay_ms(graph, steps, warm=False) for _ in range(4)]
    comb_avg = ms_step - split_avg  # the combine launch and the gap before it
    log(f"step {ms_step * 1e3:.1f} us (eager {eager_ms_step * 1e3:.1f} us); split "
        f"{split_avg * 1e3:.1f} us, combine + gap {comb_avg * 1e3:.1f} us")
    if clocks is not None:
        clocks.update(gpu_clocks_under_load(graph))
    del graph, split_graph

    # warm (cache-resident) figure for context: the same copy every step, split only
    plan.set_timing(fk.TIMING_SPLIT_ONLY)
    wgraph = _capture(lambda: [fk.residual_attn_decode(
        first.pool, plan, first.q, first.Bk, first.Bv, first.btab, first.rtab, first.out,
        first.workspace, cfg.lora_scale, sm, cfg.rope_theta) for _ in range(steps)])
    plan.set_timing(fk.TIMING_OFF)
    wsplit_ms = _replay_ms(wgraph, steps)
    del wgraph

    achieved = split_bytes / (split_avg * 1e-3) / 1e9
    traffic = load_traffic(kname) if name == DECODE_WORKLOAD else None
    pct = np.percentile(np.array(reps) * 1e3, [10, 50, 90]).tolist()
    step_pct = np.percentile(np.array(step_reps) * 1e3, [10, 50, 90]).tolist()
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
                     "kernel": f"decode_mfma_kernel (split-K decode)" if kname == "mfma"
                               else "residual_attn_generic (split-K decode)",
                     "algorithmic_bytes_per_launch": split_bytes,
                     "avg_launch_us": split_avg * 1e3,
                     "timing": "graph of the timed K calls in split-only mode, one timed replay"},
        "step_hbm_gbs": step_bytes / (ms_step * 1e-3) / 1e9,
        "split_us_p10_p50_p90": pct,
        "step_us_p10_p50_p90": step_pct,
        "combine_and_gap_us": comb_avg * 1e3,
        "eager_ms_per_step": eager_ms_step,
        "warm_split_avg_us": wsplit_ms * 1e3,
    }


def _capture(fn):
    """fn() once eagerly, then captured as a HIP graph and replayed once (untimed)."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    return g


WARM_S = 0.2  # back-to-back replays before a timed replay


def _warm(g, seconds=WARM_S):
    """Replay g back to back for about `seconds`: after an idle gap (graph capture on the
    host, set-up) the device takes some milliseconds to return to its working clocks, and
    a decode step in a serving loop runs right after the previous one."""
    import torch
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()


def _replay_ms(g, calls, warm=True):
    """Per-call ms of one timed replay of a graph of `calls` calls (events on the replay
    stream, synchronised before and after), after back-to-back warm replays."""
    import torch
    if warm:
        _warm(g)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / calls


def gpu_clocks_under_load(graph, seconds=1.5):
    """GPU clocks, power and power cap (rocm-smi) read while `graph` replays back to back."""
    import subprocess
    import threading

    import torch
    res = {}

    # rocm-smi is a Python script: run it with this interpreter (no `env` re-exec), and not
    # at all under a profiler whose preloaded library would initialise the GPU in the child
    smi = "/opt/rocm/bin/rocm-smi"
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or not os.path.exists(smi):
        return {"under_load_error": "not read (profiler preloaded or rocm-smi missing)"}

    def read():
        time.sleep(seconds / 3)
        try:
            r = subprocess.run([sys.executable, smi, "--showclocks", "--showpower",
                                "--showmaxpower", "--json"], capture_output=True, text=True,
                               timeout=30)
            card = next(iter(json.loads(r.stdout).values()))
            res["under_load"] = {k: v for k, v in card.items()
                                 if "clk" in k.lower() or "power" in k.lower()}
        except Exception as e:  # no rocm-smi or no permission: record why
            res["under_load_error"] = repr(e)[:200]

    th = threading.Thread(target=read)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        graph.replay()
        torch.cuda.synchronize()
    th.join()
    return res


def _graph_ms(fn, steps):
    """Per-call ms of `steps` calls of fn captured as one HIP graph (warm replays, then one
    timed replay)."""
    g = _capture(lambda: [fn() for _ in range(steps)])
    return _replay_ms(g, steps)


def _split_us(plan, fn, steps):
    """Split-kernel time per call in us: `steps` calls with the plan in split-only mode,
    captured as a graph and replayed (timed like the whole call)."""
    from lora_shared_prefix_amd import forkkv as fk
    plan.set_timing(fk.TIMING_SPLIT_ONLY)
    try:
        ms = _graph_ms(fn, steps)
    finally:
        plan.set_timing(fk.TIMING_OFF)
    return ms * 1e3


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
    plain_split = _split_us(ab.plan, dec, steps)
    out["plain_decode"] = {"ms_per_call": plain_ms, "split_avg_us": plain_split}

    out["serving_loop"] = serving_loop(cfg, x, ops, agents, 64)

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
    f_split = _split_us(fb.plan, fdec, steps)
    f_bytes, _ = algorithmic_bytes(cfg, L0 + N * cfg.suffix_len)
    out["frozen_tail_decode"] = {
        "ms_per_call": f_ms, "split_avg_us": f_split,
        "split_hbm_gbs": f_bytes / (f_split * 1e-6) / 1e9,
        "trunk": f"{L0} tokens, the last 7 in a shared read-only page"}
    del fb

    # decoupled eviction: 64 shared trunk pages leave every holder, fresh pages are mapped
    # back into the agents (host bookkeeping), and the recomputed base rows are stored
    # through one holder (base pool only; the residual pages never left)
    bf = torch.bfloat16
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


def _microbench_lib():
    import ctypes as C
    path = os.path.join(ROOT, "lora_shared_prefix_amd", "libforkkv_microbench.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    L = C.CDLL(path)
    L.mb_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_int,
                                 C.c_void_p]
    L.mb_mfma_bf16.argtypes = [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_void_p]
    L.mb_mfma_chains.restype = C.c_int
    L.mb_pipe_probe.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_void_p,
                                C.c_int, C.c_void_p]
    return L


def pipe_probes():
    """How the matrix cores of a SIMD share it with another wave's work: 256 workgroups of
    512 threads (one per compute unit; waves w and w + 4 share a SIMD), waves 0-3 running 16
    bf16 16x16x32 MFMAs per trip, waves 4-7 64 FMAs, 64 exp2 or 16 ds_read_b128 per trip
    (or both waves that same work).  Returns ns per trip for each combination."""
    import torch
    L = _microbench_lib()
    sp = torch.cuda.current_stream().cuda_stream
    ops = torch.tensor([0x3F80] * 8 + [0x3D00] * 8, dtype=torch.int16, device="cuda")
    blocks, iters = 256, 5000
    out = torch.zeros(blocks * 8, dtype=torch.float32, device="cuda")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    def ns(mode, mfma, chains):
        assert L.mb_pipe_probe(mode, mfma, chains, ops.data_ptr(), iters, out.data_ptr(),
                               blocks, sp) == 0
        t0.record()
        L.mb_pipe_probe(mode, mfma, chains, ops.data_ptr(), iters, out.data_ptr(), blocks, sp)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e6 / iters

    res = {f"16 MFMA, {c} chain(s), other wave idle": ns(0, 1, c) for c in (1, 2, 4, 16)}
    for mode, what in ((1, "64 FMA"), (2, "64 exp2"), (3, "16 ds_read_b128")):
        res[f"{what} alone"] = ns(mode, 0, 4)
        res[f"{what} beside 16 MFMA (4 chains)"] = ns(mode, 1, 4)
        res[f"{what} on both waves of each SIMD"] = ns(mode, 2, 4)
    return {"ns_per_trip": res, "setup": f"{blocks} workgroups x 512 threads, {iters} trips"}


def measured_ceilings():
    """The box's own ceilings, each self-checked: a read-only streaming reduction over 1 GiB
    (four times the 256 MB Infinity Cache) and a bf16 16x16x32 MFMA loop."""
    import torch
    L = _microbench_lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # read-only stream: int32 ones, so every pass must sum to the word count
    n_bytes = 1 << 30
    buf = torch.ones(n_bytes // 4, dtype=torch.int32, device="cuda")
    passes = 20
    best = None
    names = {0: "4 loads in flight", 1: "8 loads in flight", 2: "8 non-temporal loads in flight"}
    for variant in (0, 1, 2):
        for blocks in (2048, 8192):
            part = torch.zeros(blocks, dtype=torch.int64, device="cuda")
            for _ in range(passes):  # back to back: the device at its working clocks
                assert L.mb_stream_read(buf.data_ptr(), n_bytes, part.data_ptr(), blocks,
                                        variant, sp) == 0
            t0.record()
            for _ in range(passes):
                L.mb_stream_read(buf.data_ptr(), n_bytes, part.data_ptr(), blocks, variant, sp)
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / passes
            assert int(part.sum().item()) == n_bytes // 4, "stream-read checksum"
            if best is None or ms < best[0]:
                best = (ms, f"{blocks} blocks x 256 threads, {names[variant]}")
    read_ms = best[0]
    del buf, part
    # bf16 MFMA loop: A = 1, B = 1/32 (exact in bf16), so each MFMA adds 1.0 per element
    ops = torch.tensor([0x3F80] * 8 + [0x3D00] * 8, dtype=torch.int16, device="cuda")
    mblocks, iters = 256 * 8, 2048
    chains = L.mb_mfma_chains()
    out = torch.zeros(mblocks * 4, dtype=torch.float32, device="cuda")
    assert L.mb_mfma_bf16(ops.data_ptr(), iters, out.data_ptr(), mblocks, sp) == 0
    torch.cuda.synchronize()
    t0.record()
    for _ in range(5):
        L.mb_mfma_bf16(ops.data_ptr(), iters, out.data_ptr(), mblocks, sp)
    t1.record()
    torch.cuda.synchronize()
    mfma_ms = t0.elapsed_time(t1) / 5
    assert bool(torch.all(out == float(4 * chains * iters))), "MFMA-loop checksum"
    flops = mblocks * 4 * chains * iters * 2 * 16 * 16 * 32
    return {"hbm_read_gbs": n_bytes / (read_ms * 1e-3) / 1e9,
            "hbm_read_test": f"read-only sum of 1 GiB, best of 6 launch shapes ({best[1]}, "
                             f"16 B loads), {passes} passes, checksum ok",
            "mfma_bf16_tflops": flops / (mfma_ms * 1e-3) / 1e12,
            "mfma_test": f"{mblocks * 4} waves x {chains} chains x {iters} "
                         "v_mfma_f32_16x16x32_bf16, checksum ok"}


def serving_loop(cfg, x, ops, agents, steps):
    """A serving loop of decode with append at the decode workload's shape (one input copy):
    three rounds of `steps` steps in a row on one plan (the median round is reported).  Each step the host reserves every agent's next
    token (one batched call); at a page crossing (every 16 steps here: the agents' lengths
    are multiples of 16) it also updates the device tables in place and rebuilds and
    re-uploads the plan; then the step runs -- as an eager call, and in a second pass as a
    replay of one captured call (the plan's device lengths advance inside each call, so the
    same graph serves every step).  Reported per step: wall time with all host work, GPU
    time, the host's share (Python included) and the part of it spent in the library's own
    host calls (batched append, plan rebuild, upload)."""
    import numpy as np
    import torch

    from lora_shared_prefix_amd.session import DeviceBatch, workload_geom

    geom = workload_geom(cfg)
    sm = 1.0 / np.sqrt(cfg.head_dim)
    N, Hkv, d, r = cfg.n_agents, cfg.num_kv_heads, cfg.head_dim, cfg.rank
    bf = torch.bfloat16
    rows = {"k_new": torch.randn(N, Hkv, d, dtype=bf, device="cuda"),
            "v_new": torch.randn(N, Hkv, d, dtype=bf, device="cuda"),
            "rk_new": torch.randn(N, r, dtype=bf, device="cuda"),
            "rv_new": torch.randn(N, r, dtype=bf, device="cuda")}
    res = {}
    rounds = 3  # the host share is noisy on a shared host: the median round is reported
    for mode in ("eager", "graph"):
        b = DeviceBatch(geom, x, ops, agents, x["perm_b"], x["perm_r"], plan=False)
        b.pool.append_batch(b.handles, 1)
        b.refresh_tables(extra_pages=rounds * steps // 16 + 2)
        b.make_plan()
        call = lambda: b.decode_append(rows, cfg.lora_scale, sm, cfg.rope_theta)
        call()  # first step (untimed): compiles nothing, warms the device
        g = None
        if mode == "graph":
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call()
        torch.cuda.synchronize()
        per_round = []
        for _ in range(rounds):
            host, rebuilds, recaptures = 0.0, 0, 0
            b.lib_host_s = 0.0
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t_wall = time.perf_counter()
            t0.record()
            for _ in range(steps):
                th = time.perf_counter()
                same, _ = b.next_step()
                rebuilds += int(b.lens[0] % 16 == 1)
                host += time.perf_counter() - th
                if g is not None and not same:  # the plan outgrew its capacities: capture anew
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        call()  # (recorded, not run)
                    recaptures += 1
                if g is not None:
                    g.replay()
                else:
                    call()
            t1.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t_wall
            gpu_ms = t0.elapsed_time(t1)
            per_round.append({"steps": steps, "page_crossings": rebuilds, "recaptures": recaptures,
                              "wall_us_per_step": wall / steps * 1e6,
                              "gpu_us_per_step": gpu_ms / steps * 1e3,
                              "host_us_per_step": host / steps * 1e6,
                              "library_host_us_per_step": b.lib_host_s / steps * 1e6,
                              "agent_tokens_per_s": N * steps / wall})
        med = sorted(per_round, key=lambda r: r["wall_us_per_step"])[rounds // 2]
        res[mode] = dict(med, rounds=rounds,
                         wall_us_per_step_rounds=[r["wall_us_per_step"] for r in per_round],
                         library_host_us_per_step_rounds=[r["library_host_us_per_step"]
                                                          for r in per_round])
        del b, g
        torch.cuda.empty_cache()
    log("serving loop: " + json.dumps(res))
    return res


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
    ap.add_argument("--pipe-probes", action="store_true",
                    help="time the SIMD pipe-sharing probes and exit")
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
    if args.pipe_probes:
        print(json.dumps(pipe_probes()))
        return
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
    clocks = {"rocm": torch.version.hip}
    d = bench_decode(args.workload, args.steps, args.warmup, kernel, args.pages_per_item,
                     args.copies, clocks=clocks)
    cfg, x, ops, agents = d.pop("_cfg"), d.pop("_x"), d.pop("_ops"), d.pop("_agents")
    ceiling = copy_bandwidth_gbs()
    log(f"device copy bandwidth {ceiling:.0f} GB/s (read + write bytes / time, 1 GiB copy)")
    torch.cuda.empty_cache()
    ceilings = measured_ceilings()
    ceilings["copy_read_write_gbs"] = ceiling
    log(f"measured ceilings: {json.dumps(ceilings)}")
    rl = d["roofline"]
    rl["peak_measured"] = ceilings["hbm_read_gbs"]
    rl["frac_of_measured"] = rl["achieved"] / ceilings["hbm_read_gbs"]
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
        "step_us_p10_p50_p90": d["step_us_p10_p50_p90"],
        "combine_and_gap_us": d["combine_and_gap_us"],
        "eager_ms_per_step": d["eager_ms_per_step"],
        "warm_split_avg_us": d["warm_split_avg_us"],
        "ceilings": ceilings,
        "gpu": clocks,
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
                "combine_and_gap_us": o["combine_and_gap_us"], "config": o["config"]}
        result["other_decode_workloads"] = others
    if not args.no_next and args.workload == DECODE_WORKLOAD:
        torch.cuda.empty_cache()
        result["next_rows"] = bench_next_rows(cfg, x, ops, agents, max(10, args.steps // 2))
    if not args.no_prefill:
        torch.cuda.empty_cache()  # the decode inputs are freed by now
        result["prefill"] = bench_prefill(args.steps, args.warmup)
        result["prefill"]["peak_measured_tflops"] = ceilings["mfma_bf16_tflops"]
        result["prefill"]["mfma_frac_of_measured"] = (result["prefill"]["tflops"]
                                                      / ceilings["mfma_bf16_tflops"])
    if args.cpu_sample > 0:
        log("timing the fp64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(cfg, x, ops, agents, args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
