"""Bench: paged-KV GQA split-KV decode attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload mixed] [--gpus 1]

One step = the whole hot path over one decode batch: host plan (uniform tiles,
greedy bin-packing) written into mapped pinned memory that the kernels read in
place, the split-KV partial kernel and the log-sum-exp combine kernel, all on one
stream. Inputs (seeded, synthetic) are resident in HBM before timing starts. After
an untimed ramp (--ramp-ms of steps, so the GPU's clocks have risen) and W warmup
steps, exactly K steps are timed by wall clock between synchronisations; the decode
kernel is timed with HIP events on every --event-every-th of them. After the timed
loop, read probes (libpkv_probe.so) measure this part's own HBM read ceilings, and
the step is also reported as a percentage of the random 4 KB page gather. Prints ONE
JSON line on stdout; progress goes to stderr.

value = algorithmic bytes / wall time per step (GB/s). Algorithmic bytes: K and V of
every valid token, Q, the bf16 output, the block-table entries used, seq_lens and
(FP8) the page scales; split-KV partials are excluded.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention achieved HBM GB/s (% of peak) + µs/step, mixed KV lengths"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD's published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partial_traffic.json")
KERNEL_SOURCES = ["paged_kv_gqa_amd/csrc/decode_partial.hip", "paged_kv_gqa_amd/csrc/kernels.hpp"]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per decode_partial launch from the committed counter summary, if it
    was taken on the current kernel source and this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, algo_bytes):
    """Time the fp64 CPU oracle on the same workload (one full step)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    log("cpu baseline: timing the oracle on the full batch")
    t0 = time.perf_counter()
    oracle.decode_attention(inp)
    dt = time.perf_counter() - t0
    return {"value": round(algo_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": "one full step of the same workload (all %d requests x %d kv heads), "
                      "fp64 numpy, on this host's cores" % (inp.batch, inp.num_kv_heads),
            "host_cpus": len(os.sched_getaffinity(0))}


def read_probe(dev, nbytes=4 << 30, reps=10):
    """HBM read ceilings of this part, measured by libpkv_probe.so after the timed loop:
    a contiguous non-temporal stream and a gather of 4 KB pages in random order
    (decode's access pattern at page size 16), both over a 4 GiB buffer; each the best
    of three grid sizes (256-thread workgroups). GB/s."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_gqa_amd", "libpkv_probe.so"))
    vp = ctypes.c_void_p
    lib.pkvp_stream_read.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int, vp]
    lib.pkvp_page_gather.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int, vp]
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    npages = nbytes // 4096
    gen = torch.Generator().manual_seed(0)
    perm = torch.randperm(npages, generator=gen, dtype=torch.int32).to(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = vp(torch.cuda.current_stream().cuda_stream)

    def rate(launch):
        if launch() != 0:
            raise RuntimeError("read probe launch failed")
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            launch()
        b.record()
        torch.cuda.synchronize()
        return nbytes / (a.elapsed_time(b) / reps / 1e3) / 1e9

    s = max(rate(lambda: lib.pkvp_stream_read(vp(buf.data_ptr()), nbytes, vp(sink.data_ptr()),
                                              grid, stream)) for grid in (2048, 8192, 16384))
    g = max(rate(lambda: lib.pkvp_page_gather(vp(buf.data_ptr()), vp(perm.data_ptr()), npages,
                                              vp(sink.data_ptr()), grid, stream))
            for grid in (1024, 2048, 4096))
    del buf, perm, sink
    torch.cuda.empty_cache()
    return s, g


def ramp(step, ms):
    """Untimed steps for at least `ms` milliseconds before the warmup steps: the GPU
    raises its clocks over the first tens of milliseconds of load after idling (input
    generation), longer than a few warmup steps last. Returns the number of steps."""
    import torch
    n = 0
    t_end = time.perf_counter() + ms / 1e3
    while time.perf_counter() < t_end:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def timed_steps(step, K, every):
    """Time exactly K steps (synchronised before and after). The hot kernel is timed with
    HIP events recorded around its launch on every `every`-th of those steps: each
    recorded event costs its step GPU time (~3 us), so events on every step would slow
    the loop they measure. Returns (wall seconds, mean kernel seconds, launches timed)."""
    import numpy as np
    import torch
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for i in range(0, K, max(1, every))}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(ev.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = float(np.mean([a.elapsed_time(b) for a, b in ev.values()])) / 1e3
    return wall, kern, len(ev)


PREFILL_METRIC = "causal prefill attention TFLOP/s over the paged KV cache"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, AMD's published figure


def prefill_cpu_baseline(p, stride=16):
    """Time the fp64 CPU oracle on a sample of the prefill workload: kv head 0 of
    every request, every ``stride``-th query token (flops counted for those rows)."""
    import numpy as np
    from oracle.prefill import prefill_attention
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    c = p.cache
    G = c.num_q_heads // c.num_kv_heads
    rows, flops = {}, 0
    for b in range(p.batch):
        n, L = int(p.q_lens[b]), int(c.seq_lens[b])
        rows[b] = list(range(0, n, stride))
        flops += sum(4 * c.head_dim * G * (L - n + t + 1) for t in rows[b])
    log("cpu baseline: timing the oracle on kv head 0, every %d-th token" % stride)
    t0 = time.perf_counter()
    prefill_attention(p, pairs=[(b, 0) for b in range(p.batch)], rows=rows)
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": "kv head 0 of every request, every %d-th query token (%.3g flops), "
                      "fp64 numpy, host cores" % (stride, flops),
            "host_cpus": len(os.sched_getaffinity(0))}


def prefill_main(args):
    """One step = host tile plan (copied to the device) + the prefill kernel over one
    batch of the named prefill workload."""
    import numpy as np
    import torch

    import synth
    import paged_kv_gqa_amd as pkv

    cfg = synth.ALL_PREFILL[args.prefill]
    log("generating %s inputs (seed %d)" % (args.prefill, args.seed))
    p = synth.make_prefill_inputs(cfg, seed=args.seed)
    c = p.cache
    flops = synth.prefill_flops(p)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    qd = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if c.kv_format == "bf16":
        k = torch.from_numpy(c.k_cache.view(np.int16)).view(torch.bfloat16).to(dev)
        v = torch.from_numpy(c.v_cache.view(np.int16)).view(torch.bfloat16).to(dev)
        ks = vs = None
    else:
        k, v = torch.from_numpy(c.k_cache).to(dev), torch.from_numpy(c.v_cache).to(dev)
        ks, vs = torch.from_numpy(c.k_scale).to(dev), torch.from_numpy(c.v_scale).to(dev)
    bt = torch.from_numpy(c.block_table).to(dev)
    cu = torch.from_numpy(p.cu_q).to(dev)
    kl = torch.from_numpy(c.seq_lens).to(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((int(p.cu_q[-1]), c.num_q_heads), dtype=torch.float32, device=dev)
    runner = pkv.PagedPrefill(num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
                              head_dim=c.head_dim, page_size=c.page_size, kv_format=c.kv_format)
    q_lens_h, kv_lens_h = p.q_lens.copy(), c.seq_lens.copy()

    def step(evs=None):
        items = runner.plan(q_lens_h, kv_lens_h)
        if evs is not None:
            evs[0].record()
        runner(qd, cu, kl, bt, q_lens_h, kv_lens_h, c.scale, k_cache=k, v_cache=v, k_scale=ks,
               v_scale=vs, out=out, lse=lse, items=items)
        if evs is not None:
            evs[1].record()

    n_ramp = ramp(step, args.ramp_ms)
    log("ramp: %d untimed steps; warmup %d steps" % (n_ramp, args.warmup))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    log("timing %d steps" % K)
    wall, kern_s, n_timed = timed_steps(step, K, args.event_every)
    value = flops / (wall / K) / 1e12
    achieved = flops / kern_s / 1e12
    n_items = int(runner.last_items.shape[0])
    log("%.1f us/step, %.1f TFLOP/s; prefill kernel %.1f us avg (%.1f TFLOP/s, %.1f%% of bf16 peak)"
        % (wall / K * 1e6, value, kern_s * 1e6, achieved, 100 * achieved / MFMA_BF16_PEAK_TFLOPS))
    rec = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ramp_steps": n_ramp,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if c.kv_format == "bf16" else "fp8 KV, bf16 MFMA",
        "data": "synthetic",
        "config": {
            "workload": cfg["desc"],
            "batch": p.batch,
            "q_lens": p.q_lens.tolist(),
            "kv_lens": c.seq_lens.tolist(),
            "heads": "%d q / %d kv" % (c.num_q_heads, c.num_kv_heads),
            "head_dim": c.head_dim,
            "page_size": c.page_size,
            "work_items": n_items,
            "flops_per_step": flops,
            "step": "host tile plan (copied to the device) + prefill kernel",
        },
        "roofline": {
            "kernel": "prefill",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": round(kern_s * 1e6, 2),
            "launches_timed": "%d of the %d timed steps (HIP events on every %d-th)" % (
                n_timed, K, args.event_every),
        },
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = prefill_cpu_baseline(p)
    print(json.dumps(rec), flush=True)


def percentiles(us):
    import numpy as np
    a = np.asarray(us, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def step_distribution(step, dev, n=50, flush_mib=512):
    """Per-step GPU time of `step` (events on the current stream around the whole step),
    back to back and with the caches flushed before every step: a fill kernel writes
    `flush_mib` MiB (twice the 256 MB MALL, far beyond the L2s) outside the events."""
    import torch
    scratch = torch.empty(flush_mib << 20, dtype=torch.uint8, device=dev)
    out = {}
    for flush in (False, True):
        evs = []
        for i in range(n):
            if flush:
                scratch.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        out["flushed" if flush else "back_to_back"] = percentiles([a.elapsed_time(b) * 1e3 for a, b in evs])
    del scratch
    return out


def host_plan_us(inp, tile_tokens, num_workers, reps=1000):
    """Median wall time of the host planner (tile choice + plan) over `reps` calls."""
    import numpy as np
    import paged_kv_gqa_amd as pkv
    sl = inp.seq_lens
    T, N, _ = pkv.pkv_plan_query(sl, inp.q_len, inp.num_q_heads, inp.num_kv_heads, inp.head_dim,
                                 inp.page_size, inp.kv_format, tile_tokens, num_workers)
    bufs = (np.empty((N, 4), np.int32), np.empty(num_workers + 1, np.int32),
            np.empty(inp.batch + 1, np.int32))
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        T, N, _ = pkv.pkv_plan_query(sl, inp.q_len, inp.num_q_heads, inp.num_kv_heads, inp.head_dim,
                                     inp.page_size, inp.kv_format, tile_tokens, num_workers)
        pkv.pkv_plan(sl, inp.q_len, inp.num_kv_heads, T, num_workers, out=bufs)
        times.append((time.perf_counter() - t0) * 1e6)
    return percentiles(times)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ramp-ms", type=float, default=200.0,
                    help="untimed steps for at least this long before the warmup steps "
                         "(the GPU's clocks rise over the first tens of ms of load)")
    ap.add_argument("--event-every", type=int, default=5,
                    help="time the hot kernel with HIP events on every N-th timed step")
    ap.add_argument("--workload", default="mixed")
    ap.add_argument("--q-len", type=int, default=0,
                    help="override the workload's query tokens per request (draft tokens)")
    ap.add_argument("--q-heads", type=int, default=0,
                    help="override the workload's query heads (rows per kv head = q heads / kv heads x q_len)")
    ap.add_argument("--tile-tokens", type=int, default=0)
    ap.add_argument("--num-workers", type=int, default=0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--block-sparse", type=float, default=None, metavar="KEEP",
                    help="block-sparse decode: each (request, kv head, page) attended with "
                         "probability KEEP (seeded), plus the pages of the query tokens")
    ap.add_argument("--append", action="store_true",
                    help="start every step with the fused KV append (rotary embedding of q "
                         "and the new k rows, paged write, fp8 quantise-on-write) of the "
                         "batch's newest tokens")
    ap.add_argument("--graph", action="store_true",
                    help="with --device-plan: time the step replayed from a HIP graph captured once "
                         "(the kernel is timed on eager steps)")
    ap.add_argument("--device-plan", action="store_true",
                    help="build the plan on the GPU (pkv_plan_device) from device seq_lens "
                         "instead of on the host")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many MiB "
                         "(a known-size kernel for scaling HBM counters)")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the HBM read-ceiling probes")
    ap.add_argument("--no-distribution", action="store_true",
                    help="skip the per-step time distribution (back to back and cache-flushed)")
    ap.add_argument("--dist-steps", type=int, default=100)
    ap.add_argument("--prefill", default=None, metavar="WORKLOAD",
                    help="time variable-length causal prefill on a prefill workload "
                         "(prefill_varlen, prefill_long, prefill_chunk_fp8) instead of decode")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.graph and (not args.device_plan or args.block_sparse is not None):
        print("--graph needs --device-plan (a host plan cannot be replayed) and no --block-sparse",
              file=sys.stderr)
        sys.exit(2)
    if args.prefill is not None:
        prefill_main(args)
        return

    import numpy as np
    import torch

    import synth
    import paged_kv_gqa_amd as pkv

    cfg = dict(synth.ALL[args.workload])
    if args.q_len:
        cfg["q_len"] = args.q_len
        cfg["desc"] += "; q_len set to %d" % args.q_len
    if args.q_heads:
        cfg["num_q_heads"] = args.q_heads
        cfg["desc"] += "; q heads set to %d" % args.q_heads
    log("generating %s inputs (seed %d)" % (args.workload, args.seed))
    inp = synth.make_inputs(cfg, seed=args.seed)
    out_bytes = inp.batch * inp.q_len * inp.num_q_heads * inp.head_dim * 2
    mask_h = mask_d = None
    if args.block_sparse is not None:
        mask_h = synth.make_block_mask(inp, args.block_sparse, seed=1)
        algo = synth.sparse_algorithmic_bytes(inp, mask_h)
        partial_algo = synth.sparse_algorithmic_bytes(inp, mask_h, decode_only=True)
    else:
        algo = synth.algorithmic_bytes(inp)
        partial_algo = algo - out_bytes          # what decode_partial itself must move
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if inp.kv_format == "bf16":
        k = torch.from_numpy(inp.k_cache.view(np.int16)).view(torch.bfloat16).to(dev)
        v = torch.from_numpy(inp.v_cache.view(np.int16)).view(torch.bfloat16).to(dev)
        ks = vs = None
    else:
        k = torch.from_numpy(inp.k_cache).to(dev)
        v = torch.from_numpy(inp.v_cache).to(dev)
        ks = torch.from_numpy(inp.k_scale).to(dev)
        vs = torch.from_numpy(inp.v_scale).to(dev)
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl_dev = torch.from_numpy(inp.seq_lens).to(dev)
    if args.append:
        algo += synth.append_algorithmic_bytes(inp)
        kn_h, vn_h, _ = synth.new_token_rows(inp, seed=2)
        as_bf16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        k_new, v_new = as_bf16(kn_h), as_bf16(vn_h)
        cos_h, sin_h = synth.rope_tables(inp.block_table.shape[1] * inp.page_size, inp.head_dim)
        rope_cos, rope_sin = torch.from_numpy(cos_h).to(dev), torch.from_numpy(sin_h).to(dev)
        q_rot = torch.empty_like(q)
    if mask_h is not None:
        mask_d = torch.from_numpy(mask_h).to(dev)
    seq_lens_h = inp.seq_lens.copy()
    runner = pkv.PagedDecode(num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                             head_dim=inp.head_dim, page_size=inp.page_size,
                             kv_format=inp.kv_format, q_len=inp.q_len,
                             tile_tokens=args.tile_tokens, num_workers=args.num_workers,
                             device_plan=args.device_plan)
    out = torch.empty((inp.batch, inp.q_len, inp.num_q_heads, inp.head_dim), dtype=torch.bfloat16,
                      device=dev)

    def step(events=None):
        q_step = q
        if args.append:
            runner.append(k_new, v_new, k, v, bt, sl_dev, q=q, q_out=q_rot, rope_cos=rope_cos,
                          rope_sin=rope_sin, k_scale=ks, v_scale=vs)
            q_step = q_rot
        runner(q_step, k, v, bt, seq_lens_h, inp.scale, k_scale=ks, v_scale=vs, seq_lens=sl_dev,
               out=out, partial_events=events, block_mask=mask_d, block_mask_h=mask_h)

    n_ramp = ramp(step, args.ramp_ms)
    log("ramp: %d untimed steps; warmup %d steps" % (n_ramp, args.warmup))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.device_plan:
        info = runner.plan_info()
        if info["status"] != 0:
            raise RuntimeError("device plan failed: %s" % info)
        plan = dict(T=info["T"], N=info["N"], W=runner.num_workers)
        step_desc = "device plan (pkv_plan_device) + decode_partial + combine"
    else:
        plan = runner.last_plan
        step_desc = "host plan (read in place by the kernels) + decode_partial + combine"
        if plan["N"] == inp.batch * inp.num_kv_heads and mask_h is None:
            step_desc = ("host plan (read in place by the kernels) + decode_partial (one tile per "
                         "request: it writes the final rows, no combine)")
    if mask_h is not None:
        step_desc = "block mask compaction + " + step_desc
    if args.append:
        step_desc = "fused KV append (rotary, paged write%s) + " % (
            ", fp8 quantise-on-write" if inp.kv_format != "bf16" else "") + step_desc
    log("plan: tile %d tokens, %d items, %d workers" % (plan["T"], plan["N"], plan["W"]))

    K = args.steps
    log("timing %d steps" % K)
    wall, kern_avg_s, n_timed = timed_steps(step, K, args.event_every)
    if args.graph:
        # The same step captured once; the graph's replays are the timed steps.
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_desc += ", replayed from a HIP graph"
    ms_per_step = wall / K * 1e3
    value = algo / (wall / K) / 1e9
    achieved = partial_algo / kern_avg_s / 1e9
    traffic = (measured_traffic(args.workload)
               if mask_h is None and not (args.q_len or args.q_heads) else None)
    log("%.1f us/step, %.1f GB/s (%.1f%% of 8 TB/s); decode_partial %.1f us avg (%.1f GB/s)" % (
        ms_per_step * 1e3, value, 100 * value / HBM_PEAK_GBS, kern_avg_s * 1e6, achieved))

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ramp_steps": n_ramp,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.kv_format,
        "data": "synthetic",
        "config": {
            "workload": cfg["desc"] + ("" if mask_h is None else
                                       "; block-sparse: each (request, kv head, page) attended "
                                       "with probability %g (seed 1) plus the query pages"
                                       % args.block_sparse),
            "batch": inp.batch,
            "sum_seq_lens": int(inp.seq_lens.sum()),
            "q_len": inp.q_len,
            "heads": "%d q / %d kv" % (inp.num_q_heads, inp.num_kv_heads),
            "head_dim": inp.head_dim,
            "page_size": inp.page_size,
            "tile_tokens": plan["T"],
            "work_items": plan["N"],
            "num_workers": plan["W"],
            "algorithmic_bytes_per_step": algo,
            "step": step_desc,
        },
        "roofline": {
            "kernel": "decode_partial",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": partial_algo,
            "avg_launch_us": round(kern_avg_s * 1e6, 2),
            "launches_timed": "%d of the %d timed steps (HIP events on every %d-th)" % (
                n_timed, K, args.event_every),
        },
    }
    if not args.no_distribution:
        log("step distribution: back to back and flushed, %d steps each" % args.dist_steps)
        dist = step_distribution((lambda: g.replay()) if args.graph else (lambda: step()), dev,
                                 n=args.dist_steps)
        dist["host_plan_us"] = None if args.device_plan else host_plan_us(
            inp, args.tile_tokens, plan["W"])
        dist["plan_upload_us"] = 0.0 if not args.device_plan else None
        dist["note"] = ("GPU time per whole step from events on the step's stream; flushed = a "
                        "512 MiB fill before every step, outside the events. The host plan is "
                        "written into mapped pinned memory that the kernels read in place, so "
                        "there is no plan upload." if not args.device_plan else
                        "GPU time per whole step; the plan is built on the device inside the step.")
        for kind in ("back_to_back", "flushed"):
            dist[kind]["GBs_at_median"] = round(algo / (dist[kind]["median"] * 1e-6) / 1e9, 1)
        rec["timing"] = dist
        log("flushed step median %.1f us (p10 %.1f, p90 %.1f); back to back %.1f us" % (
            dist["flushed"]["median"], dist["flushed"]["p10"], dist["flushed"]["p90"],
            dist["back_to_back"]["median"]))
    if not args.no_read_probe:
        s_gbs, g_gbs = read_probe(dev)
        rec["read_probe"] = {
            "stream_GBs": round(s_gbs, 1),
            "page_gather_GBs": round(g_gbs, 1),
            "buffer_GiB": 4,
            "step_pct_of_page_gather": round(100 * value / g_gbs, 1),
            "kernel_pct_of_page_gather": round(100 * achieved / g_gbs, 1),
            "note": "this part's measured read ceilings (libpkv_probe.so, after the timed "
                    "loop): a contiguous stream and a random 4 KB page gather with "
                    "non-temporal whole-line loads, the decode kernel's pattern",
        }
        log("read probe: stream %.0f GB/s, 4 KB page gather %.0f GB/s; step at %.1f%%, "
            "decode kernel at %.1f%% of the gather" % (s_gbs, g_gbs, 100 * value / g_gbs,
                                                       100 * achieved / g_gbs))
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: %d bytes read and written" % n)
        del src, dst
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, algo)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
