#!/usr/bin/env python3
"""Benchmark one decode step of paged MQA/GQA attention on one MI355X.

A step is the whole hot path over one batch: kv_append of every sequence's
new token into its page, then decode attention over the sequence's context
(the split pass with its log-sum-exp merge, or the single pass when the
workload uses one split), issued as one paged_decode_step call: one kernel
for groups of up to 16 q heads, the reduce kernel after it for wider ones;
above 1536 (sequence, kv head) pairs the library launches the append apart,
ahead of the attention. Inputs are seeded synthetic data already
resident in HBM. R replicas of the KV pools rotate step to step so that the
256 MB Infinity Cache cannot serve the working set. The R steps of one
rotation (one per replica) are captured once as a HIP graph and replayed, as a
decode engine captures a whole model step: the timed steps are the GPU's own
time, not Python's launch overhead or one graph launch per layer.

Prints ONE JSON line: metric / value (KV GB/s of the step) / unit, timing,
`roofline` for the attention kernel (algorithmic bytes per launch / its
average event-timed launch duration, against 8 TB/s) and `cpu_baseline`
(the fp64 oracle timed on this host over a bounded sample of the same
workload).

The default 400 warm-up steps are there because the first milliseconds of
replays after capture run up to 10% slow (seen on the wide MQA workload);
the 1000 timed steps then take well under a second on every workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
  python bench.py --workload proj_qkv   # a decode projection (M == 1 GEMM)
  python bench.py --copy-only BYTES     # plain copy kernel for counter scaling

A decode-projection workload (proj_qkv, proj_qkv_w8a16, proj_o, lm_head,
mlp_w8a16_4864) times one gemm_m1_transposed call per step instead, over
replicas of the transposed weight, against the same HBM roofline.
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
DEFAULT_WORKLOAD = "gqa_llama"
METRIC = "decode-attn KV GB/s (% of HBM peak) + us/call, GQA 32q/8kv d128 batch 32"
PROFILE_DIR = os.path.join(ROOT, "profiles")
# what a kernel binary is built from: its sources and the build flags
KERNEL_SOURCES = [os.path.join(ROOT, "paged_mqa_gqa_amd", "csrc", f)
                  for f in ("decode_attn.hip", "device_common.h", "launch.h")] + [
    os.path.join(ROOT, "paged_mqa_gqa_amd", "build.py")]
GEMM_SOURCES = [os.path.join(ROOT, "paged_mqa_gqa_amd", "csrc", f)
                for f in ("gemm_m1.hip", "device_common.h", "launch.h")] + [
    os.path.join(ROOT, "paged_mqa_gqa_amd", "build.py")]
ATTN_LAUNCHES_PER_GRAPH = 8
LAUNCH_REPS = 5             # repetitions of the per-launch event timing
KV_DTYPE_CODE = {"fp16": 0, "fp8_e4m3fn": 1, "int8": 2}     # enum pa_kv_dtype


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--splits", type=int, default=0, help="override the split count")
    ap.add_argument("--replicas", type=int, default=0, help="override pool replicas")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--separate-append", action="store_true",
                    help="issue kv_append and the attention call as two launches")
    ap.add_argument("--copy-only", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES, --steps times")
    return ap.parse_args()


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for path in sources or KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, prefix="decode_attn", sources=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (attention, or with prefix "gemm_m1" and the GEMM sources, the decode
    projection), if it was taken on the current kernel sources; else None."""
    path = os.path.join(PROFILE_DIR, f"{prefix}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def step_fuses_append(w) -> bool:
    """Whether the library's decode step appends inside the attention kernel
    for this workload (it issues the append apart for large pair counts)."""
    import paged_mqa_gqa_amd as pa
    cfg = w.cfg
    d = pa.PaDims(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                  cfg.block_size, w.num_pages, cfg.max_blocks, KV_DTYPE_CODE[cfg.kv_dtype])
    return pa.step_fuses_append(d)


def attention_algorithmic_bytes(w, with_append=True) -> int:
    """Bytes one decode step must move at minimum: K/V of every attended
    token, q, the fp16 output, the block-table entries of those tokens, the
    context lengths and positions, (fp8) the scales, and the appended rows
    (fp16 in, cache format out; left out with `with_append=False`, for the
    attention launch alone). Split partials are this implementation's
    overhead and are not counted."""
    cfg = w.cfg
    L = w.context_lens.astype("int64")
    nblk = -(-L // cfg.block_size)
    qb = cfg.num_seqs * cfg.num_q_heads * cfg.head_dim * 2
    scales = 0 if cfg.kv_dtype == "fp16" else 2 * cfg.num_kv_heads * 4
    rows = cfg.num_seqs * cfg.num_kv_heads * cfg.head_dim * 2     # K and V
    append = rows * 2 + rows * cfg.kv_bytes_per_elem
    if not with_append:
        append = 0
    return int(w.kv_bytes() + 2 * qb + int(nblk.sum()) * 4 * cfg.num_kv_heads
               + cfg.num_seqs * 8 + scales + append)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of the same step."""
    import oracle
    threads = blas_threads()
    from workloads.device import remap_pages
    cfg = w.cfg
    ks, vs = w.kv_scales()
    nk, nv, pos = w.new_tokens()
    seqs_done, kv_done, t_total = 0, 0, 0.0
    for b in range(cfg.num_seqs):
        # compact pool of this sequence's pages, all tokens but the last (untimed)
        sub = remap_pages(w, [b])
        kp, vp = oracle.empty_pools(sub.num_pages, cfg.num_kv_heads, cfg.block_size,
                                    cfg.head_dim, cfg.kv_dtype)
        K, V, sid, p = sub.tokens([b], upto_last=True)
        kp, vp = oracle.kv_append(kp, vp, sub.block_table, sid, p, K, V, cfg.kv_dtype, ks, vs)
        t0 = time.perf_counter()
        kp, vp = oracle.kv_append(kp, vp, sub.block_table, [b], pos[b:b + 1], nk[b:b + 1],
                                  nv[b:b + 1], cfg.kv_dtype, ks, vs)
        oracle.decode(sub.q, kp, vp, sub.block_table, sub.context_lens, sub.scale,
                      cfg.kv_dtype, ks, vs, seqs=[b])
        t_total += time.perf_counter() - t0
        seqs_done += 1
        kv_done += int(w.context_lens[b]) * cfg.num_kv_heads * cfg.head_dim * 2 * \
            cfg.kv_bytes_per_elem
        if t_total >= budget_s:
            break
    return {
        "value": round(kv_done / t_total / 1e9, 4), "unit": "GB/s",
        "cores": int(threads), "kind": "oracle",
        "sample": f"{seqs_done} of {cfg.num_seqs} sequences of {cfg.name}, one decode "
                  f"step each (append + fp64 attention), {t_total:.1f} s; "
                  f"KV bytes attended / oracle time",
        "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
    }


def copy_only(nbytes: int, steps: int):
    """A plain streaming kernel of known size (reads nbytes, writes nbytes):
    the reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = nbytes // 2
    src = torch.randn(n, device="cuda", dtype=torch.float32).to(torch.float16)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 2, "copy_bytes_written": n * 2,
                      "launches": steps}), flush=True)


def time_graphs(stream, step_graphs, rotation_graph, launch_graph, launches, steps, warmup):
    """Replay `warmup` then exactly `steps` steps (whole rotations as one graph
    each, the rest one step graph at a time), synchronised on both sides and
    timed on the host; then the average duration of one launch from HIP
    events on `stream` around replays of `launch_graph` (`launches` launches
    back to back), measured LAUNCH_REPS times. Returns (ms per step, us per
    launch as the median of the repetitions, (min, max) of them)."""
    import torch
    R = len(step_graphs)

    def run_steps(k):
        for _ in range(k // R):
            rotation_graph.replay()
        for r in range(k % R):
            step_graphs[r].replay()

    with torch.cuda.stream(stream):
        run_steps(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        run_steps(steps)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    reps = max(4, steps // launches)
    samples = []
    for _ in range(LAUNCH_REPS):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            launch_graph.replay()
            e0.record(stream)
            for _ in range(reps):
                launch_graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        samples.append(e0.elapsed_time(e1) * 1e3 / (reps * launches))
    samples.sort()
    return ms_step, samples[len(samples) // 2], (samples[0], samples[-1])


def capture(stream, fn):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    return g


def split_ranges(pa, dw, S):
    """Token ranges the split pass actually cuts per (sequence, kv head) for
    this batch and split cap (read back from one untimed two-pass call)."""
    import torch
    if S == 1:
        return {"max": 1, "mean": 1.0}
    ws = pa.paged_decode_attn_splitk(dw.q, dw.k_pages, dw.v_pages, dw.block_table,
                                     dw.context_lens, dw.scale, S, dw.k_scale, dw.v_scale)
    torch.cuda.synchronize()
    B, Hq, d = dw.q.shape
    Hkv = dw.k_pages.shape[1]
    cnt = pa.split_views(ws, B, Hq, Hkv, S, d)[2].cpu().numpy()
    live = (dw.context_lens.cpu().numpy() > 0)
    c = cnt[live]
    return {"max": int(c.max()), "mean": round(float(c.mean()), 2)}


def bench_attention(args):
    import torch
    import paged_mqa_gqa_amd as pa
    from workloads import CONFIGS, Workload
    from workloads.device import DeviceWorkload

    cfg = CONFIGS[args.workload]
    w = Workload(cfg)
    S = args.splits or cfg.num_splits
    kvb = w.kv_bytes()
    R = args.replicas or max(1, min(8, -(-1_000_000_000 // kvb)))
    print(f"[bench] {cfg.name}: building inputs, KV {kvb / 1e6:.1f} MB, "
          f"{R} replica(s), {S} split(s)", file=sys.stderr, flush=True)

    dw = DeviceWorkload(w, upto_last=True)
    ranges = split_ranges(pa, dw, S)
    pools = [(dw.k_pages, dw.v_pages)] + [(dw.k_pages.clone(), dw.v_pages.clone())
                                          for _ in range(R - 1)]
    stream = torch.cuda.Stream()     # the stream every kernel goes to
    ws = pa.splitk_workspace(dw.q, dw.k_pages, dw.block_table, S)
    out = torch.empty_like(dw.q)
    group = cfg.num_q_heads // cfg.num_kv_heads
    # whether the library's step appends inside the attention kernel (it
    # issues the append as a launch of its own for large pair counts)
    fused = step_fuses_append(w) and not args.separate_append

    def attention(r):
        kp, vp = pools[r]
        pa.paged_decode_attn_splitk_merged(dw.q, kp, vp, dw.block_table,
                                           dw.context_lens, dw.scale, S, ws,
                                           dw.k_scale, dw.v_scale, out=out,
                                           stream=stream)

    def step(r):
        # kv_append + attention in one library call (appending the same
        # token again on later rotations writes the same bytes)
        kp, vp = pools[r]
        if args.separate_append:
            pa.kv_append(dw.new_k, dw.new_v, kp, vp, dw.block_table, dw.positions,
                         k_scale=dw.k_scale, v_scale=dw.v_scale, stream=stream)
            attention(r)
            return
        pa.paged_decode_step(dw.q, dw.new_k, dw.new_v, dw.positions, kp, vp,
                             dw.block_table, dw.context_lens, dw.scale, S, ws,
                             dw.k_scale, dw.v_scale, out=out, stream=stream)

    # eager run of every call once (first-use work stays out of the graphs)
    with torch.cuda.stream(stream):
        for r in range(R):
            step(r)
    torch.cuda.synchronize()
    step_graphs = [capture(stream, lambda r=r: step(r)) for r in range(R)]
    rotation_graph = capture(stream, lambda: [step(r) for r in range(R)])
    # the attention launch on its own: the step itself when the append is
    # fused into it, else the attention call the step makes after its append
    one = step if fused else attention
    with torch.cuda.stream(stream):
        one(0)
    torch.cuda.synchronize()
    attn_graph = capture(stream, lambda: [one(i % R) for i in range(ATTN_LAUNCHES_PER_GRAPH)])
    torch.cuda.synchronize()
    ms_step, attn_avg_us, attn_range = time_graphs(stream, step_graphs, rotation_graph, attn_graph,
                                       ATTN_LAUNCHES_PER_GRAPH, args.steps, args.warmup)

    value = kvb / (ms_step * 1e-3) / 1e9
    alg = attention_algorithmic_bytes(w, with_append=fused)
    achieved = alg / (attn_avg_us * 1e-6) / 1e9
    traffic = measured_traffic(cfg.name)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    if S == 1:
        attn_desc, kernel = "single pass", "decode_attn_kernel"
    elif group <= 16:
        attn_desc, kernel = "split pass with in-kernel merge", "decode_attn_stream_kernel"
    else:
        attn_desc = "split pass + reduce kernel"
        kernel = "decode_attn_stream_kernel (+ splitk_reduce_kernel)"
    attn_desc += (", kv_append fused into it" if fused
                  else ", kv_append as its own launch before it")
    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.kv_dtype,
        "data": "synthetic (seeded; no dataset or weights involved)",
        "config": {
            "workload": cfg.name, "batch": cfg.num_seqs, "q_heads": cfg.num_q_heads,
            "kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
            "block_size": cfg.block_size, "kv_dtype": cfg.kv_dtype,
            "context_tokens": int(w.context_lens.sum()), "kv_bytes": int(kvb),
            "splits": S, "ranges_per_pair": ranges, "pool_replicas": R,
            "step": f"kv_append + attention ({attn_desc}); the {R} steps of a replica "
                    f"rotation captured as one HIP graph",
        },
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "us_per_step": round(ms_step * 1e3, 2),
        "attn_us_per_call": round(attn_avg_us, 2),
        "attn_kv_gbs": round(kvb / (attn_avg_us * 1e-6) / 1e9, 2),
        "context_tokens_per_s": round(float(w.context_lens.sum()) / (ms_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "algorithmic_bytes_per_launch": alg,
            "launch_us": round(attn_avg_us, 3),
            "launch_us_min_max": [round(attn_range[0], 3), round(attn_range[1], 3)],
        },
        "cpu_baseline": cpu,
    }


def gemm_cpu_baseline(cfg, x, w, s, budget_s):
    """The fp64 oracle of the decode projection, as it stands, repeated for
    about budget_s seconds; weight bytes per second."""
    from oracle import gemm
    wt = gemm.transpose(w)
    st = gemm.transpose(s) if s is not None else None
    n, t = 0, 0.0
    while t < budget_s and n < 1000:
        t0 = time.perf_counter()
        gemm.gemm_m1(x, wt, st, cfg.group)
        t += time.perf_counter() - t0
        n += 1
    return {"value": round(cfg.weight_bytes * n / t / 1e9, 4), "unit": "GB/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{n} fp64 oracle products of {cfg.name} in {t:.1f} s; weight bytes "
                      f"/ oracle time (the transposes untimed)",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def gemm_algorithmic_bytes(cfg) -> int:
    """Bytes one decode-projection call must move: the weights (and their
    group scales), the activation rows in and the fp16 output out."""
    return cfg.weight_bytes + cfg.M * cfg.K * 2 + cfg.M * cfg.N * 2


def bench_gemm(args):
    import torch
    import paged_mqa_gqa_amd as pa
    from workloads import GEMM_CONFIGS, make_gemm

    cfg = GEMM_CONFIGS[args.workload]
    x, w, s = make_gemm(cfg)
    R = args.replicas or max(1, min(32, -(-1_000_000_000 // cfg.weight_bytes)))
    print(f"[bench] {cfg.name}: M {cfg.M} K {cfg.K} N {cfg.N} {cfg.w_dtype}, weights "
          f"{cfg.weight_bytes / 1e6:.1f} MB, {R} replica(s)", file=sys.stderr, flush=True)
    xd = torch.from_numpy(x).cuda()
    wd = torch.from_numpy(w).cuda()
    sd = torch.from_numpy(s).cuda() if s is not None else None
    # the load-time transposed copies, R of them so that the 256 MB Infinity
    # Cache cannot hold the weights a step reads
    wts = [pa.transpose_weights(wd) for _ in range(R)]
    sts = [pa.transpose_weights(sd) if sd is not None else None for _ in range(R)]
    del wd
    y = torch.empty((cfg.M, cfg.N), dtype=torch.float16, device="cuda")
    stream = torch.cuda.Stream()

    def step(r):
        pa.gemm_m1_transposed(xd, wts[r], sts[r], cfg.group, out=y, stream=stream)

    with torch.cuda.stream(stream):
        for r in range(R):
            step(r)
    torch.cuda.synchronize()
    step_graphs = [capture(stream, lambda r=r: step(r)) for r in range(R)]
    rotation_graph = capture(stream, lambda: [step(r) for r in range(R)])
    launches = max(8, R)
    launch_graph = capture(stream, lambda: [step(i % R) for i in range(launches)])
    torch.cuda.synchronize()
    ms_step, us_launch, us_range = time_graphs(stream, step_graphs, rotation_graph, launch_graph,
                                     launches, args.steps, args.warmup)
    alg = gemm_algorithmic_bytes(cfg)
    value = alg / (ms_step * 1e-3) / 1e9
    traffic = measured_traffic(cfg.name, "gemm_m1", GEMM_SOURCES)
    achieved = alg / (us_launch * 1e-6) / 1e9
    cpu = None if args.no_cpu_baseline else gemm_cpu_baseline(cfg, x, w, s,
                                                               min(args.cpu_seconds, 10.0))
    return {
        "metric": "decode projection weight GB/s (% of HBM peak) + us/call",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16" if cfg.w_dtype == "fp16" else "int8 weights, fp16 activations",
        "data": "synthetic (seeded random weights and activations)",
        "config": {"workload": cfg.name, "M": cfg.M, "K": cfg.K, "N": cfg.N,
                   "weights": cfg.w_dtype, "group": cfg.group if cfg.w_dtype == "int8" else None,
                   "weight_bytes": cfg.weight_bytes, "weight_replicas": R,
                   "step": "one gemm_m1_transposed call; the R calls of a replica rotation "
                           "captured as one HIP graph"},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "us_per_step": round(ms_step * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "gemm_m1_kernel",
                     "algorithmic_bytes_per_launch": alg, "launch_us": round(us_launch, 3),
                     "launch_us_min_max": [round(us_range[0], 3), round(us_range[1], 3)]},
        "cpu_baseline": cpu,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: --gpus {args.gpus} is not supported "
              f"(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.copy_only:
        copy_only(args.copy_only, args.steps)
        return
    import torch
    import paged_mqa_gqa_amd as pa
    from workloads import GEMM_CONFIGS
    torch.cuda.init()
    pa.load()
    res = bench_gemm(args) if args.workload in GEMM_CONFIGS else bench_attention(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
