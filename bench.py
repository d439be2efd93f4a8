#!/usr/bin/env python3
"""Benchmark one decode step of paged MQA/GQA attention on one MI355X.

A step is the whole hot path over one batch: kv_append of every sequence's
new token into its page, then decode attention (split pass plus
log-sum-exp merge, or the single pass when the workload uses one split).
Inputs are seeded synthetic data already resident in HBM; R replicas of the
KV pools rotate step to step so that the 256 MB Infinity Cache cannot serve
the working set.

Prints ONE JSON line: metric / value (KV GB/s of the step) / unit, timing,
`roofline` for the attention kernel (algorithmic bytes per launch / its
average event-timed duration, against 8 TB/s) and `cpu_baseline` (the fp64
oracle timed on this host over a bounded sample of the same workload).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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
KERNEL_SRC = os.path.join(ROOT, "paged_mqa_gqa_amd", "csrc", "decode_attn.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--splits", type=int, default=0, help="override the split count")
    ap.add_argument("--replicas", type=int, default=0, help="override pool replicas")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, f"decode_attn_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_algorithmic_bytes(w) -> int:
    """Bytes decode attention must move at minimum: K/V of every attended
    token, q, the block-table entries of those tokens, the context lengths
    and the fp16 output (split partials are this implementation's overhead,
    not counted)."""
    cfg = w.cfg
    L = w.context_lens.astype("int64")
    nblk = -(-L // cfg.block_size)
    qb = cfg.num_seqs * cfg.num_q_heads * cfg.head_dim * 2
    return int(w.kv_bytes() + 2 * qb + int(nblk.sum()) * 4 * cfg.num_kv_heads
               + cfg.num_seqs * 4)


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of the same step."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    from workloads.device import remap_pages
    cfg = w.cfg
    ks, vs = w.fp8_scales()
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
        "host_cpus": os.cpu_count(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: --gpus {args.gpus} is not supported "
              f"(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import paged_mqa_gqa_amd as pa
    from workloads import CONFIGS, Workload
    from workloads.device import DeviceWorkload

    torch.cuda.init()
    pa.load()
    cfg = CONFIGS[args.workload]
    w = Workload(cfg)
    S = args.splits or cfg.num_splits
    kvb = w.kv_bytes()
    R = args.replicas or max(1, min(8, -(-1_000_000_000 // kvb)))
    print(f"[bench] {cfg.name}: building inputs, KV {kvb / 1e6:.1f} MB, "
          f"{R} replica(s), {S} split(s)", file=sys.stderr, flush=True)

    dw = DeviceWorkload(w, upto_last=True)
    pools = [(dw.k_pages, dw.v_pages)] + [(dw.k_pages.clone(), dw.v_pages.clone())
                                          for _ in range(R - 1)]
    stream = torch.cuda.Stream()     # the stream every kernel goes to
    d = pa.dims(cfg.num_seqs, cfg.num_q_heads, dw.k_pages, dw.block_table)
    ws = pa.splitk_workspace(dw.q, dw.k_pages, dw.block_table, S)
    out = torch.empty_like(dw.q)
    torch.cuda.synchronize()

    def step(i, ev=None):
        kp, vp = pools[i % R]
        pa.kv_append(dw.new_k, dw.new_v, kp, vp, dw.block_table, dw.positions,
                     k_scale=dw.k_scale, v_scale=dw.v_scale, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        if S == 1:
            pa.paged_decode_attn(dw.q, kp, vp, dw.block_table, dw.context_lens,
                                 dw.scale, dw.k_scale, dw.v_scale, out=out, stream=stream)
            if ev is not None:
                ev[1].record(stream)
        else:
            pa.paged_decode_attn_splitk_merged(dw.q, kp, vp, dw.block_table,
                                               dw.context_lens, dw.scale, S, ws,
                                               dw.k_scale, dw.v_scale, out=out,
                                               stream=stream)
            if ev is not None:
                ev[1].record(stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            step(i, events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_step = elapsed * 1e3 / args.steps
    attn_us = [a.elapsed_time(b) * 1e3 for a, b in events]
    attn_avg_us = float(np.mean(attn_us))
    value = kvb / (ms_step * 1e-3) / 1e9
    alg = attention_algorithmic_bytes(w)
    achieved = alg / (attn_avg_us * 1e-6) / 1e9
    traffic = measured_traffic(cfg.name)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    res = {
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
        "dtype": "fp16" if cfg.kv_dtype == "fp16" else "fp8_e4m3fn",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "batch": cfg.num_seqs, "q_heads": cfg.num_q_heads,
            "kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
            "block_size": cfg.block_size, "kv_dtype": cfg.kv_dtype,
            "context_tokens": int(w.context_lens.sum()), "splits": S,
            "pool_replicas": R, "step": "kv_append + attention" +
            (" (single pass)" if S == 1 else " (split pass with in-kernel merge)"),
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
            "kernel": ("decode_attn_kernel (single pass)" if S == 1 else
                       "decode_attn_streamk_kernel (split pass, merged)"),
            "algorithmic_bytes_per_launch": alg,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
