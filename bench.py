#!/usr/bin/env python3
"""Throughput of the MI355X FMHA forward pass on one GPU (one JSON line).

A step is one call of the whole forward pass (fmha_fwd: tile scheduling, Q/K/V
loads, Q.K^T, masking, online softmax, P.V, epilogue) over one batch of
synthetic input already resident in HBM. The default workload is the bf16
varlen-causal d=128 case the headline figure is quoted on: 32768 tokens in 8
documents (cu_seqlens = round(linspace(0, 32768, 9))), 32 heads, seed 0.

Timing follows the FA4 spill issue's protocol (W warm-up steps, then K timed
steps; GPU events on the stream the kernel runs on). value = counted FLOP of
K steps / elapsed time, with FLOP = 4*h*sum(sq*sk)*d halved for causal.

Extra objects on the same line:
  roofline      achieved TFLOP/s of the FMHA kernel against MI355X's published
                dense bf16 MFMA peak, plus HBM traffic from committed rocprofv3
                counter summaries when they were taken on the current kernel
                source (else null);
  cpu_baseline  the fp64 CPU oracle timed on this host on a bounded sample of
                the same workload (one document, several heads), in the same unit.

Options: --workload c1|c2|c3|c4|c5 (other workloads, for measurement only),
--no-cpu-baseline, --counters (a short run for rocprofv3 --pmc: a copy kernel
of known size, then a few steps).
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

MI355X_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # published dense MFMA peaks
MI355X_HBM_GBPS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "head_attention_forward_fmha_amd", "csrc", "fmha_fwd_kernel.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fmha_fwd_traffic.json")

SHORT = {"c1": "c1_tiny_dense", "c2": "c2_dense_2225", "c3": "c3_varlen_causal_8k",
         "c4": "c4_varlen_causal_32k", "c5": "c5_causal_fp8pv_32k"}


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4", choices=sorted(SHORT) + sorted(SHORT.values()))
    ap.add_argument("--variant", default="auto", choices=["auto", "four_wave", "pingpong"],
                    help="kernel variant (auto picks by problem size)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-heads", type=int, default=16)
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 --pmc: copy kernel of known size, then steps")
    return ap.parse_args()


def device_inputs(w, dev):
    import numpy as np
    import torch
    from synthetic import workload_inputs
    inp = workload_inputs(w)
    d = dict(q=inp.q.to(dev), k=inp.k.to(dev),
             cu_q=torch.from_numpy(np.asarray(inp.cu_q, np.int32)).to(dev),
             cu_k=torch.from_numpy(np.asarray(inp.cu_k, np.int32)).to(dev))
    if w.fp8_pv:
        d["v8"] = inp.v_e4m3.to(dev)
        d["vs"] = inp.v_scale.to(dev)
    else:
        d["v"] = inp.v.to(dev)
    d["out"] = torch.empty((w.total_q, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    d["lse"] = torch.empty((w.heads, w.total_q), dtype=torch.float32, device=dev)
    return inp, d


def make_step(w, d, variant="auto"):
    import head_attention_forward_fmha_amd as fm
    mq, mk = w.max_seqlen_q, w.max_seqlen_k
    if w.fp8_pv:
        def step():
            fm.fwd_fp8pv(d["q"], d["k"], d["v8"], d["vs"], d["cu_q"], d["cu_k"], mq, mk,
                         causal=w.causal, softmax_scale=w.softmax_scale, out=d["out"],
                         lse=d["lse"], variant=variant)
    else:
        def step():
            fm.fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], mq, mk, causal=w.causal,
                   softmax_scale=w.softmax_scale, out=d["out"], lse=d["lse"], variant=variant)
    return step


def time_steps(step, steps, warmup):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # whole-region events plus per-step events (median, as the FA4 issue reports)
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for a, b in per:
        a.record(stream)
        step()
        b.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    each = sorted(a.elapsed_time(b) for a, b in per)
    return total_ms, each


def load_traffic(w):
    """Per-launch HBM bytes from committed counter summaries, if current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        entry = t.get(w.name)
        if entry is None or entry.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return float(entry["hbm_bytes_per_launch"])
    except Exception:
        return None


def cpu_baseline(w, inp, sample_heads):
    """Time the fp64 oracle on one document x sample_heads heads of the workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cu_q = np.asarray(inp.cu_q)
    doc = int(np.argmax(np.diff(cu_q)))
    heads = list(range(min(sample_heads, w.heads)))
    sq = int(cu_q[doc + 1] - cu_q[doc])
    v = inp.v
    if w.fp8_pv:
        v = oracle.dequantize_v(inp.v_e4m3, inp.v_scale)
    t0 = time.perf_counter()
    oracle.attention(inp.q, inp.k, v, inp.cu_q, inp.cu_k, w.causal, w.softmax_scale,
                     heads=heads, docs=[doc])
    dt = time.perf_counter() - t0
    flops = 4.0 * len(heads) * sq * sq * w.head_dim / (2.0 if w.causal else 1.0)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"document {doc} ({sq} tokens) x {len(heads)} of {w.heads} heads, "
                      f"fp64 numpy, {dt:.1f} s wall; same FLOP count convention"}


def run_counters(w, d, step):
    """A copy of known size (calibrates FETCH_SIZE/WRITE_SIZE), then a few steps."""
    import torch
    n = 256 * 1024 * 1024
    a = torch.empty(n, dtype=torch.uint8, device=d["q"].device).fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    print(json.dumps({"counters_run": w.name, "copy_bytes": n, "steps": 3}), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this FMHA forward pass has no multi-GPU path "
              "(heads/documents would shard across GPUs with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from synthetic import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)
    name = SHORT.get(args.workload, args.workload)
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    inp, d = device_inputs(w, dev)
    step = make_step(w, d, args.variant)
    if args.counters:
        run_counters(w, d, step)
        return
    total_ms, each = time_steps(step, args.steps, args.warmup)
    flops = w.flops()
    ms_per_step = total_ms / args.steps
    value = flops * args.steps / (total_ms * 1e-3) / 1e12
    dtype = "bf16+fp8" if w.fp8_pv else "bf16"
    peak = MI355X_PEAK_TFLOPS["bf16"]
    traffic = load_traffic(w)
    roof = {"bound": "mfma", "achieved": round(value, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(value / peak, 4), "traffic": traffic,
            "kernel": "fmha::fmha_fwd_kernel", "algorithmic_flop_per_launch": flops,
            "algorithmic_hbm_bytes_per_launch": w.hbm_bytes(),
            "achieved_hbm_gbps": round(w.hbm_bytes() / (ms_per_step * 1e-3) / 1e9, 1)}
    if w.fp8_pv:
        # Q.K^T at the bf16 rate, P.V at the fp8 rate: the harmonic blend of the two peaks
        roof["peak_blended_bf16_fp8"] = 1.0 / (0.5 / MI355X_PEAK_TFLOPS["bf16"] +
                                               0.5 / MI355X_PEAK_TFLOPS["fp8"])
        roof["frac_blended"] = round(value / roof["peak_blended_bf16_fp8"], 4)
    line = {
        "metric": "FMHA fwd TFLOP/s and % of MI355X dense bf16 MFMA peak, d=128, 1 GPU",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "median_ms": round(each[len(each) // 2], 4), "min_ms": round(each[0], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.description, "name": w.name, "total_tokens": w.total_q,
                   "docs": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "causal": w.causal, "seed": w.seed, "fp8_pv": w.fp8_pv,
                   "kernel_variant": args.variant},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_sample_heads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
