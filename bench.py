#!/usr/bin/env python3
"""Throughput of the MI355X FMHA forward pass on one GPU (one JSON line).

A step is one call of the whole forward pass (fmha_fwd: tile scheduling, Q/K/V
loads, Q.K^T, masking, online softmax, P.V, epilogue) over one batch of
synthetic input already resident in HBM. The default workload is the bf16
varlen-causal d=128 case the headline figure is quoted on: 32768 tokens in 8
documents (cu_seqlens = round(linspace(0, 32768, 9))), 32 heads, seed 0.

Timing follows the FA4 spill issue's protocol (W warm-up steps, then K timed
steps; GPU events on the stream the kernel runs on). The defaults (100 timed
steps; warm-up steps for about 0.1 s of estimated work, at least 30, e.g. 91
for c4 and 728 for c3) let the GPU clock settle first: the first tens of
milliseconds after idle run at lower clocks. value = counted FLOP of
K steps / elapsed time, with FLOP = 4*h*sum(sq*sk)*d halved for causal.

Extra objects on the same line:
  roofline      counted FLOP per launch / average launch duration (per-step
                events) against MI355X's published dense bf16 MFMA peak, plus
                HBM traffic per launch from committed rocprofv3 counter
                summaries when they were taken on the current kernel sources
                (else null);
  cpu_baseline  the fp64 CPU oracle timed on this host on a bounded sample of
                the same workload (whole document x head units), in the same unit.

--step bwd times the backward pass (fmha_bwd, given the forward's O and LSE and
a fixed upstream gradient dO = 2 O / n, the gradient of the FA4 issue's loss
mean(O^2)); --step fwd_bwd times the forward followed by the backward, the step
that issue benchmarks. Backward FLOP are counted as 2.5 times the forward's
(five products of the forward's size instead of two: S and dP recomputed,
dV, dK, dQ), the usual convention; the kernels execute seven (dQ recomputes S
and dP). The roofline object then brackets the whole fmha_bwd call (its three
launches, on one stream); rocprofv3 summaries give the per-kernel split.

Options: --workload c1|c2|c3|c4|c5 (other workloads, for measurement only:
x_varlen_noncausal_32k, x_short_q_long_k, x_causal_fp4pv_32k, x_causal_bf16_32k),
--splits N|auto
(the split-KV pass), --trace coarse|detailed (pipeline summary of a traced launch),
--variant, --no-cpu-baseline, --counters (a short run for rocprofv3 --pmc: a
copy kernel of known size, then a few steps), --summarize-counters and
--summarize-trace (turn rocprofv3 CSV output into the committed summaries).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}   # published dense MFMA peaks
MI355X_HBM_GBPS = 8000.0
CSRC = os.path.join(ROOT, "head_attention_forward_fmha_amd", "csrc")
KERNEL_SOURCES = ("fmha_fwd_kernel.hip", "fmha_device.h", "fmha_kernel_params.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fmha_fwd_traffic.json")
KERNEL_NAMES = {"four_wave": "fmha::fmha_fwd_kernel", "pingpong": "fmha::fmha_fwd_pingpong_kernel",
                "pipelined": "fmha::fmha_fwd_pipe_kernel", "wide": "fmha::fmha_fwd_wide_kernel"}
# counted FLOP of the oracle sample: about 10-30 s of fp64 numpy on a 16-core host
CPU_SAMPLE_FLOP = 4e11

SHORT = {"c1": "c1_tiny_dense", "c2": "c2_dense_2225", "c3": "c3_varlen_causal_8k",
         "c4": "c4_varlen_causal_32k", "c5": "c5_causal_fp8pv_32k"}


def kernel_source_hash() -> str:
    """Hash of the device sources; counter figures taken on other sources are stale."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pv_format(w) -> int:
    """The kernels' P.V format template argument: 0 bf16, 1 fp8 e4m3, 2 fp4 e2m1."""
    return 2 if w.fp4_pv else 1 if w.fp8_pv else 0


def kernel_template_name(w, variant, split=False):
    if variant in ("pipelined", "wide"):
        return f"{KERNEL_NAMES[variant]}<{w.head_dim}, {str(w.causal).lower()}>"
    return (f"{KERNEL_NAMES[variant]}<{w.head_dim}, {str(w.causal).lower()}, {pv_format(w)}, "
            f"{str(split).lower()}>")


def timed_kernel_resources(w, variant, split=False):
    """The compiler's resource report entry of the timed forward kernel (None if
    the report written by the build is missing)."""
    from head_attention_forward_fmha_amd import build as fb
    return fb.kernel_resources(fb.mangled_kernel_name(variant, w.head_dim, w.causal,
                                                      pv_format(w), split))


def bwd_kernel_resources(w):
    """Resource report entries of the two backward kernels, by role."""
    from head_attention_forward_fmha_amd import build as fb
    return {role: fb.kernel_resources(fb.mangled_kernel_name(fam, w.head_dim, w.causal))
            for role, fam in (("dq", "bwd_dq"), ("dkdv", "bwd_dkdv"))}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clock ramps up over the first tens of milliseconds of work: the
    # default warm-up covers about 0.1 s of work, and the timed steps about
    # 100 ms of c4
    ap.add_argument("--steps", type=int, default=100)
    # default: at least 30 steps and about 0.1 s of estimated work (at 1 PFLOP/s
    # counted), so that the clock has settled also for the short workloads
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="c4",
                    choices=sorted(SHORT) + sorted(SHORT.values()) +
                    ["x_varlen_noncausal_32k", "x_short_q_long_k", "x_causal_fp4pv_32k",
                     "x_causal_bf16_32k"])
    ap.add_argument("--variant", default="auto", choices=["auto", "four_wave", "pingpong", "pipelined", "wide"],
                    help="kernel variant (auto picks by problem size)")
    ap.add_argument("--splits", default=None,
                    help="run the split-KV pass (bf16) with this many key splits, or 'auto'; "
                         "the workspace is allocated once, outside the timed region")
    ap.add_argument("--trace", choices=["coarse", "detailed"], default=None,
                    help="after the warm-up, one traced launch of the causal ping-pong kernel; "
                         "prints the pipeline summary instead of the throughput line")
    ap.add_argument("--step", choices=["fwd", "bwd", "fwd_bwd"], default="fwd",
                    help="what one timed step runs (bf16 workloads for bwd and fwd_bwd)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-flop", type=float, default=CPU_SAMPLE_FLOP,
                    help="counted FLOP of the oracle sample (whole document x head units)")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 --pmc: copy kernel of known size, then steps")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --counters run into an entry of the traffic file")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="print a rocprofv3 --stats kernel_stats.csv as a text table")
    ap.add_argument("--summarize-sq", metavar="COUNTER_CSV",
                    help="print the SQ/GRBM counters of a --counters run per FMHA launch, with "
                         "the MFMA FLOP, exp2 and MFMA-busy checks against the workload")
    ap.add_argument("--sustain", type=float, default=None, metavar="SECONDS",
                    help="after the warm-up, run the step back to back for SECONDS and print "
                         "one line (launches, us per step, TFLOP/s): a load under which the "
                         "board's clock and power can be read (amd-smi metric -p -c)")
    ap.add_argument("--microbench", action="store_true",
                    help="instead of a step: instruction-throughput microbenchmarks (exp2, FMA, "
                         "P conversions, MFMA, LDS reads and their overlap), one JSON line")
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
    elif w.fp4_pv:
        d["v4"] = inp.v_e2m1.to(dev)
        d["vx"] = inp.v_mx_scale.to(dev)
    else:
        d["v"] = inp.v.to(dev)
    d["out"] = torch.empty((w.total_q, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    d["lse"] = torch.empty((w.heads, w.total_q), dtype=torch.float32, device=dev)
    return inp, d


def make_step(w, d, variant="auto", splits=None):
    import head_attention_forward_fmha_amd as fm
    import torch
    mq, mk = w.max_seqlen_q, w.max_seqlen_k
    if splits is not None:
        if w.fp8_pv or w.fp4_pv:
            raise SystemExit("split-KV runs the bf16 path only")
        n = (fm.splitkv_num_splits(w.batch, mq, mk, w.heads, w.causal, variant)
             if splits == "auto" else int(splits))
        nbytes = fm.splitkv_workspace_size(w.total_q, w.heads, w.head_dim, n)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=d["q"].device) if nbytes else None
        d["splits"] = n

        def step():
            fm.fwd_splitkv(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], mq, mk, causal=w.causal,
                           softmax_scale=w.softmax_scale, out=d["out"], lse=d["lse"],
                           num_splits=n, workspace=ws, variant=variant)
        return step
    if w.fp8_pv:
        def step():
            fm.fwd_fp8pv(d["q"], d["k"], d["v8"], d["vs"], d["cu_q"], d["cu_k"], mq, mk,
                         causal=w.causal, softmax_scale=w.softmax_scale, out=d["out"],
                         lse=d["lse"], variant=variant)
    elif w.fp4_pv:
        def step():
            fm.fwd_fp4pv(d["q"], d["k"], d["v4"], d["vx"], d["cu_q"], d["cu_k"], mq, mk,
                         causal=w.causal, softmax_scale=w.softmax_scale, out=d["out"],
                         lse=d["lse"], variant=variant)
    else:
        def step():
            fm.fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], mq, mk, causal=w.causal,
                   softmax_scale=w.softmax_scale, out=d["out"], lse=d["lse"], variant=variant)
    return step


def make_bwd_step(w, d, with_fwd):
    """The backward (or forward + backward) step. O and LSE come from one forward
    pass; dO = 2 O / n (the loss gradient, computed once: it is elementwise work
    outside the attention) stays fixed, which does not change the work done."""
    import head_attention_forward_fmha_amd as fm
    import torch
    if w.fp8_pv or w.fp4_pv:
        raise SystemExit("the backward pass is bf16")
    mq, mk = w.max_seqlen_q, w.max_seqlen_k
    fwd_args = (d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], mq, mk)
    fm.fwd(*fwd_args, causal=w.causal, softmax_scale=w.softmax_scale, out=d["out"], lse=d["lse"])
    n = d["out"].numel()
    d["dout"] = (d["out"].float() * (2.0 / n)).to(torch.bfloat16)
    ws = torch.empty(fm.bwd_workspace_size(w.total_q, w.heads), dtype=torch.uint8,
                     device=d["q"].device)
    dq, dk, dv = (torch.empty_like(d[x]) for x in ("q", "k", "v"))

    def bwd():
        fm.bwd(d["q"], d["k"], d["v"], d["out"], d["dout"], d["lse"], d["cu_q"], d["cu_k"], mq,
               mk, causal=w.causal, softmax_scale=w.softmax_scale, dq=dq, dk=dk, dv=dv,
               workspace=ws)
    if not with_fwd:
        return bwd

    def step():
        fm.fwd(*fwd_args, causal=w.causal, softmax_scale=w.softmax_scale, out=d["out"],
               lse=d["lse"])
        bwd()
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


def load_traffic(w, variant):
    """Per-launch HBM bytes from committed counter summaries, if taken on these sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    entry = t.get(f"{w.name}/{variant}")
    if entry is None or entry.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return float(entry["hbm_bytes_per_launch"])


def cpu_baseline(w, inp, sample_flop, step="fwd"):
    """Time the fp64 oracle on a bounded sample of the workload.

    The sample is whole (document, head) units, longest documents first and heads
    in order, until their counted FLOP (the same convention as the GPU figure)
    reaches sample_flop or the workload is exhausted. step "bwd" times the
    backward oracle (with a fixed N(0, 1) dO), "fwd_bwd" both."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    cu_q, cu_k = np.asarray(inp.cu_q), np.asarray(inp.cu_k)
    order = sorted(range(len(cu_q) - 1), key=lambda b: -(cu_q[b + 1] - cu_q[b]))
    if w.fp8_pv:
        v = oracle.dequantize_v(inp.v_e4m3, inp.v_scale)
    elif w.fp4_pv:
        v = oracle.mx_dequantize_v(inp.v_e2m1, inp.v_mx_scale, w.head_dim)
    else:
        v = inp.v
    mult = {"fwd": 1.0, "bwd": 2.5, "fwd_bwd": 3.5}[step]
    dout = None
    if step != "fwd":
        from synthetic import make_dout
        dout = make_dout(w.total_q, w.heads, w.head_dim, seed=w.seed)
    done, units, parts, dt = 0.0, 0, [], 0.0
    for b in order:
        sq, sk = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b])
        per_head = mult * 4.0 * sq * sk * w.head_dim / (2.0 if w.causal else 1.0)
        if per_head == 0:
            continue
        n_heads = int(min(w.heads, max(1, np.ceil((sample_flop - done) / per_head))))
        t0 = time.perf_counter()
        if step != "bwd":
            oracle.attention(inp.q, inp.k, v, inp.cu_q, inp.cu_k, w.causal, w.softmax_scale,
                             heads=list(range(n_heads)), docs=[b])
        if step != "fwd":
            oracle.attention_backward(inp.q, inp.k, v, dout, inp.cu_q, inp.cu_k, w.causal,
                                      w.softmax_scale, heads=list(range(n_heads)), docs=[b])
        dt += time.perf_counter() - t0
        done += n_heads * per_head
        units += n_heads
        parts.append(f"doc {b} ({sq} tokens) x {n_heads} heads")
        if done >= sample_flop:
            break
    return {"value": done / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{units} (document, head) units: {'; '.join(parts)}; "
                      f"{done / 1e9:.1f} GFLOP counted ({step}), fp64 numpy, {dt:.1f} s wall"}


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


def run_trace(w, d, step, args):
    """Warm up untraced, then one traced launch; print the pipeline summary."""
    import head_attention_forward_fmha_amd as fm
    import numpy as np
    import torch
    from head_attention_forward_fmha_amd import pipeline_trace
    if not w.causal or w.head_dim != 128:
        raise SystemExit("the pipeline trace covers causal d=128 launches")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pv = "e4m3" if w.fp8_pv else "e2m1" if w.fp4_pv else "bf16"
    v = d["v8"] if w.fp8_pv else d["v4"] if w.fp4_pv else d["v"]
    vs = d["vs"] if w.fp8_pv else d["vx"] if w.fp4_pv else None
    def traced():
        return fm.fwd_trace(d["q"], d["k"], v, d["cu_q"], d["cu_k"], w.max_seqlen_q,
                            w.max_seqlen_k, pv=pv, v_scale=vs, softmax_scale=w.softmax_scale,
                            detailed=args.trace == "detailed", traced_workgroups=32)
    traced()                       # loads the traced kernel's code
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    _, _, trace = traced()
    end.record()
    torch.cuda.synchronize()
    summary = pipeline_trace.summarize(trace.cpu().numpy().view(np.uint64))
    summary.update({"trace": args.trace, "workload": w.name, "pv": pv, "traced_workgroups": 32,
                    "launch_us": round(start.elapsed_time(end) * 1e3, 1)})
    print(json.dumps(summary), flush=True)


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_counters(fetch_csv, write_csv, copy_bytes=256 * 1024 * 1024):
    """HBM bytes per FMHA launch from a --counters run under rocprofv3 --pmc.

    FETCH_SIZE and WRITE_SIZE are KiB per dispatch. Each is scaled by the ratio of
    the bytes the copy kernel of known size moved to what the counter read for it,
    then averaged over the FMHA dispatches of the run."""
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r["Counter_Name"] == counter]
        per = {}
        for r in rows:
            key = (r["Dispatch_Id"], r["Kernel_Name"], int(r["Grid_Size"]))
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        copies = [v for (_, name, grid), v in per.items()
                  if "copyBuffer" in name and v * 1024 > copy_bytes / 8]
        fmha = [(name, v) for (_, name, _), v in per.items() if "fmha_fwd" in name]
        if len(copies) != 1 or not fmha:
            raise SystemExit(f"{path}: expected one {copy_bytes}-byte copy and FMHA dispatches")
        factor = copy_bytes / (copies[0] * 1024)
        names = {n for n, _ in fmha}
        if len(names) != 1:
            raise SystemExit(f"{path}: more than one FMHA kernel: {sorted(names)}")
        kib = sum(v for _, v in fmha) / len(fmha)
        out[counter] = {"kib_per_dispatch": kib, "copy_factor": factor,
                        "bytes_per_launch": kib * 1024 * factor, "dispatches": len(fmha),
                        "kernel": names.pop()}
    return out


def run_sustained(w, step, seconds, warmup):
    """The step back to back for `seconds` (synchronising every 50 steps)."""
    import time
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n, t0 = 0, time.time()
    e0.record()
    while time.time() - t0 < seconds:
        for _ in range(50):
            step()
        torch.cuda.synchronize()
        n += 50
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    print(json.dumps({"workload": w.name, "sustained_s": round(time.time() - t0, 1), "steps": n,
                      "us_per_step": round(ms * 1e3, 1),
                      "tflops": round(w.flops() / (ms * 1e-3) / 1e12, 1)}), flush=True)


def visible_scores(w):
    """Score elements the method evaluates an exp2 for: per (document, head),
    the (query, key) pairs the mask leaves visible (bottom-right causal)."""
    import numpy as np
    total = 0
    for sq, sk in w.doc_lens:
        if w.causal:
            i = np.arange(sq, dtype=np.int64)
            total += int(np.clip(i + 1 + sk - sq, 0, sk).sum())
        else:
            total += sq * sk
    return total * w.heads


def summarize_sq(csv_path, w, simds=1024, xcds=8):
    """Per-launch averages of the counters of a rocprofv3 --pmc --counters run,
    kernel by kernel (the forward's one kernel, or the backward's dQ and dK/dV
    kernels), and the checks the counters present allow:
    MFMA FLOP = 512 x the MFMA MOPS counters, against the counted forward FLOP
    (the kernel also multiplies the masked part of its diagonal tiles);
    transcendental instructions x 64 lanes per visible score (one exp2 per
    score, plus the rescale exp2s and the epilogue's log);
    MFMA busy cycles per SIMD over the elapsed cycles per XCD (GRBM_GUI_ACTIVE
    sums the XCDs);
    LDS bank- and address-conflict stall cycles over the cycles the LDS spends
    on indexed (ds_read/ds_write) work, and per LDS instruction."""
    per = {}
    for r in _counter_rows(csv_path):
        name = r["Kernel_Name"]
        if "fmha_fwd" not in name and "fmha_bwd" not in name:
            continue
        d = per.setdefault(name, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{csv_path}: no FMHA dispatches")
    lines = []
    for name in sorted(per):
        disp = per[name]
        counters = sorted({c for d in disp.values() for c in d})
        avg = {c: sum(d.get(c, 0.0) for d in disp.values()) / len(disp) for c in counters}
        if lines:
            lines.append("")
        lines.append(f"{len(disp)} dispatches of {name}")
        for c in counters:
            lines.append(f"  {c:32s} {avg[c]:.4e}")
        fwd = "fmha_fwd" in name
        mops = sum(v for c, v in avg.items() if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
        if mops and fwd:
            lines.append(f"  MFMA FLOP (512 x MOPS)           {512 * mops:.4e}  "
                         f"= {512 * mops / w.flops():.4f} x the counted {w.flops():.4e}")
        elif mops:
            lines.append(f"  MFMA FLOP (512 x MOPS)           {512 * mops:.4e}  "
                         f"= {512 * mops / w.flops():.4f} x the counted forward {w.flops():.4e}")
        if "SQ_INSTS_VALU_TRANS_F32" in avg and fwd:
            vis = visible_scores(w)
            lines.append(f"  transcendental lane ops / visible score  "
                         f"{64 * avg['SQ_INSTS_VALU_TRANS_F32'] / vis:.4f}  "
                         f"({vis:.4e} visible scores)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
            busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
            elapsed = avg["GRBM_GUI_ACTIVE"] / xcds
            lines.append(f"  MFMA busy per SIMD / elapsed     {busy:.4e} / {elapsed:.4e} = "
                         f"{busy / elapsed:.3f}")
        for c, what in (("SQ_LDS_BANK_CONFLICT", "bank-conflict"),
                        ("SQ_LDS_ADDR_CONFLICT", "address-conflict")):
            if c not in avg:
                continue
            if avg.get("SQ_LDS_IDX_ACTIVE"):
                lines.append(f"  LDS {what} cycles / indexed LDS cycles  "
                             f"{avg[c] / avg['SQ_LDS_IDX_ACTIVE']:.4f}")
            if avg.get("SQ_INSTS_LDS"):
                lines.append(f"  LDS {what} cycles / LDS instruction     "
                             f"{avg[c] / avg['SQ_INSTS_LDS']:.4f}")
    return "\n".join(lines)


def summarize_trace(stats_csv):
    rows = _counter_rows(stats_csv)
    lines = [f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                     f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
                     f"{float(r['Percentage']):>6.2f}  {r['Name']}")
    return "\n".join(lines)


def bwd_line(w, args, inp, d, step, total_ms, each):
    """The JSON line of a --step bwd / fwd_bwd run."""
    import head_attention_forward_fmha_amd as fm
    mult = 2.5 if args.step == "bwd" else 3.5
    flops = mult * w.flops()
    value = flops * args.steps / (total_ms * 1e-3) / 1e12
    if args.step == "bwd":
        bwd_ms = sum(each) / len(each)
    else:
        # time the backward call alone for the roofline of its kernels
        bwd = make_bwd_step(w, d, with_fwd=False)
        _, each_b = time_steps(bwd, max(10, args.steps // 2), 5)
        bwd_ms = sum(each_b) / len(each_b)
    achieved = 2.5 * w.flops() / (bwd_ms * 1e-3) / 1e12
    peak = MI355X_PEAK_TFLOPS["bf16"]
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None,
            "kernel": f"fmha_bwd call: fmha::fmha_bwd_dq_kernel<{w.head_dim}, "
                      f"{str(w.causal).lower()}>, "
                      f"fmha::fmha_bwd_dkdv_kernel<{w.head_dim}, {str(w.causal).lower()}>",
            "launch_avg_us": round(bwd_ms * 1e3, 2),
            "algorithmic_flop_per_launch": 2.5 * w.flops()}
    line = {
        "metric": ("FMHA bwd" if args.step == "bwd" else "FMHA fwd+bwd") +
                  " TFLOP/s (bwd counted as 2.5x the fwd FLOP), d=%d, 1 GPU" % w.head_dim,
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 4),
        "median_ms": round(each[len(each) // 2], 4), "min_ms": round(each[0], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.description, "name": w.name, "total_tokens": w.total_q,
                   "docs": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "causal": w.causal, "seed": w.seed, "step": args.step,
                   "kernel_variant": fm.auto_variant(w.batch, w.max_seqlen_q, w.heads)},
        "roofline": roof,
        "kernel_resources": bwd_kernel_resources(w),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_sample_flop, args.step)
    return line


def main():
    args = parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_sq:
        from synthetic import EXTRA_WORKLOADS, WORKLOADS
        w = {**WORKLOADS, **EXTRA_WORKLOADS}[SHORT.get(args.workload, args.workload)]
        print(summarize_sq(args.summarize_sq, w))
        return
    if args.summarize_counters:
        # the counters must have been taken on the current sources: the entry is
        # stamped with their hash, and a later change of the kernel voids it
        from synthetic import EXTRA_WORKLOADS, WORKLOADS
        w = {**WORKLOADS, **EXTRA_WORKLOADS}[SHORT.get(args.workload, args.workload)]
        c = summarize_counters(*args.summarize_counters)
        kernel = c["FETCH_SIZE"]["kernel"]
        variant = ("pingpong" if "pingpong" in kernel else
                   "pipelined" if "pipe_kernel" in kernel else
                   "wide" if "wide_kernel" in kernel else "four_wave")
        table = {}
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                table = json.load(f)
        table[f"{w.name}/{variant}"] = {
            "kernel": kernel, "kernel_source_sha256_16": kernel_source_hash(),
            "hbm_bytes_per_launch": round(c["FETCH_SIZE"]["bytes_per_launch"] +
                                          c["WRITE_SIZE"]["bytes_per_launch"]),
            "algorithmic_hbm_bytes_per_launch": w.hbm_bytes(),
            "fetch_kib_per_dispatch": round(c["FETCH_SIZE"]["kib_per_dispatch"], 1),
            "fetch_copy_factor": round(c["FETCH_SIZE"]["copy_factor"], 4),
            "write_kib_per_dispatch": round(c["WRITE_SIZE"]["kib_per_dispatch"], 1),
            "write_copy_factor": round(c["WRITE_SIZE"]["copy_factor"], 4),
            "dispatches": c["FETCH_SIZE"]["dispatches"]}
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(table[f"{w.name}/{variant}"], indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this FMHA forward pass has no multi-GPU path "
              "(heads/documents would shard across GPUs with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.microbench:
        if not torch.cuda.is_available():
            raise SystemExit("bench.py --microbench needs a GPU")
        from head_attention_forward_fmha_amd import microbench
        props = torch.cuda.get_device_properties(0)
        cus = props.multi_processor_count
        rows = microbench.run_all(cus)
        print(json.dumps({"microbench": "instruction throughput in isolation", "device": props.name,
                          "gcn_arch": getattr(props, "gcnArchName", ""), "cus": cus,
                          "cycles": "shader clock (s_memtime), per wave, median over the device",
                          "rows": rows}))
        return
    from synthetic import EXTRA_WORKLOADS, WORKLOADS
    import head_attention_forward_fmha_amd as fm
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)
    name = SHORT.get(args.workload, args.workload)
    w = {**WORKLOADS, **EXTRA_WORKLOADS}[name]
    dev = torch.device("cuda:0")
    inp, d = device_inputs(w, dev)
    if args.step == "fwd":
        step = make_step(w, d, args.variant, args.splits)
    else:
        if args.splits is not None or args.trace or args.variant != "auto":
            raise SystemExit("--step bwd/fwd_bwd runs the default forward variant, unsplit")
        step = make_bwd_step(w, d, with_fwd=args.step == "fwd_bwd")
    if args.warmup is None:
        est_s = (w.flops() * (3.5 if args.step == "fwd_bwd" else 2.5 if args.step == "bwd"
                              else 1.0)) / 1e15
        args.warmup = max(30, min(5000, int(math.ceil(0.1 / max(est_s, 1e-9)))))
    if args.counters:
        run_counters(w, d, step)
        return
    if args.trace:
        run_trace(w, d, step, args)
        return
    if args.sustain is not None:
        run_sustained(w, step, args.sustain, args.warmup)
        return
    total_ms, each = time_steps(step, args.steps, args.warmup)
    if args.step != "fwd":
        print(json.dumps(bwd_line(w, args, inp, d, step, total_ms, each)), flush=True)
        return
    flops = w.flops()
    ms_per_step = total_ms / args.steps
    value = flops * args.steps / (total_ms * 1e-3) / 1e12
    # one launch per step (split-KV: the split kernel and the merge): the per-step
    # events bracket the whole pass
    launch_ms = sum(each) / len(each)
    achieved = flops / (launch_ms * 1e-3) / 1e12
    dtype = "bf16+fp8" if w.fp8_pv else "bf16+e2m1" if w.fp4_pv else "bf16"
    peak = MI355X_PEAK_TFLOPS["bf16"]
    variant = (args.variant if args.variant != "auto"
               else fm.auto_variant(w.batch, w.max_seqlen_q, w.heads))
    if args.variant == "auto" and d.get("splits", 1) > 1:
        # the library's automatic choice counts split work items: the 8-wave
        # kernel from 128 items of 256 query rows
        items = -(-w.max_seqlen_q // 256) * w.heads * w.batch * d["splits"]
        variant = "pingpong" if items >= 128 else "four_wave"
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": load_traffic(w, variant),
            "kernel": kernel_template_name(w, variant, "splits" in d),
            "launch_avg_us": round(launch_ms * 1e3, 2),
            "algorithmic_flop_per_launch": flops,
            "algorithmic_hbm_bytes_per_launch": w.hbm_bytes(),
            "algorithmic_hbm_gbps": round(w.hbm_bytes() / (launch_ms * 1e-3) / 1e9, 1)}
    if w.fp8_pv:
        # Q.K^T at the bf16 rate, P.V at the fp8 rate: the harmonic blend of the two peaks
        roof["peak_blended_bf16_fp8"] = 1.0 / (0.5 / MI355X_PEAK_TFLOPS["bf16"] +
                                               0.5 / MI355X_PEAK_TFLOPS["fp8"])
        roof["frac_blended"] = round(achieved / roof["peak_blended_bf16_fp8"], 4)
    if w.fp4_pv:
        # Q.K^T at the bf16 rate, P.V at the fp4 rate
        roof["peak_blended_bf16_fp4"] = 1.0 / (0.5 / MI355X_PEAK_TFLOPS["bf16"] +
                                               0.5 / MI355X_PEAK_TFLOPS["fp4"])
        roof["frac_blended"] = round(achieved / roof["peak_blended_bf16_fp4"], 4)
    line = {
        "metric": "FMHA fwd TFLOP/s and % of MI355X dense bf16 MFMA peak, d=128, 1 GPU",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "median_ms": round(each[len(each) // 2], 4), "min_ms": round(each[0], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.description, "name": w.name, "total_tokens": w.total_q,
                   "docs": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "causal": w.causal, "seed": w.seed, "fp8_pv": w.fp8_pv, "fp4_pv": w.fp4_pv,
                   "kernel_variant": variant, "key_splits": d.get("splits", 1)},
        "roofline": roof,
        "kernel_resources": timed_kernel_resources(w, variant, "splits" in d),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_sample_flop)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
