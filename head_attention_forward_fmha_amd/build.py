"""Builds libfmha.so (HIP kernels + C ABI) and libfmha_microbench.so (the
instruction-throughput microbenchmarks) for gfx950 with hipcc, in-tree.

Usage: python -m head_attention_forward_fmha_amd.build [--verbose]

The library is linked against the HIP runtime with an rpath that prefers
torch's bundled libamdhip64.so, so that a process which imports torch first
and then loads this library uses exactly one HIP runtime (both carry the
SONAME libamdhip64.so.7). The compiler's kernel resource report
(-Rpass-analysis=kernel-resource-usage) is saved next to the library and
checked: every kernel must use no scratch and spill no registers.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfmha.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
RESOURCE_REPORT = os.path.join(PKG_DIR, "libfmha.resource-usage.txt")
SOURCES = ["fmha_fwd_kernel.hip", "fmha_merge.hip", "fmha_bwd_kernel.hip", "fmha_api.hip"]
# instruction-throughput microbenchmarks (measurement support, include/fmha_microbench.h)
MICROBENCH_SOURCE = "microbench.hip"
MICROBENCH_LIB_PATH = os.path.join(PKG_DIR, "libfmha_microbench.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay disabled; hipcc -O3 would otherwise form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libfmha.so")


def _torch_lib_dir():
    try:
        import torch
        return os.path.join(os.path.dirname(torch.__file__), "lib")
    except Exception:
        return None


def parse_resource_report(text: str) -> dict:
    """Map kernel name -> {field: value} from clang's kernel-resource-usage remarks.

    The remarks look like
      <file>:<line>:<col>: remark: Function Name: <symbol> [-Rpass-analysis=...]
      <file>:<line>:<col>: remark:     VGPRs Spill: 0 [-Rpass-analysis=...]
    """
    kernels = {}
    cur = None
    for line in text.splitlines():
        m = re.search(r"remark:\s+Function Name:\s+(\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?):\s+(\S+)\s+\[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return kernels


def check_resources(kernels: dict) -> list:
    """Return a list of violations (scratch use or spills) in a parsed report."""
    bad = []
    for name, f in kernels.items():
        if "ScratchSize [bytes/lane]" not in f or "VGPRs Spill" not in f:
            bad.append(f"{name}: resource report incomplete ({sorted(f)})")
            continue
        if f.get("ScratchSize [bytes/lane]", "0") != "0":
            bad.append(f"{name}: scratch {f.get('ScratchSize [bytes/lane]')} B/lane")
        for key in ("VGPRs Spill", "SGPRs Spill"):
            if f.get(key, "0") != "0":
                bad.append(f"{name}: {key} {f[key]}")
    return bad


# kernel families -> the Itanium-mangled prefix of their template instances
_MANGLED_PREFIX = {
    "pingpong": "_ZN4fmha24fmha_fwd_pingpong_kernel",
    "four_wave": "_ZN4fmha15fmha_fwd_kernel",
    "pipelined": "_ZN4fmha20fmha_fwd_pipe_kernel",
    "wide": "_ZN4fmha20fmha_fwd_wide_kernel",
    "bwd_dkdv": "_ZN4fmha12_GLOBAL__N_120fmha_bwd_dkdv_kernel",
    "bwd_dq": "_ZN4fmha12_GLOBAL__N_118fmha_bwd_dq_kernel",
}


def mangled_kernel_name(family: str, head_dim: int, causal: bool = False, pv: int = 0,
                        split: bool = False) -> str:
    """The symbol of one kernel instance, as the resource report names it.

    Template arguments: head dim, causal, P.V format (0 bf16, 1 fp8, 2 fp4) and
    key split for the forward kernels; the ping-pong's untraced instance."""
    b = lambda v: "ELb1" if v else "ELb0"  # noqa: E731
    pre = _MANGLED_PREFIX[family]
    if family == "pingpong":
        return (f"{pre}ILi{head_dim}{b(causal)}ELi{pv}{b(split)}ENS_12NoPhaseTraceEEEvNS_9FwdParamsE")
    if family == "four_wave":
        return f"{pre}ILi{head_dim}{b(causal)}ELi{pv}{b(split)}EEEvNS_9FwdParamsE"
    if family in ("pipelined", "wide"):
        return f"{pre}ILi{head_dim}{b(causal)}EEEvNS_9FwdParamsE"
    return f"{pre}ILi{head_dim}{b(causal)}EEEvNS_9BwdParamsE"


def kernel_resources(symbol: str, report_path: str = RESOURCE_REPORT):
    """Registers, scratch, spills, occupancy and LDS of one kernel from the saved
    resource report, or None when the report or the kernel is missing."""
    if not os.path.exists(report_path):
        return None
    with open(report_path) as f:
        entry = parse_resource_report(f.read()).get(symbol)
    if entry is None:
        return None

    def num(key):
        v = entry.get(key)
        return int(v) if v is not None and v.isdigit() else None

    return {"symbol": symbol, "vgprs": num("VGPRs"), "agprs": num("AGPRs"),
            "sgprs": num("TotalSGPRs"),
            "scratch_bytes_per_lane": num("ScratchSize [bytes/lane]"),
            "vgpr_spill": num("VGPRs Spill"), "sgpr_spill": num("SGPRs Spill"),
            "occupancy_waves_per_simd": num("Occupancy [waves/SIMD]"),
            "lds_bytes_per_block": num("LDS Size [bytes/block]")}


def _compile(hipcc: str, src_path: str, obj: str, includes, verbose: bool) -> str:
    cmd = [hipcc, *HIP_FLAGS, *[a for d in includes for a in ("-I", d)],
           "-Rpass-analysis=kernel-resource-usage", "-c", src_path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src_path)}")
    return r.stderr


def build(verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor
    hipcc = _hipcc()
    build_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(build_dir, exist_ok=True)
    jobs = [(os.path.join(CSRC, src), os.path.join(build_dir, src + ".o"), (INCLUDE, CSRC))
            for src in SOURCES]
    # the microbenchmark library: one source, its own shared object
    mb_obj = os.path.join(build_dir, MICROBENCH_SOURCE + ".o")
    jobs.append((os.path.join(CSRC, MICROBENCH_SOURCE), mb_obj, (INCLUDE,)))
    # the sources compile independently; a few at a time keeps memory modest
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as pool:
        reports = list(pool.map(lambda j: _compile(hipcc, j[0], j[1], j[2], verbose), jobs))
    objs = [j[1] for j in jobs[:len(SOURCES)]]
    rpaths = [d for d in (_torch_lib_dir(), "/opt/rocm/lib") if d]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           *[f"-Wl,-rpath,{d}" for d in rpaths]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libfmha.so failed")
    os.replace(tmp, LIB_PATH)
    tmp = MICROBENCH_LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, mb_obj,
           *[f"-Wl,-rpath,{d}" for d in rpaths]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libfmha_microbench.so failed")
    os.replace(tmp, MICROBENCH_LIB_PATH)
    text = "\n".join(reports)
    with open(RESOURCE_REPORT, "w") as f:
        f.write(text)
    bad = check_resources(parse_resource_report(text))
    if bad:
        raise RuntimeError("kernel resource gate failed (scratch or spills):\n  " + "\n  ".join(bad))
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
