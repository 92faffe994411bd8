"""Instruction-throughput microbenchmarks on the current GPU (libfmha_microbench.so).

"Kernel Bottleneck Tuning (validated on FA4 FP4/FP8 PV, GB300)", section 1:
measure what each instruction sustains in isolation, with independent
dependency chains and a cycle counter, before budgeting a kernel with it. The
library times one wave per measurement (shader-clock cycles, s_memtime); this
module turns the cycles into per-compute-unit rates:

  vector ops       lane operations per clock per CU = waves * 64 / cycles
  MFMA             FLOP per clock per CU = waves * FLOP per instruction / cycles,
                   and the device rate at the nominal 2.4 GHz and the CU count
  LDS reads        bytes per clock per CU = waves * 1024 / cycles

The argument marshalling is all that happens here; every measurement runs in
the library's kernels (include/fmha_microbench.h).
"""

from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfmha_microbench.so")

EXPORTED_SYMBOLS = ("fmha_microbench_run",)

# FMHA_MB_* of include/fmha_microbench.h
BENCHMARKS = {
    "exp2": 0, "fma": 1, "cvt_bf16": 2, "cvt_e4m3": 3, "cvt_e2m1": 4, "exp2_e4m3": 5,
    "mfma_bf16": 6, "mfma_e4m3": 7, "lds_b128": 8, "mfma_lds_b128": 9, "mfma_with_valu": 10,
    "softmax": 11, "exp2_poly": 12, "exp2_with_fma": 13,
}
MFMA_FLOP = {"mfma_bf16": 2 * 32 * 32 * 16, "mfma_e4m3": 2 * 32 * 32 * 64,
             "mfma_lds_b128": 2 * 32 * 32 * 16, "mfma_with_valu": 2 * 32 * 32 * 16}
NOMINAL_GHZ = 2.4

_lib = None


def load_library():
    """Load libfmha_microbench.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m head_attention_forward_fmha_amd.build`")
        import torch  # noqa: F401  (one HIP runtime: torch's, loaded first)
        lib = ctypes.CDLL(LIB_PATH)
        lib.fmha_microbench_run.restype = ctypes.c_int32
        lib.fmha_microbench_run.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_double)]
        _lib = lib
    return _lib


def run_raw(name: str, waves_per_simd: int, iters: int):
    """(cycles per instruction or op per wave, secondary figure) of one benchmark."""
    out = (ctypes.c_double * 2)()
    st = load_library().fmha_microbench_run(BENCHMARKS[name], int(waves_per_simd), int(iters),
                                            out)
    if st != 0:
        raise RuntimeError(f"fmha_microbench_run({name}, {waves_per_simd}, {iters}): status {st}")
    return float(out[0]), float(out[1])


# (name, waves per SIMD, iterations); iterations sized for a few ms each
PLAN = (
    ("exp2", 1, 4000), ("exp2", 2, 4000), ("fma", 1, 4000), ("fma", 2, 4000),
    ("cvt_bf16", 2, 4000), ("cvt_e4m3", 2, 4000), ("cvt_e2m1", 2, 4000),
    ("exp2_e4m3", 2, 2000), ("softmax", 1, 400), ("softmax", 2, 400),
    ("mfma_bf16", 1, 400), ("mfma_bf16", 2, 400), ("mfma_e4m3", 1, 200),
    ("lds_b128", 1, 400), ("lds_b128", 2, 400),
    ("mfma_lds_b128", 1, 400), ("mfma_lds_b128", 2, 400),
    ("mfma_with_valu", 2, 400),
    ("exp2_poly", 1, 2000), ("exp2_poly", 2, 2000),
    ("exp2_with_fma", 1, 2000), ("exp2_with_fma", 2, 2000),
)


def run_all(cus: int, plan=PLAN):
    """Every benchmark of `plan`; a list of result dicts with the derived rates."""
    rows = []
    for name, wps, iters in plan:
        cyc, sec = run_raw(name, wps, iters)
        waves = 4 * wps
        row = {"bench": name, "waves_per_simd": wps, "iters": iters, "cycles": round(cyc, 3)}
        if name in MFMA_FLOP:
            mfma_waves = 4 if name == "mfma_with_valu" else waves
            flop_clk = mfma_waves * MFMA_FLOP[name] / cyc
            row["flop_per_clk_cu"] = round(flop_clk, 1)
            row["tflops_at_2p4ghz"] = round(flop_clk * cus * NOMINAL_GHZ * 1e9 / 1e12, 1)
            if name == "mfma_lds_b128":
                row["lds_bytes_per_clk_cu"] = round(waves * 1024 / cyc, 1)
            if name == "mfma_with_valu":
                row["valu_cycles_per_iter"] = round(sec, 1)
        elif name == "lds_b128":
            row["lds_bytes_per_clk_cu"] = round(waves * 1024 / cyc, 1)
        elif name == "softmax":
            row["cycles_per_iter"] = row.pop("cycles")
        else:
            row["lane_ops_per_clk_cu"] = round(waves * 64 / cyc, 1)
        rows.append(row)
    return rows
