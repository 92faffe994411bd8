"""CPU tests of the microbenchmark library: it loads without a GPU, exports what
include/fmha_microbench.h declares, its benchmark numbering matches the header,
and it refuses bad arguments before any HIP call."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmha_microbench.h")
LIB = os.path.join(ROOT, "head_attention_forward_fmha_amd", "libfmha_microbench.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfmha_microbench.so not built")


def _header_text():
    return re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)


def test_library_exports_every_declared_symbol():
    from head_attention_forward_fmha_amd import microbench
    declared = sorted(set(re.findall(r"\b(fmha_[a-z0-9_]+)\s*\(", _header_text())))
    assert declared == sorted(microbench.EXPORTED_SYMBOLS)
    lib = microbench.load_library()
    for name in declared:
        assert hasattr(lib, name), name


def test_benchmark_numbers_match_the_header():
    from head_attention_forward_fmha_amd import microbench
    defs = dict(re.findall(r"#define FMHA_MB_([A-Z0-9_]+) (\d+)", open(HEADER).read()))
    count = int(defs.pop("COUNT"))
    assert {k.lower(): int(v) for k, v in defs.items()} == microbench.BENCHMARKS
    assert sorted(microbench.BENCHMARKS.values()) == list(range(count))
    assert {n for n, _, _ in microbench.PLAN} == set(microbench.BENCHMARKS)


@pytest.mark.parametrize("which, wps, iters", [
    (-1, 1, 10), (14, 1, 10),         # unknown benchmark
    (0, 0, 10), (0, 5, 10),           # waves per SIMD outside 1..4
    (0, 1, 0), (0, 1, (1 << 20) + 1), # iteration count outside 1..2^20
    (10, 1, 10), (10, 3, 10),         # MFMA beside VALU needs exactly 2 waves per SIMD
])
def test_bad_arguments_are_refused_without_a_launch(which, wps, iters):
    from head_attention_forward_fmha_amd import microbench
    out = (ctypes.c_double * 2)(-7.0, -7.0)
    assert microbench.load_library().fmha_microbench_run(which, wps, iters, out) == 1
    assert list(out) == [-7.0, -7.0]


def test_null_result_is_refused():
    from head_attention_forward_fmha_amd import microbench
    assert microbench.load_library().fmha_microbench_run(0, 1, 10, None) == 1


def test_polynomial_exp2_is_accurate_to_bf16_and_beyond():
    """The FMA-path 2^x the microbenchmark times (exp2_poly in csrc/microbench.hip),
    restated in fp32 numpy: range reduction x = n + f by adding and subtracting
    1.5 * 2^23, a degree-3 polynomial for 2^f, n added to the exponent field.
    Against np.exp2 it stays within 7.6e-5 relative (about 13.7 bits, beyond the
    2^-9 of a bf16 P) from the clamp at -125 up to 8, the range a lazily
    rescaled softmax feeds it; at -126 the exponent field would reach zero
    (a subnormal encoding), which the clamp avoids."""
    import numpy as np
    f32 = np.float32
    x = np.concatenate([np.linspace(-125, 8, 400001), np.arange(-125, 9)]).astype(f32)
    rnd = f32(12582912.0)
    xc = np.maximum(x, f32(-125))
    t = (xc + rnd).astype(f32)
    n = (t - rnd).astype(f32)
    fr = (xc - n).astype(f32)
    c3, c2, c1, c0 = (f32(0.05517132207751274), f32(0.24261054396629333),
                      f32(0.6932609677314758), f32(0.9999281167984009))
    p = ((c3 * fr + c2).astype(f32) * fr + c1).astype(f32)
    p = (p * fr + c0).astype(f32)
    bits = (p.view(np.int32).astype(np.int64) + (t.view(np.int32).astype(np.int64) << 23)) % (1 << 32)
    y = bits.astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.abs(fr).max() <= 0.5
    rel = np.abs(y / np.exp2(x.astype(np.float64)) - 1)
    assert rel.max() < 7.6e-5, rel.max()
