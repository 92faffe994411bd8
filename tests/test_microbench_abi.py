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
    (-1, 1, 10), (12, 1, 10),         # unknown benchmark
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
