"""CPU tests of the C-ABI boundary: the library loads without a GPU, exports every
function include/fmha.h declares, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmha.h")
LIB = os.path.join(ROOT, "head_attention_forward_fmha_amd", "libfmha.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfmha.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fmha_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert names == sorted(["fmha_fwd", "fmha_fwd_fp8pv", "fmha_fwd_variant",
                            "fmha_fwd_fp8pv_variant", "fmha_fwd_fp4pv", "fmha_fwd_fp4pv_variant",
                            "fmha_fwd_splitkv", "fmha_fwd_splitkv_workspace_size",
                            "fmha_fwd_splitkv_num_splits", "fmha_merge_partials", "fmha_fwd_trace",
                            "fmha_bwd", "fmha_bwd_workspace_size", "fmha_bwd_noalloc",
                            "fmha_fwd_auto_variant", "fmha_validate_cu_seqlens",
                            "fmha_status_string", "fmha_abi_version"])


def test_library_exports_every_declared_symbol():
    import head_attention_forward_fmha_amd as fm
    lib = fm.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(fm.EXPORTED_SYMBOLS) == set(_declared_functions())
    assert fm.abi_version() == (1 << 16) | 5


def test_status_strings():
    import head_attention_forward_fmha_amd as fm
    assert fm.status_string(0) == "ok"
    assert fm.status_string(1) == "invalid argument"
    assert fm.status_string(2) == "unsupported configuration"
    assert fm.status_string(3) == "kernel launch failed"
    assert fm.status_string(99) == "unknown status"


def _call_fwd(**kw):
    """Call fmha_fwd with fake (never dereferenced) aligned pointers."""
    import head_attention_forward_fmha_amd as fm
    lib = fm.load_library()
    a = dict(q=0x10000, k=0x20000, v=0x30000, cu_q=None, cu_k=None, batch=1, total_q=128,
             total_k=128, max_q=128, max_k=128, heads=2, d=64, causal=0, scale=0.125,
             out=0x40000, lse=0x50000)
    a.update(kw)
    return lib.fmha_fwd(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], a["batch"], a["total_q"],
                        a["total_k"], a["max_q"], a["max_k"], a["heads"], a["d"], a["causal"],
                        ctypes.c_float(a["scale"]), a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), 2),
    (dict(d=256), 2),
    (dict(heads=0), 1),
    (dict(batch=-1), 1),
    (dict(total_q=-5), 1),
    (dict(causal=2), 1),
    (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(scale=float("inf")), 1),
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(k=0x20008), 1),          # misaligned
    (dict(lse=0x50002), 1),
    (dict(total_q=100), 1),        # dense: total != batch * max_seqlen
    (dict(cu_q=0x60000), 1),       # only one cu_seqlens pointer
    (dict(heads=70000), 2),
    # 32-bit offsets: heads * d * (total + 64) must stay below 2^31 (here 2 * 64: 16777152
    # is the first total past it; the limit without the 64-row headroom took it)
    (dict(total_k=16777152, max_k=16777152), 2),
    (dict(total_q=16777152, max_q=16777152), 2),
])
def test_fwd_rejects_bad_arguments(kw, status):
    assert _call_fwd(**kw) == status


def test_variant_must_be_known():
    import head_attention_forward_fmha_amd as fm
    lib = fm.load_library()
    args = [0x10000, 0x20000, 0x30000, None, None, 1, 128, 128, 128, 128, 2, 64, 0,
            ctypes.c_float(0.125), 0x40000, 0x50000]
    assert lib.fmha_fwd_variant(*args, 5, None) == 1
    assert lib.fmha_fwd_variant(*args, -1, None) == 1
    fargs = [0x10000, 0x20000, 0x30000, 0x70000, None, None, 1, 128, 128, 128, 128, 2, 128, 0,
             ctypes.c_float(0.125), 0x40000, 0x50000]
    assert lib.fmha_fwd_fp8pv_variant(*fargs, 7, None) == 1
    # the pipelined and 64-row-wave kernels have no fp8 P.V form
    assert lib.fmha_fwd_fp8pv_variant(*fargs, 3, None) == 2
    assert lib.fmha_fwd_fp8pv_variant(*fargs, 4, None) == 2


@pytest.mark.parametrize("batch,max_q,heads,want", [
    (8, 4096, 32, "pingpong"),     # 16 blocks of 256 rows x 8 docs x 32 heads = 4096
    (1, 32768, 16, "pingpong"),    # 2048 blocks
    (4, 2048, 32, "pingpong"),     # exactly 1024
    (1, 2225, 16, "pingpong"),     # 9 x 16 = 144 blocks
    (1, 2048, 16, "pingpong"),     # 8 x 16 = 128, the threshold
    (1, 2047, 15, "four_wave"),    # 120
    (1, 128, 2, "four_wave"),
    (0, 0, 1, "four_wave"),
])
def test_auto_variant(batch, max_q, heads, want):
    import head_attention_forward_fmha_amd as fm
    assert fm.auto_variant(batch, max_q, heads) == want


def test_auto_variant_rejects_negative_sizes():
    import head_attention_forward_fmha_amd as fm
    with pytest.raises(ValueError):
        fm.auto_variant(-1, 10, 1)


def test_fwd_empty_problem_is_a_no_op():
    # no kernel is launched (so no GPU is needed) when there is nothing to compute
    assert _call_fwd(batch=0, total_q=0, total_k=0, max_q=0, max_k=0, q=None, k=None, v=None,
                     out=None, lse=None) == 0


def test_fp8_rejects_head_dim_64_and_missing_scale():
    import head_attention_forward_fmha_amd as fm
    lib = fm.load_library()
    args = [0x10000, 0x20000, 0x30000, 0x70000, None, None, 1, 128, 128, 128, 128, 2, 64, 0,
            ctypes.c_float(0.125), 0x40000, 0x50000, None]
    assert lib.fmha_fwd_fp8pv(*args) == 2
    args[12] = 128
    args[3] = None
    assert lib.fmha_fwd_fp8pv(*args) == 1


def test_fp4_argument_checks():
    import head_attention_forward_fmha_amd as fm
    lib = fm.load_library()
    # q, k, v codes, exponents, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, heads, d, ...
    args = [0x10000, 0x20000, 0x30000, 0x70000, None, None, 1, 128, 128, 128, 128, 2, 64, 0,
            ctypes.c_float(0.125), 0x40000, 0x50000, None]
    assert lib.fmha_fwd_fp4pv(*args) == 2          # head_dim 64
    args[12] = 128
    args[3] = None
    assert lib.fmha_fwd_fp4pv(*args) == 1          # exponents missing
    args[3] = 0x70002
    assert lib.fmha_fwd_fp4pv(*args) == 1          # exponents not 4-byte aligned
    args[3] = 0x70000
    args[2] = 0x30008
    assert lib.fmha_fwd_fp4pv(*args) == 1          # codes not 16-byte aligned
    args[2] = 0x30000
    vargs = args[:-1]
    assert lib.fmha_fwd_fp4pv_variant(*vargs, 3, None) == 2   # no pipelined fp4 kernel
    assert lib.fmha_fwd_fp4pv_variant(*vargs, 4, None) == 2   # nor a 64-row-wave one
    assert lib.fmha_fwd_fp4pv_variant(*vargs, 5, None) == 1
    # nothing to compute: no launch, no GPU needed
    empty = [None, None, None, None, None, None, 0, 0, 0, 0, 0, 2, 128, 1,
             ctypes.c_float(0.125), None, None, None]
    assert lib.fmha_fwd_fp4pv(*empty) == 0


def test_splitkv_argument_checks():
    import head_attention_forward_fmha_amd as fm
    lib = fm.load_library()
    assert fm.splitkv_workspace_size(2225, 16, 128, 3) == 3 * 2225 * 16 * 129 * 4
    assert fm.splitkv_workspace_size(10, 2, 96, 2) == 0
    assert fm.splitkv_workspace_size(10, 2, 64, 0) == 0
    assert fm.splitkv_workspace_size(10, 2, 64, 65) == 0
    base = [0x10000, 0x20000, 0x30000, None, None, 1, 128, 128, 128, 128, 2, 64, 0,
            ctypes.c_float(0.125), 0x40000, 0x50000]
    need = fm.splitkv_workspace_size(128, 2, 64, 2)
    ok_tail = [2, 0x80000, need, 0, None]
    for i, bad, status in ((0, 0, 1), (0, 65, 1), (1, None, 1), (1, 0x80008, 1),
                           (2, need - 1, 1), (3, 3, 2), (3, 4, 2), (3, 9, 1)):
        tail = list(ok_tail)
        tail[i] = bad
        assert lib.fmha_fwd_splitkv(*base, *tail) == status, (i, bad)
    # nothing to compute: no launch, workspace not needed
    empty = [None, None, None, None, None, 0, 0, 0, 0, 0, 2, 64, 0, ctypes.c_float(0.125),
             None, None]
    assert lib.fmha_fwd_splitkv(*empty, 2, None, 0, 0, None) == 0
    # merge: part count, head_dim, alignment
    margs = [0x10000, 0x20000, 2, 100, 4, 128, 0x30000, 0x40000, None]
    for i, bad, status in ((2, 0, 1), (2, 65, 1), (5, 96, 2), (0, 0x10008, 1), (6, 0x30008, 1),
                           (1, 0x20002, 1), (0, None, 1)):
        a = list(margs)
        a[i] = bad
        assert lib.fmha_merge_partials(*a) == status, (i, bad)
    a = list(margs)
    a[3] = 0
    assert lib.fmha_merge_partials(*a) == 0


def test_trace_argument_checks():
    import head_attention_forward_fmha_amd as fm
    lib = fm.load_library()
    need = 2 * 8 * fm.TRACE_EVENTS_PER_WAVE * 8
    # pv, q, k, v, v_scale, cu_q, cu_k, batch, tq, tk, mq, mk, heads, d, causal, scale, out, lse
    base = [0, 0x10000, 0x20000, 0x30000, None, None, None, 1, 256, 256, 256, 256, 2, 128, 1,
            ctypes.c_float(0.088), 0x40000, 0x50000]
    # every call below has one bad argument: the checks return before any launch
    tail = [0, 2, 0x80000, need, None]              # detailed, workgroups, trace, bytes, stream
    for i, bad, status in ((0, 3, 1), (13, 64, 2), (14, 0, 2), (4, 0x70002, 1)):
        b = list(base)
        b[i] = bad
        assert lib.fmha_fwd_trace(*b, *tail) == status, (i, bad)
    b = list(base)
    b[0] = 1                                         # e4m3 needs its per-head scales
    assert lib.fmha_fwd_trace(*b, *tail) == 1
    for i, bad in ((0, 2), (1, 0), (1, 4097), (2, None), (2, 0x80004), (3, need - 1)):
        t = list(tail)
        t[i] = bad
        assert lib.fmha_fwd_trace(*base, *t) == 1, (i, bad)


def test_bwd_argument_checks():
    import head_attention_forward_fmha_amd as fm
    lib = fm.load_library()
    assert lib.fmha_bwd_workspace_size(300, 4) == 2 * 300 * 4 * 4
    assert lib.fmha_bwd_workspace_size(-1, 4) == 0 and lib.fmha_bwd_workspace_size(3, 0) == 0
    need = 2 * 256 * 2 * 4
    # q, k, v, out, dout, lse, cu_q, cu_k, batch, tq, tk, mq, mk, heads, d, causal, scale,
    # dq, dk, dv, workspace, bytes, stream
    base = [0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000, None, None, 1, 256, 256,
            256, 256, 2, 128, 1, ctypes.c_float(0.088), 0x70000, 0x80000, 0x90000, 0xa0000,
            need, None]
    # every call below has one bad argument: the checks return before any launch
    for i, bad, status in ((4, None, 1), (5, None, 1), (17, None, 1), (18, None, 1),
                           (19, None, 1), (4, 0x50008, 1), (17, 0x70002, 1), (19, 0x90004, 1),
                           (20, None, 1), (20, 0xa0008, 1), (21, need - 1, 1), (14, 96, 2),
                           (15, 2, 1), (16, ctypes.c_float(0.0), 1), (9, 255, 1)):
        b = list(base)
        b[i] = bad
        assert lib.fmha_bwd(*b) == status, (i, bad)
    # nothing to compute: no launch
    empty = [None] * 8 + [0, 0, 0, 0, 0, 2, 64, 0, ctypes.c_float(0.125)] + [None] * 4 + [0, None]
    assert lib.fmha_bwd(*empty) == 0


def test_bwd_noalloc_argument_checks():
    """fmha_bwd_noalloc checks fmha_bwd's arguments, then its scratch limit
    (heads * total_q * 8 bytes <= FMHA_NOALLOC_SCRATCH_BYTES), before any HIP
    call."""
    import head_attention_forward_fmha_amd as fm
    lib = fm.load_library()
    header = open(os.path.join(ROOT, "include", "fmha.h")).read()
    assert "#define FMHA_NOALLOC_SCRATCH_BYTES (16u << 20)" in header
    assert fm.NOALLOC_SCRATCH_BYTES == 16 << 20
    # q, k, v, out, dout, lse, cu_q, cu_k, batch, tq, tk, mq, mk, heads, d, causal, scale,
    # dq, dk, dv, stream
    base = [0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000, None, None, 1, 256, 256,
            256, 256, 2, 128, 1, ctypes.c_float(0.088), 0x70000, 0x80000, 0x90000, None]
    for i, bad, status in ((4, None, 1), (5, None, 1), (17, None, 1), (18, None, 1),
                           (19, None, 1), (17, 0x70002, 1), (14, 96, 2), (15, 2, 1)):
        b = list(base)
        b[i] = bad
        assert lib.fmha_bwd_noalloc(*b) == status, (i, bad)
    # over the limit: 2^21 + 1 rows of one head, or 2 heads of 2^20 + 64 tokens
    limit_rows = fm.NOALLOC_SCRATCH_BYTES // 8
    for heads, tq in ((1, limit_rows + 1), (2, limit_rows // 2 + 64)):
        b = list(base)
        b[9], b[10], b[11], b[12], b[13], b[14] = tq, tq, tq, tq, heads, 64
        assert lib.fmha_bwd_noalloc(*b) == 2, (heads, tq)
    empty = [None] * 8 + [0, 0, 0, 0, 0, 2, 64, 0, ctypes.c_float(0.125)] + [None] * 4
    assert lib.fmha_bwd_noalloc(*empty) == 0


def test_bwd_noalloc_binding_reports_the_limit():
    import torch
    import head_attention_forward_fmha_amd as fm
    rows = fm.NOALLOC_SCRATCH_BYTES // 8 // 64 + 1      # 64 heads: one token over the limit
    q = torch.zeros(rows, 64, 64, dtype=torch.bfloat16)
    lse = torch.zeros(64, rows)
    with pytest.raises(fm.FmhaError, match="scratch"):
        fm.bwd_noalloc(q, q, q, q, q, lse, q, q, q)


def test_splitkv_num_splits_choice():
    import head_attention_forward_fmha_amd as fm
    # one value per size; splitting pays only when the query blocks do not fill the device
    c4 = fm.splitkv_num_splits(8, 4096, 4096, 32, causal=True)
    assert c4 == 1
    # c2's 144 blocks of 256 rows: measured, splitting does not pay (the split
    # items' overheads and the merge outweigh the idle compute units)
    assert fm.splitkv_num_splits(1, 2225, 2225, 16) == 1
    assert fm.splitkv_num_splits(1, 512, 32768, 16) >= 4  # short queries, long keys
    assert fm.splitkv_num_splits(1, 64, 8192, 8) > 4      # few query rows, long keys
    assert fm.splitkv_num_splits(1, 128, 64, 2) == 1      # a single key tile cannot split
    with pytest.raises(ValueError):
        fm.splitkv_num_splits(-1, 10, 10, 1)
    with pytest.raises(ValueError):
        fm.splitkv_num_splits(1, 10, 10, 1, variant="pipelined")


@pytest.mark.parametrize("cu,total,max_s,ok", [
    ([0, 2048, 4096, 6144, 8192], 8192, 2048, True),
    ([0, 2048, 4096, 6144, 8192], 8192, 2047, False),   # a doc longer than max_seqlen
    ([0, 10, 5, 20], 20, 15, False),                     # decreasing
    ([1, 10], 10, 10, False),                            # does not start at 0
    ([0, 10], 11, 10, False),                            # does not end at total
    ([0, 0, 0, 7], 7, 7, True),                          # empty documents are fine
    ([0], 0, 0, True),
])
def test_validate_cu_seqlens(cu, total, max_s, ok):
    import head_attention_forward_fmha_amd as fm
    assert fm.validate_cu_seqlens(np.array(cu, np.int32), total, max_s) is ok


def test_resource_gate_parser():
    from head_attention_forward_fmha_amd.build import check_resources, parse_resource_report
    # the format clang prints: location first, then "remark:"
    r = "[-Rpass-analysis=kernel-resource-usage]"
    text = (f"a.hip:10:1: remark: Function Name: kern {r}\n"
            "   10 | void kern() {\n"
            f"a.hip:10:1: remark:     VGPRs: 200 {r}\n"
            f"a.hip:10:1: remark:     ScratchSize [bytes/lane]: 16 {r}\n"
            f"a.hip:10:1: remark:     SGPRs Spill: 0 {r}\n"
            f"a.hip:10:1: remark:     VGPRs Spill: 3 {r}\n"
            f"a.hip:20:1: remark: Function Name: good {r}\n"
            f"a.hip:20:1: remark:     ScratchSize [bytes/lane]: 0 {r}\n"
            f"a.hip:20:1: remark:     SGPRs Spill: 0 {r}\n"
            f"a.hip:20:1: remark:     VGPRs Spill: 0 {r}\n")
    k = parse_resource_report(text)
    assert k["kern"]["VGPRs"] == "200" and k["kern"]["VGPRs Spill"] == "3"
    bad = check_resources(k)
    assert len(bad) == 2 and all(b.startswith("kern") for b in bad)
    # a kernel whose report lacks the fields fails too
    assert check_resources({"x": {}})


def test_built_kernels_have_no_scratch_or_spills():
    from head_attention_forward_fmha_amd.build import (RESOURCE_REPORT, check_resources,
                                                       parse_resource_report)
    if not os.path.exists(RESOURCE_REPORT):
        pytest.skip("resource report not present (library built elsewhere)")
    kernels = parse_resource_report(open(RESOURCE_REPORT).read())
    assert sum("fmha_fwd" in k for k in kernels) >= 16
    assert check_resources(kernels) == []


def test_binding_variant_names_match_the_header():
    """The binding's variant names map to the values include/fmha.h defines."""
    from head_attention_forward_fmha_amd import _lib
    header = open(os.path.join(ROOT, "include", "fmha.h")).read()
    defined = {m.group(1).lower(): int(m.group(2))
               for m in re.finditer(r"#define FMHA_VARIANT_(\w+) (\d+)", header)}
    assert defined == _lib.VARIANTS
