"""CPU tests of bench.py's counter summaries: the visible-score count that the
transcendental counter is checked against, and the per-launch reduction of a
rocprofv3 counter CSV (rows per XCD and dispatch, summed per dispatch, then
averaged over the FMHA dispatches; other kernels ignored)."""

import importlib.util
import os

import numpy as np

from synthetic import Workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("fmha_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _brute_visible(doc_lens, heads, causal):
    n = 0
    for sq, sk in doc_lens:
        for i in range(sq):
            for j in range(sk):
                # bottom-right causal: key j visible to query i iff j <= i + sk - sq
                n += (not causal) or (j <= i + sk - sq)
    return n * heads


def test_visible_scores_matches_brute_force():
    b = _bench()
    for causal in (False, True):
        for lens in (((5, 5), (3, 7), (9, 2), (0, 4), (4, 0)), ((1, 1),), ((17, 33), (33, 17))):
            w = Workload("t", "t", heads=3, head_dim=64, causal=causal, doc_lens=lens)
            assert b.visible_scores(w) == _brute_visible(lens, 3, causal), (causal, lens)


def test_summarize_sq_sums_xcds_and_averages_dispatches(tmp_path):
    b = _bench()
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    kern = "void fmha::fmha_fwd_pingpong_kernel<128, true, 0, false>(fmha::FwdParams)"
    for disp, scale in ((1, 1.0), (2, 3.0)):
        for xcd in range(8):
            rows.append(f'{disp},"{kern}",SQ_INSTS_VALU_MFMA_MOPS_BF16,{scale * 100}')
            rows.append(f'{disp},"{kern}",SQ_INSTS_VALU_TRANS_F32,{scale * 10}')
            rows.append(f'{disp},"{kern}",SQ_VALU_MFMA_BUSY_CYCLES,{scale * 1024}')
            rows.append(f'{disp},"{kern}",GRBM_GUI_ACTIVE,{scale * 4096}')
    rows.append('3,"__amd_rocclr_copyBuffer",SQ_INSTS_VALU_TRANS_F32,999999')
    p = tmp_path / "c.csv"
    p.write_text("\n".join(rows) + "\n")
    w = Workload("t", "t", heads=1, head_dim=128, causal=False, doc_lens=((8, 8),))
    text = b.summarize_sq(str(p), w)
    assert text.startswith("2 dispatches")
    mops = 2.0 * 8 * 100           # mean over dispatches of the 8-XCD sum
    assert f"{mops:.4e}" in text
    flop_line = [l for l in text.splitlines() if "MFMA FLOP" in l][0]
    assert f"{512 * mops:.4e}" in flop_line and f"{512 * mops / w.flops():.4f}" in flop_line
    trans = 2.0 * 8 * 10
    vis = 64
    assert f"{64 * trans / vis:.4f}" in text
    busy = 2.0 * 8 * 1024 / 1024
    elapsed = 2.0 * 8 * 4096 / 8
    assert f"{busy / elapsed:.3f}" in text
    assert "999999" not in text and "copyBuffer" not in text


def test_summarize_sq_splits_backward_kernels_and_reports_lds_conflicts(tmp_path):
    b = _bench()
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    dq = "void fmha::fmha_bwd_dq_kernel<128, true>(fmha::BwdParams)"
    dkdv = "void fmha::fmha_bwd_dkdv_kernel<128, true>(fmha::BwdParams)"
    for disp, kern, conflict in ((1, dq, 5.0), (2, dkdv, 0.0), (3, dq, 15.0), (4, dkdv, 0.0)):
        for xcd in range(8):
            rows.append(f'{disp},"{kern}",SQ_LDS_BANK_CONFLICT,{conflict}')
            rows.append(f'{disp},"{kern}",SQ_LDS_IDX_ACTIVE,1000')
            rows.append(f'{disp},"{kern}",SQ_INSTS_LDS,50')
            rows.append(f'{disp},"{kern}",SQ_INSTS_VALU_TRANS_F32,7')
    p = tmp_path / "c.csv"
    p.write_text("\n".join(rows) + "\n")
    w = Workload("t", "t", heads=1, head_dim=128, causal=True, doc_lens=((8, 8),))
    text = b.summarize_sq(str(p), w)
    blocks = text.split("\n\n")
    assert len(blocks) == 2
    by_kernel = {blk.splitlines()[0]: blk for blk in blocks}
    assert set(by_kernel) == {f"2 dispatches of {dq}", f"2 dispatches of {dkdv}"}
    q = by_kernel[f"2 dispatches of {dq}"]
    # mean over the two dQ dispatches of the 8-XCD sums: conflicts 80, indexed cycles 8000
    assert "bank-conflict cycles / indexed LDS cycles  0.0100" in q
    assert "bank-conflict cycles / LDS instruction     0.2000" in q
    assert "bank-conflict cycles / indexed LDS cycles  0.0000" in by_kernel[f"2 dispatches of {dkdv}"]
    # the visible-score check belongs to the forward kernels only
    assert "visible score" not in text
