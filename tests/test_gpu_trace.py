"""GPU tests of the pipeline trace (fmha_fwd_trace).

The traced launch runs the same ping-pong kernel arithmetic as the forward
pass, so its outputs must equal the untraced kernel's bit for bit, for every
P.V format and both trace modes, and meet the oracle's bars as the forward
pass does ("Kernel Bottleneck Tuning", section 6: every build, instrumented or
not, is checked against the reference). The records must follow the kernel's schedule:
a work item of n key tiles runs slot pairs j = 0 .. n, so a wave records one
item start, 2n + 3 slot starts (one before each slot and one after the last
barrier, which opens the epilogue) and, per slot, one phase-end mark (coarse)
or three (detailed), with non-decreasing times.
"""

import numpy as np
import pytest
import torch

from head_attention_forward_fmha_amd import pipeline_trace as pt
from synthetic import make_inputs

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _inputs(lens, heads, pv, seed, with_host=False):
    inp = make_inputs(lens, heads, 128, seed=seed, fp8_pv=pv == "e4m3", fp4_pv=pv == "e2m1")
    dev = _dev()
    v = {"bf16": inp.v, "e4m3": inp.v_e4m3, "e2m1": inp.v_e2m1}[pv].to(dev)
    vs = {"bf16": None, "e4m3": inp.v_scale, "e2m1": inp.v_mx_scale}[pv]
    cu = torch.from_numpy(np.asarray(inp.cu_q, np.int32)).to(dev)
    ck = torch.from_numpy(np.asarray(inp.cu_k, np.int32)).to(dev)
    args = (inp.q.to(dev), inp.k.to(dev), v, None if vs is None else vs.to(dev), cu, ck,
            int(np.diff(inp.cu_q).max()), int(np.diff(inp.cu_k).max()))
    return (args, inp) if with_host else args


def _check_against_oracle(pv, inp, o, lse, what):
    """The forward pass's parity checks, applied to a traced launch's outputs."""
    import oracle
    from tests import test_gpu_fmha as gf
    from tests import test_gpu_fp4 as g4
    scale = float(np.float32(1.0 / np.sqrt(128)))
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    if pv == "bf16":
        o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, True, scale)
        gf._check(o, lse, o_ref, l_ref, what=what)
    elif pv == "e4m3":
        o_ref, l_ref = oracle.attention_fp8pv(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                              inp.cu_k, True, scale)
        emu = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                              inp.cu_k, True, scale)
        gf._check(o, lse, o_ref, l_ref, fp8=True, emu=emu, what=what)
    else:
        tq, h = inp.q.shape[0], inp.q.shape[1]
        emu = oracle.attention_fp4pv_emulated(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                              inp.cu_k, True, scale)
        o_x, l_x = oracle.attention_fp4pv(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                          inp.cu_k, True, scale)
        g4._check(o.reshape(tq * h, -1), lse.T.reshape(-1), emu, o_x.reshape(tq * h, -1),
                  l_x.T.reshape(-1), what=what)


def _untraced(pv, q, k, v, vs, cu, ck, mq, mk):
    import head_attention_forward_fmha_amd as fm
    if pv == "bf16":
        return fm.fwd(q, k, v, cu, ck, mq, mk, causal=True, variant="pingpong")
    if pv == "e4m3":
        return fm.fwd_fp8pv(q, k, v, vs, cu, ck, mq, mk, causal=True, variant="pingpong")
    return fm.fwd_fp4pv(q, k, v, vs, cu, ck, mq, mk, causal=True, variant="pingpong")


@pytest.mark.parametrize("pv", ["bf16", "e4m3", "e2m1"])
@pytest.mark.parametrize("detailed", [False, True])
def test_traced_outputs_equal_the_untraced_kernel(pv, detailed):
    import head_attention_forward_fmha_amd as fm
    args, inp = _inputs(((700, 700), (333, 333), (1, 1), (1300, 1300)), 4, pv, seed=3,
                        with_host=True)
    o0, l0 = _untraced(pv, *args)
    q, k, v, vs, cu, ck, mq, mk = args
    o1, l1, trace = fm.fwd_trace(q, k, v, cu, ck, mq, mk, pv=pv, v_scale=vs, detailed=detailed,
                                 traced_workgroups=8)
    torch.cuda.synchronize()
    _check_against_oracle(pv, inp, o1, l1, what=f"traced {pv} detailed={detailed}")
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    s = pt.summarize(trace.cpu().numpy().view(np.uint64))
    assert s["waves"] > 0 and s["period"] > 0
    assert 0.05 < s["mfma_busy_share"] < 0.95 and 0.0 <= s["mfma_wait_p_share"] < 0.9
    if detailed:
        assert s["mean_cycles"]["qk"] > 0 and s["mean_cycles"]["softmax"] > 0


@pytest.mark.parametrize("detailed", [False, True])
def test_records_follow_the_schedule(detailed):
    """One document of 512 rows and one head: two causal work items of 256 rows
    (8 and 4 key tiles). The persistent grid gives each its own workgroup."""
    import head_attention_forward_fmha_amd as fm
    q, k, v, vs, cu, ck, mq, mk = _inputs(((512, 512),), 1, "bf16", seed=4)
    _, _, trace = fm.fwd_trace(q, k, v, cu, ck, mq, mk, detailed=detailed, traced_workgroups=8)
    torch.cuda.synchronize()
    tr = trace.cpu().numpy().view(np.uint64)
    marks_per_slot = 3 if detailed else 1
    seen = set()
    for wg in range(tr.shape[0]):
        for wave in range(8):
            ev = pt.decode_wave(tr[wg, wave])
            if not ev:
                continue
            times = [t for _, t in ev]
            assert all(a <= b for a, b in zip(times, times[1:]))
            assert [i for i, (e, _) in enumerate(ev) if e == pt.EV_ITEM] == [0], (wg, wave)
            n_slot_marks = sum(1 for e, _ in ev if e == pt.EV_SLOT)
            n_tiles = (n_slot_marks - 3) // 2
            assert 2 * n_tiles + 3 == n_slot_marks and n_tiles in (4, 8)
            seen.add(n_tiles)
            assert len(ev) == 1 + n_slot_marks + marks_per_slot * (2 * n_tiles + 2)
    assert seen == {4, 8}


def test_non_causal_trace_is_unsupported():
    import head_attention_forward_fmha_amd as fm
    lib = fm.load_library()
    q, k, v, vs, cu, ck, mq, mk = _inputs(((128, 128),), 2, "bf16", seed=5)
    trace = torch.zeros((1, 8, fm.TRACE_EVENTS_PER_WAVE), dtype=torch.int64, device=q.device)
    import ctypes
    st = lib.fmha_fwd_trace(0, q.data_ptr(), k.data_ptr(), v.data_ptr(), None, cu.data_ptr(),
                            ck.data_ptr(), 1, 128, 128, 128, 128, 2, 128, 0, ctypes.c_float(0.088),
                            torch.empty_like(q).data_ptr(), None, 0, 1, trace.data_ptr(),
                            trace.numel() * 8, None)
    assert st == 2
