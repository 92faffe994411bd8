"""fmha_bwd_noalloc (the backward without a workspace argument) against fmha_bwd.

The entry point is for callers that cannot allocate device memory. It runs
the same kernels as fmha_bwd with the library's fixed per-GPU scratch array as
the workspace, so its dQ, dK, dV must equal fmha_bwd's bit for bit (stronger
than the backward's derived bar against the oracle, which both also meet).
Two calls in a row, the second on a smaller problem, check that nothing of
the first call's scratch contents leaks into the second.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from synthetic import make_dout, make_inputs

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _problem(lens, heads, d, seed, dev):
    inp = make_inputs(lens, heads, d, seed=seed)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq = torch.from_numpy(np.asarray(inp.cu_q, np.int32)).to(dev)
    ck = torch.from_numpy(np.asarray(inp.cu_k, np.int32)).to(dev)
    mq = int(np.diff(inp.cu_q).max())
    mk = int(np.diff(inp.cu_k).max())
    return inp, q, k, v, cq, ck, mq, mk


def _noalloc_through_the_abi(lib, q, k, v, o, dout, lse, cq, ck, mq, mk, causal, scale):
    """One fmha_bwd_noalloc call with raw pointers (outputs preallocated, NaN)."""
    nan = float("nan")
    dq, dk, dv = (torch.full_like(t, nan) for t in (q, k, v))
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.fmha_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              dout.data_ptr(), lse.data_ptr(), cq.data_ptr(), ck.data_ptr(),
                              cq.numel() - 1, q.shape[0], k.shape[0], mq, mk, q.shape[1],
                              q.shape[2], int(causal), ctypes.c_float(scale), dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), ctypes.c_void_p(stream))
    assert st == 0, st
    return dq, dk, dv


@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_equals_the_workspace_entry_point_on_two_calls(causal):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    lib = fm.load_library()
    scale = float(np.float32(1 / np.sqrt(128)))
    # the first call is larger (more rows of D and LSE*log2e in the scratch),
    # the second smaller and with other values
    for lens, heads, seed in ((((1000, 1000), (333, 333), (1, 1), (700, 701)), 4, 3),
                              (((200, 200), (77, 90)), 2, 4)):
        inp, q, k, v, cq, ck, mq, mk = _problem(lens, heads, 128, seed, dev)
        o, lse = fm.fwd(q, k, v, cq, ck, mq, mk, causal=causal, softmax_scale=scale)
        dout = (make_dout(q.shape[0], heads, 128, seed=seed).float() * 0.01).to(torch.bfloat16)
        dout = dout.to(dev)
        ref = fm.bwd(q, k, v, o, dout, lse, cq, ck, mq, mk, causal=causal, softmax_scale=scale)
        got = _noalloc_through_the_abi(lib, q, k, v, o, dout, lse, cq, ck, mq, mk, causal, scale)
        torch.cuda.synchronize()
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert not torch.isnan(g).any(), f"{name}: unwritten output"
            assert torch.equal(g, r), f"{name} differs from fmha_bwd (lens={lens})"
        # and the derived backward bar against the oracle on the smaller problem
        if heads == 2:
            want, t = oracle.attention_backward(inp.q, inp.k, inp.v, dout.cpu(), inp.cu_q,
                                                inp.cu_k, causal, scale, rounding_scale=True)
            for name, g, r, tt in zip(("dQ", "dK", "dV"), got, want, t):
                gg = g.float().cpu().numpy().astype(np.float64)
                assert np.all(np.abs(gg - r) <= 8 * tt + 2.0 ** -8 * np.abs(r)), name


def test_noalloc_binding_matches_bwd():
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    inp, q, k, v, cq, ck, mq, mk = _problem(((300, 300), (129, 129)), 3, 64, 5, dev)
    o, lse = fm.fwd(q, k, v, cq, ck, mq, mk, causal=True)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    dout = dout.to(dev)
    ref = fm.bwd(q, k, v, o, dout, lse, cq, ck, mq, mk, causal=True)
    outs = tuple(torch.empty_like(t) for t in (q, k, v))
    got = fm.bwd_noalloc(q, k, v, o, dout, lse, *outs, cq, ck, mq, mk, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(g, r) for g, r in zip(got, ref))
