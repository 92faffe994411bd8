"""GPU parity of the backward pass (fmha_bwd) against the fp64 oracle.

Bar. The pages fix no precision for the backward; the reading taken is the
forward's arithmetic, bf16 operands of every matrix product with fp32
accumulation. Each gradient element is a sum whose terms carry one bf16
rounding each (P in dV, dS in dQ and dK, and D = dO . O taken from the bf16 O),
so its error is of the order of the oracle's rounding scale T (the root sum of
squares of those terms' worst-case rounding errors; see oracle/backward.py).
An element g passes when

    |g - g_ref| <= 8 T + 2^-8 |g_ref|,

2^-8 |g_ref| covering the output's own rounding to bf16. An emulation of these
roundings stays within 6 T on the CPU (tests/test_oracle_backward.py), and T is
about 0.1 % of a gradient's rms, so a masking or indexing mistake fails.

Inputs. Two paths: (a) the step's own path, the library's forward followed by
its backward, and (b) the backward alone given the oracle's O (rounded to bf16)
and LSE (rounded to fp32), which isolates the backward kernels. dO is an
independent N(0, 1) bf16 draw, or the gradient of mean(O^2) taken from the
oracle's O. Every expected value comes from the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic import WORKLOADS, make_dout, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

K_SCALE = 8.0      # multiple of the rounding scale
RTOL = 2.0 ** -8  # the output's own bf16 rounding


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _cu(x, dev):
    return torch.from_numpy(np.asarray(x, np.int32)).to(dev)


def _gpu_bwd(inp, dout, causal, scale, out=None, lse=None):
    """The library's forward (unless out/lse are given) and backward; fp64 numpy grads."""
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = _cu(inp.cu_q, dev), _cu(inp.cu_k, dev)
    mq = int(np.diff(inp.cu_q).max()) if len(inp.cu_q) > 1 else 0
    mk = int(np.diff(inp.cu_k).max()) if len(inp.cu_k) > 1 else 0
    if out is None:
        out, lse = fm.fwd(q, k, v, cq, ck, mq, mk, causal=causal, softmax_scale=scale)
    else:
        out, lse = out.to(dev), lse.to(dev)
    nan = float("nan")
    dq = torch.full_like(q, nan)
    dk = torch.full_like(k, nan)
    dv = torch.full_like(v, nan)
    fm.bwd(q, k, v, out, dout.to(dev), lse, cq, ck, mq, mk, causal=causal, softmax_scale=scale,
           dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]


def _check(got, ref, scale, what):
    for name, g, r, t in zip(("dQ", "dK", "dV"), got, ref, scale):
        assert not np.isnan(g).any(), f"{what}: NaN in {name} (unwritten or invalid)"
        if r.size == 0:
            continue
        err = np.abs(g - r)
        tol = K_SCALE * t + RTOL * np.abs(r)
        bad = err > tol
        if bad.any():
            i = np.unravel_index(np.argmax(err / np.maximum(tol, 1e-300)), err.shape)
            raise AssertionError(f"{what}: {name} {bad.sum()} of {bad.size} out of tolerance; "
                                 f"worst at {i}: gpu {g[i]:.4e} ref {r[i]:.4e} scale {t[i]:.3e}")


def _parity(lens, heads, d, causal, seed=0, scale=None, isolated=False):
    inp = make_inputs(lens, heads, d, seed=seed)
    dout = make_dout(inp.q.shape[0], heads, d, seed=seed)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    out = lse = None
    if isolated:
        o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, causal, scale)
        out = torch.from_numpy(o_ref).to(torch.bfloat16)
        lse = torch.from_numpy(l_ref).to(torch.float32).contiguous()
    got = _gpu_bwd(inp, dout, causal, scale, out, lse)
    ref, t = oracle.attention_backward(inp.q, inp.k, inp.v, dout, inp.cu_q, inp.cu_k, causal,
                                       scale, rounding_scale=True)
    _check(got, ref, t, f"lens={lens} h={heads} d={d} causal={causal} isolated={isolated}")
    return got


RAGGED = [
    ((1, 1),), ((65, 65),), ((200, 200),), ((129, 129), (1, 1), (64, 64), (300, 300)),
    ((100, 300),), ((300, 100),), ((70, 0),), ((0, 50), (40, 40)),
    ((5, 5), (0, 0), (130, 7), (7, 130)),
]


@pytest.mark.parametrize("lens", RAGGED)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_ragged_and_empty(lens, causal, d):
    _parity(lens, 3, d, causal, seed=len(lens) + d)


def test_bwd_long_causal_document_one_pair_per_item_group():
    """Causal items are dispatched in groups of about 64: a document of 8300
    tokens has 65 blocks of 128 rows, so its groups hold one (document, head)
    pair each, while the short second document's pairs share groups."""
    _parity(((8300, 8300), (300, 300)), 2, 64, True)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_isolated_from_the_forward(causal):
    """The backward alone, given the oracle's O and LSE."""
    _parity(((257, 257), (90, 300), (300, 90)), 2, 128, causal, seed=3, isolated=True)


def test_bwd_c1_tiny_dense():
    w = WORKLOADS["c1_tiny_dense"]
    inp = workload_inputs(w)
    dout = make_dout(w.total_q, w.heads, w.head_dim, seed=w.seed)
    got = _gpu_bwd(inp, dout, w.causal, w.softmax_scale)
    ref, t = oracle.attention_backward(inp.q, inp.k, inp.v, dout, inp.cu_q, inp.cu_k, w.causal,
                                       w.softmax_scale, rounding_scale=True)
    _check(got, ref, t, w.name)


@pytest.mark.timeout(600)
def test_bwd_c2_dense_2225_full():
    """c2's shape (2225 rows, ragged last block) at full size: every gradient
    element of every head against the oracle."""
    w = WORKLOADS["c2_dense_2225"]
    inp = workload_inputs(w)
    dout = make_dout(w.total_q, w.heads, w.head_dim, seed=w.seed)
    got = _gpu_bwd(inp, dout, w.causal, w.softmax_scale)
    ref, t = oracle.attention_backward(inp.q, inp.k, inp.v, dout, inp.cu_q, inp.cu_k, w.causal,
                                       w.softmax_scale, rounding_scale=True)
    _check(got, ref, t, f"{w.name} full")


@pytest.mark.timeout(600)
def test_bwd_c3_full():
    """c3 at full size with the benchmark step's dO = 2 O / n (n = numel(O), O the
    oracle's forward output), every gradient element of every document and head
    against the oracle (about half a minute of fp64 on the host's cores)."""
    w = WORKLOADS["c3_varlen_causal_8k"]
    inp = workload_inputs(w)
    n = w.total_q * w.heads * w.head_dim
    o_ref, _ = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, w.causal,
                                w.softmax_scale)
    dout = torch.from_numpy(2.0 * o_ref / n).float().to(torch.bfloat16)
    got = _gpu_bwd(inp, dout, w.causal, w.softmax_scale)
    print("c3 backward: oracle on every row", flush=True)
    ref, t = oracle.attention_backward(inp.q, inp.k, inp.v, dout, inp.cu_q, inp.cu_k, w.causal,
                                       w.softmax_scale, rounding_scale=True)
    _check(got, ref, t, f"{w.name} full")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c4_varlen_causal_32k"])
def test_bwd_varlen_causal_full_size_four_heads(name):
    """The varlen causal step's shapes at full size, with dO on the scale of the
    benchmark loss's gradient 2 O / n (n = numel(O)): exactly 2 O / n from the
    oracle's O on the checked (document, head) pairs, an N(0, 1) draw times
    2 / n elsewhere. Every document of four heads is checked element by element
    (the oracle's cost), every gradient for finiteness."""
    w = WORKLOADS[name]
    inp = workload_inputs(w)
    rng = np.random.default_rng(5)
    docs = list(range(len(w.doc_lens)))
    heads = sorted(int(h) for h in rng.choice(w.heads, 4, replace=False))
    n = w.total_q * w.heads * w.head_dim
    dout = make_dout(w.total_q, w.heads, w.head_dim, seed=w.seed).float() * (2.0 / n)
    o_ref, _ = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, w.causal,
                                w.softmax_scale, heads=heads, docs=docs)
    for b in docs:
        q0, q1 = int(inp.cu_q[b]), int(inp.cu_q[b + 1])
        for h in heads:
            dout[q0:q1, h] = torch.from_numpy(2.0 * o_ref[q0:q1, h] / n).float()
    dout = dout.to(torch.bfloat16)
    got = _gpu_bwd(inp, dout, w.causal, w.softmax_scale)
    ref, t = oracle.attention_backward(inp.q, inp.k, inp.v, dout, inp.cu_q, inp.cu_k, w.causal,
                                       w.softmax_scale, heads=heads, docs=docs,
                                       rounding_scale=True)
    for b in docs:
        q0, q1 = int(inp.cu_q[b]), int(inp.cu_q[b + 1])
        k0, k1 = int(inp.cu_k[b]), int(inp.cu_k[b + 1])
        sel = [slice(q0, q1), slice(k0, k1), slice(k0, k1)]
        pick = [lambda x, s=s_: x[s][:, heads] for s_ in sel]
        _check([f(g) for f, g in zip(pick, got)], [f(r) for f, r in zip(pick, ref)],
               [f(x) for f, x in zip(pick, t)], f"{name} doc {b} heads {heads}")
    assert all(np.isfinite(g).all() for g in got)


@pytest.mark.timeout(600)
def test_bwd_single_document_32k_one_head():
    """The third shape the FA4 spill issue times fwd+bwd: one 32768-token causal
    document, 16 heads, d = 128, at full size with dO = 2 O / n on the checked
    head (from the library's own forward O, which is the step's input), an
    N(0, 1) draw times 2 / n elsewhere. Checked on every dQ, dK and dV element
    of one head, every gradient for finiteness."""
    import head_attention_forward_fmha_amd as fm
    from synthetic import EXTRA_WORKLOADS
    w = EXTRA_WORKLOADS["x_causal_bf16_32k"]
    inp = workload_inputs(w)
    dev = _dev()
    cq = torch.from_numpy(np.asarray(inp.cu_q, np.int32)).to(dev)
    o_dev, _ = fm.fwd(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), cq, cq, w.max_seqlen_q,
                      w.max_seqlen_k, causal=True, softmax_scale=w.softmax_scale)
    n = w.total_q * w.heads * w.head_dim
    head = 5
    dout = make_dout(w.total_q, w.heads, w.head_dim, seed=w.seed).float() * (2.0 / n)
    dout[:, head] = o_dev[:, head].float().cpu() * (2.0 / n)
    dout = dout.to(torch.bfloat16)
    got = _gpu_bwd(inp, dout, True, w.softmax_scale)
    ref, t = oracle.attention_backward(inp.q, inp.k, inp.v, dout, inp.cu_q, inp.cu_k, True,
                                       w.softmax_scale, heads=[head], rounding_scale=True)
    _check([g[:, [head]] for g in got], [r[:, [head]] for r in ref],
           [x[:, [head]] for x in t], f"{w.name} head {head}, every row and key")
    assert all(np.isfinite(g).all() for g in got)


def test_bwd_dense_layout_matches_packed():
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    b, s, h, d = 2, 300, 4, 128
    inp = make_inputs(((s, s),) * b, h, d, seed=9)
    dout = make_dout(b * s, h, d, seed=9)
    packed = _gpu_bwd(inp, dout, True, float(np.float32(1 / np.sqrt(d))))
    q, k, v = (t.to(dev).reshape(b, s, h, d) for t in (inp.q, inp.k, inp.v))
    out, lse = fm.fwd(q, k, v, causal=True)
    dq, dk, dv = fm.bwd(q, k, v, out, dout.to(dev).reshape(b, s, h, d), lse, causal=True)
    torch.cuda.synchronize()
    for g, p in zip((dq, dk, dv), packed):
        assert np.array_equal(g.float().cpu().numpy().reshape(b * s, h, d), p)


def test_bwd_deterministic_repeats():
    inp = make_inputs(((1000, 1000), (777, 777)), 4, 128, seed=21)
    dout = make_dout(inp.q.shape[0], 4, 128, seed=21)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    g0 = _gpu_bwd(inp, dout, True, scale)
    for _ in range(3):
        g = _gpu_bwd(inp, dout, True, scale)
        assert all(np.array_equal(a, b) for a, b in zip(g, g0))


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_stale_lds_is_never_read(causal):
    from tests.gpu_support import poison_lds
    dev = _dev()
    for lens in (((65, 65),), ((300, 300), (77, 77))):
        poison_lds(torch.cuda.current_stream(dev).cuda_stream)
        _parity(lens, 3, 128, causal, seed=41)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_rows_after_the_last_document_are_never_read(causal):
    """Q, K, V, O and dO are views of the first rows of buffers whose next 128
    rows hold NaN. Both documents end inside a 64-row tile, so the backward's
    tile copies reach past the last row; they must read zeros (the buffer range
    check), never the NaN rows, which would spread NaN into dQ, dK and dV."""
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    heads, d, pad = 2, 128, 128
    lens = ((50, 70), (90, 77))               # total_q = 140, total_k = 147
    inp = make_inputs(lens, heads, d, seed=37)
    dout = make_dout(inp.q.shape[0], heads, d, seed=37)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    cq, ck = _cu(inp.cu_q, dev), _cu(inp.cu_k, dev)
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, causal, scale)

    def padded(x):
        buf = torch.full((x.shape[0] + pad,) + tuple(x.shape[1:]), float("nan"),
                         dtype=torch.bfloat16, device=dev)
        buf[:x.shape[0]] = x.to(dev)
        return buf[:x.shape[0]]

    q, k, v = padded(inp.q), padded(inp.k), padded(inp.v)
    out = padded(torch.from_numpy(o_ref).to(torch.bfloat16))
    lse = torch.from_numpy(l_ref).to(torch.float32).contiguous().to(dev)
    do = padded(dout)
    nan = float("nan")
    dq, dk, dv = torch.full_like(q, nan), torch.full_like(k, nan), torch.full_like(v, nan)
    fm.bwd(q, k, v, out, do, lse, cq, ck, 90, 77, causal=causal, softmax_scale=scale,
           dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    ref, t = oracle.attention_backward(inp.q, inp.k, inp.v, dout, inp.cu_q, inp.cu_k, causal,
                                       scale, rounding_scale=True)
    _check(got, ref, t, f"NaN-padded inputs, causal={causal}")
