"""GPU parity of the HIP forward pass against the fp64 oracle, through the C ABI.

Bar (bf16): |O_gpu - O_ref| <= 1e-2 + 1e-2 |O_ref| elementwise and
|LSE_gpu - LSE_ref| <= 1e-3 on finite rows, -inf rows matching exactly.
Bar (fp8 P.V): |O_gpu - O_ref| <= 5e-2 + 5e-2 |O_ref|, LSE as for bf16 (the row
sum is taken before P is rounded to e4m3). That bar alone passes an all-zero O
on long rows (|O| is about 0.01 there), so fp8 outputs are also held to the
method's own quantised result (``oracle.attention_fp8pv_emulated``) at the
bf16 bar, widened only by the oracle's fp32-ambiguity and subnormal-band
allowances. In the small-document edge cases (not c5) an fp8 element may also
exceed the stated bar by no more than the method's own pinned rounding bound
plus the bf16 bar: rows with a few keys can, by the method itself.

Every check also reports the error normalised by the row RMS of O_ref and
holds it to a derived bar (tests/parity.py), which stays sharp on long rows.

The five workloads are checked at their full sizes in the launch configuration
the benchmark times: c1, c2, c3 and c4 on every output, c5 on every row of one
head and on sampled (token, head) rows of all heads, which the oracle computes
one by one (each from its complete score row). Edge cases cover ragged tails, empty documents, sq != sk with causal
bottom-right alignment, d = 64, and tiny documents.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from synthetic import WORKLOADS, make_inputs, workload_inputs
from tests.parity import NORMALISED_BAR, error_summary, fp8_emulation_check

pytestmark = pytest.mark.gpu

VARIANTS = ["four_wave", "pingpong", "pipelined", "wide"]
VARIANTS_FP8 = ["four_wave", "pingpong"]   # the pipelined and 64-row-wave kernels are bf16 only

O_ATOL = O_RTOL = 1e-2
O_ATOL_FP8 = O_RTOL_FP8 = 5e-2
LSE_ATOL = 1e-3


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _run(inp, causal, scale, heads, d, fp8=False, max_q=None, max_k=None, variant="auto"):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    q, k = inp.q.to(dev), inp.k.to(dev)
    cq = torch.from_numpy(np.asarray(inp.cu_q, np.int32)).to(dev)
    ck = torch.from_numpy(np.asarray(inp.cu_k, np.int32)).to(dev)
    lq = np.diff(np.asarray(inp.cu_q))
    lk = np.diff(np.asarray(inp.cu_k))
    mq = int(lq.max()) if max_q is None else max_q
    mk = int(lk.max()) if max_k is None else max_k
    out = torch.full((q.shape[0], heads, d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((heads, q.shape[0]), float("nan"), dtype=torch.float32, device=dev)
    if fp8:
        fm.fwd_fp8pv(q, k, inp.v_e4m3.to(dev), inp.v_scale.to(dev), cq, ck, mq, mk, causal=causal,
                     softmax_scale=scale, out=out, lse=lse, variant=variant)
    else:
        fm.fwd(q, k, inp.v.to(dev), cq, ck, mq, mk, causal=causal, softmax_scale=scale, out=out,
               lse=lse, variant=variant)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(o, lse, o_ref, lse_ref, fp8=False, what="", emu=None, stated_fp8_bar=True):
    """The stated bar against the exact oracle; the normalised error against the
    exact oracle (bf16) or against the emulated method ``emu`` (fp8, rows in
    o's row order after reshaping to [rows, d]).

    fp8 edge cases (``stated_fp8_bar=False``): on a row with a handful of
    visible keys the method's own rounding of P to e4m3 (each weight within
    2^-4) can move O past the stated absolute term (pinned on the CPU in
    tests/test_oracle_fp8.py); there an element also passes within the
    oracle's bound on that rounding plus the bf16 bar. Every row is still held
    to the emulated method at the bf16 bar. The c5 workload, the configuration
    the fp8 bar is stated for, is held to the stated bar alone."""
    atol, rtol = (O_ATOL_FP8, O_RTOL_FP8) if fp8 else (O_ATOL, O_RTOL)
    assert not np.isnan(o).any(), f"{what}: NaN in O (unwritten or invalid output)"
    err = np.abs(o - o_ref)
    tol = atol + rtol * np.abs(o_ref)
    if fp8 and not stated_fp8_bar:
        tol = np.maximum(tol, emu.bound.reshape(o.shape) + O_ATOL + O_RTOL * np.abs(o_ref))
    bad = err > tol
    if bad.any():
        idx = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} O elements out of tolerance; worst at {idx}: "
                             f"gpu {o[idx]} ref {o_ref[idx]} (max abs err {err.max():.3e})")
    d = o.shape[-1]
    if not fp8:
        summ = error_summary(o.reshape(-1, d), o_ref.reshape(-1, d), atol, rtol)
    else:
        assert emu is not None, "fp8 outputs are also checked against the emulated method"
        o2 = o.reshape(-1, d)
        ok = fp8_emulation_check(o2, emu)
        assert ok.all(), (f"{what}: {int((~ok).sum())} rows off the emulated fp8 method; first "
                          f"row {int(np.argmin(ok))}")
        # normalised error with the fp32 allowances taken off first
        allow = emu.ambiguity + emu.slack
        summ = error_summary(o2, emu.out, 1e-2, 1e-2, extra=allow)
        resid = np.maximum(np.abs(o2 - emu.out) - allow, 0.0)
        rms = np.sqrt((emu.out ** 2).mean(axis=1))
        live = rms > 0
        summ["max_normalised_err"] = float((resid[live].max(axis=1) / rms[live]).max()) \
            if live.any() else 0.0
    print(f"{what}: max abs err {summ['max_abs_err']:.3e}, max normalised err "
          f"{summ['max_normalised_err']:.3e}, rms err {summ['rms_err']:.3e}, over bar "
          f"{summ['n_over_bar']}, worst at {summ['worst_location']}")
    assert summ["max_normalised_err"] <= NORMALISED_BAR, (
        f"{what}: normalised O error {summ['max_normalised_err']:.3e} > {NORMALISED_BAR} "
        f"(row {summ['worst_normalised_row']})")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse), ~fin), f"{what}: -inf LSE rows differ"
    if fin.any():
        lerr = np.abs(lse[fin] - lse_ref[fin])
        assert lerr.max() <= LSE_ATOL, f"{what}: LSE max err {lerr.max():.3e}"


def _full_parity(lens, heads, d, causal, seed=0, scale=None, fp8=False, max_q=None, max_k=None,
                 variant="auto"):
    inp = make_inputs(lens, heads, d, seed=seed, fp8_pv=fp8)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    o, lse = _run(inp, causal, scale, heads, d, fp8=fp8, max_q=max_q, max_k=max_k, variant=variant)
    emu = None
    if fp8:
        o_ref, lse_ref = oracle.attention_fp8pv(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                                inp.cu_k, causal, scale)
        emu = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                              inp.cu_k, causal, scale)
    else:
        o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, causal, scale)
    _check(o, lse, o_ref, lse_ref, fp8=fp8, emu=emu, stated_fp8_bar=False,
           what=f"lens={lens} h={heads} d={d} causal={causal} variant={variant}")
    return inp, o, lse


def _sample_rows(cu, heads, n_random, seed):
    """(token, head) samples: tile-boundary rows of every document plus random rows."""
    rng = np.random.default_rng(seed)
    cu = np.asarray(cu, np.int64)
    s = set()
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        for r in (0, 1, 31, 32, 63, 64, 127, 128, 129, e - a - 129, e - a - 2, e - a - 1):
            if 0 <= r < e - a:
                s.add((a + r, int(rng.integers(heads))))
    for t in rng.integers(0, int(cu[-1]), n_random):
        s.add((int(t), int(rng.integers(heads))))
    return sorted(s)


def _sampled_parity(w, n_random=1500, seed=0, variant="auto"):
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal, w.softmax_scale, w.heads, w.head_dim, fp8=w.fp8_pv,
                  variant=variant)
    samples = _sample_rows(inp.cu_q, w.heads, n_random, seed)
    emu = None
    if w.fp8_pv:
        o_ref, l_ref = oracle.attention_fp8pv_sampled(inp.q, inp.k, inp.v_e4m3, inp.v_scale,
                                                      inp.cu_q, inp.cu_k, w.causal,
                                                      w.softmax_scale, samples)
        emu = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                              inp.cu_k, w.causal, w.softmax_scale,
                                              samples=samples)
    else:
        o_ref, l_ref = oracle.attention_sampled(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, w.causal,
                                                w.softmax_scale, samples)
    t = np.array([a for a, _ in samples])
    hh = np.array([b for _, b in samples])
    _check(o[t, hh], lse[hh, t], o_ref, l_ref, fp8=w.fp8_pv, what=w.name, emu=emu)
    # every output element was written and finite
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    return o, lse


# ---------------------------------------------------------------- the five workloads

def test_c1_tiny_dense_full():
    w = WORKLOADS["c1_tiny_dense"]
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal, w.softmax_scale, w.heads, w.head_dim)
    g = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                             "c1_tiny_dense_seed0.npz"), allow_pickle=False)
    _check(o, lse, g["o"], g["lse"], what="c1")


def test_c2_dense_2225_full():
    w = WORKLOADS["c2_dense_2225"]
    _full_parity(w.doc_lens, w.heads, w.head_dim, w.causal)


def test_c2_dense_layout_matches_packed():
    """The dense [b,s,h,d] call (no cu_seqlens) equals the packed call bitwise."""
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    inp = make_inputs(((300, 300), (300, 300)), 4, 128, seed=5)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq = torch.from_numpy(inp.cu_q).to(dev)
    o1, l1 = fm.fwd(q, k, v, cq, cq, 300, 300)
    o2, l2 = fm.fwd(q.view(2, 300, 4, 128), k.view(2, 300, 4, 128), v.view(2, 300, 4, 128))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(2, 300, 4, 128), o2)
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("variant", ["auto", "pipelined", "wide"])
def test_c3_varlen_causal_8k_full(variant):
    """c3 at full size, every (token, head, d) output against the full oracle."""
    w = WORKLOADS["c3_varlen_causal_8k"]
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal, w.softmax_scale, w.heads, w.head_dim, variant=variant)
    o_ref, lse_ref = _c3_oracle()
    _check(o, lse, o_ref, lse_ref, what=f"{w.name} {variant}")


_C3_CACHE = {}


def _c3_oracle():
    """The full c3 oracle (a few seconds on the host's cores), computed once."""
    if "c3" not in _C3_CACHE:
        w = WORKLOADS["c3_varlen_causal_8k"]
        inp = workload_inputs(w)
        _C3_CACHE["c3"] = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, w.causal,
                                           w.softmax_scale)
    return _C3_CACHE["c3"]


@pytest.mark.timeout(600)
def test_c4_varlen_causal_32k_full():
    """c4, the headline workload, at full size in the launch configuration the
    benchmark times: every (token, head, d) output against the full oracle
    (about a minute of fp64 on the host's cores)."""
    w = WORKLOADS["c4_varlen_causal_32k"]
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal, w.softmax_scale, w.heads, w.head_dim)
    print("c4: oracle on every row", flush=True)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, w.causal,
                                      w.softmax_scale)
    _check(o, lse, o_ref, lse_ref, what=w.name)


@pytest.mark.parametrize("variant", ["pipelined", "wide"])
def test_c4_varlen_causal_32k_sampled_variant(variant):
    _sampled_parity(WORKLOADS["c4_varlen_causal_32k"], n_random=1000, variant=variant)


@pytest.mark.parametrize("variant", ["pipelined", "wide"])
def test_c2_dense_2225_variant(variant):
    w = WORKLOADS["c2_dense_2225"]
    _full_parity(w.doc_lens, w.heads, w.head_dim, w.causal, variant=variant)


def test_c5_causal_fp8pv_32k_sampled():
    """c5 at full size on sampled rows: the stated fp8 bar against the exact
    attention of the dequantised V, and the emulated method at the bf16 bar."""
    _sampled_parity(WORKLOADS["c5_causal_fp8pv_32k"], n_random=600)


@pytest.mark.timeout(600)
def test_c5_causal_fp8pv_32k_one_head_every_row():
    """c5 at full size: every row of one head (all 32768, so every position of
    the long persistent items) at the stated fp8 bar against the exact
    attention of the dequantised V, and every other row of that head against
    the emulated method at the bf16 bar."""
    w = WORKLOADS["c5_causal_fp8pv_32k"]
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal, w.softmax_scale, w.heads, w.head_dim, fp8=True)
    head = 5
    rows = np.arange(int(inp.cu_q[-1]))
    print("c5: exact oracle on every row of one head", flush=True)
    o_ref, l_ref = oracle.attention_fp8pv_sampled(inp.q, inp.k, inp.v_e4m3, inp.v_scale,
                                                  inp.cu_q, inp.cu_k, w.causal, w.softmax_scale,
                                                  [(int(t), head) for t in rows])
    err = np.abs(o[rows, head] - o_ref)
    tol = O_ATOL_FP8 + O_RTOL_FP8 * np.abs(o_ref)
    assert (err <= tol).all(), f"{int((err > tol).sum())} O elements of head {head} off the bar"
    assert np.abs(lse[head, rows] - l_ref).max() <= LSE_ATOL
    sub = rows[::2]
    print("c5: emulated method on every other row of that head", flush=True)
    emu = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                          inp.cu_k, w.causal, w.softmax_scale,
                                          samples=[(int(t), head) for t in sub])
    _check(o[sub, head], lse[head, sub], o_ref[::2], l_ref[::2], fp8=True, emu=emu,
           what=f"{w.name} head {head}")


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("lens", [
    ((1, 1),), ((63, 63),), ((65, 65),), ((127, 127),), ((129, 129),), ((200, 200),),
    ((129, 129), (1, 1), (64, 64), (300, 300)),
])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("variant", VARIANTS)
def test_ragged_lengths(lens, causal, d, variant):
    _full_parity(lens, 3, d, causal, seed=len(lens) + d, variant=variant)


@pytest.mark.parametrize("lens", [
    ((100, 300),), ((300, 100),), ((1, 129),), ((129, 1),), ((70, 0),), ((0, 50), (40, 40)),
    ((5, 5), (0, 0), (130, 7), (7, 130)),
])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("variant", VARIANTS)
def test_unequal_and_empty_documents(lens, causal, variant):
    _full_parity(lens, 2, 128, causal, seed=7, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_many_small_documents(variant):
    rng = np.random.default_rng(3)
    lens = tuple((int(x), int(x)) for x in rng.integers(0, 200, 40))
    for causal in (False, True):
        _full_parity(lens, 4, 128, causal, seed=11, variant=variant)


def _edge_mix(n_random, max_len, seed):
    """Documents for a persistent launch with more work items than the grid
    holds (every workgroup walks several items, so each item's loads are
    issued under the previous item's end): random lengths mixed with a
    single-token document, key-less and query-less documents, sq < sk and
    sq > sk under bottom-right causal alignment, and tails just past a tile."""
    rng = np.random.default_rng(seed)
    edge = ((1, 1), (10, 0), (0, 12), (13, 40), (40, 13), (257, 257), (65, 65), (0, 0))
    rand = tuple((int(x), int(x)) for x in rng.integers(1, max_len, n_random))
    mixed = list(rand)
    for i, e in enumerate(edge):
        mixed.insert((7 * i + 3) % (len(mixed) + 1), e)
    return tuple(mixed)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("variant", ["four_wave", "pingpong", "wide"])
def test_persistent_items_with_edge_documents(d, variant):
    # 40 documents x 16 heads x 3 blocks of 256 rows: far more items than the
    # 256 workgroups of the persistent grid, empty ones included
    lens = _edge_mix(32, 600, seed=21)
    _full_parity(lens, 16, d, True, seed=22, variant=variant)


def test_fp8_persistent_items_with_edge_documents():
    lens = _edge_mix(22, 400, seed=23)
    _full_parity(lens, 12, 128, True, fp8=True, seed=24, variant="pingpong")


@pytest.mark.parametrize("variant", VARIANTS_FP8)
def test_fp8_small_cases(variant):
    for lens, causal in ((((200, 200),), True), (((129, 129), (64, 64)), False),
                         (((100, 300), (300, 100)), True), (((600, 600), (1, 1)), True)):
        _full_parity(lens, 2, 128, causal, fp8=True, seed=13, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_nonstandard_scale_and_large_scores(variant):
    # a large scale makes every row nearly one-hot: the max-subtraction must hold
    _full_parity(((256, 256),), 2, 128, True, scale=1.0, seed=17, variant=variant)
    _full_parity(((600, 600),), 2, 64, False, scale=0.5, seed=18, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_max_seqlen_larger_than_needed(variant):
    # a generous max_seqlen only adds empty work items
    _full_parity(((100, 100), (50, 50)), 2, 128, True, max_q=1000, max_k=1000, seed=19,
                 variant=variant)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("fp8", [False, True])
def test_kernel_variants_agree_bitwise(causal, fp8):
    """The 4-wave and ping-pong kernels run the same per-row arithmetic in the
    same tile order (the pipelined kernel checks its maximum per 32 keys, so it
    agrees with them only within rounding)."""
    lens = ((1000, 1000), (333, 333), (1, 1), (700, 701))
    inp = make_inputs(lens, 4, 128, seed=29, fp8_pv=fp8)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    o1, l1 = _run(inp, causal, scale, 4, 128, fp8=fp8, variant="four_wave")
    o2, l2 = _run(inp, causal, scale, 4, 128, fp8=fp8, variant="pingpong")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- bitwise properties

@pytest.mark.parametrize("variant", VARIANTS)
def test_deterministic_repeats(variant):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    inp = make_inputs(((1000, 1000), (777, 777)), 8, 128, seed=21)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq = torch.from_numpy(inp.cu_q).to(dev)
    ref_o, ref_l = fm.fwd(q, k, v, cq, cq, 1000, 1000, causal=True, variant=variant)
    for _ in range(20):
        o, l = fm.fwd(q, k, v, cq, cq, 1000, 1000, causal=True, variant=variant)
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


@pytest.mark.parametrize("variant", VARIANTS)
def test_causal_future_keys_do_not_leak(variant):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    inp = make_inputs(((500, 500),), 4, 128, seed=23)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq = torch.from_numpy(inp.cu_q).to(dev)
    o1, l1 = fm.fwd(q, k, v, cq, cq, 500, 500, causal=True, variant=variant)
    i = 200
    k2, v2 = k.clone(), v.clone()
    k2[i + 1:] = k2[i + 1:] * 3 + 1
    v2[i + 1:] = -v2[i + 1:]
    o2, l2 = fm.fwd(q, k2, v2, cq, cq, 500, 500, causal=True, variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(o1[:i + 1], o2[:i + 1]) and torch.equal(l1[:, :i + 1], l2[:, :i + 1])
    assert not torch.equal(o1[i + 1:], o2[i + 1:])


@pytest.mark.parametrize("variant", VARIANTS)
def test_documents_are_isolated_and_match_per_document_calls(variant):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    lens = ((300, 300), (129, 129), (513, 513))
    inp = make_inputs(lens, 4, 128, seed=25)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq = torch.from_numpy(inp.cu_q).to(dev)
    o, l = fm.fwd(q, k, v, cq, cq, 513, 513, causal=True, variant=variant)
    for b in range(3):
        a, e = int(inp.cu_q[b]), int(inp.cu_q[b + 1])
        ob, lb = fm.fwd(q[a:e].contiguous(), k[a:e].contiguous(), v[a:e].contiguous(), causal=True,
                        variant=variant)
        torch.cuda.synchronize()
        assert torch.equal(ob, o[a:e]) and torch.equal(lb, l[:, a:e])


@pytest.mark.parametrize("variant", VARIANTS)
def test_causal_row0_is_v0_exactly(variant):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    inp = make_inputs(((64, 64), (200, 200)), 4, 128, seed=27)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq = torch.from_numpy(inp.cu_q).to(dev)
    o, l = fm.fwd(q, k, v, cq, cq, 200, 200, causal=True, variant=variant)
    torch.cuda.synchronize()
    for a in (0, 64):
        assert torch.equal(o[a], v[a])
        ref = 0.08838834764831845 * (q[a].double().cpu() * k[a].double().cpu()).sum(-1)
        assert torch.allclose(l[:, a].double().cpu(), ref, atol=1e-4, rtol=0)


@pytest.mark.parametrize("variant", ["pipelined", "wide"])
def test_bf16_only_variants_reject_fp8(variant):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    inp = make_inputs(((128, 128),), 2, 128, seed=31, fp8_pv=True)
    with pytest.raises(fm.FmhaError):
        fm.fwd_fp8pv(inp.q.to(dev), inp.k.to(dev), inp.v_e4m3.to(dev), inp.v_scale.to(dev),
                     variant=variant)


# ---------------------------------------------------------------- stale LDS

@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_stale_lds_is_never_read(variant, causal, d):
    """Every LDS byte a pass reads was written by that pass: with the LDS of all
    CUs filled with NaN bit patterns beforehand, the outputs stay finite and
    match the oracle (lengths with ragged tiles and several copy rounds)."""
    from tests.gpu_support import poison_lds
    dev = _dev()
    for lens in (((65, 65),), ((130, 130),), ((300, 300), (77, 77))):
        poison_lds(torch.cuda.current_stream(dev).cuda_stream)
        _full_parity(lens, 3, d, causal, seed=41, variant=variant)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("variant", VARIANTS_FP8)
@pytest.mark.parametrize("causal", [False, True])
def test_rows_after_the_last_document_are_never_read(fp8, variant, causal):
    """K and V are views of the first total_k rows of buffers whose next 128
    rows hold NaN (e4m3 NaN codes for fp8 V). The last document ends inside a
    64-key tile, so its last tile's copies reach past total_k; they must read
    zeros (the buffer range check), never the NaN rows, which would turn O into
    NaN through P = 0 times NaN."""
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    heads, d = 2, 128
    lens = ((50, 70), (90, 77))               # total_k = 147: 19 keys into its third tile
    inp = make_inputs(lens, heads, d, seed=31, fp8_pv=fp8)
    total_q, total_k = inp.q.shape[0], inp.k.shape[0]
    pad = 128
    k_buf = torch.full((total_k + pad, heads, d), float("nan"), dtype=torch.bfloat16, device=dev)
    k_buf[:total_k] = inp.k.to(dev)
    k = k_buf[:total_k]
    cq = torch.from_numpy(np.asarray(inp.cu_q, np.int32)).to(dev)
    ck = torch.from_numpy(np.asarray(inp.cu_k, np.int32)).to(dev)
    scale = float(np.float32(1 / np.sqrt(d)))
    if fp8:
        v_buf = torch.full((total_k + pad, heads, d), 0x7F, dtype=torch.uint8, device=dev)
        v_buf[:total_k] = inp.v_e4m3.to(dev)
        o, lse = fm.fwd_fp8pv(inp.q.to(dev), k, v_buf[:total_k], inp.v_scale.to(dev), cq, ck, 90,
                              77, causal=causal, softmax_scale=scale, variant=variant)
        o_ref, l_ref = oracle.attention_fp8pv(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                              inp.cu_k, causal, scale)
        emu = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                              inp.cu_k, causal, scale)
    else:
        emu = None
        v_buf = torch.full((total_k + pad, heads, d), float("nan"), dtype=torch.bfloat16,
                           device=dev)
        v_buf[:total_k] = inp.v.to(dev)
        o, lse = fm.fwd(inp.q.to(dev), k, v_buf[:total_k], cq, ck, 90, 77, causal=causal,
                        softmax_scale=scale, variant=variant)
        o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, causal, scale)
    torch.cuda.synchronize()
    _check(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
           o_ref, l_ref, fp8=fp8, what=f"NaN-padded K/V, fp8={fp8}, {variant}", emu=emu)
