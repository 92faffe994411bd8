"""GPU parity of the fp4 P.V forward pass (MXFP4 V, per-group e2m1 P) against the oracle.

The fp4 method ("Kernel Bottleneck Tuning (validated on FA4 FP4/FP8 PV, GB300)",
section 4) quantises P, so the kernel is held to two oracles:

  * the method's quantised result (``oracle.attention_fp4pv_emulated``), at the
    bf16 bar |O - O_emu| <= 1e-2 + 1e-2 |O_emu|. Where the fp32 scores may take
    a rounding decision the other way (a scaled value next to an e2m1
    midpoint, a group exponent argument next to an integer; the oracle lists
    each such decision with its signed effect on O), the row must lie within
    that bar of one of the method's outcomes, each decision taken one way or
    the other; the bar itself is never widened;
  * the exact attention of the dequantised inputs (``oracle.attention_fp4pv``):
    |O - O_exact| <= bound + 1e-2 + 1e-2 |O_exact|, with the oracle's
    elementwise bound on the P quantisation error, for every row;
  * LSE against the exact scores: |LSE - LSE_ref| <= 1e-3, -inf rows exactly.
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic import EXTRA_WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

VARIANTS_FP4 = ["four_wave", "pingpong"]
O_ATOL = O_RTOL = 1e-2
LSE_ATOL = 1e-3


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _run(inp, causal, scale, heads, d=128, max_q=None, max_k=None, variant="auto"):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    cq = torch.from_numpy(np.asarray(inp.cu_q, np.int32)).to(dev)
    ck = torch.from_numpy(np.asarray(inp.cu_k, np.int32)).to(dev)
    lq, lk = np.diff(np.asarray(inp.cu_q)), np.diff(np.asarray(inp.cu_k))
    mq = int(lq.max()) if max_q is None else max_q
    mk = int(lk.max()) if max_k is None else max_k
    tq = inp.q.shape[0]
    out = torch.full((tq, heads, d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((heads, tq), float("nan"), dtype=torch.float32, device=dev)
    fm.fwd_fp4pv(inp.q.to(dev), inp.k.to(dev), inp.v_e2m1.to(dev), inp.v_mx_scale.to(dev), cq, ck,
                 mq, mk, causal=causal, softmax_scale=scale, out=out, lse=lse, variant=variant)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(o, lse, emu, o_exact, lse_exact, what):
    """o [n, d], lse [n] of the samples; emu an oracle FP4Emulation of the same samples."""
    assert not np.isnan(o).any(), f"{what}: NaN in O (unwritten or invalid output)"
    bar = O_ATOL + O_RTOL * np.abs(emu.out)
    off = [i for i in range(o.shape[0])
           if not oracle.fp4.outcome_within(o[i], emu.out[i], emu.alternatives[i], emu.slack[i],
                                            bar[i])]
    if off:
        i = off[0]
        j = int(np.argmax(np.abs(o[i] - emu.out[i]) - bar[i]))
        raise AssertionError(f"{what}: {len(off)} rows off every outcome of the emulated method; "
                             f"first row {i} ({len(emu.alternatives[i])} ambiguous decisions), "
                             f"d={j}: gpu {o[i, j]} emu {emu.out[i, j]} exact {o_exact[i, j]}")
    err_x = np.abs(o - o_exact)
    tol_x = emu.bound + O_ATOL + O_RTOL * np.abs(o_exact)
    bad_x = err_x > tol_x
    assert not bad_x.any(), f"{what}: {bad_x.sum()} O elements outside the quantisation bound"
    fin = np.isfinite(lse_exact)
    assert np.array_equal(np.isneginf(lse), ~fin), f"{what}: -inf LSE rows differ"
    if fin.any():
        lerr = np.abs(lse[fin] - lse_exact[fin])
        assert lerr.max() <= LSE_ATOL, f"{what}: LSE max err {lerr.max():.3e}"


def _full_parity(lens, heads, causal, seed=0, scale=None, max_q=None, max_k=None,
                 variant="auto"):
    inp = make_inputs(lens, heads, 128, seed=seed, fp4_pv=True)
    scale = float(np.float32(1.0 / np.sqrt(128))) if scale is None else scale
    o, lse = _run(inp, causal, scale, heads, max_q=max_q, max_k=max_k, variant=variant)
    tq = inp.q.shape[0]
    emu = oracle.attention_fp4pv_emulated(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                          inp.cu_k, causal, scale)
    o_x, l_x = oracle.attention_fp4pv(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                      inp.cu_k, causal, scale)
    # emulation rows are (token, head) in token-major order
    _check(o.reshape(tq * heads, -1), lse.T.reshape(-1), emu, o_x.reshape(tq * heads, -1),
           l_x.T.reshape(-1), what=f"lens={lens} h={heads} causal={causal} variant={variant}")
    return inp, o, lse


@pytest.mark.parametrize("lens", [
    ((1, 1),), ((31, 31),), ((33, 33),), ((65, 65),), ((129, 129),), ((200, 200),),
    ((129, 129), (1, 1), (64, 64), (300, 300)),
])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("variant", VARIANTS_FP4)
def test_fp4_ragged_lengths(lens, causal, variant):
    _full_parity(lens, 3, causal, seed=len(lens) + 5, variant=variant)


@pytest.mark.parametrize("lens", [
    # documents starting inside a 32-token block, so that tiles are widened and
    # the first keys masked
    ((13, 13), (50, 50), (70, 40), (0, 20), (45, 100)),
    ((13, 13), (10, 0), (20, 20)),          # no keys, starting mid-block
    ((100, 300),), ((300, 100),), ((1, 129),), ((129, 1),), ((70, 0),), ((0, 50), (40, 40)),
    ((5, 5), (0, 0), (130, 7), (7, 130)),
])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("variant", VARIANTS_FP4)
def test_fp4_unaligned_unequal_and_empty_documents(lens, causal, variant):
    _full_parity(lens, 2, causal, seed=17, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS_FP4)
def test_fp4_many_small_documents(variant):
    rng = np.random.default_rng(5)
    lens = tuple((int(x), int(x)) for x in rng.integers(0, 150, 30))
    for causal in (False, True):
        _full_parity(lens, 2, causal, seed=23, variant=variant)


def test_fp4_persistent_items_with_edge_documents():
    """More work items than the persistent grid holds (each workgroup walks
    several, loading the next under the current one's end), with documents
    that start inside a 32-token block, key-less and query-less documents,
    sq != sk, and a single-token document among random lengths."""
    rng = np.random.default_rng(25)
    lens = [(int(x), int(x)) for x in rng.integers(1, 400, 22)]
    for i, e in enumerate(((1, 1), (10, 0), (0, 12), (13, 40), (40, 13), (257, 257), (33, 33))):
        lens.insert((5 * i + 2) % (len(lens) + 1), e)
    _full_parity(tuple(lens), 12, True, seed=26, variant="pingpong")


@pytest.mark.parametrize("variant", VARIANTS_FP4)
def test_fp4_large_scores_and_scale(variant):
    # a large softmax scale gives peaked rows, groups far below the row maximum
    # and repeated raises of the running maximum
    _full_parity(((300, 300), (77, 77)), 2, True, seed=9, scale=0.6, variant=variant)
    _full_parity(((300, 300),), 2, False, seed=10, scale=0.02, variant=variant)


def test_fp4_x_causal_32k_sampled():
    """The 32768-token single-document causal fp4 workload at full size, in the
    launch configuration the benchmark times, on sampled rows."""
    w = EXTRA_WORKLOADS["x_causal_fp4pv_32k"]
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal, w.softmax_scale, w.heads)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rng = np.random.default_rng(0)
    rows = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 4095, 16384, 32766, 32767}
    rows |= {int(t) for t in rng.integers(0, w.total_q, 150)}
    samples = sorted((t, int(rng.integers(w.heads))) for t in rows)
    emu = oracle.attention_fp4pv_emulated(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                          inp.cu_k, True, w.softmax_scale, samples=samples)
    o_x, l_x = oracle.attention_fp4pv_sampled(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                              inp.cu_k, True, w.softmax_scale, samples)
    t = np.array([a for a, _ in samples])
    hh = np.array([b for _, b in samples])
    _check(o[t, hh], lse[hh, t], emu, o_x, l_x, what=w.name)


@pytest.mark.timeout(600)
def test_fp4_x_causal_32k_one_head_every_8th_row():
    """The 32768-token single-document causal fp4 workload at full size: every
    8th row of one head, so positions across the whole length of the long
    persistent items, against the emulated method and the exact bound."""
    w = EXTRA_WORKLOADS["x_causal_fp4pv_32k"]
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal, w.softmax_scale, w.heads)
    head = 11
    samples = [(int(t), head) for t in range(0, w.total_q, 8)]
    print("fp4 32k: emulated method on every 8th row of one head", flush=True)
    emu = oracle.attention_fp4pv_emulated(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                          inp.cu_k, True, w.softmax_scale, samples=samples)
    o_x, l_x = oracle.attention_fp4pv_sampled(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                              inp.cu_k, True, w.softmax_scale, samples)
    t = np.array([a for a, _ in samples])
    _check(o[t, head], lse[head, t], emu, o_x, l_x, what=f"{w.name} head {head}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp4_kernel_variants_agree_bitwise(causal):
    lens = ((1000, 1000), (333, 333), (1, 1), (700, 701))
    inp = make_inputs(lens, 4, 128, seed=29, fp4_pv=True)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    o1, l1 = _run(inp, causal, scale, 4, variant="four_wave")
    o2, l2 = _run(inp, causal, scale, 4, variant="pingpong")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("variant", VARIANTS_FP4)
def test_fp4_deterministic_repeats(variant):
    inp = make_inputs(((1000, 1000), (777, 777)), 8, 128, seed=21, fp4_pv=True)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    o0, l0 = _run(inp, True, scale, 8, variant=variant)
    for _ in range(10):
        o, l = _run(inp, True, scale, 8, variant=variant)
        assert np.array_equal(o, o0) and np.array_equal(l, l0)


@pytest.mark.parametrize("variant", ["pipelined", "wide"])
def test_fp4_bf16_only_variants_are_rejected(variant):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    inp = make_inputs(((128, 128),), 2, 128, seed=31, fp4_pv=True)
    with pytest.raises(fm.FmhaError):
        fm.fwd_fp4pv(inp.q.to(dev), inp.k.to(dev), inp.v_e2m1.to(dev), inp.v_mx_scale.to(dev),
                     variant=variant)


@pytest.mark.parametrize("variant", VARIANTS_FP4)
@pytest.mark.parametrize("causal", [False, True])
def test_fp4_stale_lds_is_never_read(variant, causal):
    """With the LDS of all CUs filled with NaN bit patterns beforehand, outputs
    stay finite and match the oracles (ragged tiles, several copy rounds)."""
    from tests.gpu_support import poison_lds
    dev = _dev()
    for lens in (((65, 65),), ((130, 130),), ((300, 300), (77, 77))):
        poison_lds(torch.cuda.current_stream(dev).cuda_stream)
        _full_parity(lens, 3, causal, seed=41, variant=variant)
