"""Pins for the oracle's OCP e4m3 decoder/encoder and the fp8 P.V oracles.

The method's P quantisation ("Kernel Bottleneck Tuning (validated on FA4
FP4/FP8 PV, GB300)", sections 4 and 5: P rounded to e4m3 with its scale folded
into the exp2 argument) has no printed values on the pages, so the emulation
is pinned by the format's definition, two independently written roundings, a
pure-Python brute force, closed forms, cases where the quantisation is exact,
its independence from the integer maximum, constructed ties and planted
mistakes.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
from synthetic import make_inputs, quantize_v_e4m3
from tests.parity import fp8_emulation_check

LN2_SCALE = float(np.float32(math.log(2.0)))   # c = scale * log2 e within 3e-9 of 1


def test_decode_known_values():
    # values fixed by the e4m3 definition (bias 7, 3 mantissa bits, no inf)
    table = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x30: 0.5, 0x7E: 448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0xB8: -1.0, 0xFE: -448.0}
    for c, val in table.items():
        assert oracle.e4m3_decode(np.uint8(c)) == val, hex(c)
    assert np.isnan(oracle.e4m3_decode(np.uint8(0x7F)))
    assert np.isnan(oracle.e4m3_decode(np.uint8(0xFF)))


def test_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_encode_matches_torch_rne():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(20000) * 100, g.standard_normal(5000) * 1e-2,
                        np.array([448.0, 464.0, -464.0, 2.0 ** -10, 3 * 2.0 ** -11, 0.0, 1.0625,
                                  1.1875, 2.0 ** -7, 240.0, 248.0])])
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x)
    # +0/-0 both decode to zero; compare values
    assert np.array_equal(oracle.e4m3_decode(got), oracle.e4m3_decode(ref))
    # ties go to the even code: 464 lies halfway between 448 (0x7E) and 480 (not finite)
    assert oracle.e4m3_encode(np.array([464.0]))[0] == 0x7E
    assert oracle.e4m3_encode(np.array([1.0625]))[0] == 0x38   # halfway 1.0/1.125 -> even
    assert oracle.e4m3_encode(np.array([1.1875]))[0] == 0x3A   # halfway 1.125/1.25 -> even


def test_roundtrip_all_finite_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    back = oracle.e4m3_encode(vals[fin])
    assert np.array_equal(oracle.e4m3_decode(back), vals[fin])


def test_dequantize_and_fp8_oracle_compose():
    inp = make_inputs(((24, 24),), 2, 16, seed=1, fp8_pv=True)
    vhat = oracle.dequantize_v(inp.v_e4m3, inp.v_scale)
    # the quantised V stays within e4m3's relative rounding error of the bf16 V
    v = inp.v.double().numpy()
    scale = inp.v_scale.double().numpy()[None, :, None]
    err = np.abs(vhat - v)
    assert np.all(err <= np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * scale) + 1e-12)
    o, lse = oracle.attention_fp8pv(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q, inp.cu_k,
                                    True, 0.25)
    o2, lse2 = oracle.attention(inp.q, inp.k, vhat, inp.cu_q, inp.cu_k, True, 0.25)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_quantizer_scale_is_amax_over_448():
    v = torch.randn(100, 3, 16).to(torch.bfloat16)
    codes, scale = quantize_v_e4m3(v)
    amax = v.float().abs().amax(dim=(0, 2))
    assert torch.allclose(scale, amax / 448.0)
    dec = oracle.e4m3_decode(codes.numpy())
    assert np.nanmax(np.abs(dec)) <= 448.0 and not np.isnan(dec).any()


# ---------------------------------------------------------------- the method's P rounding

def test_round_e4m3_matches_the_exhaustive_encoder():
    g = np.random.default_rng(1)
    codes = np.arange(127, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    mids = (vals[1:] + vals[:-1]) / 2.0
    x = np.concatenate([np.abs(g.standard_normal(30000)) * 50, np.abs(g.standard_normal(10000))
                        * 1e-2, g.uniform(0, 2.0 ** -6, 5000), mids, vals,
                        mids * (1 + 1e-12), mids * (1 - 1e-12)])
    x = np.clip(x, 0, 448)
    assert np.array_equal(ofp8.round_e4m3(x), oracle.e4m3_decode(oracle.e4m3_encode(x)))


CASES = [
    (((9, 9),), False), (((9, 9),), True), (((5, 7), (6, 3)), True), (((40, 40),), True),
    (((3, 0), (20, 45), (7, 7)), False), (((13, 50),), True),
]


@pytest.mark.parametrize("lens,causal", CASES)
def test_emulation_matches_bruteforce(lens, causal):
    inp = make_inputs(lens, 2, 4, seed=11, fp8_pv=True)
    # scale 0.3 keeps every row's weights within 2^11 of its largest
    emu = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                          inp.cu_k, causal, 0.3)
    bf = oracle.attention_fp8pv_bruteforce(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                           inp.cu_k, causal, 0.3)
    tq, h = inp.q.shape[0], inp.q.shape[1]
    assert not emu.slack.any()          # these rows have no subnormal band
    assert np.allclose(emu.out.reshape(tq, h, -1), bf, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("lens,causal", CASES)
def test_emulation_within_bound_of_exact_and_lse_exact(lens, causal):
    inp = make_inputs(lens, 2, 8, seed=12, fp8_pv=True)
    scale = 0.35
    emu = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                          inp.cu_k, causal, scale)
    o, lse = oracle.attention_fp8pv(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q, inp.cu_k,
                                    causal, scale)
    tq, h, dv = o.shape
    assert np.all(np.abs(emu.out - o.reshape(tq * h, dv)) <= emu.bound + 1e-12)
    lse_ref = lse.T.reshape(-1)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(emu.lse))
    assert np.allclose(emu.lse[fin], lse_ref[fin], rtol=0, atol=1e-12)
    # the relative rounding of e4m3 is at most 2^-4: the bound says no more
    vhat = np.abs(oracle.dequantize_v(inp.v_e4m3, inp.v_scale))
    p_abs = np.abs(oracle.attention(inp.q, inp.k, vhat, inp.cu_q, inp.cu_k, causal, scale)[0])
    assert np.all(emu.bound <= 2.0 ** -4 * p_abs.reshape(tq * h, dv) + 1e-12)


def _pinned_scores_inputs(raw_cols, v_rows, v_scale=0.5):
    """d = 4 inputs whose raw scores q.k_j are the given values (query 0)."""
    sk = len(raw_cols)
    q = torch.zeros((1, 1, 4), dtype=torch.bfloat16)
    q[0, 0, 0] = 1.0
    k = torch.zeros((sk, 1, 4), dtype=torch.bfloat16)
    k[:, 0, 0] = torch.tensor(raw_cols, dtype=torch.float32)
    codes = torch.from_numpy(oracle.e4m3_encode(np.asarray(v_rows, np.float64))).view(sk, 1, 4)
    return q, k, codes, torch.tensor([v_scale], dtype=torch.float32)


def test_exact_when_every_weight_is_an_e4m3_value():
    # c = 1 (to 3e-9) and integer scores: every 2^(c r) is a power of two (to 3e-8),
    # which e4m3 holds exactly, so the quantised P equals P
    raw = [6, 5, 5, 3, 0, -2, 4]
    v = np.random.default_rng(2).integers(-8, 9, (len(raw), 4)) / 4.0
    q, k, codes, vs = _pinned_scores_inputs(raw, v)
    emu = oracle.attention_fp8pv_emulated(q, k, codes, vs, [0, 1], [0, len(raw)], False,
                                          LN2_SCALE)
    w = np.exp2(np.array(raw, dtype=np.float64))
    assert np.allclose(emu.out[0], 0.5 * (w @ v) / w.sum(), rtol=1e-7, atol=1e-12)
    assert not emu.ambiguity.any() and not emu.slack.any()


def test_single_visible_key_closed_form():
    # causal row 0 sees key 0 only; it is the first tile's maximum, so it maps
    # exactly to 2^5: O = scale * codes_0 = V_hat_0 exactly
    inp = make_inputs(((40, 40),), 1, 8, seed=13, fp8_pv=True)
    tau = 0.3
    emu = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                          inp.cu_k, True, tau, samples=[(0, 0), (1, 0)])
    vhat = oracle.dequantize_v(inp.v_e4m3, inp.v_scale)
    assert np.array_equal(emu.out[0], vhat[0, 0])
    # row 1 sees keys 0 and 1: the larger maps exactly, the other to R(w), w < 1
    c = float(np.float32(tau)) / math.log(2.0)
    s = (inp.q[1, 0].double() @ inp.k[:2, 0].double().T).numpy()
    w = np.exp2(c * (s - s.max()))
    rw = ofp8.round_e4m3(w * 32) / 32
    want = (rw @ vhat[:2, 0]) / w.sum()
    assert np.allclose(emu.out[1], want, rtol=1e-12, atol=1e-15)


def test_quantised_weight_does_not_depend_on_the_whole_steps():
    # 2^(a + K - 5) e4m3(2^(c s - a - K + 5)) for every whole K that keeps the
    # value in e4m3's normal range and under 448: always the same number,
    # 2^a R(2^(c s - a)); the fractional anchor a alone fixes the grid
    g = np.random.default_rng(3)
    cs = g.uniform(-4, 4, 5000)
    a = 0.3717
    w = cs - a
    ref = (ofp8.round_e4m3(np.exp2(w - np.floor(w)) * 8) / 8 * np.exp2(np.floor(w))
           * 2.0 ** a)
    for k in (4, 5, 7):
        x = np.exp2(cs - a - k + 5)
        ok = (x >= 2.0 ** -6) & (x <= 448)
        got = ofp8.round_e4m3(x) * 2.0 ** (a + k - 5)
        assert ok.mean() > 0.5
        assert np.allclose(got[ok], ref[ok], rtol=1e-15, atol=0)


def test_log_domain_fold_equals_post_exp_scaling():
    # section 4's refactoring: adding the scale's log2 to the exp2 argument gives
    # the codes that multiplying by the scale after the exp2 gives, so the error
    # against the exact result is the same
    x = np.linspace(-30, 0, 2001)
    folded = oracle.e4m3_encode(np.minimum(np.exp2(x + 5.0), 448.0))
    post = oracle.e4m3_encode(np.minimum(np.exp2(x) * 32.0, 448.0))
    assert np.array_equal(folded, post)
    exact = np.exp2(x)
    e1 = np.abs(oracle.e4m3_decode(folded) / 32.0 - exact)
    e2 = np.abs(oracle.e4m3_decode(post) / 32.0 - exact)
    assert np.array_equal(e1, e2)


def test_ambiguity_at_an_e4m3_midpoint_is_the_other_rounding():
    # scores 8 and 0: the anchor is c * 8, so key 0 maps to 32 exactly and key 1
    # to x = 2^(5 - 8c); tau puts 8c within 1e-7 of log2(32/17), so x sits next
    # to 17, the midpoint between the e4m3 values 16 and 18. Its other rounding
    # moves O by the e4m3 step at x (2) in units of 2^(anchor - 5)
    target = math.log2(32.0 / 17.0) - 3e-8
    tau = float(np.float32(target / 8.0 * math.log(2.0)))
    c = tau / math.log(2.0)
    v = [[1.0, 0.0, -2.0, 0.5], [0.0, 1.0, 0.0, -0.25]]
    q, k, codes, vs = _pinned_scores_inputs([8, 0], v)
    emu = oracle.attention_fp8pv_emulated(q, k, codes, vs, [0, 1], [0, 2], False, tau)
    x = 2.0 ** (5 - 8 * c)
    assert abs(x / 17.0 - 1) < 1e-6
    assert emu.key_tie[0] == 1
    l = 1.0 + 2.0 ** (-8 * c)                       # weights relative to the anchor
    want = 0.5 * 2.0 * 2.0 ** -5 * np.abs(np.array(v[1])) / l
    assert np.allclose(emu.ambiguity[0], want, rtol=1e-9, atol=0)
    # away from the midpoint (x = 17.5) there is none
    tau2 = float(np.float32(math.log2(32.0 / 17.5) / 8.0 * math.log(2.0)))
    emu2 = oracle.attention_fp8pv_emulated(q, k, codes, vs, [0, 1], [0, 2], False, tau2)
    assert emu2.key_tie[0] == 0 and not emu2.ambiguity.any()


def test_subnormal_band_gets_a_bounded_allowance():
    # scale 1 and scores 40 apart: every other key is 2^-57 of the largest, deep
    # in the band where e4m3 rounds to 0 or a subnormal depending on M; the
    # allowance covers it and stays below 2^-12 of |V| per key here
    raw = [40, 0, 0, 1, 2]
    v = np.ones((5, 4))
    q, k, codes, vs = _pinned_scores_inputs(raw, v, v_scale=1.0)
    emu = oracle.attention_fp8pv_emulated(q, k, codes, vs, [0, 1], [0, 5], False, 1.0)
    assert np.all(emu.slack > 0) and np.all(emu.slack < 4 * 2.0 ** -12)
    assert np.allclose(emu.out[0], 1.0, rtol=2.0 ** -4)


def test_zero_or_wrong_head_output_fails_the_long_row_check():
    """On the long single-document workload (32768 keys, h = 16, d = 128) the
    stated fp8 bar 5e-2 + 5e-2 |O| passes an all-zero O on most late rows
    (|O| is about 0.01 there); the check against the emulated method at the
    bf16 bar does not: zero, wrong-head and wrong-row outputs all fail it."""
    from synthetic import WORKLOADS, workload_inputs
    w = WORKLOADS["c5_causal_fp8pv_32k"]
    inp = workload_inputs(w)
    rng = np.random.default_rng(0)
    rows = sorted({int(t) for t in rng.integers(16384, 32768, 24)})
    samples = [(t, int(rng.integers(w.heads))) for t in rows]
    emu = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                          inp.cu_k, True, w.softmax_scale, samples=samples)
    o_x, _ = oracle.attention_fp8pv_sampled(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                            inp.cu_k, True, w.softmax_scale, samples)
    # the method itself passes, and the exact attention passes the stated bar
    assert fp8_emulation_check(emu.out, emu).all()
    assert np.all(np.abs(emu.out - o_x) <= 5e-2 + 5e-2 * np.abs(o_x))
    zero = np.zeros_like(emu.out)
    assert np.mean(np.all(np.abs(zero - o_x) <= 5e-2 + 5e-2 * np.abs(o_x), axis=1)) > 0.5
    assert not fp8_emulation_check(zero, emu).any()
    # another head of the same token, and the next token of the same head
    other = [(t, (hh + 1) % w.heads) for t, hh in samples]
    emu_o = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                            inp.cu_k, True, w.softmax_scale, samples=other)
    assert not fp8_emulation_check(emu_o.out, emu).any()
    nxt = [(t + 1, hh) for t, hh in samples]
    emu_n = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                            inp.cu_k, True, w.softmax_scale, samples=nxt)
    assert not fp8_emulation_check(emu_n.out, emu).any()
    # the fp32 allowances stay small against the bar on these rows (measured:
    # 35 to 88 keys per row next to a midpoint, together at most 0.24 of the bar)
    bar = 1e-2 + 1e-2 * np.abs(emu.out)
    assert ((emu.ambiguity + emu.slack) / bar).max() < 0.5


def test_method_can_exceed_the_stated_bar_on_a_few_key_row():
    """A counterexample to the stated fp8 bar holding on every short row: the
    third query of a 242-token causal document (three visible keys) in the
    mixed-length edge case of the GPU parity tests (seed 24, 12 heads). The
    method's own rounding of the three weights to e4m3 moves element 14 of head
    10 by 0.053 from the exact attention, past 5e-2 + 5e-2 |O| = 0.0505, and
    within the oracle's bound on that rounding (which is what the GPU check
    allows there, besides holding the kernel to the emulated method)."""
    rng = np.random.default_rng(23)
    edge = ((1, 1), (10, 0), (0, 12), (13, 40), (40, 13), (257, 257), (65, 65), (0, 0))
    lens = [(int(x), int(x)) for x in rng.integers(1, 400, 22)]
    for i, e in enumerate(edge):
        lens.insert((7 * i + 3) % (len(lens) + 1), e)
    inp = make_inputs(tuple(lens), 12, 128, seed=24, fp8_pv=True)
    b = 8
    assert lens[b] == (242, 242) and int(inp.cu_q[b]) == 916
    sq = slice(int(inp.cu_q[b]), int(inp.cu_q[b + 1]))
    sk = slice(int(inp.cu_k[b]), int(inp.cu_k[b + 1]))
    q, k, v8 = inp.q[sq], inp.k[sk], inp.v_e4m3[sk]
    cu = np.array([0, 242])
    scale = float(np.float32(1.0 / np.sqrt(128)))
    o, _ = oracle.attention_fp8pv(q, k, v8, inp.v_scale, cu, cu, True, scale)
    emu = oracle.attention_fp8pv_emulated(q, k, v8, inp.v_scale, cu, cu, True, scale)
    row = 2 * 12 + 10
    err = abs(emu.out[row, 14] - o[2, 10, 14])
    assert err > 5e-2 + 5e-2 * abs(o[2, 10, 14])
    assert err <= emu.bound[row, 14] + 1e-12
    # the relaxed GPU tolerance covers it with room to spare
    assert err <= emu.bound[row, 14] + 1e-2 + 1e-2 * abs(o[2, 10, 14])


@pytest.mark.parametrize("lens,causal", [
    (((200, 200),), True), (((129, 129), (64, 64)), False), (((100, 300), (300, 100)), True),
    (((600, 600), (1, 1)), True), (((200, 200), (77, 77), (129, 129)), True),
])
def test_method_meets_the_stated_bar_on_short_rows(lens, causal):
    """With the first tile's largest key mapped exactly, the method's own P
    rounding keeps these cases' short rows (one key, a few keys whose V cancel)
    within the stated fp8 bar 5e-2 + 5e-2 |O| of the exact attention, and
    within its bound (not every short row: see the counterexample above)."""
    inp = make_inputs(lens, 2, 128, seed=13, fp8_pv=True)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    o, _ = oracle.attention_fp8pv(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q, inp.cu_k,
                                  causal, scale)
    emu = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                          inp.cu_k, causal, scale)
    o2 = o.reshape(emu.out.shape)
    err = np.abs(emu.out - o2)
    assert np.all(err <= emu.bound + 1e-12)
    assert np.all(err <= 5e-2 + 5e-2 * np.abs(o2))
