"""Pins for the oracle's e2m1 codec, the MXFP4 V format and the fp4 P.V oracles.

The fp4 P.V method ("Kernel Bottleneck Tuning (validated on FA4 FP4/FP8 PV,
GB300)", section 4, log-domain refactoring) quantises P per group of keys with
a power-of-two scale read off the group's largest score. Nothing on the pages
prints values for it, so the oracle is pinned by the format's definition, two
independently written encoders, brute force, closed forms and cases where the
quantisation is exact.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp4 as ofp4
from synthetic import make_inputs, quantize_v_mxfp4
from synthetic import _e2m1_codes as synthetic_e2m1_codes

# OCP MX v1.0, FP4 E2M1: the value of every code
E2M1_TABLE = {0: 0.0, 1: 0.5, 2: 1.0, 3: 1.5, 4: 2.0, 5: 3.0, 6: 4.0, 7: 6.0}
LN2_SCALE = float(np.float32(math.log(2.0)))   # makes c = fp32(scale * log2 e) exactly 1


def test_decode_matches_format_table():
    for c, val in E2M1_TABLE.items():
        assert ofp4.e2m1_decode(c) == val
        assert ofp4.e2m1_decode(c | 8) == -val
    vals = ofp4.e2m1_decode(np.arange(8))
    assert np.all(np.diff(vals) > 0)            # positive codes are ordered by value
    # one explicit mantissa bit: every normal value is 1 or 1.5 times a power of two
    for v in vals[2:]:
        f = v / 2.0 ** math.floor(math.log2(v))
        assert f in (1.0, 1.5)


def test_encoders_agree_and_round_to_nearest_even():
    g = np.random.default_rng(3)
    x = np.concatenate([g.uniform(-7, 7, 50000), g.uniform(-0.6, 0.6, 5000),
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 6.0, 6.5, 100.0,
                                  0.0, 0.2499, 0.2501, 5.0001, 4.9999])])
    mine = ofp4.e2m1_encode(x)
    other = synthetic_e2m1_codes(torch.from_numpy(x.astype(np.float32))).numpy()
    assert np.array_equal(ofp4.e2m1_decode(mine), ofp4.e2m1_decode(other))
    dec = ofp4.e2m1_decode(mine)
    grid = np.array(sorted(set(E2M1_TABLE.values()) | {-v for v in E2M1_TABLE.values()}))
    # nearest (after saturation at +-6)
    xs = np.clip(x, -6, 6)
    best = np.abs(xs[:, None] - grid[None, :]).min(axis=1)
    assert np.all(np.abs(xs - dec) == best)
    # ties to the even code
    for v, want in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
                    (-5.0, 0xE)]:
        assert ofp4.e2m1_encode(np.array([v]))[0] == want, v


def test_mx_quantiser_scale_rule_and_nearest():
    g = torch.Generator().manual_seed(5)
    v = (torch.randn(100, 3, 8, generator=g) * torch.tensor([1e-3, 1.0, 50.0]).view(1, 3, 1))
    v[40:64, 1, 2] = 0.0                          # one all-zero block (tokens 32..63)
    v[32:40, 1, 2] = 0.0
    v = v.to(torch.bfloat16)
    packed, scales = quantize_v_mxfp4(v)
    assert packed.shape == (100, 3, 4) and scales.shape == (4, 3, 8)
    vf = v.double().numpy()
    x = scales.numpy().astype(np.int64) - 127
    for b in range(4):
        amax = np.abs(vf[32 * b:32 * b + 32]).max(axis=0)
        nz = amax > 0
        ratio = amax[nz] / np.exp2(x[b][nz])
        assert np.all((ratio >= 4.0) & (ratio < 8.0))       # X = floor(log2 amax) - 2
        assert np.all(x[b][~nz] == -127)
    vh = ofp4.mx_dequantize_v(packed, scales, 8)
    # every element is a nearest e2m1 value at its block's scale
    step = np.exp2(x[np.arange(100) // 32])
    grid = np.array(sorted(set(E2M1_TABLE.values()) | {-v for v in E2M1_TABLE.values()}))
    xs = np.clip(vf / step, -6, 6)
    best = np.abs(xs[..., None] - grid).min(axis=-1)
    assert np.allclose(np.abs(xs - vh / step), best, rtol=0, atol=0)


def test_mx_packing_order_and_exact_roundtrip():
    # values representable at the block scale come back exactly; even d is the low nibble
    vals = np.array([6.0, -0.5, 1.5, 0.0, 3.0, -4.0, 1.0, 2.0])
    v = np.tile(vals, (64, 2, 1)) * np.array([1.0, 0.25])[None, :, None]
    v[40, 0, :] *= -1
    vt = torch.from_numpy(v).to(torch.bfloat16)
    packed, scales = quantize_v_mxfp4(vt)
    assert np.array_equal(ofp4.mx_dequantize_v(packed, scales, 8), v)
    # d = 0 (amax 6, exponent 0) in the low nibble; d = 1 (amax 0.5, exponent -3,
    # so -0.5 is coded as -4) in the high nibble
    b = packed.numpy()
    assert scales.numpy()[0, 0, 0] == 127 and scales.numpy()[0, 0, 1] == 124
    assert int(b[0, 0, 0]) == int(ofp4.e2m1_encode(np.array([6.0]))[0]) | (
        int(ofp4.e2m1_encode(np.array([-4.0]))[0]) << 4)


def test_mx_blocks_are_local():
    inp = make_inputs(((70, 70),), 2, 8, seed=2, fp4_pv=True)
    v2 = inp.v.clone()
    v2[5] *= 64                                   # token 5 lies in block 0
    p2, s2 = quantize_v_mxfp4(v2)
    assert torch.equal(s2[1:], inp.v_mx_scale[1:])
    assert torch.equal(p2[32:], inp.v_e2m1[32:])


CASES = [
    (((9, 9),), False), (((9, 9),), True), (((5, 7), (6, 3)), True), (((40, 40),), True),
    (((3, 0), (20, 45), (7, 7)), False), (((13, 50),), True),
]


@pytest.mark.parametrize("lens,causal", CASES)
def test_emulation_matches_bruteforce(lens, causal):
    inp = make_inputs(lens, 2, 4, seed=11, fp4_pv=True)
    emu = ofp4.attention_fp4pv_emulated(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                        inp.cu_k, causal, 0.5)
    bf = ofp4.attention_fp4pv_bruteforce(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                         inp.cu_k, causal, 0.5)
    tq, h = inp.q.shape[0], inp.q.shape[1]
    got = emu.out.reshape(tq, h, -1)
    assert np.allclose(got, bf, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("lens,causal", CASES)
def test_emulation_within_bound_of_exact_and_lse_exact(lens, causal):
    inp = make_inputs(lens, 2, 8, seed=12, fp4_pv=True)
    scale = 0.35
    emu = ofp4.attention_fp4pv_emulated(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                        inp.cu_k, causal, scale)
    o, lse = ofp4.attention_fp4pv(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q, inp.cu_k,
                                  causal, scale)
    tq, h, dv = o.shape
    exact = o.reshape(tq * h, dv)
    err = np.abs(emu.out - exact)
    assert np.all(err <= emu.bound + 1e-12)
    lse_ref = lse.T.reshape(-1)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(emu.lse))
    # the emulation works with the fp32-rounded exp2-domain scale c, as the kernel
    # does, which moves LSE by about 1e-8 against the exact tau * log2 e
    assert np.allclose(emu.lse[fin], lse_ref[fin], rtol=0, atol=1e-6)


def _pinned_scores_inputs(raw_cols, v_rows):
    """d = 4 inputs whose raw scores q.k_j are the given integers (row 0)."""
    sk = len(raw_cols)
    q = torch.zeros((1, 1, 4), dtype=torch.bfloat16)
    q[0, 0, 0] = 1.0
    k = torch.zeros((sk, 1, 4), dtype=torch.bfloat16)
    k[:, 0, 0] = torch.tensor(raw_cols, dtype=torch.float32)
    v = torch.from_numpy(np.asarray(v_rows, dtype=np.float64)).to(torch.bfloat16).view(sk, 1, 4)
    packed, scales = quantize_v_mxfp4(v)
    return q, k, packed, scales


def test_exact_when_every_scaled_value_is_representable():
    # c = 1; raw scores are integers within 3 below their group's maximum, so each
    # 2^(r - E_G) is 4, 2, 1 or 1/2 and the quantised P equals P
    assert ofp4.fp32_log2e_scale(LN2_SCALE) == 1.0
    g = np.random.default_rng(4)
    # block 0: keys 0..31 with maximum 10; block 1: keys 32..52 with maximum 1
    raw = np.concatenate([[10], g.integers(7, 11, 31), [1], g.integers(-2, 2, 20)]).tolist()
    vrows = np.array([E2M1_TABLE[int(c)] for c in g.integers(0, 8, 4 * len(raw))]).reshape(-1, 4)
    q, k, vp, vs = _pinned_scores_inputs(raw, vrows)
    cu_q, cu_k = np.array([0, 1]), np.array([0, len(raw)])
    emu = ofp4.attention_fp4pv_emulated(q, k, vp, vs, cu_q, cu_k, False, LN2_SCALE)
    # the unquantised result with c = 1: sum 2^r_j V_j / sum 2^r_j
    w = np.exp2(np.array(raw, dtype=np.float64))
    assert np.allclose(emu.out[0], (w @ vrows) / w.sum(), rtol=1e-12, atol=1e-14)


def test_value_below_the_group_grid_is_dropped():
    # group maximum 10 -> E_G = 8; a key at 6 scales to 2^-2 = 0.25, the midpoint
    # between 0 and 0.5, which rounds to the even code 0: that key's P is lost
    raw = [10, 9, 6]
    vrows = [[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0]]
    q, k, vp, vs = _pinned_scores_inputs(raw, vrows)
    cu = np.array([0, 1]), np.array([0, 3])
    emu = ofp4.attention_fp4pv_emulated(q, k, vp, vs, cu[0], cu[1], False, LN2_SCALE)
    l = 2.0 ** 10 + 2.0 ** 9 + 2.0 ** 6
    assert np.allclose(emu.out[0], [2.0 ** 10 / l, 2.0 ** 9 / l, 0.0, 0.0], rtol=1e-14)


def test_single_visible_key_closed_form():
    # causal row 0 sees key 0 only: O = e2m1(x) / x * V_hat_0 with
    # x = 2^(c r - ceil(c r - log2 6)) in (3, 6]
    inp = make_inputs(((40, 40),), 1, 8, seed=13, fp4_pv=True)
    scale = 0.3
    emu = ofp4.attention_fp4pv_emulated(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                        inp.cu_k, True, scale, samples=[(0, 0)])
    c = ofp4.fp32_log2e_scale(scale)
    r = float(inp.q[0, 0].double() @ inp.k[0, 0].double())
    e = math.ceil(float(np.float32(np.float64(np.float32(r)) * c - np.float32(ofp4.LOG2_6))))
    x = 2.0 ** (c * r - e)
    assert 3.0 < x <= 6.0
    vh = ofp4.mx_dequantize_v(inp.v_e2m1, inp.v_mx_scale, 8)[0, 0]
    want = ofp4.e2m1_decode(ofp4.e2m1_encode(np.array([x])))[0] / x * vh
    assert np.allclose(emu.out[0], want, rtol=1e-12, atol=1e-15)


def test_log_domain_fold_equals_post_exp_division():
    # section 4's refactoring: dividing 2^(c r - m) by the group scale 2^(E_G - m)
    # after the exp gives the same codes as subtracting E_G inside the exp2, and
    # the same error against the exact result
    inp = make_inputs(((200, 200),), 1, 16, seed=14, fp4_pv=True)
    c = ofp4.fp32_log2e_scale(0.25)
    qf = inp.q[:, 0].double().numpy()
    kf = inp.k[:, 0].double().numpy()
    raw = qf @ kf.T
    x, codes, e, _ = ofp4.quantize_p_row_block(raw, np.arange(200), c)
    m = (c * raw).max(axis=1, keepdims=True)
    post = np.exp2(c * raw - m) / np.exp2(e - m)
    codes_post = ofp4.e2m1_encode(post)
    assert np.array_equal(ofp4.e2m1_decode(codes), ofp4.e2m1_decode(codes_post))
    assert np.all(x <= 6.0 * (1 + 1e-6)) and np.all(x.max(axis=1) > 3.0 - 1e-9)


def test_group_codes_depend_only_on_their_block():
    inp = make_inputs(((96, 96),), 1, 16, seed=15, fp4_pv=True)
    c = ofp4.fp32_log2e_scale(0.25)
    qf = inp.q[:, 0].double().numpy()
    kf = inp.k[:, 0].double().numpy()
    raw = qf @ kf.T
    _, codes, e, _ = ofp4.quantize_p_row_block(raw, np.arange(96), c)
    raw2 = raw.copy()
    raw2[:, 70] += 40.0                           # key 70 is in block 2
    _, codes2, e2, _ = ofp4.quantize_p_row_block(raw2, np.arange(96), c)
    assert np.array_equal(codes[:, :64], codes2[:, :64]) and np.array_equal(e[:, :64], e2[:, :64])
    assert not np.array_equal(e[:, 64:], e2[:, 64:])


def test_groups_follow_packed_token_blocks():
    # a document starting at token 20 has its first group cut at token 32
    inp = make_inputs(((20, 20), (50, 50)), 1, 8, seed=16, fp4_pv=True)
    c = ofp4.fp32_log2e_scale(0.3)
    k0 = 20
    qf = inp.q[k0:, 0].double().numpy()
    kf = inp.k[k0:, 0].double().numpy()
    raw = qf @ kf.T
    _, _, e, _ = ofp4.quantize_p_row_block(raw, np.arange(k0, 70), c)
    # keys 20..31 share one exponent per row, 32..63 another, 64..69 a third
    assert np.all(e[:, :12] == e[:, :1]) and np.all(e[:, 12:44] == e[:, 12:13])
    assert np.all(e[:, 44:] == e[:, 44:45])
