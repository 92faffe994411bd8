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
LN2_SCALE = float(np.float32(math.log(2.0)))   # makes c = scale * log2 e within 3e-9 of 1


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
    # the row sum keeps the unquantised values, so LSE is the exact one
    assert np.allclose(emu.lse[fin], lse_ref[fin], rtol=0, atol=1e-12)


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
    # c = 1 (to 3e-9); raw scores are integers within 3 below their group's
    # maximum, so each 2^(c r - E_G) is 4, 2, 1 or 1/2 (to 3e-8), far from every
    # rounding midpoint, and the quantised P equals P to 3e-8
    assert abs(ofp4.log2e_scale(LN2_SCALE) - 1.0) < 3e-9
    g = np.random.default_rng(4)
    # block 0: keys 0..31 with maximum 10; block 1: keys 32..52 with maximum 1
    raw = np.concatenate([[10], g.integers(7, 11, 31), [1], g.integers(-2, 2, 20)]).tolist()
    vrows = np.array([E2M1_TABLE[int(c)] for c in g.integers(0, 8, 4 * len(raw))]).reshape(-1, 4)
    q, k, vp, vs = _pinned_scores_inputs(raw, vrows)
    cu_q, cu_k = np.array([0, 1]), np.array([0, len(raw)])
    emu = ofp4.attention_fp4pv_emulated(q, k, vp, vs, cu_q, cu_k, False, LN2_SCALE)
    # the unquantised result with c = 1: sum 2^r_j V_j / sum 2^r_j
    w = np.exp2(np.array(raw, dtype=np.float64))
    assert np.allclose(emu.out[0], (w @ vrows) / w.sum(), rtol=1e-7, atol=1e-12)
    assert not emu.ambiguity.any()


def test_value_below_the_group_grid_is_dropped():
    # group maximum 10 -> E_G = 8; a key at 5 scales to 2^-3 = 0.125, below the
    # midpoint 0.25 between 0 and 0.5, so it rounds to 0: that key's P is lost
    raw = [10, 9, 5]
    vrows = [[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0]]
    q, k, vp, vs = _pinned_scores_inputs(raw, vrows)
    cu = np.array([0, 1]), np.array([0, 3])
    emu = ofp4.attention_fp4pv_emulated(q, k, vp, vs, cu[0], cu[1], False, LN2_SCALE)
    c = ofp4.log2e_scale(LN2_SCALE)
    l = 2.0 ** (10 * c) + 2.0 ** (9 * c) + 2.0 ** (5 * c)
    # the kept keys' P_hat are the grid values 2^8 * 4 and 2^8 * 2
    assert np.allclose(emu.out[0], [2.0 ** 10 / l, 2.0 ** 9 / l, 0.0, 0.0], rtol=1e-14)
    assert not emu.ambiguity.any()


def test_single_visible_key_closed_form():
    # causal row 0 sees key 0 only: O = e2m1(x) / x * V_hat_0 with
    # x = 2^(c r - ceil(c r - log2 6)) in (3, 6]
    inp = make_inputs(((40, 40),), 1, 8, seed=13, fp4_pv=True)
    scale = 0.3
    emu = ofp4.attention_fp4pv_emulated(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                        inp.cu_k, True, scale, samples=[(0, 0)])
    c = float(np.float32(scale)) / math.log(2.0)
    r = float(inp.q[0, 0].double() @ inp.k[0, 0].double())
    e = math.ceil(c * r - math.log2(6.0))
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
    c = ofp4.log2e_scale(0.25)
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
    c = ofp4.log2e_scale(0.25)
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
    c = ofp4.log2e_scale(0.3)
    k0 = 20
    qf = inp.q[k0:, 0].double().numpy()
    kf = inp.k[k0:, 0].double().numpy()
    raw = qf @ kf.T
    _, _, e, _ = ofp4.quantize_p_row_block(raw, np.arange(k0, 70), c)
    # keys 20..31 share one exponent per row, 32..63 another, 64..69 a third
    assert np.all(e[:, :12] == e[:, :1]) and np.all(e[:, 12:44] == e[:, 12:13])
    assert np.all(e[:, 44:] == e[:, 44:45])


# ---------------------------------------------------------------- the ambiguity term

def _nearest_e2m1(x):
    """Nearest e2m1 value, ties to the even code (written out for the pins)."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    x = min(x, 6.0)
    return grid[min(range(8), key=lambda i: (abs(grid[i] - x), i % 2))]


def _mx_exact_rows(rows):
    """V rows whose MXFP4 encoding is exact (values 0 or 1 per column)."""
    return [list(map(float, r)) for r in rows]


def test_ambiguity_is_zero_away_from_ties():
    # integer scores 10, 9, 5 with c = 1 (to 3e-9): every scaled value sits at
    # least 1e-3 from a midpoint and the group argument 7.415 far from an integer
    q, k, vp, vs = _pinned_scores_inputs([10, 9, 5], _mx_exact_rows(np.eye(3, 4)))
    emu = ofp4.attention_fp4pv_emulated(q, k, vp, vs, [0, 1], [0, 3], False, LN2_SCALE)
    assert not emu.ambiguity.any() and not emu.group_tie.any() and emu.key_tie[0] == 0


def test_ambiguity_at_an_e2m1_midpoint_is_the_other_rounding():
    # key 2 at raw score 6: x = 2^(6c - 8) = 0.25 (1 + 1e-8), a hair above the
    # midpoint between 0 and 0.5, inside the fp32 window (its score error bound
    # alone is 4 * 2^-24 * 6 = 1.4e-6). fp64 rounds it up to 0.5; the other
    # branch rounds it to 0, which moves O by 0.5 * 2^E * |V_2| / l
    raw = [10, 9, 6]
    v = _mx_exact_rows(np.eye(3, 4))
    q, k, vp, vs = _pinned_scores_inputs(raw, v)
    emu = ofp4.attention_fp4pv_emulated(q, k, vp, vs, [0, 1], [0, 3], False, LN2_SCALE)
    c = ofp4.log2e_scale(LN2_SCALE)
    x = 2.0 ** (6 * c - 8)
    assert 0.25 < x < 0.25 * (1 + 1e-7)
    assert emu.key_tie[0] == 1 and not emu.group_tie.any()
    l = sum(2.0 ** (c * r - 10 * c) for r in raw)
    want = 0.5 * 2.0 ** (8 - 10 * c) * np.abs(np.array(v[2])) / l
    assert np.allclose(emu.ambiguity[0], want, rtol=1e-12, atol=0)
    # the listed alternative is the signed change: rounding down loses the key
    assert len(emu.alternatives[0]) == 1
    assert np.allclose(emu.alternatives[0][0], -0.5 * 2.0 ** (8 - 10 * c) * np.array(v[2]) / l,
                       rtol=1e-12, atol=0)
    # fp64 took the upper branch: key 2 contributes 2^8 * 0.5 to O's third column
    assert np.isclose(emu.out[0, 2], 0.5 * 2.0 ** (8 - 10 * c) / l, rtol=1e-12)


@pytest.mark.parametrize("side", [+1, -1])
def test_ambiguity_at_a_group_exponent_tie_is_the_other_grid(side):
    # group maximum 8 and c chosen so that c * 8 - log2 6 lies within 1e-6 of
    # 6 (fp32 tau moves it by < 6e-7): E_G may be 6 or 7. The ambiguity is the
    # other grid's effect, sum_j |P_alt_j - P_hat_j| |V_j| / l, computed here
    # with a separately written nearest-e2m1
    target = 6.0 + side * 2e-7
    tau = float(np.float32((target + math.log2(6.0)) / 8.0 * math.log(2.0)))
    c = tau / math.log(2.0)
    a = 8 * c - math.log2(6.0)
    assert abs(a - 6.0) < 1e-6
    raw = [8, 7, 5]
    v = _mx_exact_rows([[1, 0, 0, 0], [0, 1, 0, 0], [1, 0, 1, 0]])
    q, k, vp, vs = _pinned_scores_inputs(raw, v)
    emu = ofp4.attention_fp4pv_emulated(q, k, vp, vs, [0, 1], [0, 3], False, tau)
    assert emu.group_tie[0]
    e = math.ceil(a)
    e_alt = e - 1 if a > 6.0 else e + 1
    m = 8 * c
    l = sum(2.0 ** (c * r - m) for r in raw)
    p_hat = [_nearest_e2m1(2.0 ** (c * r - e)) * 2.0 ** (e - m) for r in raw]
    p_alt = [_nearest_e2m1(2.0 ** (c * r - e_alt)) * 2.0 ** (e_alt - m) for r in raw]
    want = sum(abs(pa - ph) * np.abs(np.array(vr)) for pa, ph, vr in zip(p_alt, p_hat, v)) / l
    assert np.any(want > 0)
    # no scaled value of either grid is near a midpoint here, so the group tie
    # is the whole ambiguity
    assert emu.key_tie[0] == 0
    assert np.allclose(emu.ambiguity[0], want, rtol=1e-12, atol=0)
    signed = sum((pa - ph) * np.array(vr) for pa, ph, vr in zip(p_alt, p_hat, v)) / l
    assert len(emu.alternatives[0]) == 1
    assert np.allclose(emu.alternatives[0][0], signed, rtol=1e-12, atol=0)
    out = sum(ph * np.array(vr) for ph, vr in zip(p_hat, v)) / l
    assert np.allclose(emu.out[0], out, rtol=1e-12)


def test_group_tie_window_closes_away_from_the_integer():
    # the same construction with the argument 1e-3 from the integer: no tie
    tau = float(np.float32((6.001 + math.log2(6.0)) / 8.0 * math.log(2.0)))
    q, k, vp, vs = _pinned_scores_inputs([8, 7, 5], _mx_exact_rows(np.eye(3, 4)))
    emu = ofp4.attention_fp4pv_emulated(q, k, vp, vs, [0, 1], [0, 3], False, tau)
    assert not emu.group_tie.any() and not emu.ambiguity.any()


def test_planted_wider_window_is_caught(monkeypatch):
    # a mistake that inflates the window (here: the safety factor times 1e4)
    # makes ties out of keys that are nowhere near one; the zero-away-from-ties
    # pin must then fail
    from oracle import fp32_window
    monkeypatch.setattr(fp32_window, "SAFETY", 2e4)
    q, k, vp, vs = _pinned_scores_inputs([10, 9, 5], _mx_exact_rows(np.eye(3, 4)))
    inp = make_inputs(((300, 300),), 2, 128, seed=3, fp4_pv=True)
    emu = ofp4.attention_fp4pv_emulated(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                        inp.cu_k, True, float(np.float32(1 / math.sqrt(128))))
    assert (emu.ambiguity > 0).mean() > 0.2


def test_ambiguity_share_and_size_on_a_realistic_case():
    """On the mixed-length d = 128 case the GPU parity tests use (seed 29):
    how many rows hold a decision fp32 may take the other way, and how large
    its effect is against the bf16 bar. The GPU check does not add that effect
    to the bar; it accepts O only within the bar of one of the method's
    outcomes (each decision taken one way or the other), so the emulation
    itself passes, and an all-zero or wrong-head O fails every row."""
    lens = ((1000, 1000), (333, 333), (1, 1), (700, 701))
    inp = make_inputs(lens, 4, 128, seed=29, fp4_pv=True)
    scale = float(np.float32(1 / math.sqrt(128)))
    emu = ofp4.attention_fp4pv_emulated(inp.q, inp.k, inp.v_e2m1, inp.v_mx_scale, inp.cu_q,
                                        inp.cu_k, True, scale)
    bar = 1e-2 + 1e-2 * np.abs(emu.out)
    n_dec = np.array([a.shape[0] for a in emu.alternatives])
    rows_amb = (n_dec > 0).mean()
    ratio = (emu.ambiguity / bar).max()
    # measured: 11.8% of rows hold 1 to 3 decisions; the largest total effect is
    # 8.9 times the bar (one key of a short early row flipping between 2 and 3)
    assert rows_amb < 0.2, rows_amb
    assert n_dec.max() <= 10          # every outcome is enumerated, none allowed in bulk
    assert ratio < 20.0, ratio
    assert not np.any(emu.slack)
    n = emu.out.shape[0]
    for i in range(n):
        assert ofp4.outcome_within(emu.out[i], emu.out[i], emu.alternatives[i], emu.slack[i],
                                   bar[i])
    h = 4
    checked = 0
    for i in range(n):
        if not np.any(np.abs(emu.out[i]) > 3e-2):
            continue     # rows of a one-key document can be all-small
        checked += 1
        assert not ofp4.outcome_within(np.zeros_like(emu.out[i]), emu.out[i],
                                       emu.alternatives[i], emu.slack[i], bar[i])
        other = i + 1 if (i % h) < h - 1 else i - 1          # same token, another head
        assert not ofp4.outcome_within(emu.out[other], emu.out[i], emu.alternatives[i],
                                       emu.slack[i], bar[i])
    assert checked > 0.9 * n
