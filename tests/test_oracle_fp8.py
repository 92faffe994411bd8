"""Pins for the oracle's OCP e4m3 decoder/encoder and the fp8 P.V oracle."""

import numpy as np
import pytest
import torch

import oracle
from synthetic import make_inputs, quantize_v_e4m3


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


def test_emulated_p_quantisation_within_fp8_tolerance():
    inp = make_inputs(((200, 200), (57, 57)), 2, 32, seed=2, fp8_pv=True)
    tau = float(np.float32(1 / np.sqrt(32)))
    o, lse = oracle.attention_fp8pv(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q, inp.cu_k,
                                    True, tau)
    oe, le = oracle.attention_fp8pv_emulated(inp.q, inp.k, inp.v_e4m3, inp.v_scale, inp.cu_q,
                                             inp.cu_k, True, tau)
    assert np.all(np.abs(oe - o) <= 5e-2 + 5e-2 * np.abs(o))
    # the row sum uses the unquantised exp2 values, so LSE stays exact
    np.testing.assert_allclose(le, lse, atol=1e-12, rtol=0)
    # P scale inside the exponent vs multiplied after exp2: identical codes
    x = np.linspace(-30, 0, 1001)
    a = oracle.e4m3_encode(np.minimum(np.exp2(x + 8.0), 448.0))
    b = oracle.e4m3_encode(np.minimum(np.exp2(x) * 256.0, 448.0))
    assert np.array_equal(a, b)


def test_quantizer_scale_is_amax_over_448():
    v = torch.randn(100, 3, 16).to(torch.bfloat16)
    codes, scale = quantize_v_e4m3(v)
    amax = v.float().abs().amax(dim=(0, 2))
    assert torch.allclose(scale, amax / 448.0)
    dec = oracle.e4m3_decode(codes.numpy())
    assert np.nanmax(np.abs(dec)) <= 448.0 and not np.isnan(dec).any()
