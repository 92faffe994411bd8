"""The Python binding rejects inconsistent shapes before any library call.

These run on the CPU: every check below raises while marshalling arguments,
so no kernel is launched and no device memory is touched. A wrong-sized
tensor that slipped through would make the kernels read or write past its
allocation (the C ABI only sees pointers and the sizes it is told).
"""

import pytest
import torch

import head_attention_forward_fmha_amd as fm

bf = torch.bfloat16


def _packed(tq=128, tk=128, h=2, d=64):
    return (torch.zeros(tq, h, d, dtype=bf), torch.zeros(tk, h, d, dtype=bf),
            torch.zeros(tk, h, d, dtype=bf))


def test_dense_k_v_must_have_q_batch():
    q = torch.zeros(2, 128, 2, 64, dtype=bf)
    k = torch.zeros(1, 128, 2, 64, dtype=bf)
    v = torch.zeros(1, 128, 2, 64, dtype=bf)
    with pytest.raises(ValueError, match="batch"):
        fm.fwd(q, k, v)
    with pytest.raises(ValueError, match="batch"):
        fm.fwd_splitkv(q, k, v, num_splits=2)
    with pytest.raises(ValueError):
        fm.bwd(q, k, v, q, q, torch.zeros(2, 256))


def test_dense_v_must_have_k_seqlen():
    q = torch.zeros(2, 128, 2, 64, dtype=bf)
    k = torch.zeros(2, 128, 2, 64, dtype=bf)
    v = torch.zeros(2, 64, 2, 64, dtype=bf)
    with pytest.raises(ValueError):
        fm.fwd(q, k, v)


def test_packed_v_must_have_k_tokens():
    q, k, _ = _packed()
    v = torch.zeros(100, 2, 64, dtype=bf)
    with pytest.raises(ValueError):
        fm.fwd(q, k, v)
    with pytest.raises(ValueError):
        fm.fwd_fp8pv(q.new_zeros(128, 2, 128), k.new_zeros(128, 2, 128),
                     torch.zeros(100, 2, 128, dtype=torch.uint8), torch.ones(2))


@pytest.mark.parametrize("bad_out", [
    torch.zeros(127, 2, 64, dtype=bf),                  # too few rows
    torch.zeros(128, 2, 64, dtype=torch.float32),       # wrong dtype
    torch.zeros(128, 2, 128, dtype=bf)[:, :, :64],      # not contiguous
    torch.zeros(128, 4, 64, dtype=bf),                  # wrong heads
])
def test_caller_out_is_checked(bad_out):
    q, k, v = _packed()
    with pytest.raises((ValueError, TypeError)):
        fm.fwd(q, k, v, out=bad_out)
    with pytest.raises((ValueError, TypeError)):
        fm.fwd_splitkv(q, k, v, out=bad_out, num_splits=2)


@pytest.mark.parametrize("bad_lse", [
    torch.zeros(2, 127),                    # too short
    torch.zeros(128, 2),                    # transposed
    torch.zeros(2, 128, dtype=torch.float64),
    torch.zeros(2 * 128),                   # flat
])
def test_caller_lse_is_checked(bad_lse):
    q, k, v = _packed()
    with pytest.raises((ValueError, TypeError)):
        fm.fwd(q, k, v, lse=bad_lse)


def test_fp8_and_fp4_outputs_are_checked():
    q = torch.zeros(128, 2, 128, dtype=bf)
    k = torch.zeros(128, 2, 128, dtype=bf)
    v8 = torch.zeros(128, 2, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):
        fm.fwd_fp8pv(q, k, v8, torch.ones(2), out=torch.zeros(64, 2, 128, dtype=bf))
    with pytest.raises(ValueError):
        fm.fwd_fp8pv(q, k, v8, torch.ones(2), lse=torch.zeros(2, 64))
    v4 = torch.zeros(128, 2, 64, dtype=torch.uint8)
    sc = torch.zeros(4, 2, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):
        fm.fwd_fp4pv(q, k, v4, sc, out=torch.zeros(128, 2, 64, dtype=bf))
    with pytest.raises(ValueError):
        fm.fwd_fp4pv(q, k, v4, torch.zeros(3, 2, 128, dtype=torch.uint8))


def test_merge_outputs_are_checked():
    o_part = torch.zeros(3, 100, 2, 64)
    lse_part = torch.zeros(3, 2, 100)
    with pytest.raises(ValueError):
        fm.merge_partials(o_part, lse_part, out=torch.zeros(99, 2, 64, dtype=bf))
    with pytest.raises(ValueError):
        fm.merge_partials(o_part, lse_part, lse=torch.zeros(2, 99))


def test_trace_inputs_are_checked():
    q = torch.zeros(256, 2, 128, dtype=bf)
    k = torch.zeros(256, 2, 128, dtype=bf)
    cu = torch.tensor([0, 256], dtype=torch.int32)
    with pytest.raises(ValueError):     # bf16 v shorter than k
        fm.fwd_trace(q, k, torch.zeros(200, 2, 128, dtype=bf), cu, cu, 256, 256)
    with pytest.raises(ValueError):     # e4m3 scale per head
        fm.fwd_trace(q, k, torch.zeros(256, 2, 128, dtype=torch.uint8), cu, cu, 256, 256,
                     pv="e4m3", v_scale=torch.ones(3))
    with pytest.raises(ValueError):     # e4m3 without a scale
        fm.fwd_trace(q, k, torch.zeros(256, 2, 128, dtype=torch.uint8), cu, cu, 256, 256,
                     pv="e4m3")
    with pytest.raises(ValueError):     # e2m1 codes are d/2 bytes per row
        fm.fwd_trace(q, k, torch.zeros(256, 2, 128, dtype=torch.uint8), cu, cu, 256, 256,
                     pv="e2m1", v_scale=torch.zeros(8, 2, 128, dtype=torch.uint8))
    with pytest.raises(ValueError):     # e2m1 exponent rows: ceil(total_k / 32)
        fm.fwd_trace(q, k, torch.zeros(256, 2, 64, dtype=torch.uint8), cu, cu, 256, 256,
                     pv="e2m1", v_scale=torch.zeros(7, 2, 128, dtype=torch.uint8))


def test_bwd_gradients_and_lse_are_checked():
    q, k, v = _packed(d=128)
    lse = torch.zeros(2, 128)
    with pytest.raises(ValueError):
        fm.bwd(q, k, v, q, q, lse, dq=torch.zeros(64, 2, 128, dtype=bf))
    with pytest.raises(ValueError):
        fm.bwd(q, k, v, q, q, torch.zeros(2, 64))
