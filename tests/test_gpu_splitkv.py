"""GPU parity of the split-KV forward pass and of the partial-result merge.

fmha_fwd_splitkv computes the same function as fmha_fwd, so it is held to the
bf16 bar against the oracle (|O - O_ref| <= 1e-2 + 1e-2 |O_ref|, LSE within
1e-3, -inf rows exact). Its workspace partials, merged by the oracle's own
merge, must give the oracle's attention too (which checks the split kernels
apart from the GPU merge), and fmha_merge_partials alone is checked against the
oracle's merge on synthetic partials, including empty parts and empty rows.
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

O_ATOL = O_RTOL = 1e-2
LSE_ATOL = 1e-3


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _run(inp, causal, scale, heads, d, num_splits, variant="auto", workspace=None, split=True):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq = torch.from_numpy(np.asarray(inp.cu_q, np.int32)).to(dev)
    ck = torch.from_numpy(np.asarray(inp.cu_k, np.int32)).to(dev)
    mq = int(np.diff(inp.cu_q).max())
    mk = int(np.diff(inp.cu_k).max())
    out = torch.full((q.shape[0], heads, d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((heads, q.shape[0]), float("nan"), dtype=torch.float32, device=dev)
    if split:
        fm.fwd_splitkv(q, k, v, cq, ck, mq, mk, causal=causal, softmax_scale=scale, out=out,
                       lse=lse, num_splits=num_splits, workspace=workspace, variant=variant)
    else:
        fm.fwd(q, k, v, cq, ck, mq, mk, causal=causal, softmax_scale=scale, out=out, lse=lse,
               variant=variant)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(o, lse, o_ref, lse_ref, what):
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    err = np.abs(o - o_ref)
    bad = err > O_ATOL + O_RTOL * np.abs(o_ref)
    assert not bad.any(), f"{what}: {bad.sum()} O elements out of tolerance (max {err.max():.3e})"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse), ~fin), f"{what}: -inf LSE rows differ"
    if fin.any():
        assert np.abs(lse[fin] - lse_ref[fin]).max() <= LSE_ATOL, f"{what}: LSE"


def _parity(lens, heads, d, causal, num_splits, seed=0, variant="auto"):
    inp = make_inputs(lens, heads, d, seed=seed)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _run(inp, causal, scale, heads, d, num_splits, variant=variant)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, causal, scale)
    _check(o, lse, o_ref, lse_ref,
           what=f"lens={lens} d={d} causal={causal} splits={num_splits} variant={variant}")
    return inp, o, lse


@pytest.mark.parametrize("num_splits", ["auto", 2, 3, 5])
@pytest.mark.parametrize("variant", ["four_wave", "pingpong"])
def test_c2_dense_2225_splitkv_full(num_splits, variant):
    """c2 (dense, 2225 tokens, 16 heads, ragged tail of 49 rows) at full size,
    split 2, 3 and 5 ways (144 blocks of 256 rows on 256 compute units; the
    automatic choice keeps it unsplit, as measured splitting does not pay)."""
    w = WORKLOADS["c2_dense_2225"]
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal, w.softmax_scale, w.heads, w.head_dim, num_splits, variant)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, w.causal,
                                      w.softmax_scale)
    _check(o, lse, o_ref, lse_ref, what=f"c2 splits={num_splits} {variant}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("variant", ["four_wave", "pingpong"])
def test_one_split_is_bitwise_the_unsplit_pass(causal, d, variant):
    """One split runs the unsplit pass (and needs no workspace)."""
    inp = make_inputs(((300, 300), (129, 129), (1, 1)), 4, d, seed=8)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o1, l1 = _run(inp, causal, scale, 4, d, 1, variant)
    o0, l0 = _run(inp, causal, scale, 4, d, 1, variant, split=False)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)


@pytest.mark.parametrize("lens", [
    ((1, 1),), ((65, 65),), ((200, 200),), ((129, 129), (1, 1), (64, 64), (300, 300)),
    ((100, 300),), ((300, 100),), ((70, 0),), ((0, 50), (40, 40)), ((5, 5), (0, 0), (130, 7), (7, 130)),
])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("num_splits", [2, 4, 7])
def test_splitkv_ragged_and_empty(lens, causal, num_splits):
    _parity(lens, 3, 128, causal, num_splits, seed=len(lens) + num_splits)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("variant", ["four_wave", "pingpong"])
def test_splitkv_d64_and_more_splits_than_tiles(causal, variant):
    # 65 keys are two tiles: six of the eight splits see no key at all
    _parity(((65, 65), (300, 300)), 2, 64, causal, 8, seed=4, variant=variant)
    _parity(((1000, 1000),), 2, 128, causal, 64, seed=5, variant=variant)


@pytest.mark.parametrize("causal", [False, True])
def test_workspace_partials_merge_to_attention(causal):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    lens, heads, d, n_split = ((700, 700), (333, 400)), 2, 128, 3
    inp = make_inputs(lens, heads, d, seed=12)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    tq = inp.q.shape[0]
    need = fm.splitkv_workspace_size(tq, heads, d, n_split)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev)
    _run(inp, causal, scale, heads, d, n_split, workspace=ws)
    w = ws.cpu().numpy().astype(np.float64)
    n_o = n_split * tq * heads * d
    o_parts = w[:n_o].reshape(n_split, tq * heads, d)
    lse_parts = w[n_o:].reshape(n_split, heads, tq).transpose(0, 2, 1).reshape(n_split, tq * heads)
    assert not np.isnan(o_parts).any() and not np.isnan(lse_parts).any()
    o_m, lse_m = oracle.merge_partials(o_parts, lse_parts)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, causal, scale)
    _check(o_m.reshape(tq, heads, d), lse_m.reshape(tq, heads).T, o_ref, lse_ref,
           what=f"oracle merge of the workspace partials (causal={causal})")


def test_merge_kernel_matches_the_oracle_merge():
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    rng = np.random.default_rng(7)
    for n_parts, tq, heads, d in ((1, 37, 3, 64), (5, 300, 4, 128), (64, 9, 2, 128)):
        o_parts = rng.standard_normal((n_parts, tq, heads, d)).astype(np.float32)
        lse_parts = (rng.standard_normal((n_parts, heads, tq)) * 4).astype(np.float32)
        lse_parts[rng.random((n_parts, heads, tq)) < 0.3] = -np.inf   # parts with no key
        lse_parts[:, 0, :2] = -np.inf                                  # rows with no key at all
        out, lse = fm.merge_partials(torch.from_numpy(o_parts).to(dev),
                                     torch.from_numpy(lse_parts).to(dev))
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.merge_partials(
            o_parts.reshape(n_parts, tq * heads, d),
            lse_parts.transpose(0, 2, 1).reshape(n_parts, tq * heads))
        _check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
               o_ref.reshape(tq, heads, d), lse_ref.reshape(tq, heads).T,
               what=f"merge S={n_parts} tq={tq} h={heads} d={d}")
        fin = np.isfinite(lse_ref)
        assert np.abs(lse.cpu().numpy()[fin.reshape(tq, heads).T] -
                      lse_ref.reshape(tq, heads).T[fin.reshape(tq, heads).T]).max() < 1e-5


def test_short_q_long_k_sampled():
    """The short-query workload (512 query rows x 32768 keys, 16 heads) at full
    size with the automatic split count, on sampled rows."""
    from synthetic import EXTRA_WORKLOADS
    import head_attention_forward_fmha_amd as fm
    w = EXTRA_WORKLOADS["x_short_q_long_k"]
    assert fm.splitkv_num_splits(w.batch, w.max_seqlen_q, w.max_seqlen_k, w.heads) > 1
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal, w.softmax_scale, w.heads, w.head_dim, "auto")
    rng = np.random.default_rng(2)
    samples = sorted({(int(t), int(rng.integers(w.heads))) for t in rng.integers(0, 512, 120)})
    o_ref, l_ref = oracle.attention_sampled(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, w.causal,
                                            w.softmax_scale, samples)
    t = np.array([a for a, _ in samples])
    hh = np.array([b for _, b in samples])
    _check(o[t, hh], lse[hh, t], o_ref, l_ref, what=w.name)
    assert np.isfinite(o).all() and np.isfinite(lse).all()


def test_splitkv_deterministic_repeats():
    inp = make_inputs(((1000, 1000), (777, 777)), 4, 128, seed=21)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    o0, l0 = _run(inp, True, scale, 4, 128, 5)
    for _ in range(5):
        o, l = _run(inp, True, scale, 4, 128, 5)
        assert np.array_equal(o, o0) and np.array_equal(l, l0)


@pytest.mark.parametrize("variant", ["pipelined", "wide"])
def test_splitkv_unsplit_only_variants_are_rejected(variant):
    import head_attention_forward_fmha_amd as fm
    dev = _dev()
    inp = make_inputs(((128, 128),), 2, 128, seed=31)
    with pytest.raises(fm.FmhaError):
        fm.fwd_splitkv(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), num_splits=2,
                       variant=variant)


@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_stale_lds_is_never_read(causal):
    from tests.gpu_support import poison_lds
    dev = _dev()
    for lens in (((65, 65),), ((300, 300), (77, 77))):
        poison_lds(torch.cuda.current_stream(dev).cuda_stream)
        _parity(lens, 3, 128, causal, 3, seed=41)
