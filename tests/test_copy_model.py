"""Every HBM address the kernels' copies read stays inside its allocation.

A host-side model of the copy offsets (tests/copy_model.py) is run over the
document layouts that stress them: empty documents, documents without keys or
without queries, documents starting inside a 32-token block (the e2m1 path
widens them to the block start), a last document ending at the end of the
buffer on and off a 32-token boundary, and a batch with no keys at all. A
planted mistake (copies for a tile past the last one, the kind of change
that once faulted the GPU through the unchecked e2m1 exponent load) must be
reported. Copy-placement changes are checked against this model before they
run on a GPU.
"""

import numpy as np
import pytest

from tests import copy_model as cm

LAYOUTS = {
    "empty_and_keyless": ((5, 5), (0, 0), (130, 7), (7, 130), (70, 0)),
    "mid_block_starts": ((13, 13), (50, 50), (70, 40), (0, 20), (45, 100)),
    "terminal_on_boundary": ((100, 100), (28, 28)),          # total_k = 128
    "terminal_off_boundary": ((100, 100), (47, 47)),
    "terminal_empty_on_boundary": ((64, 64), (10, 0)),        # last document has no keys
    "no_keys_at_all": ((40, 0), (7, 0)),
    "no_queries": ((0, 50), (0, 70)),
    "long_ragged": ((1000, 1000), (333, 333), (1, 1), (700, 701)),
}


def _cu(lens):
    cq = np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int64)
    return cq, ck


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("pv", ["bf16", "e4m3", "e2m1"])
@pytest.mark.parametrize("rows", [128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_copies_stay_in_bounds(layout, pv, rows, causal):
    lens = LAYOUTS[layout]
    cq, ck = _cu(lens)
    heads, d = 2, 128
    reads = cm.forward_reads(cq, ck, heads, d, causal, pv=pv, rows=rows)
    assert not reads.violations(cm.forward_sizes(int(cq[-1]), int(ck[-1]), heads, d, pv))


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("splits", [2, 3, 8])
def test_split_kv_copies_stay_in_bounds(layout, splits):
    cq, ck = _cu(LAYOUTS[layout])
    for causal in (False, True):
        reads = cm.forward_reads(cq, ck, 2, 64, causal, rows=128, num_splits=splits)
        assert not reads.violations(cm.forward_sizes(int(cq[-1]), int(ck[-1]), 2, 64))


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_copies_stay_in_bounds(layout, d, causal):
    cq, ck = _cu(LAYOUTS[layout])
    reads = cm.backward_reads(cq, ck, 2, d, causal)
    assert not reads.violations(cm.backward_sizes(int(cq[-1]), int(ck[-1]), 2, d))


def test_model_reports_a_copy_past_the_last_tile():
    """Copies for one tile past each item's last: the buffer loads of K and V
    still read zeros past the document (their range check), but the e2m1
    exponent load has no range check, and for a last document without keys at
    a 32-token boundary it reads past the exponent array."""
    cq, ck = _cu(LAYOUTS["terminal_empty_on_boundary"])
    sizes = cm.forward_sizes(int(cq[-1]), int(ck[-1]), 2, 128, "e2m1")
    good = cm.forward_reads(cq, ck, 2, 128, True, pv="e2m1", rows=256)
    assert not good.violations(sizes)
    bad = cm.forward_reads(cq, ck, 2, 128, True, pv="e2m1", rows=256, extra_tiles=1)
    v = bad.violations(sizes)
    assert v and all(s.startswith("v_scale") for s in v)
    bf = cm.forward_reads(cq, ck, 2, 128, True, pv="bf16", rows=256, extra_tiles=1)
    assert not bf.violations(cm.forward_sizes(int(cq[-1]), int(ck[-1]), 2, 128))


def test_model_reports_an_unclamped_row():
    """The backward's LSE/D loads clamp the row to the document; a query block
    whose tile runs past the last row must read the clamped row. Without the
    clamp, the last document's tile would read past the workspace."""
    cq, ck = _cu(LAYOUTS["terminal_off_boundary"])
    total_q = int(cq[-1])
    sizes = cm.backward_sizes(total_q, int(ck[-1]), 1, 64)
    reads = cm.backward_reads(cq, ck, 1, 64, False)
    assert not reads.violations(sizes)
    # the same tile rows without the clamp
    lane = np.arange(cm.LANES)
    q_start, sq = int(cq[-2]), int(cq[-1] - cq[-2])
    unclamped = cm.Reads()
    unclamped.add("workspace_lse2", (q_start + (sq // cm.TILE) * cm.TILE + lane) * 4, 4)
    assert unclamped.violations(sizes)


def test_tile_offsets_fit_the_32_bit_lane_offset():
    """The library rejects problems where heads * d * (total + 64) elements
    exceed 2^31 - 1 (fmha_fwd returns FMHA_ERR_UNSUPPORTED); below that, the
    largest tile offset plus lane offset of any copy, in bytes, stays under
    2^32, the range of the buffer loads' unsigned 32-bit offset, so no offset
    wraps onto an earlier row."""
    for heads, d in ((32, 128), (1, 64), (7, 128)):
        stride = heads * 2 * d
        total = (2 ** 31 - 1) // (heads * d) - 64      # the largest accepted total
        n_tiles = (total + cm.TILE - 1) // cm.TILE
        max_off = ((n_tiles - 1) * cm.TILE * stride + int(cm.lane_offsets(2 * d, stride).max())
                   + 16)
        assert max_off < 2 ** 32
