"""Host-side model of the kernels' HBM -> LDS copy addresses (test infrastructure).

The kernels copy K/V (forward, dQ) and Q/dO (dK/dV) tiles with raw-buffer
loads: a descriptor whose base is the (document, head) start and whose size is
the document's rows, and a per-lane byte offset that the hardware checks
against that size (offsets past it read zeros). The e2m1 V exponents and the
backward's per-row LSE/D values are loaded from plain per-lane addresses with
no such check, so those must be in bounds by construction. This module
restates, in numpy, the offsets each kernel forms (the per-lane chunk offsets
of the swizzled tile layout, the tile offsets, the exponent-row clamp, the row
clamp of the LSE/D loads) and the tiles each work item copies, and returns
every byte range that a launch reads. The tests check each range against its
allocation for empty, mid-block, terminal and key-less documents, and check
that the model reports a planted out-of-range copy.

Constants: 64-row tiles, 4 copying waves of 64 lanes, 16 bytes per lane and
copy, 1 KB copy blocks per wave; forward work items of 128 (4-wave kernel) or
256 (ping-pong) query rows; backward items of 128 rows; e2m1 exponent blocks
of 32 tokens.
"""

from __future__ import annotations

import numpy as np

TILE = 64
WAVES = 4
LANES = 64
U32 = 1 << 32


def swz(row, chunks):
    row = np.asarray(row)
    if chunks == 16:
        return ((row & 3) << 2) | ((row >> 2) & 3)
    if chunks == 4:
        return (row >> 3) & 3
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3)


def lane_offsets(row_bytes: int, stride: int) -> np.ndarray:
    """Per-lane byte offsets (relative to a tile's first row) of every copy
    instruction of every wave: lane l of wave w, copy r lands at LDS byte
    1024 (r * 4 + w) + 16 l and fetches the logical chunk stored there."""
    tile_bytes = TILE * row_bytes
    loads = tile_bytes // (WAVES * LANES * 16)
    assert loads * WAVES * LANES * 16 == tile_bytes
    chunks = row_bytes // 16
    r = np.arange(loads)[:, None, None]
    w = np.arange(WAVES)[None, :, None]
    lane = np.arange(LANES)[None, None, :]
    byte = 1024 * (r * WAVES + w) + 16 * lane
    row = byte // row_bytes
    phys = (byte % row_bytes) // 16
    return (row * stride + (phys ^ swz(row, chunks)) * 16).reshape(-1)


class Reads:
    """Byte ranges a launch reads, per named allocation."""

    def __init__(self):
        self.ranges = {}

    def add(self, name, start, length):
        start = np.asarray(start, dtype=np.int64).reshape(-1)
        self.ranges.setdefault(name, []).append((start, int(length)))

    def violations(self, sizes: dict) -> list:
        bad = []
        for name, parts in self.ranges.items():
            for start, length in parts:
                over = (start < 0) | (start + length > sizes[name])
                if over.any():
                    i = int(np.argmax(over))
                    bad.append(f"{name}: bytes [{start[i]}, {start[i] + length}) outside "
                               f"[0, {sizes[name]})")
        return bad


def _buffer_copy(reads, name, base, num_bytes, voffs, tile_off):
    """A raw-buffer copy: the 32-bit offset voff + tile_off reads 16 bytes when it
    is below the descriptor's size, zeros otherwise."""
    off = (voffs.astype(np.int64) + int(tile_off)) % U32
    hit = off < (num_bytes % U32)
    reads.add(name, base + off[hit], 16)


def _docs(cu_q, cu_k):
    return [(int(cu_q[b]), int(cu_q[b + 1]) - int(cu_q[b]), int(cu_k[b]),
             int(cu_k[b + 1]) - int(cu_k[b])) for b in range(len(cu_q) - 1)]


def forward_reads(cu_q, cu_k, heads, d, causal, pv="bf16", rows=256, num_splits=1,
                  extra_tiles=0) -> Reads:
    """Byte ranges read by one forward launch (any kernel: rows = 128 or 256).

    ``extra_tiles`` plants a mistake: copies for that many tiles past the last
    one of each work item (what an unguarded prefetch would issue)."""
    reads = Reads()
    total_k = int(cu_k[-1])
    row_bytes = 2 * d
    v_row = {"bf16": 2 * d, "e4m3": d, "e2m1": d // 2}[pv]
    k_stride, v_stride = heads * row_bytes, heads * v_row
    k_voffs = lane_offsets(row_bytes, k_stride)
    v_voffs = lane_offsets(v_row, v_stride)
    n_blocks = (total_k + 31) // 32
    vs_stride = heads * d
    for q_start, sq, k_start0, sk0 in _docs(cu_q, cu_k):
        for head in range(heads):
            for m0 in range(0, sq, rows):
                for split in range(num_splits):
                    k_start, sk, key_lo = k_start0, sk0, 0
                    if pv == "e2m1":
                        r = k_start & 31
                        k_start, sk, key_lo = k_start - r, sk + r, r
                    causal_off = sk - sq
                    kend = min(sk, max(0, m0 + rows + causal_off)) if causal else sk
                    n = (kend + TILE - 1) // TILE
                    if num_splits > 1:
                        t0 = split * n // num_splits
                        t1 = (split + 1) * n // num_splits
                        k_start, sk = k_start + t0 * TILE, sk - t0 * TILE
                        n = t1 - t0
                    # Q rows, loaded once per item (rows past the document clamped)
                    qi = np.minimum(np.arange(m0, m0 + rows), sq - 1)
                    reads.add("q", ((q_start + qi) * heads + head) * row_bytes, row_bytes)
                    k_base = k_start * k_stride + head * row_bytes
                    v_base = k_start * v_stride + head * v_row
                    for j in range(n + extra_tiles):
                        _buffer_copy(reads, "k", k_base, sk * k_stride, k_voffs,
                                     (j * TILE * k_stride) % U32)
                        _buffer_copy(reads, "v", v_base, sk * v_stride, v_voffs,
                                     (j * TILE * v_stride) % U32)
                        if pv == "e2m1":
                            blk0 = k_start // 32
                            vs_last = max(n_blocks - 1 - blk0, 0)
                            lane = np.arange(LANES)
                            rb = np.minimum(2 * j + lane // 32, vs_last)
                            reads.add("v_scale", (blk0 + rb) * vs_stride + head * d
                                      + 4 * (lane % 32), 4)
    return reads


def backward_reads(cu_q, cu_k, heads, d, causal) -> Reads:
    """Byte ranges read by the dQ and dK/dV launches of one backward pass."""
    reads = Reads()
    row_bytes = 2 * d
    stride = heads * row_bytes
    voffs = lane_offsets(row_bytes, stride)
    total_q = int(cu_q[-1])
    blk = 32 * WAVES
    lane = np.arange(LANES)
    for q_start, sq, k_start, sk in _docs(cu_q, cu_k):
        causal_off = sk - sq
        for head in range(heads):
            # dQ: per 128-query block, K/V tiles of the keys the block sees
            for m0 in range(0, sq, blk):
                qi = np.minimum(np.arange(m0, m0 + blk), sq - 1)
                for name in ("q", "dout", "out"):
                    reads.add(name, ((q_start + qi) * heads + head) * row_bytes, row_bytes)
                reads.add("lse", (head * total_q + q_start + qi) * 4, 4)
                kend = min(sk, max(0, m0 + blk + causal_off)) if causal else sk
                for j in range((kend + TILE - 1) // TILE):
                    for name in ("k", "v"):
                        _buffer_copy(reads, name, k_start * stride + head * row_bytes,
                                     sk * stride, voffs, (j * TILE * stride) % U32)
            # dK/dV: per 128-key block, Q/dO tiles of the queries that see it
            for n0 in range(0, sk, blk):
                ki = np.minimum(np.arange(n0, n0 + blk), sk - 1)
                for name in ("k", "v"):
                    reads.add(name, ((k_start + ki) * heads + head) * row_bytes, row_bytes)
                n_qt = (sq + TILE - 1) // TILE
                t0 = max(0, n0 - causal_off) // TILE if causal else 0
                for jt in range(t0, n_qt):
                    for name in ("q", "dout"):
                        _buffer_copy(reads, name, q_start * stride + head * row_bytes,
                                     sq * stride, voffs, (jt * TILE * stride) % U32)
                    r = head * total_q + q_start + np.minimum(jt * TILE + lane, sq - 1)
                    reads.add("workspace_lse2", r * 4, 4)
                    reads.add("workspace_delta", r * 4, 4)
    return reads


def forward_sizes(total_q, total_k, heads, d, pv="bf16") -> dict:
    v_row = {"bf16": 2 * d, "e4m3": d, "e2m1": d // 2}[pv]
    return {"q": total_q * heads * 2 * d, "k": total_k * heads * 2 * d,
            "v": total_k * heads * v_row, "v_scale": (total_k + 31) // 32 * heads * d}


def backward_sizes(total_q, total_k, heads, d) -> dict:
    return {"q": total_q * heads * 2 * d, "dout": total_q * heads * 2 * d,
            "out": total_q * heads * 2 * d, "k": total_k * heads * 2 * d,
            "v": total_k * heads * 2 * d, "lse": heads * total_q * 4,
            "workspace_lse2": heads * total_q * 4, "workspace_delta": heads * total_q * 4}
