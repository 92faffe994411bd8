"""Seeded synthetic inputs for the FMHA forward pass.

This module only draws and lays out inputs; it holds none of the attention
arithmetic. The CPU oracle (``oracle/``) and the HIP path both take their
inputs from here, so that a parity test compares the two on identical bytes.

Recipe (FA4 spill issue, "CuTe DSL 4.7/4.8 regression ... ~3% slower on B300",
section "Steps/Code to reproduce bug", the benchmark script): Q, K and V are
standard-normal draws stored as bf16 in a packed ``[total_tokens, heads, d]``
layout, seeded with 0, and the document boundaries are
``round(linspace(0, total, docs + 1))`` as int32. The page draws bf16 on the
GPU, which is not reproducible on a CPU; here the draw is fp32 on the CPU with
``torch.Generator().manual_seed(seed)`` in the order q, k, v, then rounded to
bf16 (round-to-nearest-even), so both sides can rebuild the same bytes.

The fp8 P.V workload additionally hands V over as OCP e4m3 codes with one fp32
scale per head: ``scale[h] = max|V[:, h, :]| / 448`` and
``codes = e4m3(clamp(V / scale[h], -448, 448))`` with round-to-nearest-even
(torch's ``float8_e4m3fn`` cast). This is input preparation for that variant;
the oracle decodes the codes with its own decoder.

The fp4 P.V workload hands V over in OCP MXFP4 along the token axis: for every
block of 32 consecutive tokens of the packed tensor, head and d, one E8M0
exponent X = floor(log2(max|V|)) - 2 (the MX rule for e2m1, whose largest
exponent is 2; -127 for an all-zero block), and e2m1 codes of V / 2^X rounded
to nearest, ties to even, saturating at 6. Codes are packed two per byte along
d (even d in the low nibble); exponents are stored as X + 127.

The backward pass takes an upstream gradient dO of q's shape: a standard-normal
draw rounded to bf16 from its own generator, seeded with seed + 1, so that it is
independent of q, k and v (``make_dout``).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """One synthetic FMHA forward workload."""

    name: str
    description: str
    heads: int
    head_dim: int
    causal: bool
    # Per-document (query length, key length); one entry per document.
    doc_lens: tuple
    # True when the tensors are laid out dense [b, s, h, d] (all docs equal).
    dense: bool = False
    fp8_pv: bool = False
    fp4_pv: bool = False
    seed: int = 0

    @property
    def batch(self) -> int:
        return len(self.doc_lens)

    @property
    def total_q(self) -> int:
        return int(sum(a for a, _ in self.doc_lens))

    @property
    def total_k(self) -> int:
        return int(sum(b for _, b in self.doc_lens))

    @property
    def max_seqlen_q(self) -> int:
        return int(max((a for a, _ in self.doc_lens), default=0))

    @property
    def max_seqlen_k(self) -> int:
        return int(max((b for _, b in self.doc_lens), default=0))

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    def flops(self) -> float:
        """Counted FLOP: 4*h*sum(sq*sk)*d, halved when causal."""
        f = 4.0 * self.heads * sum(a * b for a, b in self.doc_lens) * self.head_dim
        return f / 2.0 if self.causal else f

    def hbm_bytes(self) -> float:
        """Algorithmic HBM bytes: Q, K, V read once, O written once, LSE written once."""
        h, d = self.heads, self.head_dim
        if self.fp4_pv:   # e2m1 codes plus one exponent byte per 32 tokens
            v_bytes = 0.5 + 1.0 / 32.0
        else:
            v_bytes = 1 if self.fp8_pv else 2
        return float(self.total_q * h * d * 2 + self.total_k * h * d * (2 + v_bytes)
                     + self.total_q * h * d * 2 + self.total_q * h * 4
                     + (h * 4 if self.fp8_pv else 0))


def cu_seqlens_linspace(total: int, docs: int) -> np.ndarray:
    """round(linspace(0, total, docs + 1)) as int32, computed in fp32 like torch."""
    cu = torch.linspace(0, total, docs + 1, dtype=torch.float32).round().to(torch.int32)
    return cu.numpy().astype(np.int32)


def lens_from_cu(cu: np.ndarray) -> tuple:
    cu = np.asarray(cu, dtype=np.int64)
    return tuple((int(b - a), int(b - a)) for a, b in zip(cu[:-1], cu[1:]))


def _linspace_docs(total: int, docs: int) -> tuple:
    return lens_from_cu(cu_seqlens_linspace(total, docs))


# The five workloads. c1 is small enough for the oracle to finish in well under
# a second; c4 is the bf16 varlen-causal d=128 workload the throughput figure is
# quoted on.
WORKLOADS = {
    "c1_tiny_dense": Workload(
        "c1_tiny_dense", "tiny dense: b=1 h=2 s=128 d=64, no mask", heads=2, head_dim=64,
        causal=False, doc_lens=((128, 128),), dense=True),
    "c2_dense_2225": Workload(
        "c2_dense_2225", "dense: b=1 h=16 s=2225 d=128, no mask (ragged tail)", heads=16,
        head_dim=128, causal=False, doc_lens=((2225, 2225),), dense=True),
    "c3_varlen_causal_8k": Workload(
        "c3_varlen_causal_8k", "varlen causal: 8192 tokens / 4 docs, h=32 d=128", heads=32,
        head_dim=128, causal=True, doc_lens=_linspace_docs(8192, 4)),
    "c4_varlen_causal_32k": Workload(
        "c4_varlen_causal_32k", "varlen causal: 32768 tokens / 8 docs, h=32 d=128", heads=32,
        head_dim=128, causal=True, doc_lens=_linspace_docs(32768, 8)),
    "c5_causal_fp8pv_32k": Workload(
        "c5_causal_fp8pv_32k", "single-doc causal fp8 P.V: 32768 tokens, h=16 d=128",
        heads=16, head_dim=128, causal=True, doc_lens=_linspace_docs(32768, 1), fp8_pv=True),
}

# Extra shapes for measurement only (not among the five above): the c4 token
# layout without the causal mask, which isolates the cost of causal scheduling;
# a short query range against long keys (few query blocks: the shape split-KV
# is for); the c5 shape with P.V in fp4 (MXFP4 V, per-group e2m1 P); and the
# c5 shape in bf16, the third of the fwd+bwd shapes the FA4 spill issue times
# (one 32768-token document, 16 heads).
EXTRA_WORKLOADS = {
    "x_varlen_noncausal_32k": Workload(
        "x_varlen_noncausal_32k", "varlen non-causal: 32768 tokens / 8 docs, h=32 d=128",
        heads=32, head_dim=128, causal=False, doc_lens=_linspace_docs(32768, 8)),
    "x_short_q_long_k": Workload(
        "x_short_q_long_k", "short queries, long keys: 512 query rows x 32768 keys, h=16 d=128, "
        "no mask", heads=16, head_dim=128, causal=False, doc_lens=((512, 32768),)),
    "x_causal_fp4pv_32k": Workload(
        "x_causal_fp4pv_32k", "single-doc causal fp4 P.V: 32768 tokens, h=16 d=128",
        heads=16, head_dim=128, causal=True, doc_lens=_linspace_docs(32768, 1), fp4_pv=True),
    "x_causal_bf16_32k": Workload(
        "x_causal_bf16_32k", "single-doc causal bf16: 32768 tokens, h=16 d=128",
        heads=16, head_dim=128, causal=True, doc_lens=_linspace_docs(32768, 1)),
}


def cu_seqlens(lens) -> tuple:
    """(cu_q, cu_k) int32 prefix sums of per-document (sq, sk) lengths."""
    lq = np.array([0] + [a for a, _ in lens], dtype=np.int64)
    lk = np.array([0] + [b for _, b in lens], dtype=np.int64)
    return np.cumsum(lq).astype(np.int32), np.cumsum(lk).astype(np.int32)


def randn_bf16(shape, gen: torch.Generator) -> torch.Tensor:
    """Standard-normal fp32 draw rounded to bf16 (CPU tensor)."""
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


@dataclass
class Inputs:
    q: torch.Tensor            # bf16 [total_q, h, d] (CPU)
    k: torch.Tensor            # bf16 [total_k, h, d]
    v: torch.Tensor            # bf16 [total_k, h, d]
    cu_q: np.ndarray           # int32 [batch + 1]
    cu_k: np.ndarray           # int32 [batch + 1]
    v_e4m3: Optional[torch.Tensor] = None   # uint8 [total_k, h, d] (fp8 workloads)
    v_scale: Optional[torch.Tensor] = None  # fp32 [h]
    v_e2m1: Optional[torch.Tensor] = None   # uint8 [total_k, h, d / 2] (fp4 workloads)
    v_mx_scale: Optional[torch.Tensor] = None  # uint8 [ceil(total_k / 32), h, d]
    extra: dict = field(default_factory=dict)


def quantize_v_e4m3(v: torch.Tensor):
    """Per-head amax scaling to OCP e4m3 codes (input preparation for fp8 P.V)."""
    vf = v.float()
    amax = vf.abs().amax(dim=(0, 2))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    codes = (vf / scale[None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).contiguous(), scale.contiguous()


MX_BLOCK = 32


def _e2m1_codes(y: torch.Tensor) -> torch.Tensor:
    """Nearest e2m1 code of fp32 values, ties to the even code, saturating at 6.

    The thresholds are the midpoints of 0, .5, 1, 1.5, 2, 3, 4, 6; a midpoint
    belongs to the neighbour with the even code (0, 1, 2, 3, 4, 5, 6, 7 are the
    codes of those values).
    """
    a = y.abs()
    code = ((a > 0.25).to(torch.uint8) + (a >= 0.75).to(torch.uint8) + (a > 1.25).to(torch.uint8)
            + (a >= 1.75).to(torch.uint8) + (a > 2.5).to(torch.uint8) + (a >= 3.5).to(torch.uint8)
            + (a > 5.0).to(torch.uint8))
    neg = (y < 0) & (code != 0)
    return torch.where(neg, code | 8, code).to(torch.uint8)


def quantize_v_mxfp4(v: torch.Tensor):
    """MXFP4 along tokens (input preparation for fp4 P.V); see the module docstring.

    Returns (packed codes uint8 [t, h, d/2], exponents uint8 [ceil(t/32), h, d]).
    """
    vf = v.float()
    t, h, d = vf.shape
    nb = (t + MX_BLOCK - 1) // MX_BLOCK
    padded = torch.zeros((nb * MX_BLOCK, h, d), dtype=torch.float32)
    padded[:t] = vf
    blocks = padded.view(nb, MX_BLOCK, h, d)
    amax = blocks.abs().amax(dim=1)
    _, e = torch.frexp(amax)            # amax = f * 2^e with f in [0.5, 1): floor(log2) = e - 1
    x = torch.where(amax > 0, e - 3, torch.full_like(e, -127)).clamp(-127, 127)
    y = torch.ldexp(blocks, (-x).unsqueeze(1).to(torch.float32))
    codes = _e2m1_codes(y).view(nb * MX_BLOCK, h, d)[:t]
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed.contiguous(), (x + 127).to(torch.uint8).contiguous()


def make_inputs(lens, heads: int, head_dim: int, seed: int = 0, fp8_pv: bool = False,
                head_dim_v: Optional[int] = None, fp4_pv: bool = False) -> Inputs:
    """Draw q, k, v for documents with per-doc (sq, sk) lengths ``lens``."""
    dv = head_dim if head_dim_v is None else head_dim_v
    cu_q, cu_k = cu_seqlens(lens)
    gen = torch.Generator().manual_seed(int(seed))
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = randn_bf16((tq, heads, head_dim), gen)
    k = randn_bf16((tk, heads, head_dim), gen)
    v = randn_bf16((tk, heads, dv), gen)
    inp = Inputs(q=q, k=k, v=v, cu_q=cu_q, cu_k=cu_k)
    if fp8_pv:
        inp.v_e4m3, inp.v_scale = quantize_v_e4m3(v)
    if fp4_pv:
        inp.v_e2m1, inp.v_mx_scale = quantize_v_mxfp4(v)
    return inp


def make_dout(total_q: int, heads: int, head_dim: int, seed: int = 0) -> torch.Tensor:
    """Upstream gradient dO [total_q, heads, head_dim] bf16, N(0, 1), seeded with seed + 1."""
    gen = torch.Generator().manual_seed(int(seed) + 1)
    return randn_bf16((total_q, heads, head_dim), gen)


def workload_inputs(w: Workload, seed: Optional[int] = None) -> Inputs:
    return make_inputs(w.doc_lens, w.heads, w.head_dim,
                       seed=w.seed if seed is None else seed, fp8_pv=w.fp8_pv, fp4_pv=w.fp4_pv)
