"""MI355X-native fused multi-head attention forward pass (Python binding).

``fwd``, ``fwd_fp8pv`` and ``fwd_fp4pv`` marshal torch tensors into the C ABI of libfmha.so
(include/fmha.h); torch supplies device memory and the current HIP stream, and
every step of the forward pass runs in the library's gfx950 kernels.

The operation is the FMHA forward pass of the pages ("[BUG] Unexpected Slower
Performance in C++ CuTe (77_blackwell_fmha) vs Python CuTe DSL (fmha.py) on
Jetson Thor", Key Observation 2; "CuTe DSL 4.7/4.8 regression: FlashAttention-4
SM100 forward kernel spills registers", Steps/Code to reproduce bug): packed
varlen [total, heads, d] bf16 tensors with int32 cu_seqlens, optional causal
masking, output O and the natural-log LSE of each query row.
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

from . import _lib
from ._lib import FMHA_OK, NOALLOC_SCRATCH_BYTES, VARIANTS, FmhaError, EXPORTED_SYMBOLS  # noqa: F401

__all__ = ["fwd", "fwd_fp8pv", "fwd_fp4pv", "bwd", "bwd_noalloc", "bwd_workspace_size", "fwd_splitkv",
           "splitkv_num_splits", "NOALLOC_SCRATCH_BYTES",
           "splitkv_workspace_size", "merge_partials", "fwd_trace", "TRACE_EVENTS_PER_WAVE",
           "auto_variant", "validate_cu_seqlens", "status_string", "abi_version",
           "FmhaError", "EXPORTED_SYMBOLS", "VARIANTS", "load_library"]


def load_library():
    return _lib.load()


def status_string(status: int) -> str:
    return _lib.status_string(status)


def abi_version() -> int:
    return int(_lib.load().fmha_abi_version())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, dtype, ndim, device):
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")


def _prepare(q, k, v_like, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k):
    """Normalise dense [b,s,h,d] / packed [t,h,d] inputs to the C-ABI sizes."""
    import torch
    if q.dim() == 4:
        b, sq, h, d = q.shape
        if k.dim() != 4 or v_like.dim() != 4:
            raise ValueError("dense q [b, s, h, d] needs dense k and v")
        sk = k.shape[1]
        if k.shape[0] != b or v_like.shape[0] != b or v_like.shape[1] != sk:
            raise ValueError("dense k and v must have q's batch and the same sequence length")
        if cu_seqlens_q is not None or cu_seqlens_k is not None:
            raise ValueError("dense [b, s, h, d] inputs take no cu_seqlens")
        return dict(batch=b, total_q=b * sq, total_k=b * sk, max_q=sq, max_k=sk, heads=h, d=d,
                    cu_q=None, cu_k=None, out_shape=(b, sq, h, d), lse_len=b * sq)
    if q.dim() != 3:
        raise ValueError("q must be [total, heads, d] or [b, s, heads, d]")
    tq, h, d = q.shape
    tk = k.shape[0]
    if k.dim() != 3 or v_like.dim() != 3 or v_like.shape[0] != tk:
        raise ValueError("packed k and v must be [total_k, heads, d] with the same total_k")
    if cu_seqlens_q is None:
        if cu_seqlens_k is not None:
            raise ValueError("cu_seqlens_q and cu_seqlens_k must be given together")
        return dict(batch=1, total_q=tq, total_k=tk, max_q=tq, max_k=tk, heads=h, d=d,
                    cu_q=None, cu_k=None, out_shape=(tq, h, d), lse_len=tq)
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if cu is None or cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 vector")
        if cu.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if max_seqlen_q is None or max_seqlen_k is None:
        raise ValueError("max_seqlen_q and max_seqlen_k are required with cu_seqlens")
    return dict(batch=cu_seqlens_q.numel() - 1, total_q=tq, total_k=tk, max_q=int(max_seqlen_q),
                max_k=int(max_seqlen_k), heads=h, d=d, cu_q=cu_seqlens_q, cu_k=cu_seqlens_k,
                out_shape=(tq, h, d), lse_len=tq)


def _outputs(s, out, lse, return_lse, device):
    """The caller's out / lse (checked against the problem), or new ones."""
    import torch
    if out is None:
        out = torch.empty(s["out_shape"], dtype=torch.bfloat16, device=device)
    else:
        _check_tensor("out", out, torch.bfloat16, len(s["out_shape"]), device)
        if tuple(out.shape) != tuple(s["out_shape"]):
            raise ValueError(f"out must have shape {tuple(s['out_shape'])}, got {tuple(out.shape)}")
    if lse is None:
        if return_lse:
            lse = torch.empty((s["heads"], s["lse_len"]), dtype=torch.float32, device=device)
    else:
        _check_tensor("lse", lse, torch.float32, 2, device)
        if tuple(lse.shape) != (s["heads"], s["lse_len"]):
            raise ValueError(f"lse must have shape {(s['heads'], s['lse_len'])}, "
                             f"got {tuple(lse.shape)}")
    return out, lse


def _stream_handle(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def fwd(q, k, v, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q: Optional[int] = None,
        max_seqlen_k: Optional[int] = None, causal: bool = False,
        softmax_scale: Optional[float] = None, out=None, lse=None,
        return_lse: bool = True, variant: str = "auto") -> Tuple:
    """bf16 FMHA forward. Returns (out, lse) with lse fp32 [heads, total_q].

    q [total_q, h, d] / k, v [total_k, h, d] with cu_seqlens (int32 [batch+1]),
    or dense q [b, sq, h, d] / k, v [b, sk, h, d]. d must be 64 or 128.
    variant: "auto", "four_wave", "pingpong", "pipelined" or "wide" (kernel
    choice; same function).
    """
    import torch
    lib = _lib.load()
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, q.dim(), dev)
    _check_tensor("k", k, torch.bfloat16, q.dim(), dev)
    _check_tensor("v", v, torch.bfloat16, q.dim(), dev)
    s = _prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    if k.shape != v.shape or k.shape[-2:] != q.shape[-2:]:
        raise ValueError("k and v must match, with q's heads and head_dim")
    scale = 1.0 / math.sqrt(s["d"]) if softmax_scale is None else float(softmax_scale)
    out, lse = _outputs(s, out, lse, return_lse, dev)
    st = lib.fmha_fwd_variant(_ptr(q), _ptr(k), _ptr(v), _ptr(s["cu_q"]), _ptr(s["cu_k"]),
                              s["batch"], s["total_q"], s["total_k"], s["max_q"], s["max_k"],
                              s["heads"], s["d"], int(bool(causal)), ctypes.c_float(scale),
                              _ptr(out), _ptr(lse), VARIANTS[variant],
                              ctypes.c_void_p(_stream_handle(dev)))
    if st != FMHA_OK:
        raise FmhaError(st, "fmha_fwd")
    return out, lse


def fwd_fp8pv(q, k, v_e4m3, v_scale, cu_seqlens_q=None, cu_seqlens_k=None,
              max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
              causal: bool = False, softmax_scale: Optional[float] = None, out=None, lse=None,
              return_lse: bool = True, variant: str = "auto") -> Tuple:
    """FMHA forward with P.V in fp8 e4m3. v_e4m3 is uint8 codes, v_scale fp32 [heads]."""
    import torch
    lib = _lib.load()
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, q.dim(), dev)
    _check_tensor("k", k, torch.bfloat16, q.dim(), dev)
    _check_tensor("v_e4m3", v_e4m3, torch.uint8, q.dim(), dev)
    _check_tensor("v_scale", v_scale, torch.float32, 1, dev)
    s = _prepare(q, k, v_e4m3, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    if k.shape != v_e4m3.shape or k.shape[-2:] != q.shape[-2:] or v_scale.numel() != s["heads"]:
        raise ValueError("k, v_e4m3, v_scale shapes do not match q")
    scale = 1.0 / math.sqrt(s["d"]) if softmax_scale is None else float(softmax_scale)
    out, lse = _outputs(s, out, lse, return_lse, dev)
    st = lib.fmha_fwd_fp8pv_variant(_ptr(q), _ptr(k), _ptr(v_e4m3), _ptr(v_scale),
                                    _ptr(s["cu_q"]), _ptr(s["cu_k"]), s["batch"], s["total_q"],
                                    s["total_k"], s["max_q"], s["max_k"], s["heads"], s["d"],
                                    int(bool(causal)), ctypes.c_float(scale), _ptr(out),
                                    _ptr(lse), VARIANTS[variant],
                                    ctypes.c_void_p(_stream_handle(dev)))
    if st != FMHA_OK:
        raise FmhaError(st, "fmha_fwd_fp8pv")
    return out, lse


def fwd_fp4pv(q, k, v_e2m1, v_mx_scale, cu_seqlens_q=None, cu_seqlens_k=None,
              max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
              causal: bool = False, softmax_scale: Optional[float] = None, out=None, lse=None,
              return_lse: bool = True, variant: str = "auto") -> Tuple:
    """FMHA forward with P.V in fp4 e2m1 (MXFP4 V, per-group scaled P).

    v_e2m1 uint8 [total_k, h, d/2] (two codes per byte, even d low), v_mx_scale
    uint8 E8M0 [ceil(total_k/32), h, d]; packed [total, h, d] layout only (dense
    inputs are the packed layout with batch * seqlen tokens).
    """
    import torch
    lib = _lib.load()
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, 3, dev)
    _check_tensor("k", k, torch.bfloat16, 3, dev)
    _check_tensor("v_e2m1", v_e2m1, torch.uint8, 3, dev)
    _check_tensor("v_mx_scale", v_mx_scale, torch.uint8, 3, dev)
    s = _prepare(q, k, v_e2m1, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    tk, h, d = k.shape
    if (tuple(v_e2m1.shape) != (tk, h, d // 2) or q.shape[1:] != k.shape[1:]
            or tuple(v_mx_scale.shape) != ((tk + 31) // 32, h, d)):
        raise ValueError("k, v_e2m1, v_mx_scale shapes do not match q")
    scale = 1.0 / math.sqrt(s["d"]) if softmax_scale is None else float(softmax_scale)
    out, lse = _outputs(s, out, lse, return_lse, dev)
    st = lib.fmha_fwd_fp4pv_variant(_ptr(q), _ptr(k), _ptr(v_e2m1), _ptr(v_mx_scale),
                                    _ptr(s["cu_q"]), _ptr(s["cu_k"]), s["batch"], s["total_q"],
                                    s["total_k"], s["max_q"], s["max_k"], s["heads"], s["d"],
                                    int(bool(causal)), ctypes.c_float(scale), _ptr(out),
                                    _ptr(lse), VARIANTS[variant],
                                    ctypes.c_void_p(_stream_handle(dev)))
    if st != FMHA_OK:
        raise FmhaError(st, "fmha_fwd_fp4pv")
    return out, lse


def splitkv_workspace_size(total_q: int, num_heads: int, head_dim: int, num_splits: int) -> int:
    """Bytes of workspace fwd_splitkv needs (0 for invalid sizes)."""
    return int(_lib.load().fmha_fwd_splitkv_workspace_size(int(total_q), int(num_heads),
                                                            int(head_dim), int(num_splits)))


def splitkv_num_splits(batch: int, max_seqlen_q: int, max_seqlen_k: int, num_heads: int,
                       causal: bool = False, variant: str = "auto") -> int:
    """The split count the library suggests for this problem on the current device."""
    n = _lib.load().fmha_fwd_splitkv_num_splits(int(batch), int(max_seqlen_q), int(max_seqlen_k),
                                                 int(num_heads), int(bool(causal)),
                                                 VARIANTS[variant])
    if n < 0:
        raise ValueError("negative problem size or unknown variant")
    return int(n)


def fwd_splitkv(q, k, v, cu_seqlens_q=None, cu_seqlens_k=None,
                max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
                causal: bool = False, softmax_scale: Optional[float] = None, out=None, lse=None,
                return_lse: bool = True, num_splits="auto", workspace=None,
                variant: str = "auto") -> Tuple:
    """bf16 FMHA forward with the key range of each query block split num_splits
    ways and the parts merged (same result as ``fwd``). ``workspace`` is a device
    tensor of at least splitkv_workspace_size(...) bytes (allocated when None);
    after the call it holds the fp32 O parts [S, total_q, h, d] followed by the
    LSE parts [S, h, total_q]."""
    import torch
    lib = _lib.load()
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, q.dim(), dev)
    _check_tensor("k", k, torch.bfloat16, q.dim(), dev)
    _check_tensor("v", v, torch.bfloat16, q.dim(), dev)
    s = _prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    if k.shape != v.shape or k.shape[-2:] != q.shape[-2:]:
        raise ValueError("k and v must match, with q's heads and head_dim")
    if num_splits == "auto":
        n_split = splitkv_num_splits(s["batch"], s["max_q"], s["max_k"], s["heads"], causal,
                                     variant if variant not in ("pipelined", "wide") else "auto")
    else:
        n_split = int(num_splits)
    scale = 1.0 / math.sqrt(s["d"]) if softmax_scale is None else float(softmax_scale)
    need = splitkv_workspace_size(s["total_q"], s["heads"], s["d"], n_split)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    out, lse = _outputs(s, out, lse, return_lse, dev)
    st = lib.fmha_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(s["cu_q"]), _ptr(s["cu_k"]),
                              s["batch"], s["total_q"], s["total_k"], s["max_q"], s["max_k"],
                              s["heads"], s["d"], int(bool(causal)), ctypes.c_float(scale),
                              _ptr(out), _ptr(lse), n_split, _ptr(workspace), ws_bytes,
                              VARIANTS[variant],
                              ctypes.c_void_p(_stream_handle(dev)))
    if st != FMHA_OK:
        raise FmhaError(st, "fmha_fwd_splitkv")
    return out, lse


def bwd_workspace_size(total_q: int, num_heads: int) -> int:
    """Bytes of device workspace fmha_bwd needs (D and LSE*log2(e) per row and head)."""
    return int(_lib.load().fmha_bwd_workspace_size(int(total_q), int(num_heads)))


def bwd(q, k, v, out, dout, lse, cu_seqlens_q=None, cu_seqlens_k=None,
        max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
        causal: bool = False, softmax_scale: Optional[float] = None, dq=None, dk=None, dv=None,
        workspace=None) -> Tuple:
    """Backward pass of ``fwd``: (dq, dk, dv) bf16 given the forward's inputs, its output
    ``out``, its natural-log ``lse`` [h, total_q] and the upstream gradient ``dout``.
    ``workspace`` (allocated when None) is a device tensor of at least
    bwd_workspace_size(total_q, heads) bytes."""
    import torch
    lib = _lib.load()
    dev = q.device
    for name, t, ref in (("q", q, q), ("k", k, q), ("v", v, q), ("out", out, q),
                         ("dout", dout, q)):
        _check_tensor(name, t, torch.bfloat16, ref.dim(), dev)
    s = _prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    if k.shape != v.shape or k.shape[-2:] != q.shape[-2:]:
        raise ValueError("k and v must match, with q's heads and head_dim")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have q's shape")
    _check_tensor("lse", lse, torch.float32, 2, dev)
    if tuple(lse.shape) != (s["heads"], s["lse_len"]):
        raise ValueError("lse must be [heads, total_q]")
    scale = 1.0 / math.sqrt(s["d"]) if softmax_scale is None else float(softmax_scale)
    need = bwd_workspace_size(s["total_q"], s["heads"])
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(name, t, torch.bfloat16, ref.dim(), dev)
        if t.shape != ref.shape:
            raise ValueError(f"{name} must have the shape of its input")
    st = lib.fmha_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                      _ptr(s["cu_q"]), _ptr(s["cu_k"]), s["batch"], s["total_q"], s["total_k"],
                      s["max_q"], s["max_k"], s["heads"], s["d"], int(bool(causal)),
                      ctypes.c_float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                      ws_bytes, ctypes.c_void_p(_stream_handle(dev)))
    if st != FMHA_OK:
        raise FmhaError(st, "fmha_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q=None, cu_seqlens_k=None,
                max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
                causal: bool = False, softmax_scale: Optional[float] = None) -> Tuple:
    """``bwd`` without a workspace: the library's fixed per-GPU array of
    NOALLOC_SCRATCH_BYTES holds D and LSE*log2(e), so neither this call nor the
    library allocates (the caller passes dq, dk, dv). Calls that can overlap on
    one GPU share that array and must be ordered by the caller. Problems with
    heads * total_q above NOALLOC_SCRATCH_BYTES / 8 raise FmhaError."""
    import torch
    lib = _lib.load()
    dev = q.device
    for name, t, ref in (("q", q, q), ("k", k, q), ("v", v, q), ("out", out, q),
                         ("dout", dout, q)):
        _check_tensor(name, t, torch.bfloat16, ref.dim(), dev)
    s = _prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    if k.shape != v.shape or k.shape[-2:] != q.shape[-2:]:
        raise ValueError("k and v must match, with q's heads and head_dim")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have q's shape")
    _check_tensor("lse", lse, torch.float32, 2, dev)
    if tuple(lse.shape) != (s["heads"], s["lse_len"]):
        raise ValueError("lse must be [heads, total_q]")
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(name, t, torch.bfloat16, ref.dim(), dev)
        if t.shape != ref.shape:
            raise ValueError(f"{name} must have the shape of its input")
    if 8 * s["heads"] * s["total_q"] > NOALLOC_SCRATCH_BYTES:
        raise FmhaError(2, f"fmha_bwd_noalloc: heads * total_q = {s['heads'] * s['total_q']} "
                           f"exceeds the {NOALLOC_SCRATCH_BYTES >> 20} MiB scratch "
                           f"({NOALLOC_SCRATCH_BYTES // 8} rows)")
    scale = 1.0 / math.sqrt(s["d"]) if softmax_scale is None else float(softmax_scale)
    st = lib.fmha_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                              _ptr(s["cu_q"]), _ptr(s["cu_k"]), s["batch"], s["total_q"],
                              s["total_k"], s["max_q"], s["max_k"], s["heads"], s["d"],
                              int(bool(causal)), ctypes.c_float(scale), _ptr(dq), _ptr(dk),
                              _ptr(dv), ctypes.c_void_p(_stream_handle(dev)))
    if st != FMHA_OK:
        raise FmhaError(st, "fmha_bwd_noalloc")
    return dq, dk, dv


def merge_partials(o_part, lse_part, out=None, lse=None, return_lse: bool = True) -> Tuple:
    """Merge fp32 partial results o_part [S, total_q, h, d] / lse_part [S, h, total_q]
    over disjoint key ranges into bf16 out [total_q, h, d] and fp32 lse [h, total_q]."""
    import torch
    lib = _lib.load()
    dev = o_part.device
    _check_tensor("o_part", o_part, torch.float32, 4, dev)
    _check_tensor("lse_part", lse_part, torch.float32, 3, dev)
    n_parts, tq, h, d = o_part.shape
    if tuple(lse_part.shape) != (n_parts, h, tq):
        raise ValueError("lse_part must be [S, heads, total_q] matching o_part")
    out, lse = _outputs(dict(out_shape=(tq, h, d), heads=h, lse_len=tq), out, lse, return_lse, dev)
    st = lib.fmha_merge_partials(_ptr(o_part), _ptr(lse_part), n_parts, tq, h, d, _ptr(out),
                                 _ptr(lse), ctypes.c_void_p(_stream_handle(dev)))
    if st != FMHA_OK:
        raise FmhaError(st, "fmha_merge_partials")
    return out, lse


TRACE_EVENTS_PER_WAVE = 8192
_PV_FORMATS = {"bf16": 0, "e4m3": 1, "e2m1": 2}


def fwd_trace(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
              pv: str = "bf16", v_scale=None, softmax_scale: Optional[float] = None,
              detailed: bool = False, traced_workgroups: int = 32) -> Tuple:
    """Causal d=128 forward pass on the ping-pong kernel with a pipeline trace.

    pv: "bf16" (v bf16), "e4m3" (v codes, v_scale fp32 [heads]) or "e2m1" (v MXFP4
    codes, v_scale the E8M0 exponents). Returns (out, lse, trace) with trace
    uint64 [traced_workgroups, 8, TRACE_EVENTS_PER_WAVE] on the device (see
    head_attention_forward_fmha_amd.pipeline_trace for the records).
    """
    import torch
    lib = _lib.load()
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, 3, dev)
    _check_tensor("k", k, torch.bfloat16, 3, dev)
    if pv not in _PV_FORMATS:
        raise ValueError(f"pv must be one of {sorted(_PV_FORMATS)}")
    _check_tensor("v", v, torch.bfloat16 if pv == "bf16" else torch.uint8, 3, dev)
    tk, h, d = k.shape
    if q.shape[1:] != k.shape[1:]:
        raise ValueError("k must have q's heads and head_dim")
    if pv == "e2m1":
        if tuple(v.shape) != (tk, h, d // 2):
            raise ValueError("e2m1 v must be [total_k, heads, head_dim / 2]")
        if v_scale is None:
            raise ValueError("e2m1 v needs its E8M0 exponents (v_scale)")
        _check_tensor("v_scale", v_scale, torch.uint8, 3, dev)
        if tuple(v_scale.shape) != ((tk + 31) // 32, h, d):
            raise ValueError("e2m1 v_scale must be [ceil(total_k / 32), heads, head_dim]")
    else:
        if tuple(v.shape) != (tk, h, d):
            raise ValueError("v must have k's shape")
        if pv == "e4m3":
            if v_scale is None:
                raise ValueError("e4m3 v needs its per-head scale (v_scale)")
            _check_tensor("v_scale", v_scale, torch.float32, 1, dev)
            if v_scale.numel() != h:
                raise ValueError("e4m3 v_scale must be [heads]")
    s = _prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    scale = 1.0 / math.sqrt(s["d"]) if softmax_scale is None else float(softmax_scale)
    out = torch.empty(s["out_shape"], dtype=torch.bfloat16, device=dev)
    lse = torch.empty((s["heads"], s["lse_len"]), dtype=torch.float32, device=dev)
    trace = torch.zeros((int(traced_workgroups), 8, TRACE_EVENTS_PER_WAVE), dtype=torch.int64,
                        device=dev)
    st = lib.fmha_fwd_trace(_PV_FORMATS[pv], _ptr(q), _ptr(k), _ptr(v), _ptr(v_scale),
                            _ptr(s["cu_q"]), _ptr(s["cu_k"]), s["batch"], s["total_q"],
                            s["total_k"], s["max_q"], s["max_k"], s["heads"], s["d"], 1,
                            ctypes.c_float(scale), _ptr(out), _ptr(lse), int(bool(detailed)),
                            int(traced_workgroups), _ptr(trace),
                            trace.numel() * trace.element_size(),
                            ctypes.c_void_p(_stream_handle(dev)))
    if st != FMHA_OK:
        raise FmhaError(st, "fmha_fwd_trace")
    return out, lse, trace


def auto_variant(batch: int, max_seqlen_q: int, num_heads: int) -> str:
    """Name of the kernel variant that variant="auto" runs for this problem size."""
    v = load_library().fmha_fwd_auto_variant(int(batch), int(max_seqlen_q), int(num_heads))
    if v < 0:
        raise ValueError("negative problem size")
    return {k: n for n, k in VARIANTS.items()}[v]


def validate_cu_seqlens(cu_host, total: int, max_seqlen: int) -> bool:
    """Host-side check of a cu_seqlens array (numpy/list/CPU tensor) via the C ABI."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(cu_host, dtype=np.int32))
    st = _lib.load().fmha_validate_cu_seqlens(arr.ctypes.data_as(ctypes.c_void_p),
                                              int(arr.size) - 1, int(total), int(max_seqlen))
    return st == FMHA_OK
