"""ctypes loader for libfmha.so and the raw C-ABI prototypes (include/fmha.h).

Only argument marshalling lives here; every step of the forward pass runs in
the HIP kernels of libfmha.so. Loading fails loudly when the library has not
been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfmha.so")

FMHA_OK = 0
FMHA_ERR_INVALID_ARG = 1
FMHA_ERR_UNSUPPORTED = 2
FMHA_ERR_LAUNCH = 3
NOALLOC_SCRATCH_BYTES = 16 << 20      # FMHA_NOALLOC_SCRATCH_BYTES of include/fmha.h

VARIANTS = {"auto": 0, "four_wave": 1, "pingpong": 2, "pipelined": 3, "wide": 4}

EXPORTED_SYMBOLS = (
    "fmha_fwd",
    "fmha_fwd_fp8pv",
    "fmha_fwd_variant",
    "fmha_fwd_fp8pv_variant",
    "fmha_fwd_fp4pv",
    "fmha_fwd_fp4pv_variant",
    "fmha_fwd_splitkv",
    "fmha_fwd_splitkv_workspace_size",
    "fmha_fwd_splitkv_num_splits",
    "fmha_merge_partials",
    "fmha_fwd_trace",
    "fmha_bwd",
    "fmha_bwd_workspace_size",
    "fmha_bwd_noalloc",
    "fmha_fwd_auto_variant",
    "fmha_validate_cu_seqlens",
    "fmha_status_string",
    "fmha_abi_version",
)

_lib = None

_vp, _i32, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
_FWD_ARGS = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
             _vp, _vp, _vp]
_FWD_FP8_ARGS = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                 _f32, _vp, _vp, _vp]


class FmhaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def _single_hip_runtime_check():
    """The process must hold one HIP runtime; two would not share streams."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise RuntimeError(f"more than one HIP runtime is loaded: {sorted(real)}")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfmha.so (after torch, so that torch's HIP runtime is reused)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m head_attention_forward_fmha_amd.build` "
            "(there is no non-HIP fallback)")
    import torch  # noqa: F401  -- load torch's libamdhip64 first
    lib = ctypes.CDLL(path)
    lib.fmha_fwd.argtypes = _FWD_ARGS
    lib.fmha_fwd.restype = ctypes.c_int
    lib.fmha_fwd_fp8pv.argtypes = _FWD_FP8_ARGS
    lib.fmha_fwd_fp8pv.restype = ctypes.c_int
    lib.fmha_fwd_variant.argtypes = _FWD_ARGS[:-1] + [_i32, _vp]
    lib.fmha_fwd_variant.restype = ctypes.c_int
    lib.fmha_fwd_fp8pv_variant.argtypes = _FWD_FP8_ARGS[:-1] + [_i32, _vp]
    lib.fmha_fwd_fp8pv_variant.restype = ctypes.c_int
    # fp4 P.V: same layout as fp8 (the fourth pointer is the E8M0 exponent array)
    lib.fmha_fwd_fp4pv.argtypes = _FWD_FP8_ARGS
    lib.fmha_fwd_fp4pv.restype = ctypes.c_int
    lib.fmha_fwd_fp4pv_variant.argtypes = _FWD_FP8_ARGS[:-1] + [_i32, _vp]
    lib.fmha_fwd_fp4pv_variant.restype = ctypes.c_int
    # split-KV: fmha_fwd_variant's arguments up to lse, then num_splits, workspace,
    # workspace bytes, variant, stream
    lib.fmha_fwd_splitkv.argtypes = _FWD_ARGS[:-1] + [_i32, _vp, ctypes.c_size_t, _i32, _vp]
    lib.fmha_fwd_splitkv.restype = ctypes.c_int
    lib.fmha_fwd_splitkv_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
    lib.fmha_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.fmha_fwd_splitkv_num_splits.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
    lib.fmha_fwd_splitkv_num_splits.restype = ctypes.c_int32
    lib.fmha_merge_partials.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
    lib.fmha_merge_partials.restype = ctypes.c_int
    # pv_format, q, k, v, v_scale, cu_q, cu_k, 8 sizes/flags, scale, out, lse, detailed,
    # traced workgroups, trace, trace bytes, stream
    lib.fmha_fwd_trace.argtypes = ([_i32] + _FWD_FP8_ARGS[:-1] + [_i32, _i32, _vp, ctypes.c_size_t, _vp])
    lib.fmha_fwd_trace.restype = ctypes.c_int
    lib.fmha_bwd.argtypes = ([_vp] * 8 + [_i32] * 8 + [_f32] + [_vp] * 4 +
                             [ctypes.c_size_t, _vp])
    lib.fmha_bwd.restype = ctypes.c_int
    # fmha_bwd's arguments without workspace and workspace bytes
    lib.fmha_bwd_noalloc.argtypes = [_vp] * 8 + [_i32] * 8 + [_f32] + [_vp] * 4
    lib.fmha_bwd_noalloc.restype = ctypes.c_int
    lib.fmha_bwd_workspace_size.argtypes = [_i32, _i32]
    lib.fmha_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fmha_fwd_auto_variant.argtypes = [_i32, _i32, _i32]
    lib.fmha_fwd_auto_variant.restype = ctypes.c_int32
    lib.fmha_validate_cu_seqlens.argtypes = [_vp, _i32, _i32, _i32]
    lib.fmha_validate_cu_seqlens.restype = ctypes.c_int
    lib.fmha_status_string.argtypes = [ctypes.c_int]
    lib.fmha_status_string.restype = ctypes.c_char_p
    lib.fmha_abi_version.argtypes = []
    lib.fmha_abi_version.restype = ctypes.c_int32
    _single_hip_runtime_check()
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fmha_status_string(int(status)).decode()
