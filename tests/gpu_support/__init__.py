"""GPU test support: an LDS-poisoning kernel (test infrastructure, not product).

build() compiles lds_poison.hip into libldspoison.so next to this file (with the
same hipcc flags as the library); poison_lds() launches it on the current
stream. A GPU test poisons the LDS of every CU with NaN bit patterns before a
forward pass, so that any read of LDS the pass did not write first shows up as
a non-finite output.
"""

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lds_poison.hip")
LIB = os.path.join(HERE, "libldspoison.so")
_lib = None


def build() -> str:
    from head_attention_forward_fmha_amd.build import ARCH, HIP_FLAGS, _hipcc
    cmd = [_hipcc(), *HIP_FLAGS, "-shared", "-o", LIB + ".tmp", SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on lds_poison.hip:\n" + r.stdout + r.stderr)
    os.replace(LIB + ".tmp", LIB)
    assert ARCH == "gfx950"
    return LIB


def poison_lds(stream_handle: int, workgroups: int = 1024) -> None:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError("libldspoison.so is not built (run __graft_entry__.build())")
        _lib = ctypes.CDLL(LIB)
        _lib.lds_poison_launch.argtypes = [ctypes.c_int, ctypes.c_void_p]
        _lib.lds_poison_launch.restype = ctypes.c_int
    err = _lib.lds_poison_launch(int(workgroups), ctypes.c_void_p(stream_handle))
    if err != 0:
        raise RuntimeError(f"lds_poison_launch failed: HIP error {err}")
