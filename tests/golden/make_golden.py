"""Writes tests/golden/c1_tiny_dense_seed0.npz from the oracle alone.

The stored O/LSE are the fp64 oracle's answer for the tiny dense workload
(b=1, h=2, s=128, d=64, no mask, seed 0) together with a digest of the seeded
inputs, so that a later change to the input recipe or to the oracle's
arithmetic shows up as a test failure. Run from the repository root:

    python tests/golden/make_golden.py
"""

import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synthetic import WORKLOADS, workload_inputs  # noqa: E402


def input_digest(inp) -> str:
    h = hashlib.sha256()
    for t in (inp.q, inp.k, inp.v):
        h.update(t.contiguous().view(-1).view(dtype=__import__("torch").int16).numpy().tobytes())
    h.update(np.asarray(inp.cu_q, np.int32).tobytes())
    return h.hexdigest()


def main():
    w = WORKLOADS["c1_tiny_dense"]
    inp = workload_inputs(w)
    o, lse = oracle.attention(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, w.causal, w.softmax_scale)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_tiny_dense_seed0.npz")
    np.savez_compressed(path, o=o, lse=lse, digest=np.array(input_digest(inp)))
    print("wrote", path)


if __name__ == "__main__":
    main()
