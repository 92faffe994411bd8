"""CPU oracle for the FMHA forward pass (fp64, plain definition).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no
code with the HIP path and imports nothing from it.

Parity status per function:
  attention / attention_sampled / attention_bruteforce -- pinned (brute force,
      torch float64 SDPA, closed forms and invariants in tests/test_oracle.py);
  e4m3_decode / e4m3_encode -- pinned (format definition values, torch
      float8_e4m3fn casts);
  attention_fp8pv -- pinned through its parts (decode + attention);
  attention_fp8pv_emulated -- pinned (pure-Python brute force, the fast e4m3
      rounding against the exhaustive encoder, exactness when every weight is
      an e4m3 value, the single-key closed form, independence from the integer
      maximum, the log-domain fold against post-exp scaling, the bound against
      attention_fp8pv, constructed midpoint ties, and planted mistakes).
  e2m1_decode / e2m1_encode / mx_dequantize_v -- pinned (the e2m1 value table,
      agreement with the independently written threshold encoder of the
      synthetic inputs, nearest-value and scale-rule checks, exact round trips);
  attention_fp4pv -- pinned through its parts (MX decode + attention);
  attention_fp4pv_emulated -- pinned (pure-Python brute force, exactness when
      every scaled P is an e2m1 value, closed forms for a dropped key and a
      single visible key, the log-domain fold against post-exp division, group
      locality, the error bound against attention_fp4pv, and constructed ties:
      zero ambiguity away from them, the exact other branch at them).
  merge_partials -- pinned (attention over disjoint key ranges, each taken
      with the oracle's own masked softmax, merges to attention over all keys;
      empty ranges and empty rows).
  attention_backward -- pinned (central finite differences of the forward
      oracle, invariants of the definition, torch float64 autograd);
  loss_grad_mean_square -- pinned (torch autograd of mean(O^2)).
"""

from .reference import (DEFAULT_ROW_BLOCK, attention, attention_bruteforce, attention_rows,
                        attention_sampled, scores, softmax_rows, visible)
from .fp8 import (E4M3_MAX, FP8Emulation, attention_fp8pv, attention_fp8pv_bruteforce,
                  attention_fp8pv_emulated, attention_fp8pv_sampled, dequantize_v, e4m3_decode,
                  e4m3_encode, round_e4m3)
from .merge import merge_partials
from .backward import attention_backward, loss_grad_mean_square
from .fp4 import (E2M1_MAX, FP4Emulation, attention_fp4pv, attention_fp4pv_bruteforce,
                  attention_fp4pv_emulated, attention_fp4pv_sampled, e2m1_decode, e2m1_encode,
                  mx_dequantize_v)

__all__ = [
    "DEFAULT_ROW_BLOCK", "attention", "attention_bruteforce", "attention_rows",
    "attention_sampled", "scores", "softmax_rows", "visible", "E4M3_MAX", "attention_fp8pv",
    "attention_fp8pv_emulated", "attention_fp8pv_sampled", "dequantize_v", "e4m3_decode",
    "e4m3_encode", "FP8Emulation", "attention_fp8pv_bruteforce", "round_e4m3", "E2M1_MAX", "FP4Emulation", "attention_fp4pv", "attention_fp4pv_bruteforce",
    "attention_fp4pv_emulated", "attention_fp4pv_sampled", "e2m1_decode", "e2m1_encode",
    "mx_dequantize_v", "merge_partials", "attention_backward", "loss_grad_mean_square",
]
