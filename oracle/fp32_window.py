"""How far the GPU's fp32 arithmetic can move a quantisation decision.

TEST INFRASTRUCTURE (see ``oracle/reference.py``): imported only by tests,
``__graft_entry__.smoke()`` and the cpu_baseline leg of ``bench.py``.

The low-precision P.V methods ("Kernel Bottleneck Tuning (validated on FA4
FP4/FP8 PV, GB300)", sections 4 and 5) round each exp2 value to a short
format and, for fp4, choose each group's power-of-two scale by rounding a
log-domain argument up to an integer. The oracle takes every one of those
decisions in fp64 from the definition. A GPU computes the same quantities in
fp32, so where the exact value sits closer to a decision boundary than the
fp32 evaluation can be trusted, either outcome is a correct result of the
method. This module bounds that distance; the oracles then list the affected
elements and how far the other outcome would move O (their ``ambiguity``).

Bounds (u = 2^-24, the fp32 unit roundoff):

* a score s = q.k is a d-term dot product of exact bf16 products accumulated
  in fp32 in some order: |s32 - s| <= d u sum_t |q_t k_t| (the standard bound
  for recursive summation, valid for any order);
* the exp2-domain scale c = tau log2 e reaches the kernel rounded to fp32:
  |c32 - c| <= u c;
* an exp2 argument a = c s + b (b an exact fp32 addend, such as minus an
  integer exponent) evaluated by one fused multiply-add is off by at most
  c |s32 - s| + u c |s| + u |a| (the last term its one rounding);
* the hardware exp2 is taken to be within 2^-21 relative (4 units in the last
  place) of 2^a.

Every bound is then doubled, so a decision is called ambiguous only well
inside the region where fp32 might take the other branch, never outside it.
"""

from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24
EXP2_REL = 2.0 ** -21
SAFETY = 2.0


def score_error(absdot: np.ndarray, d: int) -> np.ndarray:
    """Bound on |s32 - s| for scores whose products have absolute sum ``absdot``."""
    return d * U32 * np.asarray(absdot, dtype=np.float64)


def arg_error(c: float, raw: np.ndarray, absdot: np.ndarray, d: int, arg: np.ndarray,
              addend_err: float = 0.0) -> np.ndarray:
    """Bound on the fp32 error of an exp2-domain argument ``arg = c * raw + b``.

    ``addend_err`` bounds the error of the addend b itself (0 when b is an
    integer, which fp32 holds exactly).
    """
    with np.errstate(invalid="ignore"):
        return (c * score_error(absdot, d) + U32 * c * np.abs(raw) + U32 * np.abs(arg)
                + addend_err)


def rel_error_of_exp2(arg_err: np.ndarray) -> np.ndarray:
    """Bound on the relative error of exp2 of an argument off by ``arg_err``."""
    return np.log(2.0) * arg_err + EXP2_REL


def within(distance: np.ndarray, err: np.ndarray) -> np.ndarray:
    """True where a decision boundary lies within SAFETY times the error bound."""
    with np.errstate(invalid="ignore"):
        return np.asarray(distance) <= SAFETY * np.asarray(err)
