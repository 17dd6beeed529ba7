"""Per-element acceptance of a bfloat16 GPU output against the oracle (test infrastructure only).

Strict band: |gpu - oracle| <= 2e-3 + 2e-2 * |oracle|, elements compared by
value (so +0 equals -0).

Where the exact result sits at a bfloat16 rounding tie of h, or the output
cancels to near zero, more than one result is correct for an fp32-accumulating
implementation: a rounding of h that lands on the other side of a tie, or fp32
sum-order differences of the size 2^-20 of the contraction's L1 mass. The pages
accept such results: their checks compare hardware summation orders with an f64
oracle inside a band [bloomery 0.3.9 release notes, New, Metal tensor ops], and
they widen a check to the range a kernel can legitimately produce rather than
reject a correct finite value [FP4-Local checkpoints on DGX Spark, §10, #704].
Those elements are "explained" when

    |gpu - oracle| <= strict + slack_h + 2^-20 * mass + ulp_bf16(oracle)

and reported separately; anything beyond is a FAIL. The 2^-20 share is for fp32
accumulation rounded to nearest; a path whose accumulation rounds otherwise passes its
own share (mass_rel), derived from that arithmetic: K additions rounded toward zero
err by at most K * 2^-23 of the mass (the worst case of recursive summation with a
one-ulp error per addition).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats as F

ATOL = 2e-3
RTOL = 2e-2
MASS_REL = 2.0 ** -20


def directed_sum_share(K: int) -> float:
    """Share of the mass that K fp32 additions rounded toward zero (one ulp each, 2^-23
    relative) can err by, with 64 more for the combination of partial sums."""
    return (K + 64) * 2.0 ** -23


@dataclass
class BandReport:
    n: int
    strict: int
    explained: int
    fail: int
    worst_excess: float       # max (|diff| - explained bound) over failing elements, else <= 0

    def ok(self) -> bool:
        return self.fail == 0

    def __str__(self):
        return (f"n={self.n} strict={self.strict} explained={self.explained} "
                f"fail={self.fail} worst_excess={self.worst_excess:.3g}")


def classify(gpu_bits, ref_bits, mass=None, slack=None, mass_rel=MASS_REL) -> BandReport:
    """Classify each GPU bfloat16 element (bits) against the oracle's rounded
    output (bits), with optional per-element mass and slack_h (float64). `mass_rel` is
    the share of the mass the accumulation may err by: 2^-20 (fp32 sums rounded to
    nearest in any order) unless a path's arithmetic fixes another."""
    g = F.bf16_bits_to_f64(np.asarray(gpu_bits, dtype=np.uint16))
    r = F.bf16_bits_to_f64(np.asarray(ref_bits, dtype=np.uint16))
    diff = np.abs(g - r)
    diff = np.where(np.isnan(diff), np.inf, diff)
    strict_bound = ATOL + RTOL * np.abs(r)
    strict = diff <= strict_bound
    bound = strict_bound + F.bf16_ulp(r)
    if mass is not None:
        bound = bound + mass_rel * np.asarray(mass)
    if slack is not None:
        bound = bound + np.asarray(slack)
    expl = (~strict) & (diff <= bound)
    fail = ~(strict | expl)
    worst = float(np.max(diff[fail] - bound[fail])) if fail.any() else float(np.max(diff - bound, initial=-np.inf))
    return BandReport(int(diff.size), int(strict.sum()), int(expl.sum()), int(fail.sum()), worst)


def classify_f32(gpu_f32, ref_f64, mass=None, slack=None) -> BandReport:
    """Same rule for unrounded fp32 intermediates (the expert rows): no final
    bfloat16 ulp term."""
    g = np.asarray(gpu_f32, dtype=np.float64)
    r = np.asarray(ref_f64, dtype=np.float64)
    diff = np.abs(g - r)
    diff = np.where(np.isnan(diff), np.inf, diff)
    strict_bound = ATOL + RTOL * np.abs(r)
    strict = diff <= strict_bound
    bound = strict_bound.copy()
    if mass is not None:
        bound = bound + MASS_REL * np.asarray(mass)
    if slack is not None:
        bound = bound + np.asarray(slack)
    expl = (~strict) & (diff <= bound)
    fail = ~(strict | expl)
    worst = float(np.max(diff[fail] - bound[fail])) if fail.any() else float(np.max(diff - bound, initial=-np.inf))
    return BandReport(int(diff.size), int(strict.sum()), int(expl.sum()), int(fail.sum()), worst)
