"""Parity metric between a computed tensor and its float64 reference.

Elementwise relative error is meaningless where the reference crosses zero, so each
element's error is scaled by |r| plus the tensor's root-mean-square:

    err_i = |g_i - r_i| / (|r_i| + rms(r)),   pass  iff  max_i err_i <= rtol

Tolerances: rtol = 1e-4 for float32 storage, 2e-2 for bfloat16 storage with a float32
state. The report also carries the raw maximum relative error over elements with
|r| >= 1e-2 * rms(r), and the normwise max|g - r| / max|r|.

A second, tighter bound (`watch`) catches regressions below the bf16 bar: a float32 result
within the float32 bar that is then rounded to nearest-even bf16 (8 significant bits, so the
rounding moves it by at most 2^-8 of its magnitude) stays within 2^-8 (1 + 1e-4) + 1e-4 on
the same metric. Where a test passes `watch`, exceeding it fails the check as well.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

RTOL = {"f32": 1e-4, "bf16": 2e-2}
# The state is float32 whatever the storage type and never rounded to bf16.
RTOL_STATE = 1e-4
# The rounding bound above, per storage type: results computed in float32 and stored in the
# storage type (not the Mamba-2 path, whose matrix-core operands are bf16 themselves).
WATCH = {"f32": RTOL["f32"], "bf16": 2.0**-8 * (1.0 + RTOL["f32"]) + RTOL["f32"]}


@dataclass
class ParityReport:
    err: float          # max |g-r| / (|r| + rms(r))
    max_rel: float      # max |g-r|/|r| over |r| >= 1e-2 rms(r)
    normwise: float     # max|g-r| / max|r|
    rtol: float
    worst_index: tuple
    count: int
    nonfinite_mismatch: int
    watch: float | None = None

    @property
    def ok(self) -> bool:
        return (self.nonfinite_mismatch == 0 and self.err <= self.rtol
                and (self.watch is None or self.err <= self.watch))

    def __str__(self) -> str:
        w = "" if self.watch is None or self.watch == self.rtol else f", watch {self.watch:.3e}"
        return (f"err={self.err:.3e} (rtol {self.rtol:.0e}{w}) max_rel={self.max_rel:.3e} "
                f"normwise={self.normwise:.3e} worst={self.worst_index} n={self.count} "
                f"nonfinite_mismatch={self.nonfinite_mismatch}")


def parity(got: np.ndarray, ref: np.ndarray, rtol: float,
           watch: float | None = None) -> ParityReport:
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    if r.size == 0:
        return ParityReport(0.0, 0.0, 0.0, rtol, (), 0, 0, watch)
    fin_g, fin_r = np.isfinite(g), np.isfinite(r)
    nonfinite_mismatch = int(np.count_nonzero(fin_g != fin_r))
    both = fin_g & fin_r
    gg, rr = np.where(both, g, 0.0), np.where(both, r, 0.0)
    rms = float(np.sqrt(np.mean(rr * rr))) if both.any() else 0.0
    diff = np.abs(gg - rr)
    denom = np.abs(rr) + rms
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(denom > 0, diff / np.where(denom > 0, denom, 1.0),
                     np.where(diff > 0, np.inf, 0.0))
    worst = int(np.argmax(e))
    big = np.abs(rr) >= 1e-2 * rms
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(big & (rr != 0), diff / np.where(rr != 0, np.abs(rr), 1.0), 0.0)
    mx = float(np.max(np.abs(rr)))
    return ParityReport(
        err=float(e.flat[worst]),
        max_rel=float(rel.max()) if rel.size else 0.0,
        normwise=float(diff.max() / mx) if mx > 0 else float(diff.max()),
        rtol=rtol,
        worst_index=tuple(int(i) for i in np.unravel_index(worst, r.shape)),
        count=int(r.size),
        nonfinite_mismatch=nonfinite_mismatch,
        watch=watch,
    )
