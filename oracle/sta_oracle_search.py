"""Plain CPU oracle for the per-head window search of Sliding Tile Attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it is used by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg.  It shares no code with the HIP library; the
attention itself comes from the forward oracle.

What the pages say (index page, "Abstract"; gptget summary page,
"Methodology", "Technical Contribution", "Novelty" and "Limitations"): the
window size of every attention head is configured automatically, from
profiling the locality of that head's attention, trading efficiency against
quality.  They give no formula.  The plainest reading, taken here:

  W1  Profiling = comparing, on calibration inputs, each head's STA output
      under a candidate window with the head's full-attention output.
  W2  The error of candidate c for head h is the relative Frobenius error
      ||O_c - O_full|| / ||O_full|| over all batch elements, tokens and
      channels of that head.
  W3  A head gets the cheapest candidate whose error is at most a threshold
      tau; cost is the number of attended key tiles per query tile,
      prod(min(w, n)); ties go to the smaller error, then to the earlier
      candidate.  If no candidate meets tau, the head gets the full window
      (the grid), whose error is zero by definition.
  W4  Several calibration inputs: their per-(head, candidate) errors are
      averaged before the choice.

Parity pins (``tests/test_oracle_search_pins.py``): a window covering the
grid has error exactly zero; a constant V makes every error zero (the
cheapest window wins); attention confined to a query's own tile makes the
1x1x1 window exact; the choice is checked against a brute-force scan of all
candidates; on a grid with partial tiles, the full window is exact and a
candidate's error matches one computed against dense attention over the
existing tokens; planted mistakes must fail a pin.
"""

from __future__ import annotations

import math
from typing import Sequence

import numpy as np

from . import sta_oracle as F

__all__ = ["window_cost", "window_errors", "select_windows", "odd_candidates", "search"]


def window_cost(window: Sequence[int], grid: Sequence[int]) -> int:
    """Attended key tiles per query tile (reading W3)."""
    we = F.effective_window(window, grid)
    return we[0] * we[1] * we[2]


def odd_candidates(grid: Sequence[int]) -> list[tuple[int, int, int]]:
    """Centred windows: on each axis every odd extent below the axis length
    plus the whole axis, in raster order."""
    axes = []
    for n in grid:
        vals = [w for w in range(1, n, 2)] + [n]
        axes.append(vals)
    return [(a, b, c) for a in axes[0] for b in axes[1] for c in axes[2]]


def window_errors(q, k, v, video: Sequence[int], tile: Sequence[int], candidates,
                  scale: float | None = None, partial: bool = False) -> np.ndarray:
    """err[h, c] = ||O_c - O_full|| / ||O_full|| for head h (reading W2).

    q, k, v: [B, heads, N, D] (natural order), any float dtype (widened to
    float64).  Uses the explicit forward oracle; small inputs only.
    partial: extents need not be multiples of the tile (the forward
    oracle's reading R11: ceil(extent / tile) tiles per axis, only existing
    tokens take part); O_full is then attention over every existing token."""
    B, heads, N, D = q.shape
    grid = F.tile_grid(video, tile, partial)
    full = F.sta_forward_explicit(q, k, v, video, tile, [grid] * heads, scale=scale, partial=partial)
    err = np.zeros((heads, len(candidates)))
    for c, w in enumerate(candidates):
        o = F.sta_forward_explicit(q, k, v, video, tile, [tuple(w)] * heads, scale=scale, partial=partial)
        for h in range(heads):
            num = math.sqrt(float(((o[:, h] - full[:, h]) ** 2).sum()))
            den = math.sqrt(float((full[:, h] ** 2).sum()))
            err[h, c] = num / den
    return err


def select_windows(err: np.ndarray, candidates, grid: Sequence[int], threshold: float):
    """Per head, the cheapest candidate with err <= threshold (reading W3);
    err may be the mean over several calibration inputs (W4)."""
    out = []
    for h in range(err.shape[0]):
        best = None
        for c, w in enumerate(candidates):
            if not err[h, c] <= threshold:
                continue
            key = (window_cost(w, grid), err[h, c], c)
            if best is None or key < best[0]:
                best = (key, tuple(int(x) for x in w))
        out.append(best[1] if best is not None else tuple(int(n) for n in grid))
    return out


def search(samples, video: Sequence[int], tile: Sequence[int], candidates, threshold: float,
           scale: float | None = None, partial: bool = False):
    """Readings W1-W4 over several calibration inputs: each sample's
    per-(head, candidate) errors (W1, W2), their arithmetic mean over the
    samples (W4), and the choice from the mean (W3).  samples: sequence of
    (q, k, v), each [B, heads, N, D].  partial: as in window_errors.
    Returns (windows, mean errors)."""
    errs = [window_errors(q, k, v, video, tile, candidates, scale=scale, partial=partial) for q, k, v in samples]
    if not errs:
        raise ValueError("no calibration samples")
    mean = np.zeros_like(errs[0])
    for e in errs:
        mean += e
    mean /= len(errs)
    return select_windows(mean, candidates, F.tile_grid(video, tile, partial), threshold), mean
