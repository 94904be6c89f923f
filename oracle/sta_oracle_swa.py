"""Plain CPU oracle for token-wise 3D sliding window attention (SWA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it is used by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg.  It shares no code with the HIP library.

What it is (index page, "Abstract"; gptget summary page, "Methodology",
"Technical Contribution" and "Novelty"): the baseline STA is contrasted with.
In token-wise SWA every query token has its own window of keys centred on
itself, so the windows of neighbouring queries differ and a block of
queries against a block of keys is often partly permitted ("mixed blocks"),
which costs a kernel masks and irregular access; STA moves the window tile
by tile instead.  The pages give no border rule or window shape for SWA;
reading taken here (S1), mirroring STA's readings R1 and R2 at token level:

  S1  The window of query token x on an axis of extent E is w' = min(w, E)
      tokens starting at clamp(x - floor((w'-1)/2), 0, E - w'): centred on
      the query, shifted inward at the borders, so every query sees exactly
      prod(w') keys.  Inside the window: ordinary softmax attention, float64.

With 1x1x1 tiles STA and SWA coincide (a tile is a token), which the pins
use.  Pins (``tests/test_oracle_swa_pins.py``): brute force by nested loops
per query, the dense case against torch's float64 attention, a 1x1x1 window
returning V itself, equality with the STA oracle for 1x1x1 tiles, the
per-query-tile form against the explicit one, planted mistakes.
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

from . import sta_oracle as F

__all__ = ["token_window_start", "swa_mask", "swa_forward_explicit", "swa_forward_query_tiles",
           "swa_union_box"]


def token_window_start(x: int, w: int, e: int) -> int:
    """Reading S1: first token of the window of query coordinate x on an
    axis of extent e (w already clamped to e)."""
    s = x - (w - 1) // 2
    return min(max(s, 0), e - w)


def swa_mask(video: Sequence[int], window: Sequence[int]) -> np.ndarray:
    """bool [N, N]: may query token n attend to key token m (natural order)."""
    coords = F.natural_coords(video)
    ok = np.ones((coords.shape[0], coords.shape[0]), dtype=bool)
    for d in range(3):
        w = min(int(window[d]), int(video[d]))
        s = np.clip(coords[:, d] - (w - 1) // 2, 0, video[d] - w)
        ok &= (coords[None, :, d] >= s[:, None]) & (coords[None, :, d] < s[:, None] + w)
    return ok


def swa_forward_explicit(q, k, v, video: Sequence[int], windows, scale: float | None = None):
    """Token-wise SWA by the explicit N x N mask (small inputs).
    q, k, v: [B, heads, N, D] in natural order; windows: one (wT, wH, wW) per
    head, in tokens.  Returns float64 [B, heads, N, D]."""
    B, heads, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ws = F._as_windows(windows, heads)
    out = np.empty((B, heads, N, v.shape[-1]))
    for h in range(heads):
        mask = swa_mask(video, ws[h])
        for b in range(B):
            out[b, h] = F.masked_softmax_attention(q[b, h], k[b, h], v[b, h], mask, scale)
    return out


def swa_union_box(c: Sequence[int], tile: Sequence[int], window: Sequence[int], video: Sequence[int]):
    """Per axis, the token range [lo, hi) covered by the windows of all
    queries of tile c (the keys a tile of queries can need)."""
    box = []
    for d in range(3):
        w = min(int(window[d]), int(video[d]))
        x0 = c[d] * tile[d]
        x1 = min(x0 + tile[d], video[d]) - 1
        box.append((token_window_start(x0, w, video[d]), token_window_start(x1, w, video[d]) + w))
    return box


def swa_forward_query_tiles(q, k, v, tile: Sequence[int], window: Sequence[int], head: int,
                            query_tiles: Iterable[Sequence[int]], scale: float | None = None,
                            batch: int = 0) -> list[np.ndarray]:
    """Token-wise SWA outputs of selected query tiles of one head (large
    inputs).  Inputs in natural layout [B, heads, T, H, W, D]; each query
    tile's keys are gathered from the union of its queries' windows and each
    query is masked to its own window.  Returns float64 [tT, tH, tW, D] per
    tile."""
    _, _, T, H, W, D = q.shape
    video = (T, H, W)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    outs = []
    for c in query_tiles:
        (t0, t1), (y0, y1), (z0, z1) = swa_union_box(c, tile, window, video)
        sl = tuple(slice(c[d] * tile[d], (c[d] + 1) * tile[d]) for d in range(3))
        qt = np.asarray(q[batch, head][sl], np.float64)
        shape = qt.shape[:3]
        qt = qt.reshape(-1, D)
        kt = np.asarray(k[batch, head, t0:t1, y0:y1, z0:z1], np.float64).reshape(-1, D)
        vt = np.asarray(v[batch, head, t0:t1, y0:y1, z0:z1], np.float64)
        vt = vt.reshape(-1, vt.shape[-1])
        qc = np.stack(np.meshgrid(*(np.arange(s.start, s.start + n) for s, n in zip(sl, shape)),
                                  indexing="ij"), axis=-1).reshape(-1, 3)
        kc = np.stack(np.meshgrid(np.arange(t0, t1), np.arange(y0, y1), np.arange(z0, z1),
                                  indexing="ij"), axis=-1).reshape(-1, 3)
        mask = np.ones((qc.shape[0], kc.shape[0]), dtype=bool)
        for d in range(3):
            w = min(int(window[d]), int(video[d]))
            s = np.clip(qc[:, d] - (w - 1) // 2, 0, video[d] - w)
            mask &= (kc[None, :, d] >= s[:, None]) & (kc[None, :, d] < s[:, None] + w)
        o = F.masked_softmax_attention(qt, kt, vt, mask, scale)
        outs.append(o.reshape(*shape, -1))
    return outs
