"""Plain CPU oracle for the backward pass of Sliding Tile Attention (STA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it is used by ``tests/`` and by ``bench.py``'s
``cpu_baseline`` leg.  It shares no code, tables or helpers with the HIP
library; the tile geometry comes from the forward oracle.

Why a backward at all: the pages report an end-to-end time after fine-tuning
with STA in place (index page, "Abstract"; gptget summary page, "Summary"
and "Experiments"), so the operator is trained through, and its gradients
are those of the forward definition.  The pages give no formula for them;
they follow from the chain rule applied to the forward oracle's definition,
written out here in float64:

  z_ij  = scale * q_i . k_j                 for permitted (i, j)
  lse_i = log sum_j exp(z_ij)               (row log-sum-exp, permitted j)
  P_ij  = exp(z_ij - lse_i)
  o_i   = sum_j P_ij v_j
  given G = dL/dO:
  dv_j  = sum_i P_ij G_i                    (over queries i that permit j)
  dP_ij = G_i . v_j
  dz_ij = P_ij * (dP_ij - sum_l P_il dP_il) (softmax Jacobian)
  dq_i  = scale * sum_j dz_ij k_j
  dk_j  = scale * sum_i dz_ij q_i

Readings R1-R5 of the forward oracle apply unchanged.  One more (numbered
as in the design notes):

  R10 The row log-sum-exp is reported in natural-log units over the
      permitted keys of the row, with the scale applied (lse_i above).

Parity pins (``tests/test_oracle_bwd_pins.py``): central finite differences
of <O, G> on small float64 problems, the dense and block-diagonal special
cases against torch's autograd of plain attention in float64, closed forms
(Q = 0 gives lse = log of the permitted-key count), invariants (the dv rows
sum to the dO rows' sum; the dk rows sum to zero), token-order equivariance,
and planted mistakes that the pins must catch.
"""

from __future__ import annotations

import itertools
import math
from typing import Iterable, Sequence

import numpy as np

from . import sta_oracle as F

__all__ = [
    "masked_attention_lse",
    "masked_attention_backward",
    "sta_backward_explicit",
    "sta_backward_query_tiles",
    "sta_backward_key_tiles",
    "query_tiles_seeing",
]


def masked_attention_lse(q: np.ndarray, k: np.ndarray, mask: np.ndarray, scale: float) -> np.ndarray:
    """Row log-sum-exp of the scaled scores over the permitted keys, [Nq]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    z = np.where(mask, scale * (q @ k.T), -np.inf)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def masked_attention_backward(q, k, v, g, mask, scale):
    """Gradients of <softmax attention(q, k, v), g> with respect to q, k, v.

    q [Nq, D], k [Nk, D], v [Nk, Dv], g [Nq, Dv], mask bool [Nq, Nk].
    Returns (o, lse, dq, dk, dv) in float64; masked pairs carry zero
    probability, so they contribute nothing anywhere.
    """
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    lse = masked_attention_lse(q, k, mask, scale)
    z = np.where(mask, scale * (q @ k.T), -np.inf)
    p = np.exp(z - lse[:, None])            # exp(-inf) = 0 off the mask
    o = p @ v
    dv = p.T @ g
    dp = g @ v.T
    dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (dz @ k)
    dk = scale * (dz.T @ q)
    return o, lse, dq, dk, dv


def sta_backward_explicit(q, k, v, g, video: Sequence[int], tile: Sequence[int], windows,
                          scale: float | None = None, coords: np.ndarray | None = None,
                          partial: bool = False):
    """STA forward and backward by the explicit N x N mask (small inputs).

    q, k, v, g: [B, heads, N, D]; token n sits at coords[n] (natural raster
    order when coords is None).  partial: extents need not be multiples of
    the tile (the forward oracle's reading R11: the last tile of an axis
    holds only the tokens that exist).  Returns a dict of float64 arrays:
    o, dq, dk, dv [B, heads, N, D] and lse [B, heads, N].
    """
    B, heads, N, D = q.shape
    grid = F.tile_grid(video, tile, partial)
    if coords is None:
        coords = F.natural_coords(video)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ws = F._as_windows(windows, heads)
    out = {name: np.empty((B, heads, N, D)) for name in ("o", "dq", "dk", "dv")}
    out["lse"] = np.empty((B, heads, N))
    for h in range(heads):
        mask = F.sta_mask(coords, coords, tile, ws[h], grid)
        for b in range(B):
            o, lse, dq, dk, dv = masked_attention_backward(q[b, h], k[b, h], v[b, h], g[b, h], mask, scale)
            out["o"][b, h], out["lse"][b, h] = o, lse
            out["dq"][b, h], out["dk"][b, h], out["dv"][b, h] = dq, dk, dv
    return out


def _tile_slice(x, c, tile, batch, head):
    tT, tH, tW = tile
    return x[batch, head, c[0] * tT:(c[0] + 1) * tT, c[1] * tH:(c[1] + 1) * tH,
             c[2] * tW:(c[2] + 1) * tW]


def _window_slice(x, c, tile, window, grid, batch, head):
    (t0, t1), (y0, y1), (z0, z1) = F.window_tiles(c, window, grid)
    tT, tH, tW = tile
    return x[batch, head, t0 * tT:t1 * tT, y0 * tH:y1 * tH, z0 * tW:z1 * tW]


def _rows(x):
    return np.asarray(x, dtype=np.float64).reshape(-1, x.shape[-1])


def sta_backward_query_tiles(q, k, v, g, tile, window, head: int,
                             query_tiles: Iterable[Sequence[int]], scale: float | None = None,
                             batch: int = 0, partial: bool = False):
    """lse and dq of selected query tiles of one head (large inputs).

    Inputs in natural layout [B, heads, T, H, W, D].  A query's gradient
    needs only its own window (the box of tokens of its key tiles).
    Returns a list of (lse [tT, tH, tW], dq [tT, tH, tW, D]) in float64
    (smaller for a partial tile: the slices stop at the video's end).
    """
    _, _, T, H, W, D = q.shape
    grid = F.tile_grid((T, H, W), tile, partial)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = []
    for c in query_tiles:
        qt, gt = _rows(_tile_slice(q, c, tile, batch, head)), _rows(_tile_slice(g, c, tile, batch, head))
        kw = _rows(_window_slice(k, c, tile, window, grid, batch, head))
        vw = _rows(_window_slice(v, c, tile, window, grid, batch, head))
        mask = np.ones((qt.shape[0], kw.shape[0]), dtype=bool)
        _, lse, dq, _, _ = masked_attention_backward(qt, kw, vw, gt, mask, scale)
        shape = _tile_slice(q, c, tile, batch, head).shape[:3]
        out.append((lse.reshape(shape), dq.reshape(*shape, D)))
    return out


def query_tiles_seeing(key_tile: Sequence[int], window: Sequence[int], grid: Sequence[int]):
    """All query tiles whose window contains key_tile, found by testing every
    tile of the grid (raster order)."""
    hits = []
    for c in itertools.product(range(grid[0]), range(grid[1]), range(grid[2])):
        box = F.window_tiles(c, window, grid)
        if all(box[d][0] <= key_tile[d] < box[d][1] for d in range(3)):
            hits.append(c)
    return hits


def sta_backward_key_tiles(q, k, v, g, tile, window, head: int,
                           key_tiles: Iterable[Sequence[int]], scale: float | None = None,
                           batch: int = 0, partial: bool = False):
    """dk and dv of selected key tiles of one head (large inputs).

    A key tile receives gradient from every query tile whose window holds
    it.  For each such query tile the row statistics (lse and
    sum_l P_il dP_il) are taken over that query tile's whole window; the
    probabilities and score gradients are then formed for the key tile's
    columns alone.  Returns a list of (dk, dv), each [tT, tH, tW, D]
    (smaller for a partial tile).
    """
    _, _, T, H, W, D = q.shape
    grid = F.tile_grid((T, H, W), tile, partial)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = []
    for kc in key_tiles:
        kt, vt = _rows(_tile_slice(k, kc, tile, batch, head)), _rows(_tile_slice(v, kc, tile, batch, head))
        dk = np.zeros_like(kt)
        dv = np.zeros_like(vt)
        for c in query_tiles_seeing(kc, window, grid):
            qt, gt = _rows(_tile_slice(q, c, tile, batch, head)), _rows(_tile_slice(g, c, tile, batch, head))
            kw = _rows(_window_slice(k, c, tile, window, grid, batch, head))
            vw = _rows(_window_slice(v, c, tile, window, grid, batch, head))
            zw = scale * (qt @ kw.T)
            m = zw.max(axis=1, keepdims=True)
            lse = m + np.log(np.exp(zw - m).sum(axis=1, keepdims=True))
            pw = np.exp(zw - lse)
            delta = (pw * (gt @ vw.T)).sum(axis=1, keepdims=True)
            p = np.exp(scale * (qt @ kt.T) - lse)
            dz = p * (gt @ vt.T - delta)
            dv += p.T @ gt
            dk += scale * (dz.T @ qt)
        shape = _tile_slice(k, kc, tile, batch, head).shape[:3]
        out.append((dk.reshape(*shape, D), dv.reshape(*shape, D)))
    return out
