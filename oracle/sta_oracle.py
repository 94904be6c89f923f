"""Plain CPU oracle for the forward pass of Sliding Tile Attention (STA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
(to check one small GPU call) and by the ``cpu_baseline`` leg of
``bench.py``.  It shares no code, tables or helpers with the HIP library.

What it computes (sources: "Fast Video Generation with Sliding Tile
Attention", arXiv 2502.04507 -- index page, section "Abstract"; gptget summary
page, sections "Methodology", "Technical Contribution" and "Novelty"):

  * The T x H x W video latent is cut into non-overlapping 3D tiles.
  * Each query tile attends to every token of every key/value tile that lies
    inside its 3D window, and to nothing else; the window moves tile by tile,
    so a (query tile, key tile) pair is either fully attended or fully
    skipped ("no mixed blocks").
  * The window size (in tiles, per axis) is chosen per attention head.
  * Inside the permitted set the operation is ordinary softmax attention.

STA therefore reaches, exactly up to floating-point rounding order, the
result of explicit masked softmax attention with a tile-aligned mask.  This
oracle is that definition written out, in float64:

  o(x) = sum_j softmax_j(scale * q(x).k_j  over permitted j) * v_j

Readings taken where the pages are silent (each is also listed in the
design notes of the repository):

  R1  Window units are tiles; a window larger than the tile grid on an axis
      is clamped to the grid (w' = min(w, n)).
  R2  Borders shift the window inward: the window of query tile c on an axis
      with n tiles starts at clamp(c - floor((w'-1)/2), 0, n - w'), so every
      query tile sees exactly prod(w') key tiles.  For an even w' the extra
      tile falls on the high side.
  R3  No causal mask, bias, dropout or extra (text) tokens.
  R4  scale defaults to 1/sqrt(head_dim).
  R5  Inputs are taken exactly as given (for bf16 workloads: the bf16 values,
      widened); all arithmetic here is float64.
  R11 (Only when asked for, ``partial=True``.)  An extent that is not a
      multiple of its tile size gets ceil(extent / tile) tiles; the last tile
      on that axis is partial.  Tile coordinates, windows and the tile-level
      mask are unchanged; only tokens that exist take part.  This equals
      padding the video to whole tiles and masking the padded keys.

Parity pins: every function below is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (brute force, dense / block-diagonal special
cases against a library attention routine, closed forms and invariants) and
by the hand-derived fixtures under ``tests/golden/``.
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

__all__ = [
    "tile_grid",
    "effective_window",
    "window_start",
    "permitted",
    "natural_coords",
    "sta_mask",
    "masked_softmax_attention",
    "sta_forward_explicit",
    "sta_forward_query_tiles",
    "window_tiles",
    "sta_flops",
]


# ---------------------------------------------------------------------------
# Tile geometry (gptget page, "Methodology": the video is partitioned into
# non-overlapping tiles and attention is done in local windows at tile level).
# ---------------------------------------------------------------------------

def tile_grid(video: Sequence[int], tile: Sequence[int], partial: bool = False) -> tuple[int, int, int]:
    """Number of tiles along (T, H, W).  Tiles do not overlap and cover the
    video, so every extent must be a multiple of its tile size -- unless
    partial is set (reading R11): then an axis has ceil(extent / tile) tiles
    and its last tile holds only the tokens that exist."""
    if len(video) != 3 or len(tile) != 3:
        raise ValueError("video and tile must have three axes (T, H, W)")
    out = []
    for e, t in zip(video, tile):
        if t <= 0 or e <= 0 or (e % t != 0 and not partial):
            raise ValueError(f"extent {e} is not a positive multiple of tile {t}")
        out.append(-(-e // t))
    return tuple(out)


def effective_window(window: Sequence[int], grid: Sequence[int]) -> tuple[int, int, int]:
    """Reading R1: a window wider than the grid is clamped to the grid."""
    if any(w < 1 for w in window):
        raise ValueError("window extents must be >= 1 tile")
    return tuple(min(int(w), int(n)) for w, n in zip(window, grid))


def window_start(c: int, w: int, n: int) -> int:
    """Reading R2: first tile of the w-tile window of query tile c on an axis of
    n tiles (w <= n): centred on c, shifted inward at the borders."""
    s = c - (w - 1) // 2
    if s < 0:
        s = 0
    if s > n - w:
        s = n - w
    return s


def permitted(qx: Sequence[int], kx: Sequence[int], tile: Sequence[int],
              window: Sequence[int], grid: Sequence[int]) -> bool:
    """Token-level predicate: may the query token at (t, y, z) = qx attend to
    the key token at kx?  True iff, on every axis, the key's tile lies inside
    the window of the query's tile."""
    w = effective_window(window, grid)
    for d in range(3):
        cq = qx[d] // tile[d]
        ck = kx[d] // tile[d]
        s = window_start(cq, w[d], grid[d])
        if not (s <= ck < s + w[d]):
            return False
    return True


def natural_coords(video: Sequence[int]) -> np.ndarray:
    """(t, y, z) of every token in natural raster order (z fastest), [N, 3]."""
    T, H, W = video
    t, y, z = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), z.ravel()], axis=1).astype(np.int64)


def sta_mask(coords_q: np.ndarray, coords_k: np.ndarray, tile: Sequence[int],
             window: Sequence[int], grid: Sequence[int]) -> np.ndarray:
    """The predicate ``permitted`` evaluated for every (query, key) token pair,
    from token coordinates alone: bool [Nq, Nk]."""
    w = effective_window(window, grid)
    ok = np.ones((coords_q.shape[0], coords_k.shape[0]), dtype=bool)
    for d in range(3):
        cq = coords_q[:, d] // tile[d]
        ck = coords_k[:, d] // tile[d]
        s = np.clip(cq - (w[d] - 1) // 2, 0, grid[d] - w[d])
        ok &= (ck[None, :] >= s[:, None]) & (ck[None, :] < s[:, None] + w[d])
    return ok


# ---------------------------------------------------------------------------
# Attention (index page, "Abstract": STA replaces 3D full attention by
# attention over the local window; inside it the operation is softmax
# attention).
# ---------------------------------------------------------------------------

def masked_softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                             mask: np.ndarray, scale: float) -> np.ndarray:
    """Explicit masked softmax attention in float64.

    q [Nq, D], k [Nk, D], v [Nk, Dv], mask bool [Nq, Nk] (every row must
    permit at least one key).  Masked scores are set to -inf, so they get
    weight exp(-inf) = 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if not mask.any(axis=1).all():
        raise ValueError("a query row has no permitted key")
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def _as_windows(windows, heads: int) -> list[tuple[int, int, int]]:
    ws = [tuple(int(x) for x in w) for w in windows]
    if len(ws) == 1 and heads > 1:
        ws = ws * heads
    if len(ws) != heads:
        raise ValueError("need one window per head")
    return ws


def sta_forward_explicit(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                         video: Sequence[int], tile: Sequence[int], windows,
                         scale: float | None = None,
                         coords: np.ndarray | None = None, partial: bool = False) -> np.ndarray:
    """STA forward by the explicit N x N mask (small inputs only).

    q, k, v: [B, heads, N, D]; token n sits at coords[n] = (t, y, z)
    (natural raster order when coords is None, so that any token order can
    be checked).  windows: one (wT, wH, wW) per head, in tiles.
    Returns float64 [B, heads, N, D].
    """
    B, heads, N, D = q.shape
    grid = tile_grid(video, tile, partial)
    if coords is None:
        coords = natural_coords(video)
    if coords.shape[0] != N:
        raise ValueError("coords do not match the token count")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ws = _as_windows(windows, heads)
    out = np.empty((B, heads, N, v.shape[-1]), dtype=np.float64)
    for h in range(heads):
        mask = sta_mask(coords, coords, tile, ws[h], grid)
        for b in range(B):
            out[b, h] = masked_softmax_attention(q[b, h], k[b, h], v[b, h], mask, scale)
    return out


def window_tiles(c: Sequence[int], window: Sequence[int], grid: Sequence[int]):
    """Per-axis tile ranges [(s, s + w')] of the window of query tile c."""
    w = effective_window(window, grid)
    return [(window_start(c[d], w[d], grid[d]), window_start(c[d], w[d], grid[d]) + w[d])
            for d in range(3)]


def sta_forward_query_tiles(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                            tile: Sequence[int], window: Sequence[int], head: int,
                            query_tiles: Iterable[Sequence[int]],
                            scale: float | None = None, batch: int = 0,
                            partial: bool = False) -> list[np.ndarray]:
    """STA forward for selected query tiles of one head (large inputs).

    q, k, v are in natural layout [B, heads, T, H, W, D] (any float dtype,
    widened to float64).  All queries of a tile share one permitted set --
    the tokens of the window's key tiles -- which, because the window is a
    box of tiles on each axis, is the box of tokens
    [s_t*tT, (s_t+w_t)*tT) x [s_y*tH, ...) x [s_z*tW, ...).
    Returns, per query tile, float64 [tT, tH, tW, D] in natural order
    (smaller for a partial tile, reading R11: slices stop at the video's end).
    """
    _, _, T, H, W, D = q.shape
    grid = tile_grid((T, H, W), tile, partial)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    tT, tH, tW = tile
    outs = []
    for c in query_tiles:
        (t0, t1), (y0, y1), (z0, z1) = window_tiles(c, window, grid)
        qt = q[batch, head, c[0] * tT:(c[0] + 1) * tT, c[1] * tH:(c[1] + 1) * tH,
               c[2] * tW:(c[2] + 1) * tW].reshape(-1, D)
        kt = k[batch, head, t0 * tT:t1 * tT, y0 * tH:y1 * tH, z0 * tW:z1 * tW].reshape(-1, D)
        vt = v[batch, head, t0 * tT:t1 * tT, y0 * tH:y1 * tH, z0 * tW:z1 * tW]
        vt = vt.reshape(-1, vt.shape[-1])
        mask = np.ones((qt.shape[0], kt.shape[0]), dtype=bool)
        o = masked_softmax_attention(np.asarray(qt, np.float64), np.asarray(kt, np.float64),
                                     np.asarray(vt, np.float64), mask, scale)
        outs.append(o.reshape(*q[batch, head, c[0] * tT:(c[0] + 1) * tT, c[1] * tH:(c[1] + 1) * tH,
                                  c[2] * tW:(c[2] + 1) * tW].shape[:3], -1))
    return outs


def sta_flops(video: Sequence[int], tile: Sequence[int], windows, head_dim: int,
              batch: int = 1) -> int:
    """Algorithmic FLOPs of one forward call, counting only attended tile
    pairs: 4 * V^2 * D per (query tile, key tile) pair (two products at
    2 FLOP per multiply-add), V = tokens per tile."""
    grid = tile_grid(video, tile)
    V = tile[0] * tile[1] * tile[2]
    total = 0
    for w in windows:
        we = effective_window(w, grid)
        total += grid[0] * grid[1] * grid[2] * we[0] * we[1] * we[2]
    return 4 * V * V * head_dim * total * batch
