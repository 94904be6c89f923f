"""Seeded synthetic STA workloads: shapes, windows and value distributions.

This module holds no attention arithmetic.  It only draws inputs, and it is
the one module that both the HIP path's callers (tests, bench, smoke) and
the CPU oracle's callers share.  The video shape (30, 48, 80) of the larger
workloads is the 720p, 5-second latent named on the gptget summary page
("Experiments"); there are no real activations here, so Q, K and V are
N(0, 1) draws of that shape instead.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "make_qkv", "make_grad_out", "make_local_qkv", "sample_query_tiles",
           "tile_count"]


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                      # seed = 1000 * index
    video: tuple                    # (T, H, W) tokens
    tile: tuple                     # (tT, tH, tW) tokens
    windows: tuple                  # one (wT, wH, wW) per head, in tiles
    head_dim: int
    dtype: str                      # "f32" or "bf16": dtype of Q, K, V
    batch: int = 1
    magnitude: tuple | None = None  # per-token magnitude range (lo, hi)
    description: str = field(default="", compare=False)

    @property
    def heads(self) -> int:
        return len(self.windows)

    @property
    def seed(self) -> int:
        return 1000 * self.index

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def tokens(self) -> int:
        return self.video[0] * self.video[1] * self.video[2]

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_heads(self, heads: int) -> "Workload":
        ws = tuple(self.windows[h % len(self.windows)] for h in range(heads))
        return Workload(self.name, self.index, self.video, self.tile, ws, self.head_dim,
                        self.dtype, self.batch, self.magnitude, self.description)


_MIXED = ((1, 1, 1), (3, 3, 3), (3, 5, 5), (5, 6, 10))

WORKLOADS = {
    "tiny": Workload("tiny", 1, (6, 16, 16), (2, 4, 4), ((3, 3, 3),) * 2, 64, "f32",
                     description="6x16x16 latent, tile 2x4x4, window 3x3x3, 2 heads, d64, fp32"),
    # head_dim 128 with 64-token tiles: the kernels' one-wave (generic)
    # variants at the larger head size.
    "generic-d128": Workload("generic-d128", 13, (8, 16, 16), (2, 4, 8), ((3, 3, 3), (1, 4, 2)), 128,
                             "bf16", description="8x16x16 latent, tile 2x4x8 (64 tokens), windows "
                                                 "3x3x3 and 1x4x2, 2 heads, d128, bf16"),
    "generic-d128-f32": Workload("generic-d128-f32", 14, (8, 16, 16), (2, 4, 8), ((3, 3, 3), (2, 1, 2)),
                                 128, "f32", description="8x16x16 latent, tile 2x4x8 (64 tokens), "
                                                         "windows 3x3x3 and 2x1x2, 2 heads, d128, fp32"),
    "small": Workload("small", 2, (12, 24, 24), (6, 8, 8), ((3, 3, 3),) * 8, 128, "bf16",
                      description="12x24x24 latent, tile 6x8x8, window 3x3x3 (covers the grid), "
                                  "8 heads, d128, bf16"),
    "720p": Workload("720p", 3, (30, 48, 80), (6, 8, 8), ((3, 3, 3),) * 24, 128, "bf16",
                     description="30x48x80 latent (115200 tokens), tile 6x8x8, window 3x3x3, "
                                 "24 heads, d128, bf16"),
    "mixed": Workload("mixed", 4, (30, 48, 80), (6, 8, 8),
                      tuple(_MIXED[h % 4] for h in range(24)), 128, "bf16",
                      description="30x48x80 latent, tile 6x8x8, 24 heads with windows cycling "
                                  "1x1x1, 3x3x3, 3x5x5, 5x6x10, d128, bf16"),
    "long": Workload("long", 5, (60, 48, 80), (6, 8, 8), ((3, 3, 3),) * 24, 128, "bf16",
                     magnitude=(0.5, 4.0),
                     description="60x48x80 latent (230400 tokens), tile 6x8x8, window 3x3x3, "
                                 "24 heads, d128, bf16, per-token magnitude U(0.5, 4)"),
    # Extents that are not multiples of the tile (partial tiles at the far
    # edges): the exact 720p latent (720 / 16 = 45 rows) and a small case
    # with partial tiles on every axis.
    "720p-exact": Workload("720p-exact", 8, (30, 45, 80), (6, 8, 8), ((3, 3, 3),) * 24, 128, "bf16",
                           description="30x45x80 latent (108000 tokens), tile 6x8x8 (last row of "
                                       "tiles holds 5 of 8 rows), window 3x3x3, 24 heads, d128, bf16"),
    "partial-small": Workload("partial-small", 9, (5, 13, 11), (2, 4, 4), ((3, 3, 3), (1, 2, 5)), 64,
                              "f32", description="5x13x11 latent, tile 2x4x4 (partial on every "
                                                 "axis), windows 3x3x3 and 1x2x5, 2 heads, d64, fp32"),
    # Token-wise sliding window attention (the baseline STA is contrasted
    # with): windows in TOKENS; tiles only group queries into work items.
    # 18x24x24 tokens = the key count of STA's 3x3x3 window of 6x8x8 tiles.
    "swa-720p": Workload("swa-720p", 10, (30, 48, 80), (6, 8, 8), ((18, 24, 24),) * 24, 128, "bf16",
                         description="token-wise SWA: 30x48x80 latent, window 18x24x24 tokens "
                                     "(10368 keys per query), 24 heads, d128, bf16"),
    "swa-small": Workload("swa-small", 11, (12, 24, 24), (6, 8, 8), ((9, 12, 12), (5, 24, 7)) * 2, 128,
                          "bf16", description="token-wise SWA: 12x24x24 latent, windows 9x12x12 and "
                                              "5x24x7 tokens, 4 heads, d128, bf16"),
    "swa-tiny": Workload("swa-tiny", 12, (6, 16, 16), (2, 4, 4), ((5, 7, 9), (3, 3, 3)), 64, "f32",
                         description="token-wise SWA: 6x16x16 latent, windows 5x7x9 and 3x3x3 tokens, "
                                     "2 heads, d64, fp32"),
    # 2D STA (an image latent: T = 1, tiles of one frame)
    "2d": Workload("2d", 6, (1, 96, 96), (1, 16, 24), ((1, 3, 3),) * 8, 128, "bf16",
                   description="2D: 96x96 latent, tile 16x24 (384 tokens), window 3x3 tiles, "
                               "8 heads, d128, bf16"),
    "2d-fine": Workload("2d-fine", 7, (1, 128, 128), (1, 8, 8),
                        ((1, 5, 5), (1, 3, 3), (1, 9, 9), (1, 1, 1)), 64, "bf16",
                        description="2D: 128x128 latent, tile 8x8, windows 5x5, 3x3, 9x9, 1x1 "
                                    "tiles, 4 heads, d64, bf16"),
}


def tile_count(w: Workload) -> tuple[int, int, int]:
    return tuple(e // t for e, t in zip(w.video, w.tile))


def make_qkv(w: Workload, device: str | torch.device = "cpu"):
    """Q, K, V in natural layout [B, heads, T, H, W, D], drawn from one
    generator seeded with 1000 * index on ``device``: Q, K, V ~ N(0, 1) in
    that order, then (if the workload has one) a per-token magnitude
    m ~ U(lo, hi) of shape [B, T, H, W] for each of Q, K, V, shared across
    heads and channels.  Finally cast (round to nearest even) to the
    workload's dtype.  Values depend on the device's generator; callers pass
    the very same tensors to both sides of a comparison."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    T, H, W = w.video
    shape = (w.batch, w.heads, T, H, W, w.head_dim)
    out = []
    for _ in range(3):
        out.append(torch.randn(shape, generator=g, device=dev, dtype=torch.float32))
    if w.magnitude is not None:
        lo, hi = w.magnitude
        for i in range(3):
            m = torch.empty((w.batch, 1, T, H, W, 1), device=dev, dtype=torch.float32)
            m.uniform_(lo, hi, generator=g)
            out[i].mul_(m)
    return tuple(x.to(w.torch_dtype) for x in out)


def make_grad_out(w: Workload, device: str | torch.device = "cpu"):
    """The upstream gradient dL/dO for backward runs, natural layout
    [B, heads, T, H, W, D]: N(0, 1) from a generator seeded with
    1000 * index + 500 on ``device``, cast to the workload's dtype.  The
    pages fine-tune on real videos; a unit normal stands in for that
    gradient."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 500)
    T, H, W = w.video
    x = torch.randn((w.batch, w.heads, T, H, W, w.head_dim), generator=g, device=dev,
                    dtype=torch.float32)
    return x.to(w.torch_dtype)


def make_local_qkv(video, lengths, head_dim: int, batch: int = 1, sharpness: float = 8.0,
                   noise: float = 0.1, seed: int = 0, dtype=torch.bfloat16,
                   device: str | torch.device = "cpu"):
    """Calibration inputs whose attention is local, one length scale per head.

    The pages profile the locality of trained heads; with no trained model
    here, head h gets queries and keys built from random Fourier features of
    the token coordinates p = (t, y, z):
        phi_h(p) = sqrt(2 / D) cos(W_h p + b_h),  W_h ~ N(0, I / l_h^2),
        b_h ~ U(0, 2 pi),
    q = sharpness * sqrt(D) * phi_h(p) + noise * N(0, 1),
    k = phi_h(p) + noise * N(0, 1),  v ~ N(0, 1),
    so that at scale 1/sqrt(D) a query's score for a key is about sharpness
    times a Gaussian of their distance with width l_h tokens, and the head
    attends to roughly its l_h-neighbourhood.  Shapes [B, heads, T, H, W, D]
    in natural order; one generator seeded with ``seed`` on ``device``."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    T, H, W = video
    heads = len(lengths)
    t, y, z = torch.meshgrid(torch.arange(T, device=dev), torch.arange(H, device=dev),
                             torch.arange(W, device=dev), indexing="ij")
    pos = torch.stack([t, y, z], dim=-1).reshape(-1, 3).float()          # [N, 3]
    qs, ks = [], []
    for h in range(heads):
        w = torch.randn((3, head_dim), generator=g, device=dev) / float(lengths[h])
        b = torch.rand((head_dim,), generator=g, device=dev) * (2 * math.pi)
        phi = math.sqrt(2.0 / head_dim) * torch.cos(pos @ w + b)          # [N, D]
        qs.append(phi * (sharpness * math.sqrt(head_dim)))
        ks.append(phi)
    q = torch.stack(qs).unsqueeze(0).expand(batch, -1, -1, -1).clone()
    k = torch.stack(ks).unsqueeze(0).expand(batch, -1, -1, -1).clone()
    q += noise * torch.randn(q.shape, generator=g, device=dev)
    k += noise * torch.randn(k.shape, generator=g, device=dev)
    v = torch.randn(q.shape, generator=g, device=dev)
    shape = (batch, heads, T, H, W, head_dim)
    return tuple(x.reshape(shape).to(dtype) for x in (q, k, v))


def sample_query_tiles(w: Workload, head: int, count: int = 64) -> list[tuple[int, int, int]]:
    """Query tiles checked for one head on large workloads: ``count`` tiles
    from a permutation seeded with 1000 * index + 1 + head, plus the 8 corner
    tiles of the grid (where windows are shifted inward)."""
    nT, nH, nW = tile_count(w)
    n = nT * nH * nW
    g = torch.Generator()
    g.manual_seed(w.seed + 1 + head)
    picks = torch.randperm(n, generator=g)[:min(count, n)].tolist()
    tiles = {(p // (nH * nW), (p // nW) % nH, p % nW) for p in picks}
    for a in (0, nT - 1):
        for b in (0, nH - 1):
            for c in (0, nW - 1):
                tiles.add((a, b, c))
    return sorted(tiles)
