"""Forward and backward parity on seeded random small plans (needs MI355X).

Twelve seeded cases draw a tile shape (volumes 32 to 384, so both forward
variants and every backward wave layout run), a tile grid of 1 to 4 tiles
per axis, sometimes extents that are not multiples of the tile (partial
tiles), 1 to 3 heads with their own windows of 1 to grid + 1
tiles (wider than the grid is clamped), head_dim 64 or 128, bf16 or fp32
inputs and batch 1 or 2; fixed cases add 384-token tiles on a multi-tile
grid at d64 (bf16) and d128 (fp32), and partial tiles on every axis with
384-token tiles at d64 and 128-token tiles at d128.  Every token is compared with the
oracles: the forward output to max 2e-2 / mean 2e-3 absolute; the row
log-sum-exp to 1e-3; each gradient to max 2e-2 / mean 2e-3 of its rms, with
the backward oracle fed the values the kernels consume for fp32 inputs
(q, k as bf16; v, dout as fp16).
"""

import sys

import numpy as np
import pytest
import torch

from oracle import sta_oracle as O
from oracle import sta_oracle_bwd as OB
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import Workload, make_grad_out, make_qkv

pytestmark = pytest.mark.gpu

TILES = [(2, 4, 4), (1, 8, 8), (2, 4, 8), (4, 4, 6), (3, 4, 8), (2, 8, 8), (1, 16, 24), (6, 8, 8)]
MAX_TOKENS = 1536


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def random_cases(n=12, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        tile = TILES[int(rng.integers(len(TILES)))]
        grid = [int(rng.integers(1, 5)) for _ in range(3)]
        while np.prod(grid) * np.prod(tile) > MAX_TOKENS:
            d = int(np.argmax(grid))
            grid[d] -= 1
        if min(grid) < 1:
            continue
        video = [tile[d] * grid[d] for d in range(3)]
        partial = bool(rng.integers(0, 4) == 0)
        if partial:
            cut = [d for d in range(3) if tile[d] > 1]
            for d in cut[:int(rng.integers(1, len(cut) + 1))]:
                video[d] -= int(rng.integers(1, tile[d]))
        heads = int(rng.integers(1, 4))
        windows = tuple(tuple(int(rng.integers(1, g + 2)) for g in grid) for _ in range(heads))
        head_dim = int(rng.choice([64, 128]))
        dtype = "bf16" if rng.integers(0, 3) else "f32"
        batch = int(rng.integers(1, 3))
        w = Workload(f"random-{len(cases)}", 200 + len(cases), tuple(video), tile, windows, head_dim, dtype,
                     batch=batch)
        cases.append((w, partial))
    return cases


CASES = random_cases() + [
    # 384-token tiles on a multi-tile grid: d64 bf16 and d128 fp32 (the
    # 384-query forward and the 4-wave dQ / 6-pair dK/dV kernels)
    (Workload("fixed-384-d64", 230, (12, 16, 16), (6, 8, 8), ((1, 2, 2), (2, 1, 2)), 64, "bf16"), False),
    (Workload("fixed-384-f32", 231, (12, 16, 16), (6, 8, 8), ((2, 2, 1), (1, 1, 1)), 128, "f32"), False),
    # partial tiles on every axis with the 384-token kernels at d64 bf16, and
    # with 128-token tiles (4-wave dQ, 4-pair dK/dV) at d128 bf16
    (Workload("fixed-384-d64-partial", 232, (11, 13, 21), (6, 8, 8), ((2, 2, 3), (1, 2, 1)), 64, "bf16"), True),
    (Workload("fixed-128-partial", 233, (5, 15, 13), (2, 8, 8), ((3, 2, 2), (2, 3, 1)), 128, "bf16"), True),
]


def consumed(q, k, v, g):
    if q.dtype != torch.float32:
        return q, k, v, g
    return (q.to(torch.bfloat16).float(), k.to(torch.bfloat16).float(), v.to(torch.float16).float(),
            g.to(torch.float16).float())


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_plan(case):
    w, partial = CASES[case]
    say(f"case {w.name}: video {w.video} tile {w.tile} windows {w.windows} d{w.head_dim} {w.dtype} "
        f"batch {w.batch} partial {partial}")
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=partial)
    assert plan.info.partial_tiles == (1 if partial else 0)
    q, k, v = make_qkv(w)
    N = int(np.prod(w.video))
    shp = (w.batch, w.heads, N, w.head_dim)
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    out = torch.full(qd.shape, float("nan"), dtype=torch.float32, device="cuda")
    out, lse = api.sta_forward_plan(plan, qd, kd, vd, out=out, scale=w.scale, lse=True)
    torch.cuda.synchronize()
    ref = O.sta_forward_explicit(*(x.reshape(shp).double().numpy() for x in (q, k, v)), w.video, w.tile,
                                 w.windows, scale=w.scale, partial=partial)
    got = out.reshape(shp).cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    d = np.abs(got - ref)
    say(f"  forward max {d.max():.2e} mean {d.mean():.2e}")
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert plan.info.bwd_supported == 1
    g = make_grad_out(w)
    dq, dk, dv = api.sta_backward_plan(plan, qd, kd, vd, out, g.cuda(), lse, scale=w.scale)
    torch.cuda.synchronize()
    cq, ck, cv, cg = consumed(q, k, v, g)
    refb = OB.sta_backward_explicit(*(x.reshape(shp).double().numpy() for x in (cq, ck, cv, cg)), w.video,
                                    w.tile, w.windows, scale=w.scale, partial=partial)
    dl = np.abs(lse.reshape(w.batch, w.heads, N).cpu().numpy().astype(np.float64) - refb["lse"])
    say(f"  lse max {dl.max():.2e}")
    assert dl.max() <= 1e-3
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        r = refb[name]
        rms = float(np.sqrt(np.mean(r * r)))
        e = np.abs(t.reshape(shp).cpu().numpy().astype(np.float64) - r)
        say(f"  {name} max/rms {e.max() / rms:.2e} mean/rms {e.mean() / rms:.2e}")
        assert np.isfinite(e).all() and e.max() <= 2e-2 * rms and e.mean() <= 2e-3 * rms
