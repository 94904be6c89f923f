"""Large tiles, forward and backward, every token (needs MI355X).

Tiles of 768 tokens run the 384-query forward with two work items per
tile and the backward's four-wave dQ and six-pair dK/dV layouts with
several items per tile; tiles of 4096 tokens, the largest a plan accepts,
run the 32-query forward with 128 work items per tile and the four-pair
dK/dV layout.  Every query tile is compared with the per-tile forward and
backward oracles (each tile's window is a box of tokens): the output to max
2e-2 / mean 2e-3 absolute, the row log-sum-exp to 1e-3, each gradient to
max 2e-2 / mean 2e-3 of its rms.
"""

import itertools
import sys

import numpy as np
import pytest
import torch

from oracle import sta_oracle as O
from oracle import sta_oracle_bwd as OB
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import Workload, make_grad_out, make_qkv

pytestmark = pytest.mark.gpu

CASES = {
    "tile-768": Workload("tile-768", 240, (12, 24, 48), (6, 8, 16), ((2, 2, 1), (1, 3, 1)), 128, "bf16"),
    "tile-4096": Workload("tile-4096", 241, (8, 32, 64), (4, 32, 32), ((1, 1, 2),), 64, "bf16"),
}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def tile_slice(c, tile):
    return tuple(slice(c[d] * tile[d], (c[d] + 1) * tile[d]) for d in range(3))


@pytest.mark.parametrize("name", list(CASES))
def test_large_tile_every_token(name):
    w = CASES[name]
    say(f"case {name}: video {w.video} tile {w.tile} windows {w.windows} d{w.head_dim} {w.dtype}")
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    assert plan.info.bwd_supported == 1
    q, k, v = make_qkv(w)
    g = make_grad_out(w)
    qd, kd, vd, gd = (x.cuda() for x in (q, k, v, g))
    out, lse = api.sta_forward_plan(plan, qd, kd, vd, scale=w.scale, lse=True)
    dq, dk, dv = api.sta_backward_plan(plan, qd, kd, vd, out, gd, lse, scale=w.scale)
    torch.cuda.synchronize()

    T, H, W = w.video
    shp = (w.batch, w.heads, T, H, W, w.head_dim)
    got = {n: t.reshape(shp).cpu().numpy().astype(np.float64) for n, t in
           (("o", out), ("dq", dq), ("dk", dk), ("dv", dv))}
    got_lse = lse.reshape(shp[:-1]).cpu().numpy().astype(np.float64)
    qn, kn, vn, gn = (x.double().numpy() for x in (q, k, v, g))
    grid = [e // t for e, t in zip(w.video, w.tile)]
    tiles = list(itertools.product(*(range(n) for n in grid)))
    ref = {n: np.zeros(shp) for n in ("o", "dq", "dk", "dv")}
    ref_lse = np.zeros(shp[:-1])
    for h in range(w.heads):
        win = w.windows[h]
        for c, o in zip(tiles, O.sta_forward_query_tiles(qn, kn, vn, w.tile, win, h, tiles, scale=w.scale)):
            ref["o"][(0, h) + tile_slice(c, w.tile)] = o
        for c, (l, d) in zip(tiles, OB.sta_backward_query_tiles(qn, kn, vn, gn, w.tile, win, h, tiles,
                                                                 scale=w.scale)):
            ref_lse[(0, h) + tile_slice(c, w.tile)] = l
            ref["dq"][(0, h) + tile_slice(c, w.tile)] = d
        for c, (a, b) in zip(tiles, OB.sta_backward_key_tiles(qn, kn, vn, gn, w.tile, win, h, tiles,
                                                               scale=w.scale)):
            ref["dk"][(0, h) + tile_slice(c, w.tile)] = a
            ref["dv"][(0, h) + tile_slice(c, w.tile)] = b

    assert np.isfinite(got["o"]).all()
    e = np.abs(got["o"] - ref["o"])
    say(f"  forward max {e.max():.2e} mean {e.mean():.2e}")
    assert e.max() <= 2e-2 and e.mean() <= 2e-3
    dl = np.abs(got_lse - ref_lse)
    say(f"  lse max {dl.max():.2e}")
    assert dl.max() <= 1e-3
    for n in ("dq", "dk", "dv"):
        rms = float(np.sqrt(np.mean(ref[n] ** 2)))
        e = np.abs(got[n] - ref[n])
        say(f"  {n} max/rms {e.max() / rms:.2e} mean/rms {e.mean() / rms:.2e}")
        assert np.isfinite(e).all() and e.max() <= 2e-2 * rms and e.mean() <= 2e-3 * rms
