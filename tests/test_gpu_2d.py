"""2D STA on the GPU (an image latent: T = 1, one-frame tiles) against the
CPU oracles: forward, lse and dq on every query tile; dk and dv on every
key tile of the coarse latent and on every 7th key tile (plus the corners)
of the fine one; heads 0 and 5 of the coarse latent, all four window sizes
of the fine one.  Tolerances as in the 3D parity tests:
forward max 2e-2 / mean 2e-3 absolute; gradients max 2e-2 / mean 2e-3 of
the reference's rms; lse 1e-3.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import sta_oracle as O
from oracle import sta_oracle_bwd as OB
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_grad_out, make_qkv

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _sl(w, c):
    return tuple(slice(c[d] * w.tile[d], (c[d] + 1) * w.tile[d]) for d in range(3))


def _rel(name, got, ref):
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.abs(np.asarray(got, np.float64) - ref)
    say(f"  {name}: max/rms {d.max() / rms:.2e} mean/rms {d.mean() / rms:.2e}")
    assert d.max() <= 2e-2 * rms and d.mean() <= 2e-3 * rms, name


@pytest.mark.parametrize("name", ["2d", "2d-fine"])
def test_2d_forward_and_backward(name):
    w = WORKLOADS[name]
    say(f"case {name}: {w.description}")
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    assert plan.info.kernel_variant == (1 if w.tile[1] * w.tile[2] % 384 == 0 else 0)
    q, k, v = make_qkv(w)
    g = make_grad_out(w)
    qc, kc, vc, gc = (x.cuda() for x in (q, k, v, g))
    out, lse = api.sta_forward_plan(plan, qc, kc, vc, scale=w.scale, lse=True)
    dq, dk, dv = api.sta_backward_plan(plan, qc, kc, vc, out, gc, lse, scale=w.scale)
    torch.cuda.synchronize()
    grid = O.tile_grid(w.video, w.tile)
    tiles = [(0, b, c) for b in range(grid[1]) for c in range(grid[2])]
    ktiles = tiles if len(tiles) <= 64 else sorted(set(tiles[::7]) | {tiles[0], tiles[-1],
                                                                     (0, 0, grid[2] - 1), (0, grid[1] - 1, 0)})
    out, lse, dq, dk, dv = (x.cpu().numpy() for x in (out, lse, dq, dk, dv))
    for h in ((0, 5) if w.heads > 4 else range(w.heads)):
        qh, kh, vh, gh = (x[:, h:h + 1].float().numpy() for x in (q, k, v, g))
        fwd = O.sta_forward_query_tiles(qh, kh, vh, w.tile, w.windows[h], 0, tiles, scale=w.scale)
        got = np.stack([out[0, h][_sl(w, c)] for c in tiles])
        d = np.abs(got - np.stack(fwd))
        say(f" head {h} window {w.windows[h]}: forward max {d.max():.2e} mean {d.mean():.2e}")
        assert d.max() <= 2e-2 and d.mean() <= 2e-3
        qr = OB.sta_backward_query_tiles(qh, kh, vh, gh, w.tile, w.windows[h], 0, tiles, scale=w.scale)
        lse_h = lse[0, h].reshape(w.video)
        dl = max(float(np.abs(lse_h[_sl(w, c)] - r[0]).max()) for c, r in zip(tiles, qr))
        say(f"  lse max {dl:.2e}")
        assert dl <= 1e-3
        _rel("dq", np.stack([dq[0, h][_sl(w, c)] for c in tiles]), np.stack([r[1] for r in qr]))
        kr = OB.sta_backward_key_tiles(qh, kh, vh, gh, w.tile, w.windows[h], 0, ktiles, scale=w.scale)
        _rel("dk", np.stack([dk[0, h][_sl(w, c)] for c in ktiles]), np.stack([r[0] for r in kr]))
        _rel("dv", np.stack([dv[0, h][_sl(w, c)] for c in ktiles]), np.stack([r[1] for r in kr]))
