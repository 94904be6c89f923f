"""Token-wise 3D sliding window attention (the baseline the pages contrast
STA with) on the GPU against its CPU oracle.  Tolerance as for STA: max
2e-2 and mean 2e-3 absolute (fp32 output; for the fp32 workload the oracle
sees the fp32 inputs, as for STA's tiny workload).  swa-tiny: every token
(generic kernel variant); swa-small: every query tile (384-query variant);
swa-720p: sampled query tiles including the corners.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import sta_oracle_swa as OS
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_qkv, sample_query_tiles, tile_count

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run(w, q, k, v):
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, token_windows=True)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    api.sta_forward_plan(plan, q, k, v, out=out, scale=w.scale)
    torch.cuda.synchronize()
    return plan, out


def test_swa_tiny_all_tokens():
    w = WORKLOADS["swa-tiny"]
    say(f"case {w.name}: {w.description}")
    q, k, v = make_qkv(w)
    plan, out = _run(w, q.cuda(), k.cuda(), v.cuda())
    assert plan.info.swa == 1 and plan.info.kernel_variant == 0
    shp = (1, w.heads, w.tokens, w.head_dim)
    ref = OS.swa_forward_explicit(*(x.reshape(shp).double().numpy() for x in (q, k, v)), w.video, w.windows,
                                  scale=w.scale)
    d = np.abs(out.reshape(shp).cpu().numpy() - ref)
    say(f"  max {d.max():.2e} mean {d.mean():.2e}")
    assert d.max() <= 2e-2 and d.mean() <= 2e-3


@pytest.mark.parametrize("name,count", [("swa-small", None), ("swa-720p", 10)])
def test_swa_tiles(name, count):
    w = WORKLOADS[name]
    say(f"case {w.name}: {w.description}")
    q, k, v = (x.cuda() for x in make_qkv(w))
    plan, out = _run(w, q, k, v)
    assert not torch.isnan(out).any().item()
    grid = tile_count(w)
    worst, tot, cnt = 0.0, 0.0, 0
    heads = range(w.heads) if w.heads <= 4 else (0, 9, 23)
    for h in heads:
        if count is None:
            tiles = [(a, b, c) for a in range(grid[0]) for b in range(grid[1]) for c in range(grid[2])]
        else:
            tiles = sample_query_tiles(w, h, count=count)
        qh, kh, vh = (x[:, h:h + 1].float().cpu().numpy() for x in (q, k, v))
        refs = OS.swa_forward_query_tiles(qh, kh, vh, w.tile, w.windows[h], 0, tiles, scale=w.scale)
        o = out[0, h].cpu().numpy()
        for c, ref in zip(tiles, refs):
            sl = tuple(slice(c[d] * w.tile[d], (c[d] + 1) * w.tile[d]) for d in range(3))
            d = np.abs(o[sl].astype(np.float64) - ref)
            worst = max(worst, float(d.max()))
            tot += float(d.sum())
            cnt += d.size
    say(f"  {cnt} outputs: max {worst:.2e} mean {tot / cnt:.2e}")
    assert worst <= 2e-2 and tot / cnt <= 2e-3
