"""GPU checks of the forward's split work items (needs MI355X).

When equal-cost work items would leave the last round of a launch to a few
compute units, the plan cuts those items into pieces of consecutive key
steps; every piece computes a partial softmax over its keys, and the last
piece of an item to finish combines them (``sta_plan_pieces`` in
include/sta.h).  Checked here, against the float64 oracle on the very same
inputs: every query tile of every split item (output within the forward's
parity bound, row log-sum-exp within 1e-3), on the workloads whose plans
split (720p, 60x48x80, 12x24x24 where every item is split, and 30x45x80
and 12x22x24 with partial tiles, whose pieces start on key-tile
boundaries; the 12x... workloads run one range of key steps per compute
unit); that two launches give the same bits (the merge does not
depend on which piece arrives last, nor the result on which work group
takes which queue entry, and every launch leaves the queue words and
arrival counters ready for the next one), also after a launch on other
values in between, i.e. the merge reads its own launch's partial results.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import sta_oracle as O
from oracle import sta_oracle_bwd as OB
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, Workload, make_qkv

MAX_ABS, MEAN_ABS, LSE_ABS = 2e-2, 2e-3, 1e-3

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def split_tiles(plan, w, partial):
    """(batch, head, query tile coordinates) of every split work item."""
    info = plan.info
    subs = info.tile_tokens // info.queries_per_item
    nT, nH, nW = O.tile_grid(w.video, w.tile, partial)
    out = []
    for it in sorted(set(plan.pieces()[:, 0].tolist())):
        rest = it // subs
        qt, bh = rest % info.n_tiles, rest // info.n_tiles
        out.append((bh // w.heads, bh % w.heads, (qt // (nH * nW), (qt // nW) % nH, qt % nW)))
    return out


def window_rows(x, w, c, b, h, grid):
    """Token rows [n, D] of the box of tokens of query tile c's window."""
    (t0, t1), (y0, y1), (z0, z1) = O.window_tiles(c, w.windows[h], grid)
    tT, tH, tW = w.tile
    s = x[b, h, t0 * tT:t1 * tT, y0 * tH:y1 * tH, z0 * tW:z1 * tW]
    return np.asarray(s, np.float64).reshape(-1, x.shape[-1])


# 12x22x24 with 6x8x8 tiles: the last tile row along H is partial, and its
# 144 items take one range of key steps per compute unit, cut on key-tile
# boundaries (a piece's first key block must hold an existing key).
SMALL_PARTIAL = Workload("small-partial", 21, (12, 22, 24), (6, 8, 8), ((3, 3, 3),) * 8, 128, "bf16")


@pytest.mark.parametrize("name", ["720p", "long", "small", "720p-exact", "small-partial"])
def test_split_items_match_oracle(name):
    w = SMALL_PARTIAL if name == "small-partial" else WORKLOADS[name]
    partial = any(e % t for e, t in zip(w.video, w.tile))
    say(f"case split {name}")
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=partial)
    pieces = plan.pieces()
    assert len(pieces) > 0 and min(pieces[:, 4].tolist()) >= 2
    q, k, v = make_qkv(w, "cuda")
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    out, lse = api.sta_forward_plan(plan, q, k, v, out=out, scale=w.scale, lse=True)
    out2, lse2 = api.sta_forward_plan(plan, q, k, v, scale=w.scale, lse=True)
    # a launch on other values in between: a merge that read another
    # launch's partial results would not give the same bits again
    api.sta_forward_plan(plan, q, k, v * 2, scale=w.scale, lse=True)
    out4, lse4 = api.sta_forward_plan(plan, q, k, v, scale=w.scale, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "two launches differ"
    assert torch.equal(out, out4) and torch.equal(lse, lse4), "a launch in between changed the result"
    qn, kn, vn = (x.float().cpu().numpy() for x in (q, k, v))
    got = out.cpu().numpy()
    got_lse = lse.reshape(w.batch, w.heads, *w.video).cpu().numpy()
    grid = O.tile_grid(w.video, w.tile, partial)
    tT, tH, tW = w.tile
    worst, worst_lse, tot, cnt = 0.0, 0.0, 0.0, 0
    tiles = split_tiles(plan, w, partial)
    for b, h, c in tiles:
        ref = O.sta_forward_query_tiles(qn, kn, vn, w.tile, w.windows[h], h, [c], scale=w.scale, batch=b,
                                        partial=partial)[0]
        sl = (slice(c[0] * tT, (c[0] + 1) * tT), slice(c[1] * tH, (c[1] + 1) * tH),
              slice(c[2] * tW, (c[2] + 1) * tW))
        g = got[b, h][sl]
        assert g.shape == ref.shape and np.isfinite(g).all(), (b, h, c)
        d = np.abs(g.astype(np.float64) - ref)
        worst = max(worst, float(d.max()))
        tot += float(d.sum())
        cnt += d.size
        assert float(d.max()) <= MAX_ABS, (b, h, c, float(d.max()))
        qrows = np.asarray(qn[b, h][sl], np.float64).reshape(-1, w.head_dim)
        kr = window_rows(kn, w, c, b, h, grid)
        ref_lse = OB.masked_attention_lse(qrows, kr, np.ones((len(qrows), len(kr)), bool), w.scale)
        dl = float(np.abs(got_lse[b, h][sl].reshape(-1) - ref_lse).max())
        worst_lse = max(worst_lse, dl)
        assert dl <= LSE_ABS, (b, h, c, dl)
    say(f"split {name}: {len(tiles)} split items, max {worst:.2e} mean {tot / cnt:.2e} lse {worst_lse:.2e}")
    assert tot / cnt <= MEAN_ABS
