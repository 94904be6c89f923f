"""V beyond fp16's range in the forward (needs MI355X).

The P.V product runs on fp16 MFMA, whose inputs hold |v| <= 65504.  A work
item whose V holds larger entries (bf16 and fp32 go to 3.4e38) gets a
non-finite O; the forward marks it, and a second kernel of the same launch
redoes every marked item with V multiplied by 2^-e and O by 2^e (exact
scalings; e from the largest |v| of the item's keys, so that it becomes
< 2^15).  Checked here, on V with a few entries far beyond fp16 (about
1.6e6) and the rest N(0, 1):

* the oracle on the same inputs: the forward's parity bound (2e-2 max,
  2e-3 mean) relative to the largest output magnitude;
* exactness: V_big = 2^6 * V_small, where V_small's largest entry lies in
  [2^14, 2^15) and no entry in [2^10, 2^14), so that every work item that
  overflows scales by exactly 2^-6 and computes V_small's products:
  out(V_big) must equal 2^6 * out(V_small) bit for bit on every query tile
  whose items are not split by key range.  A split item is redone whole
  (its pieces merge only without overflow), so its tiles differ from the
  merged pieces by summation order: they are held to the parity bound;
* the row log-sum-exp does not depend on V (bit for bit on the tiles
  checked exactly above).
"""

import sys

import numpy as np
import pytest
import torch

from oracle import sta_oracle as O
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_qkv, sample_query_tiles

pytestmark = pytest.mark.gpu

BIG = 24576.0        # 1.5 * 2^14, exact in bf16: the largest |v| of V_small
SHIFT = 6            # V_big = 2^6 V_small: largest |v| = 1.57e6


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def with_big_entries(v, seed, frac=1e-4):
    """v with a seeded random fraction of its entries set to +-BIG."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    n = v.numel()
    idx = torch.randperm(n, generator=g)[:max(1, int(n * frac))]
    sign = torch.where(torch.rand(len(idx), generator=g) < 0.5, -1.0, 1.0)
    flat = v.reshape(-1).clone()
    flat[idx.to(v.device)] = (sign * BIG).to(v.dtype).to(v.device)
    return flat.reshape(v.shape)


def split_token_mask(plan, w):
    """[B, heads, T, H, W] bool: the tokens of every query tile that holds a
    work item split by key range."""
    info = plan.info
    mask = torch.zeros((w.batch, w.heads, *w.video), dtype=torch.bool)
    if info.pieces == 0:
        return mask
    subs = info.tile_tokens // info.queries_per_item
    nT, nH, nW = O.tile_grid(w.video, w.tile)
    tT, tH, tW = w.tile
    for it in set(plan.pieces()[:, 0].tolist()):
        rest = it // subs
        qt, bh = rest % info.n_tiles, rest // info.n_tiles
        a, b, c = qt // (nH * nW), (qt // nW) % nH, qt % nW
        mask[bh // w.heads, bh % w.heads, a * tT:(a + 1) * tT, b * tH:(b + 1) * tH, c * tW:(c + 1) * tW] = True
    return mask


@pytest.mark.parametrize("name", ["tiny", "small", "720p"])
def test_v_beyond_fp16_range(name):
    w = WORKLOADS[name]
    say(f"case vrange {name}")
    q, k, v = make_qkv(w, "cuda")
    v_small = with_big_entries(v, w.seed + 77)
    vmax_small, vmax = float(v_small.abs().max()), float(v.abs().max())
    assert vmax_small == BIG and vmax < 1024
    v_big = v_small * 2 ** SHIFT
    assert bool(torch.equal(v_big / 2 ** SHIFT, v_small))
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    o_small, lse_small = api.sta_forward_plan(plan, q, k, v_small, scale=w.scale, lse=True)
    o_big, lse_big = api.sta_forward_plan(plan, q, k, v_big, scale=w.scale, lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o_big).all()
    split = split_token_mask(plan, w).to(o_big.device)
    ref_small = o_small * 2 ** SHIFT
    whole = ~split
    assert torch.equal(o_big[whole], ref_small[whole]), "scaled redo is not exact"
    if bool(split.any()):
        d = (o_big[split] - ref_small[split]).abs()
        mag = float(ref_small.abs().max())
        say(f"vrange {name}: split tiles {int(split[0, 0].sum())} tokens/head, max {float(d.max()):.3e} "
            f"relative to {mag:.3e}")
        assert float(d.max()) <= 2e-2 * mag and float(d.mean()) <= 2e-3 * mag
    # the row log-sum-exp does not see V: equal bits where the same walk
    # ran, within 1e-4 where a whole redo replaced merged pieces
    lsplit = split.reshape(lse_big.shape)
    assert torch.equal(lse_big[~lsplit], lse_small[~lsplit])
    if bool(lsplit.any()):
        assert float((lse_big[lsplit] - lse_small[lsplit]).abs().max()) <= 1e-4
    # against the oracle, on every token (small workloads) or sampled tiles
    qn, kn, vn = (x.float().cpu().numpy() for x in (q, k, v_big))
    got = o_big.cpu().numpy()
    grid = O.tile_grid(w.video, w.tile)
    tT, tH, tW = w.tile
    worst, tot, cnt, ref_abs = 0.0, 0.0, 0, 0.0
    heads = range(w.heads) if w.heads <= 8 else range(0, w.heads, 6)
    for h in heads:
        if w.tokens <= 8192:
            tiles = [(a, b, c) for a in range(grid[0]) for b in range(grid[1]) for c in range(grid[2])]
        else:
            tiles = sample_query_tiles(w, h, count=8)
        refs = O.sta_forward_query_tiles(qn, kn, vn, w.tile, w.windows[h], h, tiles, scale=w.scale)
        for c, ref in zip(tiles, refs):
            g = got[0, h, c[0] * tT:(c[0] + 1) * tT, c[1] * tH:(c[1] + 1) * tH, c[2] * tW:(c[2] + 1) * tW]
            d = np.abs(g.astype(np.float64) - ref)
            worst = max(worst, float(d.max()))
            tot += float(d.sum())
            cnt += d.size
            ref_abs = max(ref_abs, float(np.abs(ref).max()))
    # the parity bound, relative to the output's magnitude (the fp32 tiny
    # workload's error is mostly the bf16 rounding of q and k)
    say(f"vrange {name}: max |out| {ref_abs:.3e}, max err {worst:.3e}, mean err {tot / cnt:.3e}")
    assert worst <= 2e-2 * ref_abs and tot / cnt <= 2e-3 * ref_abs
