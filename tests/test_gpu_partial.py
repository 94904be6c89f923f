"""Forward and backward parity on latents whose extents are not multiples
of the tile size (partial tiles at the far edges, reading: only existing
tokens take part) against the CPU oracles with partial tiles.  Tolerance as for whole
tiles: max 2e-2, mean 2e-3 absolute.  The small case compares every token
(fp32 inputs, as the tiny workload); the exact 720p latent (30x45x80)
compares sampled query tiles, among them the partial ones.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

from oracle import sta_oracle as O
from oracle import sta_oracle_bwd as OB
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import (WORKLOADS, Workload, make_grad_out, make_qkv,
                                                      sample_query_tiles)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run(w, q, k, v, lse=False):
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=True)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    res = api.sta_forward_plan(plan, q, k, v, out=out, scale=w.scale, lse=lse)
    torch.cuda.synchronize()
    return plan, res


def test_partial_small_all_tokens():
    w = WORKLOADS["partial-small"]
    say(f"case {w.name}: {w.description}")
    q, k, v = make_qkv(w)
    plan, out = _run(w, q.cuda(), k.cuda(), v.cuda())
    assert plan.info.partial_tiles == 1
    N = w.tokens
    shp = (1, w.heads, N, w.head_dim)
    ref = O.sta_forward_explicit(*(x.reshape(shp).double().numpy() for x in (q, k, v)), w.video, w.tile,
                                 w.windows, scale=w.scale, partial=True)
    got = out.reshape(shp).cpu().numpy()
    assert np.isfinite(got).all()
    d = np.abs(got - ref)
    say(f"  max {d.max():.2e} mean {d.mean():.2e}")
    assert d.max() <= 2e-2 and d.mean() <= 2e-3


def test_720p_exact_sampled_and_edges():
    w = WORKLOADS["720p-exact"]
    say(f"case {w.name}: {w.description}")
    q, k, v = (x.cuda() for x in make_qkv(w))
    plan, (out, lse) = _run(w, q, k, v, lse=True)
    assert not torch.isnan(out).any().item()
    grid = O.tile_grid(w.video, w.tile, partial=True)
    tT, tH, tW = w.tile
    worst, tot, cnt = 0.0, 0.0, 0
    for h in (0, 11, 23):
        tiles = sample_query_tiles(w, h, count=12)
        tiles = sorted(set(tiles) | {(a, grid[1] - 1, c) for a in (0, 2, 4) for c in (0, 5, 9)})
        qh, kh, vh = (x[:, h:h + 1].float().cpu().numpy() for x in (q, k, v))
        refs = O.sta_forward_query_tiles(qh, kh, vh, w.tile, w.windows[h], 0, tiles, scale=w.scale,
                                         partial=True)
        o = out[0, h].cpu().numpy()
        for c, ref in zip(tiles, refs):
            g = o[c[0] * tT:(c[0] + 1) * tT, c[1] * tH:(c[1] + 1) * tH, c[2] * tW:(c[2] + 1) * tW]
            assert g.shape == ref.shape
            d = np.abs(g.astype(np.float64) - ref)
            worst = max(worst, float(d.max()))
            tot += float(d.sum())
            cnt += d.size
    say(f"  {cnt} outputs: max {worst:.2e} mean {tot / cnt:.2e}")
    assert worst <= 2e-2 and tot / cnt <= 2e-3


# ---------------------------------------------------------------------------
# Backward with partial tiles: the gradients of the forward definition over
# the tokens that exist (reading R11 of the forward), against the backward
# oracle with partial tiles.  Tolerance as for whole tiles: per gradient
# tensor, max 2e-2 and mean 2e-3 of its rms; lse 1e-3 absolute.  fp32 inputs
# are fed to the oracle as the kernels consume them (q, k rounded to bf16,
# v, dout to fp16).
# ---------------------------------------------------------------------------

def _check_grad(name, got, ref):
    got = np.asarray(got, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    assert np.isfinite(got).all(), name
    d = np.abs(got - ref)
    say(f"  {name}: max/rms {d.max() / rms:.2e} mean/rms {d.mean() / rms:.2e}")
    assert d.max() <= 2e-2 * rms and d.mean() <= 2e-3 * rms, name


def _consumed(x, kind):
    if x.dtype != torch.float32:
        return x
    return x.to(torch.bfloat16 if kind == "qk" else torch.float16).float()


def _backward(w, q, k, v, g):
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=True)
    assert plan.info.partial_tiles == 1 and plan.info.bwd_supported == 1
    out, lse = api.sta_forward_plan(plan, q, k, v, scale=w.scale, out_dtype=torch.float32, lse=True)
    grads = [torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device) for _ in range(3)]
    dq, dk, dv = api.sta_backward_plan(plan, q, k, v, out, g, lse, scale=w.scale,
                                       dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


# 384-token tiles (the production kernels) with every axis partial: an
# 11x21x19 latent has a 2x3x3 grid whose last tile on each axis holds 5 of
# 6, 5 of 8 and 3 of 8 rows; one head sees the whole grid, one a 1x2x3 box.
PARTIAL_384 = Workload("partial-384", 31, (11, 21, 19), (6, 8, 8), ((3, 3, 3), (1, 2, 3)), 128, "bf16",
                       description="11x21x19 latent, tile 6x8x8 (partial on every axis), 2 heads, d128, bf16")


@pytest.mark.parametrize("name", ["partial-small", "partial-384"])
def test_partial_backward_all_tokens(name):
    w = PARTIAL_384 if name == "partial-384" else WORKLOADS[name]
    say(f"case {w.name} backward: {w.description}")
    q, k, v = make_qkv(w)
    g = make_grad_out(w)
    out, lse, dq, dk, dv = _backward(w, q.cuda(), k.cuda(), v.cuda(), g.cuda())
    shp = (w.batch, w.heads, w.tokens, w.head_dim)
    cq, ck, cv, cg = _consumed(q, "qk"), _consumed(k, "qk"), _consumed(v, "v"), _consumed(g, "v")
    ref = OB.sta_backward_explicit(*(x.reshape(shp).double().numpy() for x in (cq, ck, cv, cg)), w.video,
                                   w.tile, w.windows, scale=w.scale, partial=True)
    do = np.abs(out.reshape(shp).cpu().numpy().astype(np.float64) - ref["o"])
    say(f"  o: max {do.max():.2e} mean {do.mean():.2e}")
    assert do.max() <= 2e-2 and do.mean() <= 2e-3
    dl = float(np.abs(lse.reshape(shp[:3]).cpu().numpy().astype(np.float64) - ref["lse"]).max())
    say(f"  lse: max {dl:.2e}")
    assert dl <= 1e-3
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_grad(nm, t.reshape(shp).cpu().numpy(), ref[nm])


def test_720p_exact_backward_sampled_and_edges():
    w = WORKLOADS["720p-exact"]
    say(f"case {w.name} backward: {w.description}")
    q, k, v = (x.cuda() for x in make_qkv(w))
    g = make_grad_out(w).cuda()
    _, lse, dq, dk, dv = _backward(w, q, k, v, g)
    grid = O.tile_grid(w.video, w.tile, partial=True)
    tT, tH, tW = w.tile

    def sl(x, c):
        return x[c[0] * tT:(c[0] + 1) * tT, c[1] * tH:(c[1] + 1) * tH, c[2] * tW:(c[2] + 1) * tW]

    for h in (0, 23):
        # sampled tiles plus partial ones (the last row of tiles on H) at corners and inside
        qt = sorted(set(sample_query_tiles(w, h, count=4)) | {(0, grid[1] - 1, 0), (2, grid[1] - 1, 5)})
        kt = sorted({(4, grid[1] - 1, 9), (1, grid[1] - 1, 3), (2, 2, 4)})
        qh, kh, vh, gh = (x[:, h:h + 1].float().cpu().numpy() for x in (q, k, v, g))
        refs = OB.sta_backward_query_tiles(qh, kh, vh, gh, w.tile, w.windows[h], 0, qt, scale=w.scale,
                                           partial=True)
        say(f" head {h}: {len(qt)} query tiles, {len(kt)} key tiles")
        lse_h, dq_h = lse[0, h].reshape(w.video).cpu().numpy(), dq[0, h].cpu().numpy()
        for c, (rl, _) in zip(qt, refs):
            assert sl(lse_h, c).shape == rl.shape
        dl = max(float(np.abs(sl(lse_h, c).astype(np.float64) - rl).max()) for c, (rl, _) in zip(qt, refs))
        say(f"  lse: max {dl:.2e}")
        assert dl <= 1e-3
        _check_grad("dq", np.concatenate([sl(dq_h, c).reshape(-1) for c in qt]),
                    np.concatenate([r[1].reshape(-1) for r in refs]))
        refk = OB.sta_backward_key_tiles(qh, kh, vh, gh, w.tile, w.windows[h], 0, kt, scale=w.scale,
                                         partial=True)
        dk_h, dv_h = dk[0, h].cpu().numpy(), dv[0, h].cpu().numpy()
        _check_grad("dk", np.concatenate([sl(dk_h, c).reshape(-1) for c in kt]),
                    np.concatenate([r[0].reshape(-1) for r in refk]))
        _check_grad("dv", np.concatenate([sl(dv_h, c).reshape(-1) for c in kt]),
                    np.concatenate([r[1].reshape(-1) for r in refk]))


def test_partial_autograd_function():
    """Autograd through sta_attention on a partial-tile plan (fp32 inputs;
    the oracle is fed them as the kernels consume them)."""
    w = dataclasses.replace(PARTIAL_384, dtype="f32")
    say(f"case {w.name}, fp32, autograd through sta_attention")
    q, k, v = make_qkv(w)
    g = make_grad_out(w)
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=True)
    qd, kd, vd = (x.cuda().requires_grad_(True) for x in (q, k, v))
    out = api.sta_attention(qd, kd, vd, plan, scale=w.scale)
    (out * g.cuda()).sum().backward()
    shp = (w.batch, w.heads, w.tokens, w.head_dim)
    cq, ck, cv, cg = _consumed(q, "qk"), _consumed(k, "qk"), _consumed(v, "v"), _consumed(g, "v")
    ref = OB.sta_backward_explicit(*(x.reshape(shp).double().numpy() for x in (cq, ck, cv, cg)), w.video,
                                   w.tile, w.windows, scale=w.scale, partial=True)
    for nm, t in (("dq", qd.grad), ("dk", kd.grad), ("dv", vd.grad)):
        _check_grad(nm, t.reshape(shp).cpu().numpy(), ref[nm])


def test_cached_entry_point_takes_partial_tiles():
    """sta_forward (plan cache) on the exact 720p latent: the same result as
    sta_forward_plan with a partial-tile plan, bit for bit."""
    w = WORKLOADS["720p-exact"]
    say(f"case {w.name}: sta_forward against sta_forward_plan")
    q, k, v = (x.cuda() for x in make_qkv(w))
    _, ref = _run(w, q, k, v)
    got = api.sta_forward(q, k, v, w.tile, w.windows, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    api.sta_clear_plan_cache()
