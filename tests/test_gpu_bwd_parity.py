"""GPU parity of the HIP STA backward (and the forward's row log-sum-exp)
against the CPU backward oracle (needs MI355X).

Tolerance, derived from the kernel's arithmetic: every product runs on fp16
MFMA with fp32 accumulation, and P and dS are rounded to fp16 (unit
roundoff u = 2^-11).  A gradient entry is a sum of many such rounded terms,
so its error is about u/sqrt(3) of the root of the summed squared terms,
which for terms of random sign is the entry's own size.  Per gradient
tensor (dq, dk, dv) and compared set:
    max |gpu - oracle|  <= 2e-2 * rms(oracle)
    mean |gpu - oracle| <= 2e-3 * rms(oracle)
(the forward's max/mean pair, taken relative to the gradient's own scale,
about 7x above the expected mean error).  fp32 inputs are rounded on entry
(q, k to bf16, v and dout to fp16, as the header states); the oracle is fed
those rounded values, as it is fed the bf16 values of the bf16 workloads,
so that the check measures the kernels' arithmetic.  lse (natural log): the row sum of
fp16-rounded probabilities is off by at most u relative, so
|lse - oracle| <= 1e-3 (2u with margin).
The small workloads are compared on every token; the 30x48x80 ones on
sampled query tiles (dq, lse) and key tiles (dk, dv) per head, including
corner tiles, where windows are shifted inward.
"""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import sta_oracle_bwd as OB
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_grad_out, make_qkv, tile_count

MAX_REL, MEAN_REL, LSE_ABS = 2e-2, 2e-3, 1e-3

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def check_grad(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.abs(got - ref)
    mx, mn = float(d.max()) / rms, float(d.mean()) / rms
    say(f"  {name}: rms {rms:.3e} max/rms {mx:.2e} mean/rms {mn:.2e}")
    assert mx <= MAX_REL and mn <= MEAN_REL, name


def check_lse(got, ref):
    d = float(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)).max())
    say(f"  lse: max abs {d:.2e}")
    assert d <= LSE_ABS


def run_bwd(w, q, k, v, g, grad_dtype=torch.float32, layout="natural", plan=None):
    if plan is None:
        plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    out, lse = api.sta_forward_plan(plan, q, k, v, scale=w.scale, out_dtype=torch.float32,
                                    layout=layout, lse=True)
    grads = [torch.full(q.shape, float("nan"), dtype=grad_dtype, device=q.device) for _ in range(3)]
    dq, dk, dv = api.sta_backward_plan(plan, q, k, v, out, g, lse, scale=w.scale, layout=layout,
                                       dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    return plan, out, lse, dq, dk, dv


def flat(x, w):
    return x.reshape(w.batch, w.heads, w.tokens, -1)


# ---------------------------------------------------------------------------
# Small workloads: every token
# ---------------------------------------------------------------------------

def consumed(q, k, v, g):
    """The values the backward kernels compute with: fp32 q and k rounded to
    bf16 (the forward's score precision), fp32 v and dout rounded to fp16.
    Identity for bf16 inputs (exact in fp16 within its range)."""
    if q.dtype != torch.float32:
        return q, k, v, g
    return (q.to(torch.bfloat16).float(), k.to(torch.bfloat16).float(),
            v.to(torch.float16).float(), g.to(torch.float16).float())


def _all_tokens(w, heads, grad_dtype=torch.float32):
    q, k, v = make_qkv(w)
    g = make_grad_out(w)
    _, out, lse, dq, dk, dv = run_bwd(w, q.cuda(), k.cuda(), v.cuda(), g.cuda(), grad_dtype=grad_dtype)
    q, k, v, g = consumed(q, k, v, g)
    for h in heads:
        sl = slice(h, h + 1)
        ref = OB.sta_backward_explicit(*(flat(x, w)[:, sl].double().numpy() for x in (q, k, v, g)),
                                       w.video, w.tile, [w.windows[h]], scale=w.scale)
        say(f" head {h}")
        # the forward's own bound (absolute): max 2e-2, mean 2e-3
        do = np.abs(flat(out, w)[:, sl].cpu().numpy().astype(np.float64) - ref["o"])
        say(f"  o: max {do.max():.2e} mean {do.mean():.2e}")
        assert do.max() <= 2e-2 and do.mean() <= 2e-3
        check_lse(lse[:, sl].cpu().numpy(), ref["lse"])
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            check_grad(name, flat(t, w)[:, sl].float().cpu().numpy(), ref[name])


def test_tiny_all_tokens():
    w = WORKLOADS["tiny"]
    say("case tiny backward: 6x16x16 tile 2x4x4 w333 2 heads d64 fp32")
    _all_tokens(w, range(w.heads))


@pytest.mark.parametrize("name", ["generic-d128", "generic-d128-f32"])
def test_generic_d128_all_tokens(name):
    w = WORKLOADS[name]
    say(f"case {name} backward: 8x16x16 tile 2x4x8 (one-wave kernels) 2 heads d128 {w.dtype}")
    _all_tokens(w, range(w.heads))


def test_small_all_tokens():
    w = WORKLOADS["small"]
    say("case small backward: 12x24x24 tile 6x8x8 w333 (whole grid) 8 heads d128 bf16")
    _all_tokens(w, (0, 3, 7))


def test_small_bf16_gradients():
    w = WORKLOADS["small"]
    say("case small backward, bf16 gradients, head 5")
    # bf16 storage adds up to half an ulp (2^-9 relative) per entry: the
    # bound on the max is then 2^-9 of the largest entry, within 2e-2 rms
    # for these distributions; the mean bound is checked against 3e-3 rms.
    q, k, v = make_qkv(w)
    g = make_grad_out(w)
    _, _, _, dq, dk, dv = run_bwd(w, q.cuda(), k.cuda(), v.cuda(), g.cuda(), grad_dtype=torch.bfloat16)
    ref = OB.sta_backward_explicit(*(flat(x, w)[:, 5:6].double().numpy() for x in (q, k, v, g)),
                                   w.video, w.tile, [w.windows[5]], scale=w.scale)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        got = flat(t, w)[:, 5:6].float().cpu().numpy().astype(np.float64)
        r = ref[name]
        rms = float(np.sqrt(np.mean(r * r)))
        d = np.abs(got - r)
        say(f"  {name}: max/rms {d.max() / rms:.2e} mean/rms {d.mean() / rms:.2e}")
        assert d.max() <= MAX_REL * rms + 2.0 ** -9 * np.abs(r).max()
        assert d.mean() <= 3e-3 * rms


def test_tile_major_layout_matches_natural():
    w = WORKLOADS["small"]
    say("case small backward, tile-major layout against natural")
    q, k, v = (x.cuda() for x in make_qkv(w))
    g = make_grad_out(w).cuda()
    plan, _, lse_n, dq_n, dk_n, dv_n = run_bwd(w, q, k, v, g)
    qt, kt, vt, gt = (api.sta_tile_reorder(plan, x) for x in (q, k, v, g))
    _, _, lse_t, dq_t, dk_t, dv_t = run_bwd(w, qt, kt, vt, gt, layout="tile_major", plan=plan)
    for nat, tm in ((dq_n, dq_t), (dk_n, dk_t), (dv_n, dv_t)):
        back = api.sta_tile_unreorder(plan, tm.contiguous())
        assert torch.equal(back.reshape(nat.shape), nat)
    perm = plan.perm().long().cuda()
    assert torch.equal(lse_t.reshape(w.heads, -1), lse_n.reshape(w.heads, -1)[:, perm])


def test_autograd_function():
    w = WORKLOADS["small"]
    say("case small, autograd through sta_attention (fp32 inputs), head 2")
    q, k, v = make_qkv(w)
    g = make_grad_out(w)
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    qd, kd, vd = (x.float().cuda().requires_grad_(True) for x in (q, k, v))
    out = api.sta_attention(qd, kd, vd, plan, scale=w.scale)
    (out * g.float().cuda()).sum().backward()
    ref = OB.sta_backward_explicit(*(flat(x, w)[:, 2:3].double().numpy() for x in (q, k, v, g)),
                                   w.video, w.tile, [w.windows[2]], scale=w.scale)
    for name, t in (("dq", qd.grad), ("dk", kd.grad), ("dv", vd.grad)):
        check_grad(name, flat(t, w)[:, 2:3].cpu().numpy(), ref[name])


# ---------------------------------------------------------------------------
# 30x48x80 workloads: sampled query and key tiles
# ---------------------------------------------------------------------------

def _tile_sl(w, c):
    return tuple(slice(c[d] * w.tile[d], (c[d] + 1) * w.tile[d]) for d in range(3))


def _sample_tiles(w, head, count):
    nT, nH, nW = tile_count(w)
    rng = np.random.default_rng(w.seed + 700 + head)
    picks = rng.choice(nT * nH * nW, size=count, replace=False).tolist()
    tiles = {(p // (nH * nW), (p // nW) % nH, p % nW) for p in picks}
    tiles.add((0, 0, 0))
    tiles.add((nT - 1, nH - 1, nW - 1))
    tiles.add((nT // 2, nH // 2, nW // 2))
    return sorted(tiles)


def _sampled(w, heads, n_query, n_key, key_heads=None):
    q, k, v = (x.cuda() for x in make_qkv(w))
    g = make_grad_out(w).cuda()
    say(f"  running forward+backward on the GPU")
    _, _, lse, dq, dk, dv = run_bwd(w, q, k, v, g)
    key_heads = heads if key_heads is None else key_heads
    for h in heads:
        qh, kh, vh, gh = (x[:, h:h + 1].float().cpu().numpy() for x in (q, k, v, g))
        lse_h = lse[:, h].reshape(w.video).cpu().numpy()
        dq_h = dq[:, h].cpu().numpy()
        qtiles = _sample_tiles(w, h, n_query)
        refs = OB.sta_backward_query_tiles(qh, kh, vh, gh, w.tile, w.windows[h], 0, qtiles, scale=w.scale)
        say(f" head {h} window {w.windows[h]}: {len(qtiles)} query tiles")
        check_lse(np.stack([lse_h[_tile_sl(w, c)] for c in qtiles]), np.stack([r[0] for r in refs]))
        check_grad("dq", np.stack([dq_h[0][_tile_sl(w, c)] for c in qtiles]), np.stack([r[1] for r in refs]))
        if h not in key_heads:
            continue
        ktiles = _sample_tiles(w, h + 50, n_key)
        refs = OB.sta_backward_key_tiles(qh, kh, vh, gh, w.tile, w.windows[h], 0, ktiles, scale=w.scale)
        say(f" head {h}: {len(ktiles)} key tiles")
        dk_h, dv_h = dk[:, h].cpu().numpy(), dv[:, h].cpu().numpy()
        check_grad("dk", np.stack([dk_h[0][_tile_sl(w, c)] for c in ktiles]), np.stack([r[0] for r in refs]))
        check_grad("dv", np.stack([dv_h[0][_tile_sl(w, c)] for c in ktiles]), np.stack([r[1] for r in refs]))


def test_720p_sampled():
    w = WORKLOADS["720p"]
    say("case 720p backward: 30x48x80 tile 6x8x8 w333 24 heads d128 bf16")
    _sampled(w, heads=(0, 13, 23), n_query=6, n_key=3)


def test_mixed_windows_sampled():
    w = WORKLOADS["mixed"]
    say("case mixed backward: windows 1x1x1, 3x3x3, 3x5x5, 5x6x10 (dense)")
    # dk/dv of the dense head would need every query's statistics on the CPU;
    # its dq and lse are still checked.
    _sampled(w, heads=(0, 1, 2, 3), n_query=3, n_key=2, key_heads=(0, 1, 2))


def test_long_stress_sampled():
    w = WORKLOADS["long"]
    say("case long backward: 60x48x80, per-token magnitude U(0.5, 4)")
    _sampled(w, heads=(7,), n_query=4, n_key=3)


# ---------------------------------------------------------------------------
# fp32 inputs against the unrounded definition
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "generic-d128-f32"])
def test_fp32_backward_against_unrounded_inputs(name):
    """The fp32 backward computes with q, k rounded to bf16 and v, dout to
    fp16 (the header's contract).  Against the gradients of the UNROUNDED
    fp32 inputs its error is bounded by the triangle inequality:
        |gpu - exact| <= |gpu - exact(rounded inputs)| + |exact(rounded) - exact|
    the first term by the kernels' parity bound (2e-2 max, 2e-3 mean, of the
    gradient's rms), the second computed here by the float64 oracle on both
    input sets (the cost of the input rounding alone).  Both are reported."""
    w = WORKLOADS[name]
    say(f"case {name}: fp32 backward against the unrounded inputs")
    q, k, v = make_qkv(w)
    g = make_grad_out(w)
    assert q.dtype == torch.float32
    _, out, lse, dq, dk, dv = run_bwd(w, q.cuda(), k.cuda(), v.cuda(), g.cuda())
    qr, kr, vr, gr = consumed(q, k, v, g)
    for h in range(w.heads):
        sl = slice(h, h + 1)
        exact = OB.sta_backward_explicit(*(flat(x, w)[:, sl].double().numpy() for x in (q, k, v, g)),
                                         w.video, w.tile, [w.windows[h]], scale=w.scale)
        rounded = OB.sta_backward_explicit(*(flat(x, w)[:, sl].double().numpy() for x in (qr, kr, vr, gr)),
                                           w.video, w.tile, [w.windows[h]], scale=w.scale)
        for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            got = flat(t, w)[:, sl].double().cpu().numpy()
            rms = float(np.sqrt(np.mean(exact[nm] ** 2)))
            e_round = np.abs(rounded[nm] - exact[nm]) / rms
            e_gpu = np.abs(got - exact[nm]) / rms
            say(f"  head {h} {nm}: input rounding alone max/rms {e_round.max():.2e} mean/rms "
                f"{e_round.mean():.2e}; gpu vs unrounded max/rms {e_gpu.max():.2e} mean/rms {e_gpu.mean():.2e}")
            # (the parity bound is relative to the rounded-input gradient's rms)
            rr = float(np.sqrt(np.mean(rounded[nm] ** 2))) / rms
            assert e_gpu.max() <= e_round.max() + MAX_REL * rr, nm
            assert e_gpu.mean() <= e_round.mean() + MEAN_REL * rr, nm
