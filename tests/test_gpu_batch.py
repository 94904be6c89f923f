"""Batch > 1 on the GPU: every kernel indexes its (batch, head) plane, and
the other tests run one batch element.  The small workload with batch 2
(forward and backward, every token), the partial-tile paths (forward, and
forward and backward with 384-token tiles) and the token-wise SWA path with
batch 2 (every token), each against its CPU oracle per batch
element, with the tolerances of the corresponding single-batch tests."""

import dataclasses
import sys

import numpy as np
import pytest
import torch

from oracle import sta_oracle as O
from oracle import sta_oracle_bwd as OB
from oracle import sta_oracle_swa as OS
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, Workload, make_grad_out, make_qkv

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_batch2_forward_and_backward():
    w = dataclasses.replace(WORKLOADS["small"], batch=2, windows=((3, 3, 3), (1, 2, 2), (2, 3, 1), (3, 1, 3)))
    say("case small, batch 2, 4 heads with different windows: forward and backward")
    q, k, v = make_qkv(w)
    g = make_grad_out(w)
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    qc, kc, vc, gc = (x.cuda() for x in (q, k, v, g))
    out, lse = api.sta_forward_plan(plan, qc, kc, vc, scale=w.scale, lse=True)
    dq, dk, dv = api.sta_backward_plan(plan, qc, kc, vc, out, gc, lse, scale=w.scale)
    torch.cuda.synchronize()
    N = w.tokens
    shp = (w.batch, w.heads, N, w.head_dim)
    ref = OB.sta_backward_explicit(*(x.reshape(shp).double().numpy() for x in (q, k, v, g)), w.video,
                                   w.tile, w.windows, scale=w.scale)
    d = np.abs(out.reshape(shp).cpu().numpy() - ref["o"])
    say(f"  forward max {d.max():.2e} mean {d.mean():.2e}")
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert float(np.abs(lse.reshape(w.batch, w.heads, N).cpu().numpy() - ref["lse"]).max()) <= 1e-3
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        got = t.reshape(shp).cpu().numpy()
        for b in range(w.batch):
            r = ref[name][b]
            rms = float(np.sqrt(np.mean(r * r)))
            e = np.abs(got[b] - r)
            say(f"  {name} batch {b}: max/rms {e.max() / rms:.2e} mean/rms {e.mean() / rms:.2e}")
            assert e.max() <= 2e-2 * rms and e.mean() <= 2e-3 * rms


def test_batch2_partial_tiles():
    w = dataclasses.replace(WORKLOADS["partial-small"], batch=2)
    say("case partial-small, batch 2")
    q, k, v = make_qkv(w)
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=True)
    out = api.sta_forward_plan(plan, q.cuda(), k.cuda(), v.cuda(), scale=w.scale)
    torch.cuda.synchronize()
    shp = (w.batch, w.heads, w.tokens, w.head_dim)
    ref = O.sta_forward_explicit(*(x.reshape(shp).double().numpy() for x in (q, k, v)), w.video, w.tile,
                                 w.windows, scale=w.scale, partial=True)
    d = np.abs(out.reshape(shp).cpu().numpy() - ref)
    say(f"  max {d.max():.2e} mean {d.mean():.2e}")
    assert d.max() <= 2e-2 and d.mean() <= 2e-3


def test_batch2_partial_tiles_backward():
    # 384-token tiles (the production kernels), partial on every axis
    # (11x21x19 with 6x8x8 tiles), batch 2: forward and backward, every token
    w = Workload("partial-384-b2", 32, (11, 21, 19), (6, 8, 8), ((3, 3, 3), (1, 2, 3)), 128, "bf16", batch=2)
    say("case 11x21x19, tile 6x8x8 (partial on every axis), batch 2: forward and backward")
    q, k, v = make_qkv(w)
    g = make_grad_out(w)
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=True)
    qc, kc, vc, gc = (x.cuda() for x in (q, k, v, g))
    out, lse = api.sta_forward_plan(plan, qc, kc, vc, scale=w.scale, lse=True)
    dq, dk, dv = api.sta_backward_plan(plan, qc, kc, vc, out, gc, lse, scale=w.scale)
    torch.cuda.synchronize()
    shp = (w.batch, w.heads, w.tokens, w.head_dim)
    ref = OB.sta_backward_explicit(*(x.reshape(shp).double().numpy() for x in (q, k, v, g)), w.video,
                                   w.tile, w.windows, scale=w.scale, partial=True)
    d = np.abs(out.reshape(shp).cpu().numpy() - ref["o"])
    say(f"  forward max {d.max():.2e} mean {d.mean():.2e}")
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert float(np.abs(lse.reshape(shp[:3]).cpu().numpy() - ref["lse"]).max()) <= 1e-3
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        got = t.reshape(shp).cpu().numpy()
        assert np.isfinite(got).all(), name
        for b in range(w.batch):
            r = ref[name][b]
            rms = float(np.sqrt(np.mean(r * r)))
            e = np.abs(got[b] - r)
            say(f"  {name} batch {b}: max/rms {e.max() / rms:.2e} mean/rms {e.mean() / rms:.2e}")
            assert e.max() <= 2e-2 * rms and e.mean() <= 2e-3 * rms


def test_batch2_token_windows():
    w = dataclasses.replace(WORKLOADS["swa-tiny"], batch=2)
    say("case swa-tiny, batch 2")
    q, k, v = make_qkv(w)
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, token_windows=True)
    out = api.sta_forward_plan(plan, q.cuda(), k.cuda(), v.cuda(), scale=w.scale)
    torch.cuda.synchronize()
    shp = (w.batch, w.heads, w.tokens, w.head_dim)
    ref = OS.swa_forward_explicit(*(x.reshape(shp).double().numpy() for x in (q, k, v)), w.video, w.windows,
                                  scale=w.scale)
    d = np.abs(out.reshape(shp).cpu().numpy() - ref)
    say(f"  max {d.max():.2e} mean {d.mean():.2e}")
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
