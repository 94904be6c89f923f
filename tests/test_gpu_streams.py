"""Stream handling (needs MI355X): every entry point runs on the stream it
is given.  The inputs are copied on a side stream behind a bounded spin
kernel, and the calls are made with that stream while the current stream is
the default one: a launch on any other stream would read inputs that are
not written yet, so the outputs are compared bit for bit with a plain run.
A plan released right after a launch (its forward still queued behind a
spin) gives the same bits as one that stays alive."""

import sys

import pytest
import torch

from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_grad_out, make_qkv

pytestmark = pytest.mark.gpu


def test_entry_points_run_on_the_given_stream():
    print("case side stream: small workload forward (lse), backward, reorder", file=sys.stderr, flush=True)
    w = WORKLOADS["small"]
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    q, k, v = (x.cuda() for x in make_qkv(w))
    g = make_grad_out(w).cuda()
    out, lse = api.sta_forward_plan(plan, q, k, v, scale=w.scale, lse=True)
    dq, dk, dv = api.sta_backward_plan(plan, q, k, v, out, g, lse, scale=w.scale)
    tm = api.sta_tile_reorder(plan, q)
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(50_000_000)   # a bounded spin, tens of milliseconds
        q2, k2, v2, g2 = (x.clone() for x in (q, k, v, g))
    assert torch.cuda.current_stream() == torch.cuda.default_stream()
    out2, lse2 = api.sta_forward_plan(plan, q2, k2, v2, scale=w.scale, lse=True, stream=s)
    dq2, dk2, dv2 = api.sta_backward_plan(plan, q2, k2, v2, out2, g2, lse2, scale=w.scale, stream=s)
    tm2 = api.sta_tile_reorder(plan, q2, stream=s)
    s.synchronize()
    assert torch.equal(out2, out) and torch.equal(lse2, lse)
    for a, b in ((dq2, dq), (dk2, dk), (dv2, dv)):
        assert torch.equal(a, b)
    assert torch.equal(tm2, tm)


def test_plan_released_right_after_launch():
    print("case small workload: plan released while its forward is queued", file=sys.stderr, flush=True)
    w = WORKLOADS["small"]
    keep = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    q, k, v = (x.cuda() for x in make_qkv(w))
    ref = api.sta_forward_plan(keep, q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)   # the forward below queues behind this bounded spin
    tmp = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    out = api.sta_forward_plan(tmp, q, k, v, scale=w.scale)
    del tmp                         # sta_plan_destroy waits for the queued work first
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_tables_uploaded_on_one_stream_are_awaited_by_another():
    print("case small workload: tables uploaded behind a spin on stream 1, first used on stream 2",
          file=sys.stderr, flush=True)
    w = WORKLOADS["small"]
    keep = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    q, k, v = (x.cuda() for x in make_qkv(w))
    ref = api.sta_forward_plan(keep, q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        torch.cuda._sleep(50_000_000)   # a bounded spin: the upload below queues behind it
    out1 = api.sta_forward_plan(plan, q, k, v, scale=w.scale, stream=s1)   # uploads the tables on s1
    out2 = api.sta_forward_plan(plan, q, k, v, scale=w.scale, stream=s2)   # must wait for that upload
    torch.cuda.synchronize()
    assert torch.equal(out1, ref) and torch.equal(out2, ref)
