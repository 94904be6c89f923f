"""Argument checks of the Python binding that need device tensors (needs
MI355X): mixed dtypes, a wrong output size, a host output and a token count
that does not match the video all raise ValueError before any launch; the
plan-cache entry point gives the same bits as the plan entry point."""

import sys

import pytest
import torch

from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_qkv

pytestmark = pytest.mark.gpu


def test_bad_arguments_raise_before_launch():
    print("case tiny: argument checks", file=sys.stderr, flush=True)
    w = WORKLOADS["tiny"]
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    q, k, v = (x.cuda() for x in make_qkv(w))
    q4, k4, v4 = (x.reshape(w.batch, w.heads, w.tokens, w.head_dim) for x in (q, k, v))
    with pytest.raises(ValueError, match="dtype"):
        api.sta_forward(q, k.to(torch.bfloat16), v, w.tile, w.windows)
    with pytest.raises(ValueError, match="share a dtype"):
        api.sta_forward_plan(plan, q4, k4.to(torch.bfloat16), v4)
    with pytest.raises(ValueError, match="element count"):
        api.sta_forward(q, k, v, w.tile, w.windows, out=torch.empty(q.numel() - 1, device="cuda"))
    with pytest.raises(ValueError, match="on cuda"):
        api.sta_forward_plan(plan, q4, k4, v4, out=torch.empty(q4.shape))
    with pytest.raises(ValueError, match="tokens"):
        api.sta_forward(q4, k4, v4, w.tile, w.windows, video=(w.video[0], w.video[1], w.video[2] // 2))
    torch.cuda.synchronize()


def test_cache_entry_point_matches_plan_entry_point():
    print("case tiny: sta_forward against sta_forward_plan", file=sys.stderr, flush=True)
    w = WORKLOADS["tiny"]
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    q, k, v = (x.cuda() for x in make_qkv(w))
    a = api.sta_forward(q, k, v, w.tile, w.windows, scale=w.scale)
    b = api.sta_forward_plan(plan, q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
