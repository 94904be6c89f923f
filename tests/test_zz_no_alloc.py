"""The forward entry point that allocates nothing (sta_forward_plan_noalloc,
needs MI355X).

Called through the C ABI, it must give the same bits as sta_forward_plan
(same kernels and plan, its fixed scratch array in place of an allocated
one) on two calls in a row, the second with a smaller input; it must leave
no state behind that changes a later call; and it rejects, with
STA_ERR_UNSUPPORTED and before any launch, a plan whose scratch exceeds the
array and a plan whose tables are not on the device yet.
"""

import ctypes
import sys

import pytest
import torch

from sliding_tile_attention_sta_amd import _lib as L
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_qkv

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def noalloc(plan, q, k, v, out, lse, scale):
    return L.lib().sta_forward_plan_noalloc(
        plan.handle, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr() if lse is not None else 0), float(scale),
        L.STA_BF16 if q.dtype == torch.bfloat16 else L.STA_F32, L.STA_F32, L.STA_LAYOUT_NATURAL,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def case(w):
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    q, k, v = make_qkv(w, "cuda")
    ref, ref_lse = api.sta_forward_plan(plan, q, k, v, scale=w.scale, lse=True)   # uploads the tables
    return plan, q, k, v, ref, ref_lse


def test_noalloc_matches_forward_plan_on_two_calls_second_smaller():
    big = WORKLOADS["720p"]
    smaller = big.with_heads(4)
    say("case no-alloc: 720p 24 heads, then 720p 4 heads")
    runs = []
    for w in (big, smaller):
        plan, q, k, v, ref, ref_lse = case(w)
        assert plan.info.pieces > 0 and 0 < plan.info.scratch_bytes <= 64 << 20
        out = torch.full_like(ref, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        assert noalloc(plan, q, k, v, out, lse, w.scale) == L.STA_OK
        out2 = torch.full_like(ref, float("nan"))
        assert noalloc(plan, q, k, v, out2, None, w.scale) == L.STA_OK
        torch.cuda.synchronize()
        runs.append((w.name, w.heads, torch.equal(out, ref), torch.equal(lse, ref_lse), torch.equal(out2, ref)))
        del plan, q, k, v, ref, ref_lse, out, lse, out2
    say(f"no-alloc runs: {runs}")
    for name, heads, same, same_lse, same2 in runs:
        assert same and same_lse and same2, (name, heads)
    # the allocating entry point is unaffected by the calls in between
    plan, q, k, v, ref, _ = case(smaller)
    again = api.sta_forward_plan(plan, q, k, v, scale=smaller.scale)
    torch.cuda.synchronize()
    assert torch.equal(again, ref)


def test_noalloc_rejects_before_any_launch():
    # the 12x24x24 plan splits all 144 items into 432 pieces: 90 MB of scratch
    w = WORKLOADS["small"]
    plan, q, k, v, ref, _ = case(w)
    assert plan.info.scratch_bytes > 64 << 20
    out = torch.full_like(ref, float("nan"))
    assert noalloc(plan, q, k, v, out, None, w.scale) == L.STA_ERR_UNSUPPORTED
    # a plan that never ran on the device has no tables there
    w = WORKLOADS["720p"].with_heads(2)
    fresh = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    q, k, v = make_qkv(w, "cuda")
    out2 = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    assert noalloc(fresh, q, k, v, out2, None, w.scale) == L.STA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(out2).all()
