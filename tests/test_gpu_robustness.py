"""Failure handling and buffer bounds on the GPU (needs MI355X).

* STA_TEST_FAIL_ALLOC=1: a plan whose device tables are not uploaded yet
  fails with STA_ERR_ALLOC on the device path (forward, backward, reorder)
  and writes nothing; with the variable cleared the same plan then runs and
  matches a plan that never saw the failure.
* Canary tails: every output buffer (O in fp32 and bf16, the row
  log-sum-exp, delta, dQ, dK, dV, the reordered tensor) is the head of a
  larger allocation whose tail holds a canary pattern; after the calls
  every canary is intact.
"""

import sys

import pytest
import torch

from sliding_tile_attention_sta_amd import _lib as L
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_grad_out, make_qkv

pytestmark = pytest.mark.gpu

TAIL = 4096


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def with_tail(shape, dtype, canary):
    """(view of the head with `shape`, the whole buffer); the tail holds canary."""
    n = 1
    for s in shape:
        n *= s
    buf = torch.full((n + TAIL,), canary, dtype=dtype, device="cuda")
    return buf[:n].view(shape), buf


def test_allocation_hook_on_the_device_path(monkeypatch):
    say("case small workload: STA_TEST_FAIL_ALLOC on a fresh plan")
    w = WORKLOADS["small"]
    q, k, v = make_qkv(w, "cuda")
    ref = api.sta_forward_plan(api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim), q, k, v,
                               scale=w.scale)
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    out = torch.full(q.shape, float("nan"), device="cuda")
    monkeypatch.setenv("STA_TEST_FAIL_ALLOC", "1")
    lib = L.lib()
    st = lib.sta_forward_plan(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              w.scale, L.STA_BF16, L.STA_F32, L.STA_LAYOUT_NATURAL, None)
    assert st == L.STA_ERR_ALLOC
    tm = torch.empty_like(q)
    assert lib.sta_tile_reorder(plan.handle, q.data_ptr(), tm.data_ptr(), L.STA_BF16, None) == L.STA_ERR_ALLOC
    torch.cuda.synchronize()
    assert torch.isnan(out).all(), "a failed call wrote its output"
    monkeypatch.delenv("STA_TEST_FAIL_ALLOC")
    out = api.sta_forward_plan(plan, q, k, v, out=out, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_outputs_stay_inside_their_buffers(name):
    w = WORKLOADS[name]
    say(f"case canary tails {name}")
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    q, k, v = make_qkv(w, "cuda")
    g = make_grad_out(w, "cuda")
    i = plan.info
    rows = (i.batch, i.heads, i.tokens)
    c32, c16 = 1234.5, -77.0
    o32, o32b = with_tail(q.shape, torch.float32, c32)
    lse, lseb = with_tail(rows, torch.float32, c32)
    out, lse = api.sta_forward_plan(plan, q, k, v, out=o32, lse=lse, scale=w.scale)
    o16, o16b = with_tail(q.shape, torch.bfloat16, c16)
    api.sta_forward_plan(plan, q, k, v, out=o16, scale=w.scale)
    grads = [with_tail(q.shape, torch.float32, c32) for _ in range(3)]
    delta, deltab = with_tail(rows, torch.float32, c32)
    api.sta_backward_plan(plan, q, k, v, out, g, lse, scale=w.scale, dq=grads[0][0], dk=grads[1][0],
                          dv=grads[2][0], delta=delta)
    tm, tmb = with_tail(q.shape, q.dtype, c16 if q.dtype == torch.bfloat16 else c32)
    api.sta_tile_reorder(plan, q, out=tm)
    torch.cuda.synchronize()
    for nm, buf, c in (("out fp32", o32b, c32), ("lse", lseb, c32), ("out bf16", o16b, c16),
                       ("delta", deltab, c32), ("dq", grads[0][1], c32), ("dk", grads[1][1], c32),
                       ("dv", grads[2][1], c32), ("reordered", tmb, c16 if q.dtype == torch.bfloat16 else c32)):
        assert bool((buf[-TAIL:] == c).all()), f"{nm}: canary overwritten"
    assert torch.isfinite(out).all() and torch.isfinite(grads[0][0]).all()
