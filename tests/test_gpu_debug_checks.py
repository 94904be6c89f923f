"""The kernels' bounds checks (needs MI355X): libsta_debug.so is the library
built with -DSTA_DEBUG, whose kernels check every work item code, tile-list
entry, token row, buffer offset and LDS table index they use and record a
failed check in a device word (sta_debug_flags) instead of trapping.  Each
workload below runs through both libraries -- forward with the row
log-sum-exp, and the backward where the plan supports it -- and must record
no violation and give the same bits as the release library."""

import ctypes
import sys

import pytest
import torch

from sliding_tile_attention_sta_amd import _lib as L
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_grad_out, make_qkv

pytestmark = pytest.mark.gpu

P = lambda t: ctypes.c_void_p(t.data_ptr())


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def plan_for(l, w, partial):
    h = ctypes.c_void_p()
    ws = [x for win in w.windows for x in win]
    args = (w.batch, w.heads, *w.video, (ctypes.c_int * 3)(*w.tile), (ctypes.c_int * len(ws))(*ws), w.head_dim)
    if w.name.startswith("swa"):
        st = l.sta_swa_plan_create(*args, ctypes.byref(h))
    else:
        st = l.sta_plan_create_ex(*args, L.STA_PLAN_PARTIAL_TILES if partial else 0, ctypes.byref(h))
    assert st == L.STA_OK, st
    return h


def run(l, w, layout, noalloc=False):
    partial = any(e % t for e, t in zip(w.video, w.tile))
    h = plan_for(l, w, partial)
    info = L.PlanInfo()
    assert l.sta_plan_get_info(h, ctypes.byref(info)) == 0
    q, k, v = make_qkv(w, "cuda")
    dt = L.STA_BF16 if q.dtype == torch.bfloat16 else L.STA_F32
    out = torch.full(q.shape, float("nan"), device="cuda")
    lse = torch.full((w.batch, w.heads, info.tokens), float("nan"), device="cuda")
    st = l.sta_forward_plan_lse(h, P(q), P(k), P(v), P(out), P(lse), w.scale, dt, L.STA_F32, layout, None)
    assert st == L.STA_OK, st
    res = [out, lse]
    if noalloc:
        out2 = torch.full(q.shape, float("nan"), device="cuda")
        st = l.sta_forward_plan_noalloc(h, P(q), P(k), P(v), P(out2), None, w.scale, dt, L.STA_F32, layout, None)
        assert st == L.STA_OK, st
        res.append(out2)
    if info.bwd_supported and not info.swa:
        g = make_grad_out(w, "cuda")
        delta = torch.empty_like(lse)
        grads = [torch.full(q.shape, float("nan"), device="cuda") for _ in range(3)]
        st = l.sta_backward_plan(h, P(q), P(k), P(v), P(out), P(g), P(lse), P(delta), *(P(x) for x in grads),
                                 w.scale, dt, L.STA_F32, L.STA_F32, layout, None)
        assert st == L.STA_OK, st
        res += grads
    torch.cuda.synchronize()
    assert l.sta_plan_destroy(h) == L.STA_OK
    return res


CASES = [("tiny", 0), ("small", 0), ("small", 1), ("720p-exact", 0), ("mixed", 0), ("long", 0),
         ("swa-small", 0), ("generic-d128", 0), ("2d", 0), ("partial-small", 0)]


def test_release_library_reports_no_debug_build():
    flags = ctypes.c_uint32(7)
    assert L.lib().sta_debug_flags(ctypes.byref(flags), 1) == L.STA_ERR_UNSUPPORTED and flags.value == 0


@pytest.mark.parametrize("name,layout", CASES, ids=[f"{n}-{'tm' if t else 'nat'}" for n, t in CASES])
def test_bounds_checks_clean_and_results_identical(name, layout):
    w = WORKLOADS[name]
    if name == "mixed":
        w = w.with_heads(4)   # every window size once
    say(f"case debug checks {name} layout {layout}")
    dbg = L.debug_lib()
    flags = ctypes.c_uint32()
    assert dbg.sta_debug_flags(ctypes.byref(flags), 1) == L.STA_OK
    noalloc = name in ("tiny", "720p-exact")   # plans within the no-allocation scratch
    got = run(dbg, w, layout, noalloc=noalloc)
    assert dbg.sta_debug_flags(ctypes.byref(flags), 1) == L.STA_OK
    assert flags.value == 0, f"bounds checks failed: bits {flags.value:#x}"
    ref = run(L.lib(), w, layout, noalloc=noalloc)
    assert len(got) == len(ref)
    for i, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a, b), (name, i)
