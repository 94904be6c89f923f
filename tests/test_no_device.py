"""Entry points that need a GPU, called where there is none (the CPU-only
build machine): each returns STA_ERR_HIP, none crashes, also from several
threads at once while another clears the plan cache.  Skipped where a GPU is
present.  The pointers are never dereferenced on the host (every check
before a launch is arithmetic on them), and no launch happens without a
device."""

import ctypes
import threading

import pytest
import torch

from sliding_tile_attention_sta_amd import _lib as L

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present")

TILE = (ctypes.c_int * 3)(2, 4, 4)
WIN = (ctypes.c_int * 6)(3, 3, 3, 3, 3, 3)
SHAPE = (1, 2, 6, 16, 16)
BYTES = 1 * 2 * 6 * 16 * 16 * 64 * 4


def fake(i):
    """A distinct, non-overlapping fake device address."""
    return ctypes.c_void_p(0x100000000 + i * (BYTES + 4096))


@pytest.fixture(scope="module")
def plan():
    lib = L.lib()
    h = ctypes.c_void_p()
    assert lib.sta_plan_create(*SHAPE, TILE, WIN, 64, ctypes.byref(h)) == L.STA_OK
    yield lib, h
    assert lib.sta_plan_destroy(h) == L.STA_OK


def test_every_device_entry_point_reports_no_device(plan):
    lib, h = plan
    q, k, v, o, lse, d, dq, dk, dv = (fake(i) for i in range(9))
    f32, nat = L.STA_F32, L.STA_LAYOUT_NATURAL
    assert lib.sta_forward_plan(h, q, k, v, o, 0.125, f32, f32, nat, None) == L.STA_ERR_HIP
    assert lib.sta_forward_plan_lse(h, q, k, v, o, lse, 0.125, f32, f32, nat, None) == L.STA_ERR_HIP
    assert lib.sta_forward_plan_noalloc(h, q, k, v, o, lse, 0.125, f32, f32, nat, None) == L.STA_ERR_HIP
    assert lib.sta_backward_plan(h, q, k, v, o, d, lse, fake(9), dq, dk, dv, 0.125, f32, f32, f32, nat,
                                 None) == L.STA_ERR_HIP
    assert lib.sta_tile_reorder(h, q, o, f32, None) == L.STA_ERR_HIP
    assert lib.sta_tile_unreorder(h, q, o, f32, None) == L.STA_ERR_HIP
    assert lib.sta_forward(q, k, v, o, *SHAPE, TILE, WIN, 64, 0.125, f32, f32, nat, None) == L.STA_ERR_HIP
    err = (ctypes.c_double * 2)()
    cands = (ctypes.c_int * 6)(1, 1, 1, 3, 3, 3)
    assert lib.sta_window_errors(q, k, v, *SHAPE, TILE, 64, 0.125, f32, nat, cands, 2, err,
                                 None) == L.STA_ERR_HIP
    # argument errors still come first
    assert lib.sta_forward_plan(h, q, k, v, q, 0.125, f32, f32, nat, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan(h, q, k, v, o, -1.0, f32, f32, nat, None) == L.STA_ERR_ARG
    assert lib.sta_clear_plan_cache() == L.STA_OK


def test_threads_through_the_plan_cache_without_a_device():
    lib = L.lib()
    wins = [(ctypes.c_int * 6)(*w) for w in ((3, 3, 3, 3, 3, 3), (1, 2, 3, 3, 2, 1), (2, 2, 2, 1, 1, 1))]
    bad, stop = [], threading.Event()

    def worker(i):
        for it in range(60):
            st = lib.sta_forward(fake(0), fake(1), fake(2), fake(3), *SHAPE, TILE, wins[(i + it) % 3], 64,
                                 0.125, L.STA_F32, L.STA_F32, L.STA_LAYOUT_NATURAL, None)
            if st != L.STA_ERR_HIP:
                bad.append(st)

    def clearer():
        while not stop.is_set():
            lib.sta_clear_plan_cache()

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(6)]
    c = threading.Thread(target=clearer)
    c.start()
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    stop.set()
    c.join()
    assert bad == []
    assert lib.sta_clear_plan_cache() == L.STA_OK


def test_allocation_hook_fails_plan_creation(monkeypatch):
    lib = L.lib()
    h = ctypes.c_void_p()
    monkeypatch.setenv("STA_TEST_FAIL_ALLOC", "1")
    assert lib.sta_plan_create(*SHAPE, TILE, WIN, 64, ctypes.byref(h)) == L.STA_ERR_ALLOC and not h.value
    assert lib.sta_forward(fake(0), fake(1), fake(2), fake(3), *SHAPE, TILE, WIN, 64, 0.125, L.STA_F32,
                           L.STA_F32, L.STA_LAYOUT_NATURAL, None) == L.STA_ERR_ALLOC
    monkeypatch.delenv("STA_TEST_FAIL_ALLOC")
    assert lib.sta_plan_create(*SHAPE, TILE, WIN, 64, ctypes.byref(h)) == L.STA_OK and h.value
    assert lib.sta_plan_destroy(h) == L.STA_OK
