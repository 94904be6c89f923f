"""Host-side checks of libsta.so (CPU only; no kernel is launched).

* the library loads and exports every function that include/sta.h declares;
* the plan's key-tile lists, permutation and schedule agree with the
  oracle's geometry (window starts, tile coordinates);
* every invalid argument returns its status code before any device work.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import sta_oracle as O
from sliding_tile_attention_sta_amd import _lib as L
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "sta.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sta_[a-z_]+)\s*\(", src)))


def test_header_declares_the_expected_entry_points():
    names = header_functions()
    for required in ["sta_plan_create", "sta_plan_destroy", "sta_forward", "sta_forward_plan",
                     "sta_tile_reorder", "sta_tile_unreorder", "sta_status_string"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), f"{name} declared in sta.h but not exported"
    assert set(header_functions()) == set(L.SIGNATURES), "binding and header disagree"


def test_status_strings():
    for code in [L.STA_OK, L.STA_ERR_ARG, L.STA_ERR_SHAPE, L.STA_ERR_UNSUPPORTED, L.STA_ERR_ALLOC,
                 L.STA_ERR_HIP]:
        s = L.status_string(code)
        assert s.startswith("STA_")
    assert "unknown" in L.status_string(42)


@pytest.mark.parametrize("name", ["tiny", "small", "720p", "mixed", "long", "2d", "2d-fine"])
def test_plan_matches_oracle_geometry(name):
    w = WORKLOADS[name]
    p = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    grid = O.tile_grid(w.video, w.tile)
    info = p.info
    assert tuple(info.grid) == grid
    assert info.tile_tokens == w.tile[0] * w.tile[1] * w.tile[2]
    assert info.flops == O.sta_flops(w.video, w.tile, w.windows, w.head_dim, w.batch)
    nT, nH, nW = grid
    heads = range(w.heads) if w.heads <= 8 else range(0, w.heads, 5)
    for h in heads:
        for qt in range(0, nT * nH * nW, 7 if nT * nH * nW > 64 else 1):
            c = (qt // (nH * nW), (qt // nW) % nH, qt % nW)
            (t0, t1), (y0, y1), (z0, z1) = O.window_tiles(c, w.windows[h], grid)
            want = sorted((a * nH + b) * nW + cc for a in range(t0, t1) for b in range(y0, y1)
                          for cc in range(z0, z1))
            assert p.kv_tiles(h, qt) == want


def test_perm_is_the_tile_major_order():
    w = WORKLOADS["tiny"]
    p = api.Plan(1, 2, w.video, w.tile, w.windows, w.head_dim)
    perm = p.perm().numpy()
    coords = O.natural_coords(w.video)
    T, H, W = w.video
    tT, tH, tW = w.tile
    grid = O.tile_grid(w.video, w.tile)
    assert sorted(perm.tolist()) == list(range(T * H * W))
    V = tT * tH * tW
    for pos, n in enumerate(perm):
        t, y, z = coords[n]
        tile = ((t // tT) * grid[1] + y // tH) * grid[2] + z // tW
        local = ((t % tT) * tH + y % tH) * tW + z % tW
        assert pos == tile * V + local


@pytest.mark.parametrize("name", ["720p", "mixed", "long", "small", "tiny", "720p-exact"])
def test_schedule_covers_every_item_once_and_balances_xcds(name):
    w = WORKLOADS[name]
    partial = any(e % t for e, t in zip(w.video, w.tile))
    p = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=partial)
    s = p.schedule().numpy()
    info = p.info
    subs = info.tile_tokens // info.queries_per_item
    n_items = w.batch * w.heads * info.n_tiles * subs
    if len(p.group_lists()):
        _check_group_lists(w, p, partial)
        return
    # the XCD queues interleaved (entry s * 8 + x of XCD x's queue, -1
    # padding), then the pieces of split items in the order they are taken
    n_whole = len(s) - info.pieces
    assert n_whole % 8 == 0
    whole, tail = s[:n_whole], s[n_whole:]
    assert (tail == -2 - np.arange(info.pieces)).all()
    assert ((whole == -1) | (whole >= 0)).all()
    pieces = p.pieces().numpy()
    assert len(pieces) == info.pieces
    steps = {}
    for it, a, b, g, n in pieces.tolist():
        steps.setdefault(it, []).append((a, b, g, n))
    assert sorted(whole[whole >= 0].tolist() + list(steps)) == list(range(n_items))
    # the pieces of a split item partition its key steps (on key-tile
    # boundaries when tiles are partial), and are taken one after another
    grid = O.tile_grid(w.video, w.tile, partial)
    V = info.tile_tokens
    spt = V // 32
    for it, segs in steps.items():
        h = (it // subs // info.n_tiles) % w.heads
        we = O.effective_window(w.windows[h], grid)
        assert segs[0][0] == 0 and segs[-1][1] == we[0] * we[1] * we[2] * spt
        assert all(x[1] == y[0] and x[0] < x[1] for x, y in zip(segs, segs[1:]))
        assert len({g for _, _, g, _ in segs}) == 1 and all(n == len(segs) for *_, n in segs)
        if partial:
            assert all(a % spt == 0 for a, *_ in segs)
    # per-XCD cost (block b runs on XCD b % 8): spread within one chunk of items
    cost = {}
    for h in range(w.heads):
        we = O.effective_window(w.windows[h], grid)
        cost[h] = we[0] * we[1] * we[2]
    load = [0] * 8
    for b, code in enumerate(whole.tolist()):
        if code >= 0:
            load[b % 8] += cost[(code // subs // info.n_tiles) % w.heads]
    if n_items - len(steps) >= 8 * 32:
        assert max(load) - min(load) <= 32 * max(cost.values())
    # decreasing cost along each XCD's queue (list scheduling of an LPT order)
    for x in range(8):
        q = [cost[(c // subs // info.n_tiles) % w.heads] for c in whole[x::8].tolist() if c >= 0]
        assert q == sorted(q, reverse=True)
    # split items are the cheapest ones
    if steps:
        split_cost = max(cost[(it // subs // info.n_tiles) % w.heads] for it in steps)
        assert all(cost[(c // subs // info.n_tiles) % w.heads] >= split_cost for c in whole[whole >= 0].tolist())
    # the launch has more work groups than entries (dynamic queues) or exactly
    # sched; every forward has scratch (at least the fix-up marks of its items)
    n_items = info.batch * info.heads * info.n_tiles * subs
    assert info.scratch_bytes >= 4 * (16 + (n_items + 31) // 32 + n_items)
    if info.kernel_variant == 1:
        assert info.launch_blocks >= len(s)
    else:
        assert info.launch_blocks == len(s)


def _check_group_lists(w, p, partial):
    """Per-work-group lists: work group b runs range u = (b mod 8) * 32 +
    b // 8 of the launch's key steps; the ranges, in order, walk the items
    in decreasing-cost order, each item's steps in order, and every range
    holds the same number of steps (within one alignment unit)."""
    info = p.info
    s, off = p.schedule().numpy(), p.group_lists().numpy()
    subs = info.tile_tokens // info.queries_per_item
    n_items = w.batch * w.heads * info.n_tiles * subs
    assert info.launch_blocks == 256 and len(off) == 257
    assert off[0] == 0 and off[-1] == len(s) and (np.diff(off) >= 0).all()
    assert (s != -1).all()
    pieces = p.pieces().numpy()
    assert sorted((-2 - s[s < -1]).tolist()) == list(range(info.pieces))
    grid = O.tile_grid(w.video, w.tile, partial)
    spt = info.tile_tokens // 32
    align = spt if partial else 1

    def steps_of(code):
        h = (code // subs // info.n_tiles) % w.heads
        we = O.effective_window(w.windows[h], grid)
        return we[0] * we[1] * we[2] * spt

    walk = []   # (item, first step, end step) per range entry, in range order
    per_unit = []
    for u in range(256):
        b = (u % 32) * 8 + u // 32
        n = 0
        for code in s[off[b]:off[b + 1]].tolist():
            if code >= 0:
                walk.append((code, 0, steps_of(code)))
            else:
                it, a, e, g, npc = pieces[-2 - code].tolist()
                walk.append((it, a, e))
            n += walk[-1][2] - walk[-1][1]
        per_unit.append(n)
    total = sum(per_unit)
    assert total == sum(steps_of(c) for c in range(n_items))
    assert max(per_unit) - min(per_unit) <= align
    items = []
    for (it, a, e), nxt in zip(walk, walk[1:] + [None]):
        assert a < e and a % align == 0
        if not items or items[-1][0] != it:
            assert a == 0
            items.append([it, e])
        else:
            assert a == items[-1][1]
            items[-1][1] = e
    assert sorted(it for it, _ in items) == list(range(n_items))
    assert all(e == steps_of(it) for it, e in items)
    costs = [steps_of(it) for it, _ in items]
    assert costs == sorted(costs, reverse=True)
    # pieces record their group's size
    for it, a, e, g, npc in pieces.tolist():
        assert npc == sum(1 for x in pieces.tolist() if x[3] == g)


def test_group_lists_with_partial_tiles_break_on_key_tiles():
    """12x22x24 with 6x8x8 tiles (the last H row partial): the per-unit
    ranges are whole key tiles, so every piece starts on a key tile's first
    (always existing) token."""
    from sliding_tile_attention_sta_amd.synthetic import Workload
    w = Workload("small-partial", 21, (12, 22, 24), (6, 8, 8), ((3, 3, 3),) * 8, 128, "bf16")
    p = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=True)
    assert len(p.group_lists()) == 257 and p.info.partial_tiles == 1
    _check_group_lists(w, p, True)


def test_group_lists_only_where_they_pay():
    """Per-work-group ranges replace whole items only where the balanced
    range beats one round of the costliest item by the range overhead
    (32 steps) and no item spans more than about 8 ranges: 12x24x24 with 8
    or 2 heads (144 or 36 items of 216 steps) takes them; with 1 head (18
    items, about 15 ranges each) it keeps the 4-way split; 2d (192 items of
    108 steps: 81 per range) and every launch with at least 256 items do
    not."""
    for name, heads, lists in (("small", 8, True), ("small", 2, True), ("small", 1, False), ("2d", 8, False),
                               ("720p", 24, False), ("tiny", 2, False)):
        w = WORKLOADS[name].with_heads(heads)
        i = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
        assert (len(i.group_lists()) > 0) == lists, (name, heads)
        if name == "small" and not lists:
            assert i.info.pieces == 4 * 18   # one round of the 4-way split instead
    lib = L.lib()
    n = ctypes.c_int64()
    assert lib.sta_plan_group_lists(None, None, 0, ctypes.byref(n)) == L.STA_ERR_ARG
    w = WORKLOADS["small"]
    p = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    assert lib.sta_plan_group_lists(p.handle, None, 0, ctypes.byref(n)) == L.STA_ERR_ARG and n.value == 257


def test_tail_is_split_only_where_it_pays():
    """Equal-cost items whose count is not a multiple of the chip's 256
    compute units get their tail split; the mixed-window workload, whose
    decreasing-cost order ends in one-tile items, does not."""
    for name, split in (("720p", True), ("long", True), ("small", True), ("mixed", False), ("tiny", False)):
        w = WORKLOADS[name]
        i = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim).info
        assert (i.pieces > 0) == split, name
        assert i.pieces <= 512


def _create(*args):
    h = ctypes.c_void_p()
    st = L.lib().sta_plan_create(*args, ctypes.byref(h))
    if st == L.STA_OK:
        L.lib().sta_plan_destroy(h)
    return st


def _ints(xs):
    return (ctypes.c_int * len(xs))(*xs)


def test_plan_create_errors():
    t, w1 = _ints([2, 4, 4]), _ints([3, 3, 3])
    assert _create(1, 1, 6, 16, 16, t, w1, 64) == L.STA_OK
    assert _create(1, 1, 7, 16, 16, t, w1, 64) == L.STA_ERR_SHAPE          # 7 % 2
    assert _create(1, 1, 6, 16, 18, t, w1, 64) == L.STA_ERR_SHAPE
    assert _create(1, 1, 6, 16, 16, t, w1, 96) == L.STA_ERR_UNSUPPORTED    # head_dim
    assert _create(1, 1, 6, 16, 16, _ints([1, 2, 2]), w1, 64) == L.STA_ERR_UNSUPPORTED  # 4 tokens/tile
    assert _create(1, 1, 6, 16, 16, t, _ints([0, 3, 3]), 64) == L.STA_ERR_ARG
    assert _create(0, 1, 6, 16, 16, t, w1, 64) == L.STA_ERR_ARG
    assert _create(1, 0, 6, 16, 16, t, w1, 64) == L.STA_ERR_ARG
    assert _create(1, 1, 6, 16, 16, None, w1, 64) == L.STA_ERR_ARG
    assert _create(1, 1, 6, 16, 16, t, None, 64) == L.STA_ERR_ARG
    assert _create(1, 1, 6, 16, 16, _ints([2, 0, 4]), w1, 64) == L.STA_ERR_ARG
    assert L.lib().sta_plan_create(1, 1, 6, 16, 16, t, w1, 64, None) == L.STA_ERR_ARG
    # size limits, all rejected before any list is built (each call returns at once)
    t32 = _ints([1, 1, 32])
    assert _create(1, 1, 4, 32, 64, _ints([4, 32, 64]), w1, 64) == L.STA_ERR_UNSUPPORTED  # 8192 tokens/tile
    assert _create(2, 1, 1, 2048, 1 << 20, t32, w1, 64) == L.STA_ERR_UNSUPPORTED  # 2^32 rows
    # 2^21 tiles x 33 x 33 key tiles each: more (query, key) tile pairs than int32 offsets reach
    assert _create(1, 1, 1, 2048, 32768, t32, _ints([1, 33, 33]), 64) == L.STA_ERR_UNSUPPORTED
    # 40,000 key tiles per list (1.6e9 pairs): the list outgrows the forward kernel's LDS
    assert _create(1, 1, 1, 200, 6400, t32, _ints([1, 200, 200]), 64) == L.STA_ERR_UNSUPPORTED
    assert L.lib().sta_plan_destroy(None) == L.STA_OK


def test_plan_query_errors():
    p = api.Plan(1, 2, (6, 16, 16), (2, 4, 4), [(3, 3, 3)], 64)
    lib = L.lib()
    cnt = ctypes.c_int()
    assert lib.sta_plan_kv_tiles(p.handle, 2, 0, None, 0, ctypes.byref(cnt)) == L.STA_ERR_ARG
    assert lib.sta_plan_kv_tiles(p.handle, 0, 48, None, 0, ctypes.byref(cnt)) == L.STA_ERR_ARG
    buf = (ctypes.c_int32 * 4)()
    assert lib.sta_plan_kv_tiles(p.handle, 0, 0, buf, 4, ctypes.byref(cnt)) == L.STA_ERR_ARG
    assert cnt.value == 27
    small = (ctypes.c_int32 * 10)()
    assert lib.sta_plan_perm(p.handle, small, 10) == L.STA_ERR_ARG
    n = ctypes.c_int64()
    assert lib.sta_plan_schedule(p.handle, None, 0, ctypes.byref(n)) == L.STA_ERR_ARG
    assert n.value == p.info.work_items
    assert lib.sta_plan_get_info(None, ctypes.byref(L.PlanInfo())) == L.STA_ERR_ARG


def test_forward_argument_errors_precede_device_work():
    # Every check below fails on the host, so no device is needed or touched.
    p = api.Plan(1, 2, (6, 16, 16), (2, 4, 4), [(3, 3, 3)], 64)
    lib = L.lib()
    P = ctypes.c_void_p
    q, k, v, o = P(1 << 40), P(2 << 40), P(3 << 40), P(4 << 40)
    assert lib.sta_forward_plan(None, q, k, v, o, 0.125, 0, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan(p.handle, None, k, v, o, 0.125, 0, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan(p.handle, q, k, v, None, 0.125, 0, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan(p.handle, q, k, v, o, 0.0, 0, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan(p.handle, q, k, v, o, -1.0, 0, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan(p.handle, q, k, v, o, float("nan"), 0, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan(p.handle, q, k, v, o, 0.125, 7, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan(p.handle, q, k, v, o, 0.125, 0, 7, 0, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan(p.handle, q, k, v, o, 0.125, 0, 1, 5, None) == L.STA_ERR_ARG
    # out overlapping an input
    assert lib.sta_forward_plan(p.handle, q, k, v, P((1 << 40) + 64), 0.125, 0, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_tile_reorder(p.handle, q, P((1 << 40) + 64), 0, None) == L.STA_ERR_ARG
    assert lib.sta_tile_reorder(None, q, o, 0, None) == L.STA_ERR_ARG
    assert lib.sta_tile_unreorder(p.handle, q, o, 9, None) == L.STA_ERR_ARG
    t, win = _ints([2, 4, 4]), _ints([3, 3, 3, 3, 3, 3])
    # not whole tiles: a partial-tile plan, which takes the natural layout only
    assert lib.sta_forward(q, k, v, o, 1, 2, 7, 16, 16, t, win, 64, 0.125, 0, 1, L.STA_LAYOUT_TILE_MAJOR,
                           None) == L.STA_ERR_UNSUPPORTED
    assert lib.sta_forward(q, k, v, o, 1, 2, 6, 16, 16, t, win, 80, 0.125, 0, 1, 0, None) == L.STA_ERR_UNSUPPORTED
    assert lib.sta_forward(q, k, v, o, 1, 2, 6, 16, 16, None, win, 64, 0.125, 0, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_clear_plan_cache() == L.STA_OK


# ---------------------------------------------------------------------------
# Backward plan tables
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "small", "720p", "mixed", "2d", "2d-fine"])
def test_inverse_lists_match_oracle(name):
    from oracle import sta_oracle_bwd as OB
    w = WORKLOADS[name]
    p = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    grid = O.tile_grid(w.video, w.tile)
    nT, nH, nW = grid
    heads = range(w.heads) if w.heads <= 8 else range(0, 4)
    for h in heads:
        for kt in range(0, nT * nH * nW, 5 if nT * nH * nW > 64 else 1):
            c = (kt // (nH * nW), (kt // nW) % nH, kt % nW)
            want = [(a * nH + b) * nW + cc for a, b, cc in OB.query_tiles_seeing(c, w.windows[h], grid)]
            assert p.q_tiles(h, kt) == want


@pytest.mark.parametrize("name", ["tiny", "small", "720p", "mixed", "720p-exact", "partial-small"])
def test_backward_schedules_cover_every_item_once(name):
    w = WORKLOADS[name]
    partial = any(e % t for e, t in zip(w.video, w.tile))
    p = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=partial)
    info = p.info
    assert info.bwd_supported == 1
    for which, count, per in ((0, info.bwd_items_dq, info.bwd_queries_per_item),
                              (1, info.bwd_items_dkdv, info.bwd_keys_per_item)):
        assert info.tile_tokens % per == 0
        n_items = w.batch * w.heads * info.n_tiles * (info.tile_tokens // per)
        s = p.schedule_bwd(which).numpy()
        assert len(s) == count and len(s) % 8 == 0
        assert sorted(s[s >= 0].tolist()) == list(range(n_items))
        assert (s[s < 0] == -1).all()
    subs = info.tile_tokens // info.bwd_keys_per_item
    # the dK/dV items are ordered by the length of their inverse list
    s = p.schedule_bwd(1).numpy()
    for x in range(8):
        lens = []
        for c in s[x::8].tolist():
            if c >= 0:
                rest = c // subs
                lens.append(len(p.q_tiles((rest // info.n_tiles) % w.heads, rest % info.n_tiles)))
        assert lens == sorted(lens, reverse=True)


def test_backward_argument_errors_precede_device_work():
    p = api.Plan(1, 2, (6, 16, 16), (2, 4, 4), [(3, 3, 3)], 64)
    lib = L.lib()
    P = ctypes.c_void_p
    q, k, v, o, g = P(1 << 40), P(2 << 40), P(3 << 40), P(4 << 40), P(5 << 40)
    lse, dl, dq, dk, dv = P(6 << 40), P(7 << 40), P(8 << 40), P(9 << 40), P(10 << 40)
    ok = (p.handle, q, k, v, o, g, lse, dl, dq, dk, dv, 0.125, 0, 1, 1, 0, None)

    def call(**kw):
        args = list(ok)
        names = ["plan", "q", "k", "v", "o", "g", "lse", "dl", "dq", "dk", "dv", "scale", "in_dt",
                 "out_dt", "grad_dt", "layout", "stream"]
        for key, val in kw.items():
            args[names.index(key)] = val
        return lib.sta_backward_plan(*args)

    for name in ["plan", "q", "k", "v", "o", "g", "lse", "dl", "dq", "dk", "dv"]:
        assert call(**{name: None}) == L.STA_ERR_ARG, name
    assert call(scale=0.0) == L.STA_ERR_ARG
    assert call(scale=float("inf")) == L.STA_ERR_ARG
    assert call(in_dt=3) == L.STA_ERR_ARG
    assert call(out_dt=3) == L.STA_ERR_ARG
    assert call(grad_dt=3) == L.STA_ERR_ARG
    assert call(layout=2) == L.STA_ERR_ARG
    # written buffers overlapping an input or each other
    assert call(dq=P((1 << 40) + 64)) == L.STA_ERR_ARG
    assert call(dv=P((4 << 40) + 64)) == L.STA_ERR_ARG
    assert call(dk=P((8 << 40) + 64)) == L.STA_ERR_ARG
    assert call(dl=P((6 << 40) + 4)) == L.STA_ERR_ARG
    assert call(dl=P((10 << 40) + 4)) == L.STA_ERR_ARG
    assert lib.sta_forward_plan_lse(p.handle, q, k, v, o, None, 0.125, 0, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan_lse(p.handle, q, k, v, o, P((3 << 40) + 8), 0.125, 0, 1, 0, None) == L.STA_ERR_ARG
    assert lib.sta_forward_plan_lse(None, q, k, v, o, lse, 0.125, 0, 1, 0, None) == L.STA_ERR_ARG


# ---------------------------------------------------------------------------
# Window search (host parts)
# ---------------------------------------------------------------------------

def test_window_candidates_match_oracle():
    from oracle import sta_oracle_search as OS
    for grid in [(5, 6, 10), (1, 1, 1), (3, 4, 4), (2, 7, 1)]:
        assert api.window_candidates(grid) == OS.odd_candidates(grid)


def test_window_select_matches_oracle():
    import numpy as np
    from oracle import sta_oracle_search as OS
    rng = np.random.default_rng(8)
    for grid in [(5, 6, 10), (3, 4, 4)]:
        cands = OS.odd_candidates(grid) + [(9, 1, 2), (2, 2, 2)]
        for _ in range(40):
            err = rng.uniform(0, 1, size=(5, len(cands)))
            err[:, rng.integers(len(cands))] = 0.3
            err[rng.integers(5)] = 2.0                     # a head with no candidate in range
            for tau in (0.05, 0.3, 0.7):
                assert api.window_select(err, cands, grid, tau) == OS.select_windows(err, cands, grid, tau)


def test_window_search_argument_errors():
    lib = L.lib()
    P = ctypes.c_void_p
    err = (ctypes.c_double * 4)()
    t = _ints([2, 4, 4])
    c = _ints([1, 1, 1, 3, 3, 3])
    assert lib.sta_window_errors(None, P(1), P(2), 1, 2, 6, 16, 16, t, 64, 0.125, 0, 0, c, 2, err, None) == L.STA_ERR_ARG
    # extents that are not whole tiles: partial tiles, natural layout only
    assert lib.sta_window_errors(P(1), P(2), P(3), 1, 2, 7, 16, 16, t, 64, 0.125, 0, L.STA_LAYOUT_TILE_MAJOR, c, 2,
                                 err, None) == L.STA_ERR_UNSUPPORTED
    assert lib.sta_window_errors(P(1), P(2), P(3), 1, 2, 6, 16, 16, t, 64, 0.125, 0, 0, _ints([1, 0, 1]), 1, err, None) == L.STA_ERR_ARG
    assert lib.sta_window_errors(P(1), P(2), P(3), 1, 2, 6, 16, 16, t, 80, 0.125, 0, 0, c, 2, err, None) == L.STA_ERR_UNSUPPORTED
    out = _ints([0] * 6)
    assert lib.sta_window_select(2, _ints([3, 4, 4]), c, 2, None, 0.1, out) == L.STA_ERR_ARG
    assert lib.sta_window_select(0, _ints([3, 4, 4]), c, 2, err, 0.1, out) == L.STA_ERR_ARG
    cnt = ctypes.c_int()
    assert lib.sta_window_candidates(_ints([0, 1, 1]), None, 0, ctypes.byref(cnt)) == L.STA_ERR_ARG


# ---------------------------------------------------------------------------
# Partial tiles (extents that are not multiples of the tile size)
# ---------------------------------------------------------------------------

def test_partial_plan_geometry_and_unsupported_paths():
    video, tile, window = (30, 45, 80), (6, 8, 8), (3, 3, 3)
    assert _create(1, 2, *video, _ints(list(tile)), _ints(list(window) * 2), 128) == L.STA_ERR_SHAPE
    p = api.Plan(1, 2, video, tile, [window], 128, partial_tiles=True)
    info = p.info
    grid = O.tile_grid(video, tile, partial=True)
    assert tuple(info.grid) == grid == (5, 6, 10)
    assert info.partial_tiles == 1 and info.bwd_supported == 1
    nT, nH, nW = grid
    for qt in range(0, nT * nH * nW, 3):
        c = (qt // (nH * nW), (qt // nW) % nH, qt % nW)
        (t0, t1), (y0, y1), (z0, z1) = O.window_tiles(c, window, grid)
        want = sorted((a * nH + b) * nW + cc for a in range(t0, t1) for b in range(y0, y1)
                      for cc in range(z0, z1))
        assert p.kv_tiles(0, qt) == want
    lib = L.lib()
    P = ctypes.c_void_p
    q, k, v, o = P(1 << 40), P(2 << 40), P(3 << 40), P(4 << 40)
    buf = (ctypes.c_int32 * info.tokens)()
    assert lib.sta_plan_perm(p.handle, buf, info.tokens) == L.STA_ERR_UNSUPPORTED
    assert lib.sta_tile_reorder(p.handle, q, o, 0, None) == L.STA_ERR_UNSUPPORTED
    assert lib.sta_forward_plan(p.handle, q, k, v, o, 0.125, 0, 1, L.STA_LAYOUT_TILE_MAJOR, None) == L.STA_ERR_UNSUPPORTED
    g, lse, dl, dq, dk, dv = (P(i << 40) for i in range(5, 11))
    # the backward runs on partial plans in the natural layout only
    assert lib.sta_backward_plan(p.handle, q, k, v, o, g, lse, dl, dq, dk, dv, 0.125, 0, 1, 1,
                                 L.STA_LAYOUT_TILE_MAJOR, None) == L.STA_ERR_UNSUPPORTED
    for which, per in ((0, info.bwd_queries_per_item), (1, info.bwd_keys_per_item)):
        s = p.schedule_bwd(which).numpy()
        assert sorted(s[s >= 0].tolist()) == list(range(2 * info.n_tiles * (info.tile_tokens // per)))
    h = ctypes.c_void_p()
    assert lib.sta_plan_create_ex(1, 2, *video, _ints(list(tile)), _ints(list(window) * 2), 128, 6,
                                  ctypes.byref(h)) == L.STA_ERR_ARG
    # whole tiles through the flag: an ordinary plan
    q2 = api.Plan(1, 2, (30, 48, 80), tile, [window], 128, partial_tiles=True)
    assert q2.info.partial_tiles == 0 and q2.info.bwd_supported == 1


# ---------------------------------------------------------------------------
# Token-wise SWA plans
# ---------------------------------------------------------------------------

def test_swa_plan_info_and_unsupported_paths():
    p = api.Plan(1, 2, (30, 48, 80), (6, 8, 8), [(18, 24, 24), (100, 5, 3)], 128, token_windows=True)
    info = p.info
    assert info.swa == 1 and info.bwd_supported == 0 and info.kernel_variant == 1
    # permitted pairs only: every query sees prod(min(w, extent)) keys
    assert info.flops == 4.0 * 115200 * (18 * 24 * 24 + 30 * 5 * 3) * 128
    s = p.schedule().numpy()
    assert sorted(s[s >= 0].tolist()) == list(range(2 * 300))
    lib = L.lib()
    P = ctypes.c_void_p
    q, k, v, o = P(1 << 40), P(2 << 40), P(3 << 40), P(4 << 40)
    assert lib.sta_forward_plan(p.handle, q, k, v, o, 0.125, 0, 1, L.STA_LAYOUT_TILE_MAJOR, None) == L.STA_ERR_UNSUPPORTED
    assert lib.sta_tile_reorder(p.handle, q, o, 0, None) == L.STA_ERR_UNSUPPORTED
    buf = (ctypes.c_int32 * 115200)()
    assert lib.sta_plan_perm(p.handle, buf, 115200) == L.STA_ERR_UNSUPPORTED
    h = ctypes.c_void_p()
    assert lib.sta_swa_plan_create(1, 1, 30, 47, 80, _ints([6, 8, 8]), _ints([3, 3, 3]), 128,
                                   ctypes.byref(h)) == L.STA_ERR_SHAPE
    assert lib.sta_swa_plan_create(1, 1, 30, 48, 80, _ints([6, 8, 8]), _ints([3, 0, 3]), 128,
                                   ctypes.byref(h)) == L.STA_ERR_ARG


def test_swa_schedule_with_cost_sums_beyond_int32():
    # 24 heads x 4096 query tiles x ~32k key steps: the per-item cost prefix
    # sums pass 2^31; every XCD queue must still run in decreasing cost.
    import numpy as np
    video, tile, win, heads = (64, 128, 128), (4, 8, 8), (63, 127, 127), 24
    p = api.Plan(1, heads, video, tile, [win], 128, token_windows=True)
    info = p.info
    grid = [e // t for e, t in zip(video, tile)]

    def start(x, w, e):
        return np.minimum(np.maximum(x - (w - 1) // 2, 0), e - w)

    c = np.stack(np.meshgrid(*(np.arange(g) for g in grid), indexing="ij"), -1).reshape(-1, 3)
    span = [start(c[:, d] * tile[d] + tile[d] - 1, win[d], video[d]) + win[d] - start(c[:, d] * tile[d], win[d], video[d])
            for d in range(3)]
    cost_tile = span[0] * span[1] * ((span[2] + 31) // 32)
    assert int(cost_tile.sum()) * heads > 2 ** 31
    s = p.schedule().numpy()
    codes = s[s >= 0]
    n_items = codes.size
    assert np.array_equal(np.sort(codes), np.arange(n_items))
    subs = n_items // (heads * info.n_tiles)
    assert subs * heads * info.n_tiles == n_items
    cost = cost_tile[(codes // subs) % info.n_tiles]
    full = np.full(s.shape, -1, dtype=np.int64)
    full[s >= 0] = cost
    for x in range(8):
        q = full[x::8]
        q = q[q >= 0]
        assert np.all(np.diff(q) <= 0)


# ---------------------------------------------------------------------------
# Walk order of the key-tile lists (forward, dQ) and their inverses (dK/dV)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["720p", "mixed", "2d", "small"])
def test_walk_order_is_residue_order(name):
    """The kernels walk a window's key tiles in raster order of their
    coordinates' residues modulo the window (one-to-one inside a window), and
    a key tile's query tiles by the same residue, ties in raster order; both
    lists hold exactly the tiles of the sorted queries."""
    from oracle import sta_oracle as O
    w = WORKLOADS[name]
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    grid = O.tile_grid(w.video, w.tile)
    coord = lambda t: (t // (grid[1] * grid[2]), (t // grid[2]) % grid[1], t % grid[2])
    rng = np.random.default_rng(5)
    n_tiles = grid[0] * grid[1] * grid[2]
    for h in sorted(set(range(0, w.heads, max(1, w.heads // 6))) | {w.heads - 1}):
        we = O.effective_window(w.windows[h], grid)
        res = lambda t: tuple(c % e for c, e in zip(coord(t), we))
        for t in sorted(set(rng.integers(0, n_tiles, size=12).tolist()) | {0, n_tiles - 1}):
            walk = plan.walk(0, h, t)
            assert sorted(walk) == plan.kv_tiles(h, t)
            keys = [res(x) for x in walk]
            assert keys == sorted(keys) and len(set(keys)) == len(keys), (h, t)
            inv = plan.walk(1, h, t)
            assert sorted(inv) == plan.q_tiles(h, t)
            keys = [(res(x), x) for x in inv]
            assert keys == sorted(keys), (h, t)
    with pytest.raises(L.StaError):
        plan.walk(2, 0, 0)
