"""Pins of the token-wise SWA oracle (oracle/sta_oracle_swa.py), CPU only:
brute force by nested loops, dense and identity special cases, equality
with the STA oracle for 1x1x1 tiles, the per-query-tile form, and planted
mistakes that must each fail a pin."""

import math
import types

import numpy as np
import pytest
import torch

from oracle import sta_oracle as F
from oracle import sta_oracle_swa as S


def bf_swa_keys(x, video, window):
    """Window of query x by search: among the runs of min(w, E) consecutive
    tokens inside the axis that contain x, the one whose centre is nearest x,
    ties to the later run; keys gathered by nested loops."""
    starts = []
    for d in range(3):
        e, w = video[d], min(window[d], video[d])
        best = None
        for s in range(0, e - w + 1):
            if s <= x[d] < s + w:
                off = abs(s + (w - 1) / 2.0 - x[d])
                if best is None or off < best[0] - 1e-12 or (abs(off - best[0]) < 1e-12 and s > best[1]):
                    best = (off, s)
        starts.append((best[1], w))
    T, H, W = video
    keys = []
    for t in range(starts[0][0], starts[0][0] + starts[0][1]):
        for y in range(starts[1][0], starts[1][0] + starts[1][1]):
            for z in range(starts[2][0], starts[2][0] + starts[2][1]):
                keys.append((t * H + y) * W + z)
    return sorted(keys)


def pin_bruteforce(mod, seed=3):
    rng = np.random.default_rng(seed)
    fails = []
    for _ in range(4):
        video = tuple(int(x) for x in rng.integers(2, 7, size=3))
        windows = [tuple(int(x) for x in rng.integers(1, 8, size=3)) for _ in range(2)]
        N, D = int(np.prod(video)), 3
        q, k, v = (rng.standard_normal((1, 2, N, D)) for _ in range(3))
        got = mod.swa_forward_explicit(q, k, v, video, windows, scale=0.7)
        coords = F.natural_coords(video)
        for h in range(2):
            mask = mod.swa_mask(video, windows[h])
            for n in range(N):
                keys = bf_swa_keys(tuple(coords[n]), video, windows[h])
                if np.flatnonzero(mask[n]).tolist() != keys:
                    fails.append(("mask", video, windows[h], n))
                    break
                s = 0.7 * (k[0, h, keys] @ q[0, h, n])
                p = [math.exp(x - s.max()) for x in s]
                want = sum(pi * v[0, h, j] for pi, j in zip(p, keys)) / sum(p)
                if not np.allclose(got[0, h, n], want, rtol=0, atol=1e-12):
                    fails.append(("output", video, windows[h], n))
                    break
    return fails


def pin_special_cases(mod, seed=4):
    rng = np.random.default_rng(seed)
    fails = []
    video = (3, 4, 5)
    N, D = 60, 4
    q, k, v = (rng.standard_normal((1, 2, N, D)) for _ in range(3))
    dense = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), scale=0.5).numpy()
    if not np.allclose(mod.swa_forward_explicit(q, k, v, video, [(3, 4, 5), (9, 9, 9)], scale=0.5), dense,
                       rtol=0, atol=1e-12):
        fails.append("dense")
    if not np.allclose(mod.swa_forward_explicit(q, k, v, video, [(1, 1, 1)] * 2, scale=0.5), v,
                       rtol=0, atol=1e-12):
        fails.append("identity")
    # with 1x1x1 tiles a tile is a token, and STA is token-wise SWA
    for w in [(1, 3, 2), (3, 2, 4), (2, 4, 5)]:
        a = mod.swa_forward_explicit(q, k, v, video, [w] * 2, scale=0.5)
        b = F.sta_forward_explicit(q, k, v, video, (1, 1, 1), [w] * 2, scale=0.5)
        if not np.allclose(a, b, rtol=0, atol=1e-12):
            fails.append(("sta 1x1x1", w))
    return fails


def pin_query_tiles(mod, seed=5):
    rng = np.random.default_rng(seed)
    fails = []
    video, tile = (4, 6, 8), (2, 3, 4)
    N, D = 192, 3
    q, k, v = (rng.standard_normal((1, 1, N, D)) for _ in range(3))
    for window in [(3, 3, 3), (2, 5, 6), (4, 1, 8)]:
        want = mod.swa_forward_explicit(q, k, v, video, [window], scale=0.8)[0, 0].reshape(*video, D)
        tiles = [(a, b, c) for a in range(2) for b in range(2) for c in range(2)]
        outs = mod.swa_forward_query_tiles(*(x.reshape(1, 1, *video, D) for x in (q, k, v)), tile, window, 0,
                                           tiles, scale=0.8)
        for c, o in zip(tiles, outs):
            sl = tuple(slice(c[d] * tile[d], (c[d] + 1) * tile[d]) for d in range(3))
            if not np.allclose(o, want[sl], rtol=0, atol=1e-12):
                fails.append(("tile", window, c))
    return fails


ALL_PINS = [pin_bruteforce, pin_special_cases, pin_query_tiles]


def run_pins(mod):
    fails = []
    for p in ALL_PINS:
        try:
            fails += [(p.__name__, f) for f in p(mod)]
        except Exception as e:  # a mutant may also crash
            fails.append((p.__name__, repr(e)))
    return fails


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    assert pin(S) == []


def test_union_box_holds_every_window():
    video, tile, window = (30, 48, 80), (6, 8, 8), (18, 24, 24)
    for c in [(0, 0, 0), (2, 3, 5), (4, 5, 9)]:
        box = S.swa_union_box(c, tile, window, video)
        for d in range(3):
            for x in range(c[d] * tile[d], (c[d] + 1) * tile[d]):
                s = S.token_window_start(x, window[d], video[d])
                assert box[d][0] <= s and s + window[d] <= box[d][1]


MUTANTS = [
    ("centre", "    s = x - (w - 1) // 2\n", "    s = x - w // 2\n"),
    ("mask centre", "s = np.clip(coords[:, d] - (w - 1) // 2, 0, video[d] - w)",
     "s = np.clip(coords[:, d] - w // 2, 0, video[d] - w)"),
    ("tile mask lower bound", "mask &= (kc[None, :, d] >= s[:, None])", "mask &= (kc[None, :, d] > s[:, None])"),
    ("union too small", "box.append((token_window_start(x0, w, video[d]), token_window_start(x1, w, video[d]) + w))",
     "box.append((token_window_start(x0, w, video[d]), token_window_start(x0, w, video[d]) + w))"),
    ("tile mask bound", "(kc[None, :, d] < s[:, None] + w)", "(kc[None, :, d] <= s[:, None] + w)"),
]


def _mutant(src, old, new, tag):
    assert old in src, tag
    mod = types.ModuleType("sta_oracle_swa_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new, 1), f"<mutant {tag}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("tag,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tag, old, new):
    with open(S.__file__) as f:
        src = f.read()
    assert run_pins(_mutant(src, old, new, tag)) != [], f"mutant '{tag}' survived every pin"
