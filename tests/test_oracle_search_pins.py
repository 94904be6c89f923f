"""Pins of the window-search oracle (oracle/sta_oracle_search.py), CPU only.

  * a window covering the grid has error exactly zero,
  * a constant V gives every window error zero, so the cheapest wins,
  * attention confined to each query's own tile makes the 1x1x1 window
    exact (closed form),
  * the error of a candidate against torch's float64 dense attention,
  * the choice satisfies its defining constraints on random error tables,
  * planted mistakes in a copy of the oracle must each fail a pin.
"""

import math
import types

import numpy as np
import pytest
import torch

from oracle import sta_oracle as F
from oracle import sta_oracle_search as S

VIDEO, TILE = (4, 6, 4), (2, 3, 2)
GRID = (2, 2, 2)
N, D = 96, 8


def _rand(rng, heads=2):
    return tuple(rng.standard_normal((1, heads, N, D)) for _ in range(3))


def pin_full_window_is_exact(mod, seed=1):
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng)
    cands = [(2, 2, 2), (5, 9, 3), (1, 1, 1)]
    err = mod.window_errors(q, k, v, VIDEO, TILE, cands, scale=0.4)
    fails = []
    if not (err[:, 0] == 0).all() or not (err[:, 1] == 0).all():
        fails.append(("full window error", err[:, :2].tolist()))
    if not (err[:, 2] > 0).all():
        fails.append(("1x1x1 error not positive", err[:, 2].tolist()))
    return fails


def pin_constant_v(mod, seed=2):
    rng = np.random.default_rng(seed)
    q, k, _ = _rand(rng)
    v = np.ones_like(q) * rng.standard_normal(D)
    cands = S.odd_candidates(GRID) + [(1, 2, 1)]
    err = mod.window_errors(q, k, v, VIDEO, TILE, cands, scale=0.4)
    fails = []
    if not np.allclose(err, 0.0, atol=1e-12):
        fails.append(("constant v", float(np.abs(err).max())))
    if mod.select_windows(err, cands, GRID, 1e-9) != [(1, 1, 1)] * 2:
        fails.append(("constant v choice", mod.select_windows(err, cands, GRID, 1e-9)))
    return fails


def pin_tile_confined_attention(mod):
    # q_x = alpha e_tile(x), k_y = e_tile(y): scores are alpha within the
    # query's own tile and 0 elsewhere, so with alpha = 80 every other tile
    # carries a relative weight below e^-80 and the 1x1x1 window is exact.
    coords = F.natural_coords(VIDEO)
    tid = [(c[0] // TILE[0]) * 4 + (c[1] // TILE[1]) * 2 + c[2] // TILE[2] for c in coords]
    q = np.zeros((1, 1, N, D))
    k = np.zeros((1, 1, N, D))
    for n, t in enumerate(tid):
        q[0, 0, n, t] = 80.0
        k[0, 0, n, t] = 1.0
    v = np.random.default_rng(3).standard_normal((1, 1, N, D))
    cands = [(2, 2, 2), (1, 2, 1), (1, 1, 1), (2, 1, 2)]
    err = mod.window_errors(q, k, v, VIDEO, TILE, cands, scale=1.0)
    fails = []
    if not err[0, 2] < 1e-30:
        fails.append(("1x1x1 not exact", float(err[0, 2])))
    if mod.select_windows(err, cands, GRID, 1e-20) != [(1, 1, 1)]:
        fails.append(("choice", mod.select_windows(err, cands, GRID, 1e-20)))
    return fails


def pin_error_against_dense_library(mod, seed=4):
    # grid (6, 3, 2): a 3x3x3 window is not the whole grid here
    video, tile = (6, 6, 4), (1, 2, 2)
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((1, 2, 144, D)) for _ in range(3))
    scale = 1.0 / math.sqrt(D)
    cands = [(1, 2, 1), (3, 3, 3), (5, 1, 2)]
    err = mod.window_errors(q, k, v, video, tile, cands, scale=scale)
    dense = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), scale=scale).numpy()
    fails = []
    for c, w in enumerate(cands):
        o = F.sta_forward_explicit(q, k, v, video, tile, [w] * 2, scale=scale)
        for h in range(2):
            want = np.linalg.norm(o[:, h] - dense[:, h]) / np.linalg.norm(dense[:, h])
            if abs(err[h, c] - want) > 1e-12:
                fails.append(("error", h, w, float(err[h, c]), float(want)))
    return fails


def pin_choice_constraints(mod, seed=5):
    rng = np.random.default_rng(seed)
    grid = (5, 6, 10)
    cands = S.odd_candidates(grid) + [(7, 2, 3), (2, 2, 2), (3, 3, 3)]
    fails = []
    # a window wider than the grid costs its clamped extent: (7, 2, 3) costs
    # 5 * 2 * 3 = 30 and beats (5, 1, 7) at 35
    err = np.ones((1, len(cands)))
    err[0, cands.index((7, 2, 3))] = 0.0
    err[0, cands.index((5, 1, 7))] = 0.0
    if mod.select_windows(err, cands, grid, 0.5) != [(7, 2, 3)]:
        fails.append(("clamped cost", mod.select_windows(err, cands, grid, 0.5)))
    # an error equal to the threshold is within it
    err = np.ones((1, len(cands)))
    err[0, 0] = 0.3
    if mod.select_windows(err, cands, grid, 0.3) != [cands[0]]:
        fails.append(("threshold inclusive", mod.select_windows(err, cands, grid, 0.3)))
    # nothing meets the threshold: the full window
    if mod.select_windows(np.ones((2, len(cands))), cands, grid, 0.5) != [grid] * 2:
        fails.append(("fallback", mod.select_windows(np.ones((2, len(cands))), cands, grid, 0.5)))
    for trial in range(50):
        err = rng.uniform(0, 1, size=(3, len(cands)))
        err[:, rng.integers(len(cands))] = 0.25          # an exact tie somewhere
        tau = float(rng.uniform(0.05, 0.6))
        got = mod.select_windows(err, cands, grid, tau)
        for h in range(3):
            ok = [c for c in range(len(cands)) if err[h, c] <= tau]
            if not ok:
                if got[h] != grid:
                    fails.append(("fallback", trial, h, got[h]))
                continue
            cost = lambda c: int(np.prod([min(a, n) for a, n in zip(cands[c], grid)]))
            cmin = min(cost(c) for c in ok)
            cheapest = [c for c in ok if cost(c) == cmin]
            emin = min(err[h, c] for c in cheapest)
            first = min(c for c in cheapest if err[h, c] == emin)
            if got[h] != tuple(cands[first]):
                fails.append(("choice", trial, h, got[h], cands[first]))
    return fails


def pin_search_over_samples(mod, seed=6):
    # W4 by its properties: one sample gives that sample's errors; a sample
    # given twice changes nothing; the order of the samples does not matter;
    # every mean lies between the samples' errors; the choice is W3 on it.
    rng = np.random.default_rng(seed)
    s1, s2 = _rand(rng), tuple(2.0 * x for x in _rand(rng))
    cands = S.odd_candidates(GRID) + [(1, 2, 1)]
    e1 = mod.window_errors(*s1, VIDEO, TILE, cands, scale=0.4)
    e2 = mod.window_errors(*s2, VIDEO, TILE, cands, scale=0.4)
    fails = []
    w1, m1 = mod.search([s1], VIDEO, TILE, cands, 0.3, scale=0.4)
    if not np.array_equal(m1, e1):
        fails.append(("one sample", float(np.abs(m1 - e1).max())))
    _, m11 = mod.search([s1, s1], VIDEO, TILE, cands, 0.3, scale=0.4)
    if not np.array_equal(m11, e1):
        fails.append(("duplicate sample", float(np.abs(m11 - e1).max())))
    w12, m12 = mod.search([s1, s2], VIDEO, TILE, cands, 0.3, scale=0.4)
    _, m21 = mod.search([s2, s1], VIDEO, TILE, cands, 0.3, scale=0.4)
    if not np.array_equal(m12, m21):
        fails.append(("sample order", float(np.abs(m12 - m21).max())))
    if not ((m12 >= np.minimum(e1, e2)) & (m12 <= np.maximum(e1, e2))).all() or np.array_equal(e1, e2):
        fails.append(("mean outside the samples' errors",))
    if w12 != mod.select_windows(m12, cands, GRID, 0.3) or w1 != mod.select_windows(e1, cands, GRID, 0.3):
        fails.append(("choice", w12))
    return fails


def pin_partial_grid(mod, seed=7):
    # 5x7x3 with 2x3x2 tiles: grid (3, 3, 2), the last tile of every axis
    # partial.  The grid window (and a wider one) is dense attention over the
    # existing tokens, so its error is exactly zero; a candidate's error
    # equals the one computed against torch's float64 dense attention (the
    # forward oracle's partial tiles are pinned by brute force).
    video, tile, grid = (5, 7, 3), (2, 3, 2), (3, 3, 2)
    n = 5 * 7 * 3
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((1, 2, n, D)) for _ in range(3))
    scale = 0.45
    cands = [grid, (4, 5, 9), (1, 1, 1), (3, 1, 2), (1, 3, 1)]
    err = mod.window_errors(q, k, v, video, tile, cands, scale=scale, partial=True)
    dense = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), scale=scale).numpy()
    fails = []
    if not (err[:, :2] == 0).all():
        fails.append(("full window error on a partial grid", err[:, :2].tolist()))
    for c, w in enumerate(cands[2:], 2):
        o = F.sta_forward_explicit(q, k, v, video, tile, [w] * 2, scale=scale, partial=True)
        for h in range(2):
            want = np.linalg.norm(o[:, h] - dense[:, h]) / np.linalg.norm(dense[:, h])
            if not want > 0 or abs(err[h, c] - want) > 1e-12:
                fails.append(("partial error", h, w, float(err[h, c]), float(want)))
    windows, _ = mod.search([(q, k, v)], video, tile, cands[2:], -1.0, scale=scale, partial=True)
    if windows != [grid] * 2:
        fails.append(("fallback on a partial grid", windows))
    return fails


ALL_PINS = [pin_full_window_is_exact, pin_constant_v, pin_tile_confined_attention,
            pin_error_against_dense_library, pin_choice_constraints, pin_search_over_samples,
            pin_partial_grid]


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


def test_odd_candidates():
    assert S.odd_candidates((5, 6, 10))[:3] == [(1, 1, 1), (1, 1, 3), (1, 1, 5)]
    assert len(S.odd_candidates((5, 6, 10))) == 3 * 4 * 6
    assert S.odd_candidates((1, 2, 1)) == [(1, 1, 1), (1, 2, 1)]


MUTANTS = [
    ("normalised by the candidate", "den = math.sqrt(float((full[:, h] ** 2).sum()))",
     "den = math.sqrt(float((o[:, h] ** 2).sum()))"),
    ("squared error", "err[h, c] = num / den", "err[h, c] = (num / den) ** 2"),
    ("cost without clamp", "we = F.effective_window(window, grid)", "we = tuple(window)"),
    ("tie to the larger error", "key = (window_cost(w, grid), err[h, c], c)",
     "key = (window_cost(w, grid), -err[h, c], c)"),
    ("fallback to the last candidate", "out.append(best[1] if best is not None else tuple(int(n) for n in grid))",
     "out.append(best[1] if best is not None else tuple(candidates[-1]))"),
    ("strict threshold", "if not err[h, c] <= threshold:", "if not err[h, c] < threshold:"),
    ("sum of the samples, not their mean", "    mean /= len(errs)\n", "    pass\n"),
    ("last sample only", "        mean += e\n", "        mean = e.copy()\n"),
    ("dense reference with a 3-tile window",
     "full = F.sta_forward_explicit(q, k, v, video, tile, [grid] * heads, scale=scale, partial=partial)",
     "full = F.sta_forward_explicit(q, k, v, video, tile, [(3, 3, 3)] * heads, scale=scale, partial=partial)"),
    ("partial tiles dropped from the grid", "grid = F.tile_grid(video, tile, partial)",
     "grid = tuple(e // t for e, t in zip(video, tile))"),
    ("partial flag not passed to the candidates",
     "o = F.sta_forward_explicit(q, k, v, video, tile, [tuple(w)] * heads, scale=scale, partial=partial)",
     "o = F.sta_forward_explicit(q, k, v, video, tile, [tuple(w)] * heads, scale=scale, partial=False)"),
]


def _mutant(src, old, new, tag):
    assert old in src, tag
    mod = types.ModuleType("sta_oracle_search_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new, 1), f"<mutant {tag}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("tag,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tag, old, new):
    with open(S.__file__) as f:
        src = f.read()
    assert run_pins(_mutant(src, old, new, tag)) != [], f"mutant '{tag}' survived every pin"
