"""Pins of the CPU oracle to things other than itself (CPU only).

The pages print no numeric example, so the oracle is pinned by:
  * hand-derived worked examples and window-start tables (tests/golden/),
  * an independent brute force (window chosen by search, keys gathered by
    nested loops over tiles and tokens),
  * special cases that reduce to a library routine (full window == dense
    attention, 1x1x1 window == block-diagonal attention, both against
    torch's scaled_dot_product_attention in float64),
  * closed forms (Q = 0 gives the window mean of V; a one-hot V reads the
    key-tile set back) and invariants (token-order equivariance, shifts of K
    and V, head permutation, convexity),
  * and mutation checks: textual mutants of the oracle (a wrong window
    centre, a missing clamp, a dropped scale, a dropped normaliser, a wrong
    slice) must each fail at least one pin.
"""

import importlib.util
import itertools
import json
import math
import os
import sys
import types

import numpy as np
import pytest
import torch

from oracle import sta_oracle as O
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_qkv

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Independent references used by the pins
# ---------------------------------------------------------------------------

def bf_start(c, w, n):
    """Window start by search: among the windows of min(w, n) consecutive
    tiles that lie inside the grid and contain c, the one whose centre is
    closest to c; on a tie (even windows) the later one."""
    wv = min(w, n)
    best = None
    for s in range(0, n - wv + 1):
        if s <= c < s + wv:
            off = abs((s + (wv - 1) / 2.0) - c)
            if best is None or off < best[0] - 1e-12 or (abs(off - best[0]) < 1e-12 and s > best[1]):
                best = (off, s)
    return best[1]


def bf_keys(qx, video, tile, window):
    """Key token indices (natural order) permitted for query token qx, by
    nested loops over the window's tiles and over each tile's tokens."""
    T, H, W = video
    grid = [video[i] // tile[i] for i in range(3)]
    c = [qx[i] // tile[i] for i in range(3)]
    starts = [bf_start(c[i], window[i], grid[i]) for i in range(3)]
    ext = [min(window[i], grid[i]) for i in range(3)]
    keys = []
    for a in range(starts[0], starts[0] + ext[0]):
        for b in range(starts[1], starts[1] + ext[1]):
            for cc in range(starts[2], starts[2] + ext[2]):
                for lt in range(tile[0]):
                    for ly in range(tile[1]):
                        for lz in range(tile[2]):
                            t, y, z = a * tile[0] + lt, b * tile[1] + ly, cc * tile[2] + lz
                            keys.append((t * H + y) * W + z)
    return sorted(keys)


def bf_attention(q, k, v, video, tile, windows, scale):
    """Per-query loop: gather permitted keys, softmax with math.exp in fp64."""
    B, heads, N, D = q.shape
    T, H, W = video
    out = np.zeros((B, heads, N, v.shape[-1]))
    for h in range(heads):
        for n in range(N):
            qx = (n // (H * W), (n // W) % H, n % W)
            keys = bf_keys(qx, video, tile, windows[h])
            for b in range(B):
                s = [scale * float(np.dot(q[b, h, n].astype(np.float64), k[b, h, j].astype(np.float64)))
                     for j in keys]
                m = max(s)
                p = [math.exp(x - m) for x in s]
                tot = sum(p)
                acc = np.zeros(v.shape[-1])
                for pj, j in zip(p, keys):
                    acc += pj * v[b, h, j].astype(np.float64)
                out[b, h, n] = acc / tot
    return out


def sdpa64(q, k, v, scale):
    """torch's scaled_dot_product_attention on the CPU in float64."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)) for x in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()


def rand_case(rng, max_tokens=160):
    while True:
        tile = tuple(int(x) for x in rng.integers(1, 4, size=3))
        grid = tuple(int(x) for x in rng.integers(1, 5, size=3))
        video = tuple(t * g for t, g in zip(tile, grid))
        if video[0] * video[1] * video[2] <= max_tokens:
            break
    heads = 2
    windows = [tuple(int(x) for x in rng.integers(1, 6, size=3)) for _ in range(heads)]
    return video, tile, windows


# ---------------------------------------------------------------------------
# The pin set, parameterised by the oracle module so that mutants can be run
# ---------------------------------------------------------------------------

def pin_worked_examples(mod):
    g = _load("worked_examples.json")
    fails = []
    for case in g["cases"]:
        video, tile, window = (1, 1, 4), (1, 1, 1), tuple(case["window"])
        q = np.full((1, 1, 4, 1), math.log(2.0))
        k = np.arange(4, dtype=np.float64).reshape(1, 1, 4, 1)
        v = k.copy()
        want = np.array(case["output_num"], dtype=np.float64) / np.array(case["output_den"])
        got = mod.sta_forward_explicit(q, k, v, video, tile, [window], scale=1.0)[0, 0, :, 0]
        if not np.allclose(got, want, rtol=0, atol=1e-14):
            fails.append(("explicit", case["window"], got.tolist()))
        qn, kn, vn = (x.reshape(1, 1, 1, 1, 4, 1) for x in (q, k, v))
        got2 = np.array([mod.sta_forward_query_tiles(qn, kn, vn, tile, window, 0, [(0, 0, c)], scale=1.0)[0].ravel()[0]
                         for c in range(4)])
        if not np.allclose(got2, want, rtol=0, atol=1e-14):
            fails.append(("query_tiles", case["window"], got2.tolist()))
        starts = [mod.window_tiles((0, 0, c), window, (1, 1, 4))[2][0] for c in range(4)]
        if starts != case["starts"]:
            fails.append(("starts", case["window"], starts))
    return fails


def pin_window_starts(mod):
    g = _load("window_starts.json")
    fails = []
    for ax in g["axes"]:
        we = mod.effective_window((ax["w"], 1, 1), (ax["n"], 1, 1))[0]
        got = [mod.window_start(c, we, ax["n"]) for c in range(ax["n"])]
        if got != ax["starts"] or we != ax["extent"]:
            fails.append((ax["label"], got, we))
    return fails


def pin_bruteforce(mod, cases=6, seed=7):
    rng = np.random.default_rng(seed)
    fails = []
    for _ in range(cases):
        video, tile, windows = rand_case(rng)
        N = video[0] * video[1] * video[2]
        D = 3
        q, k, v = (rng.standard_normal((1, 2, N, D)) for _ in range(3))
        grid = tuple(video[i] // tile[i] for i in range(3))
        coords = mod.natural_coords(video)
        for h in range(2):
            mask = mod.sta_mask(coords, coords, tile, windows[h], grid)
            for n in range(N):
                want = bf_keys(tuple(coords[n]), video, tile, windows[h])
                if np.flatnonzero(mask[n]).tolist() != want:
                    fails.append(("mask", video, tile, windows[h], n))
                    break
        scale = 0.7
        want = bf_attention(q, k, v, video, tile, windows, scale)
        got = mod.sta_forward_explicit(q, k, v, video, tile, windows, scale=scale)
        if not np.allclose(got, want, rtol=0, atol=1e-12):
            fails.append(("explicit", video, tile, windows))
        T, H, W = video
        q6, k6, v6 = (x.reshape(1, 2, T, H, W, D) for x in (q, k, v))
        for h in range(2):
            tiles = list(itertools.product(range(grid[0]), range(grid[1]), range(grid[2])))
            outs = mod.sta_forward_query_tiles(q6, k6, v6, tile, windows[h], h, tiles, scale=scale)
            full = np.zeros((T, H, W, D))
            for c, o in zip(tiles, outs):
                full[c[0] * tile[0]:(c[0] + 1) * tile[0], c[1] * tile[1]:(c[1] + 1) * tile[1],
                     c[2] * tile[2]:(c[2] + 1) * tile[2]] = o
            if not np.allclose(full.reshape(N, D), want[0, h], rtol=0, atol=1e-12):
                fails.append(("query_tiles", video, tile, windows[h]))
    return fails


def pin_dense_and_blockdiag(mod, seed=11):
    rng = np.random.default_rng(seed)
    fails = []
    video, tile = (4, 6, 4), (2, 3, 2)
    N, D = 96, 8
    q, k, v = (rng.standard_normal((1, 2, N, D)) for _ in range(3))
    scale = 1.0 / math.sqrt(D)
    # full window (every axis at least the grid) == dense attention
    got = mod.sta_forward_explicit(q, k, v, video, tile, [(9, 9, 9), (2, 2, 2)], scale=scale)
    if not np.allclose(got, sdpa64(q, k, v, scale), rtol=0, atol=1e-12):
        fails.append("dense")
    # 1x1x1 window == attention inside each tile
    got = mod.sta_forward_explicit(q, k, v, video, tile, [(1, 1, 1)] * 2, scale=scale)
    coords = mod.natural_coords(video)
    tid = [(x[0] // tile[0], x[1] // tile[1], x[2] // tile[2]) for x in coords]
    want = np.zeros_like(got)
    for t in set(tid):
        idx = [i for i in range(N) if tid[i] == t]
        want[:, :, idx] = sdpa64(q[:, :, idx], k[:, :, idx], v[:, :, idx], scale)
    if not np.allclose(got, want, rtol=0, atol=1e-12):
        fails.append("blockdiag")
    return fails


ALL_PINS = [pin_worked_examples, pin_window_starts, pin_bruteforce, pin_dense_and_blockdiag]


def run_pins(mod):
    fails = []
    for p in ALL_PINS:
        try:
            fails += [(p.__name__, f) for f in p(mod)]
        except Exception as e:  # a mutant may also crash
            fails.append((p.__name__, repr(e)))
    return fails


# ---------------------------------------------------------------------------
# Tests
# ---------------------------------------------------------------------------

def test_worked_examples():
    assert pin_worked_examples(O) == []


def test_window_start_tables():
    assert pin_window_starts(O) == []


def test_search_start_equals_closed_form():
    # the brute-force search and the oracle's closed form agree everywhere small
    for n in range(1, 13):
        for w in range(1, 15):
            we = min(w, n)
            for c in range(n):
                assert bf_start(c, w, n) == O.window_start(c, we, n)


def test_bruteforce_random_grids():
    assert pin_bruteforce(O, cases=10, seed=3) == []


def test_dense_and_block_diagonal_special_cases():
    assert pin_dense_and_blockdiag(O) == []


def test_pair_counts_and_flops():
    g = _load("window_starts.json")["pairs_per_head"]
    tiny, big, mixed = WORKLOADS["tiny"], WORKLOADS["720p"], WORKLOADS["mixed"]
    assert O.sta_flops(tiny.video, tiny.tile, tiny.windows, tiny.head_dim) == g["tiny"]["flops"]
    assert O.sta_flops(big.video, big.tile, big.windows, big.head_dim) == g["720p"]["flops"]
    assert O.sta_flops(mixed.video, mixed.tile, mixed.windows, mixed.head_dim) == g["mixed"]["flops"]
    grid = O.tile_grid(big.video, big.tile)
    for w, want in zip([(1, 1, 1), (3, 3, 3), (3, 5, 5), (5, 6, 10)], g["mixed"]["pairs_per_head_cycle"]):
        we = O.effective_window(w, grid)
        assert grid[0] * grid[1] * grid[2] * we[0] * we[1] * we[2] == want


def _tiny_arrays():
    w = WORKLOADS["tiny"]
    q, k, v = (x.double().numpy() for x in make_qkv(w))
    T, H, W = w.video
    N = T * H * W
    return w, q.reshape(1, w.heads, N, -1), k.reshape(1, w.heads, N, -1), v.reshape(1, w.heads, N, -1)


def test_tiny_workload_against_bruteforce():
    w, q, k, v = _tiny_arrays()
    got = O.sta_forward_explicit(q, k, v, w.video, w.tile, w.windows, scale=w.scale)
    # brute force on a subset of query tokens (every 7th) to bound the run time
    T, H, W = w.video
    rows = list(range(0, q.shape[2], 7))
    for h in range(w.heads):
        for n in rows:
            qx = (n // (H * W), (n // W) % H, n % W)
            keys = bf_keys(qx, w.video, w.tile, w.windows[h])
            s = w.scale * (k[0, h, keys] @ q[0, h, n])
            p = np.exp(s - s.max())
            want = (p @ v[0, h, keys]) / p.sum()
            assert np.allclose(got[0, h, n], want, rtol=0, atol=1e-12)


def test_tiny_query_tiles_equal_explicit():
    w, q, k, v = _tiny_arrays()
    got = O.sta_forward_explicit(q, k, v, w.video, w.tile, w.windows, scale=w.scale)
    T, H, W = w.video
    grid = O.tile_grid(w.video, w.tile)
    q6, k6, v6 = (x.reshape(1, w.heads, T, H, W, -1) for x in (q, k, v))
    g6 = got.reshape(1, w.heads, T, H, W, -1)
    tT, tH, tW = w.tile
    for h in range(w.heads):
        tiles = list(itertools.product(*(range(n) for n in grid)))
        for c, o in zip(tiles, O.sta_forward_query_tiles(q6, k6, v6, w.tile, w.windows[h], h, tiles, scale=w.scale)):
            ref = g6[0, h, c[0] * tT:(c[0] + 1) * tT, c[1] * tH:(c[1] + 1) * tH, c[2] * tW:(c[2] + 1) * tW]
            assert np.allclose(o, ref, rtol=0, atol=1e-12)


def test_token_order_equivariance():
    rng = np.random.default_rng(5)
    video, tile, windows = (4, 4, 6), (2, 2, 3), [(1, 3, 2), (3, 1, 1)]
    N, D = 96, 5
    q, k, v = (rng.standard_normal((2, 2, N, D)) for _ in range(3))
    base = O.sta_forward_explicit(q, k, v, video, tile, windows)
    perm = rng.permutation(N)
    coords = O.natural_coords(video)[perm]
    got = O.sta_forward_explicit(q[:, :, perm], k[:, :, perm], v[:, :, perm], video, tile, windows, coords=coords)
    assert np.allclose(got, base[:, :, perm], rtol=0, atol=1e-12)


def test_zero_query_gives_window_mean_and_onehot_readout():
    # Tiny geometry: 48 tiles <= head_dim 64, so V = one-hot(tile id) fits.
    w = WORKLOADS["tiny"]
    T, H, W = w.video
    N = T * H * W
    grid = O.tile_grid(w.video, w.tile)
    coords = O.natural_coords(w.video)
    tid = ((coords[:, 0] // w.tile[0]) * grid[1] + coords[:, 1] // w.tile[1]) * grid[2] + coords[:, 2] // w.tile[2]
    v = np.zeros((1, 1, N, 64))
    v[0, 0, np.arange(N), tid] = 1.0
    q = np.zeros((1, 1, N, 64))
    k = np.random.default_rng(0).standard_normal((1, 1, N, 64))
    out = O.sta_forward_explicit(q, k, v, w.video, w.tile, [(3, 3, 3)])[0, 0]
    starts = {ax["label"]: ax["starts"] for ax in _load("window_starts.json")["axes"]}
    sT, sHW = starts["tiny T"], starts["tiny H/W"]
    for n in range(0, N, 5):
        c = coords[n] // np.array(w.tile)
        expect = np.zeros(64)
        for a in range(sT[c[0]], sT[c[0]] + 3):
            for b in range(sHW[c[1]], sHW[c[1]] + 3):
                for cc in range(sHW[c[2]], sHW[c[2]] + 3):
                    expect[(a * grid[1] + b) * grid[2] + cc] = 1.0 / 27
        assert np.allclose(out[n], expect, rtol=0, atol=1e-15)
    # mean of V over the window for general V
    v2 = np.random.default_rng(1).standard_normal((1, 1, N, 4))
    out2 = O.sta_forward_explicit(np.zeros((1, 1, N, 4)), k[..., :4], v2, w.video, w.tile, [(3, 3, 3)])[0, 0]
    v2n = v2[0, 0].reshape(T, H, W, 4)
    for n in range(0, N, 11):
        c = coords[n] // np.array(w.tile)
        t0, y0, z0 = sT[c[0]] * 2, sHW[c[1]] * 4, sHW[c[2]] * 4
        box = v2n[t0:t0 + 6, y0:y0 + 12, z0:z0 + 12].reshape(-1, 4)
        assert np.allclose(out2[n], box.mean(axis=0), rtol=0, atol=1e-13)


def test_shift_invariances_head_permutation_and_convexity():
    rng = np.random.default_rng(9)
    video, tile, windows = (4, 6, 6), (2, 3, 2), [(1, 3, 3), (3, 1, 2), (2, 2, 1)]
    N, D = 144, 6
    q, k, v = (rng.standard_normal((1, 3, N, D)) for _ in range(3))
    base = O.sta_forward_explicit(q, k, v, video, tile, windows)
    u = rng.standard_normal(D)
    assert np.allclose(O.sta_forward_explicit(q, k + u, v, video, tile, windows), base, atol=1e-12)
    cshift = rng.standard_normal(D)
    assert np.allclose(O.sta_forward_explicit(q, k, v + cshift, video, tile, windows), base + cshift, atol=1e-12)
    perm = [2, 0, 1]
    got = O.sta_forward_explicit(q[:, perm], k[:, perm], v[:, perm], video, tile, [windows[p] for p in perm])
    assert np.allclose(got, base[:, perm], atol=1e-13)
    grid = O.tile_grid(video, tile)
    coords = O.natural_coords(video)
    for h in range(3):
        mask = O.sta_mask(coords, coords, tile, windows[h], grid)
        we = O.effective_window(windows[h], grid)
        V = tile[0] * tile[1] * tile[2]
        assert (mask.sum(axis=1) == V * we[0] * we[1] * we[2]).all()
        assert mask[np.arange(N), np.arange(N)].all()          # own tile always inside
        for n in range(N):
            vals = v[0, h, mask[n]]
            assert (base[0, h, n] >= vals.min(axis=0) - 1e-12).all()
            assert (base[0, h, n] <= vals.max(axis=0) + 1e-12).all()


# ---------------------------------------------------------------------------
# Mutation check: plausible mistakes planted in a copy of the oracle (on the
# CPU) must each be caught by the pins.
# ---------------------------------------------------------------------------

MUTANTS = [
    ("even-window centre", "s = np.clip(cq - (w[d] - 1) // 2, 0, grid[d] - w[d])",
     "s = np.clip(cq - w[d] // 2, 0, grid[d] - w[d])"),
    ("no upper clamp (mask)", "s = np.clip(cq - (w[d] - 1) // 2, 0, grid[d] - w[d])",
     "s = np.maximum(cq - (w[d] - 1) // 2, 0)"),
    ("start formula", "    s = c - (w - 1) // 2\n", "    s = c - w // 2\n"),
    ("no lower clamp", "    if s < 0:\n        s = 0\n", ""),
    ("window not clamped to grid", "return tuple(min(int(w), int(n)) for w, n in zip(window, grid))",
     "return tuple(int(w) for w, n in zip(window, grid))"),
    ("dropped scale", "s = scale * (q @ k.T)", "s = (q @ k.T)"),
    ("dropped normaliser", "return (p @ v) / p.sum(axis=1, keepdims=True)", "return (p @ v)"),
    ("k/v swapped", "s = scale * (q @ k.T)", "s = scale * (q @ v.T)"),
    ("window box y/z swapped", "kt = k[batch, head, t0 * tT:t1 * tT, y0 * tH:y1 * tH, z0 * tW:z1 * tW]",
     "kt = k[batch, head, t0 * tT:t1 * tT, z0 * tH:z1 * tH, y0 * tW:y1 * tW]"),
    ("strict upper bound", "(ck[None, :] < s[:, None] + w[d])", "(ck[None, :] <= s[:, None] + w[d])"),
]


def _mutant(src, old, new, tag):
    assert old in src, tag
    mod = types.ModuleType("sta_oracle_mutant")
    exec(compile(src.replace(old, new, 1), f"<mutant {tag}>", "exec"), mod.__dict__)
    return mod


def test_pins_pass_on_oracle():
    assert run_pins(O) == []


@pytest.mark.parametrize("tag,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tag, old, new):
    with open(O.__file__) as f:
        src = f.read()
    mod = _mutant(src, old, new, tag)
    assert run_pins(mod) != [], f"mutant '{tag}' survived every pin"


def test_token_predicate_matches_bruteforce():
    # the scalar predicate `permitted` against the brute-force key lists
    rng = np.random.default_rng(21)
    for _ in range(4):
        video, tile, windows = rand_case(rng, max_tokens=96)
        grid = O.tile_grid(video, tile)
        coords = O.natural_coords(video)
        for n in range(0, len(coords), 3):
            want = set(bf_keys(tuple(coords[n]), video, tile, windows[0]))
            got = {j for j in range(len(coords)) if O.permitted(coords[n], coords[j], tile, windows[0], grid)}
            assert got == want


# ---------------------------------------------------------------------------
# Partial tiles (reading R11: extents that are not multiples of the tile)
# ---------------------------------------------------------------------------

def bf_keys_partial(qx, video, tile, window):
    """Brute force with ceil(extent / tile) tiles: the window found by search
    on that grid, then every EXISTING token of its tiles by nested loops."""
    T, H, W = video
    grid = [-(-video[i] // tile[i]) for i in range(3)]
    c = [qx[i] // tile[i] for i in range(3)]
    starts = [bf_start(c[i], window[i], grid[i]) for i in range(3)]
    ext = [min(window[i], grid[i]) for i in range(3)]
    keys = []
    for a in range(starts[0], starts[0] + ext[0]):
        for b in range(starts[1], starts[1] + ext[1]):
            for cc in range(starts[2], starts[2] + ext[2]):
                for lt in range(tile[0]):
                    for ly in range(tile[1]):
                        for lz in range(tile[2]):
                            t, y, z = a * tile[0] + lt, b * tile[1] + ly, cc * tile[2] + lz
                            if t < T and y < H and z < W:
                                keys.append((t * H + y) * W + z)
    return sorted(keys)


def test_partial_tiles_against_bruteforce():
    rng = np.random.default_rng(31)
    done = 0
    while done < 6:
        tile = tuple(int(x) for x in rng.integers(2, 4, size=3))
        video = tuple(int(x) for x in rng.integers(2, 9, size=3))
        if all(v % t == 0 for v, t in zip(video, tile)) or np.prod(video) > 180:
            continue
        done += 1
        windows = [tuple(int(x) for x in rng.integers(1, 5, size=3)) for _ in range(2)]
        with pytest.raises(ValueError):
            O.tile_grid(video, tile)
        grid = O.tile_grid(video, tile, partial=True)
        N, D = int(np.prod(video)), 3
        coords = O.natural_coords(video)
        q, k, v = (rng.standard_normal((1, 2, N, D)) for _ in range(3))
        for h in range(2):
            mask = O.sta_mask(coords, coords, tile, windows[h], grid)
            for n in range(N):
                assert np.flatnonzero(mask[n]).tolist() == bf_keys_partial(tuple(coords[n]), video, tile,
                                                                           windows[h])
        got = O.sta_forward_explicit(q, k, v, video, tile, windows, scale=0.6, partial=True)
        T, H, W = video
        for h in range(2):
            for n in range(0, N, 5):
                keys = bf_keys_partial(tuple(coords[n]), video, tile, windows[h])
                s = 0.6 * (k[0, h, keys] @ q[0, h, n])
                p = np.exp(s - s.max())
                assert np.allclose(got[0, h, n], (p @ v[0, h, keys]) / p.sum(), rtol=0, atol=1e-12)
            # per-query-tile function, partial tiles included
            tiles = list(itertools.product(range(grid[0]), range(grid[1]), range(grid[2])))
            outs = O.sta_forward_query_tiles(*(x.reshape(1, 2, T, H, W, D) for x in (q, k, v)), tile,
                                             windows[h], h, tiles, scale=0.6, partial=True)
            full = np.zeros((T, H, W, D))
            for c, o in zip(tiles, outs):
                full[c[0] * tile[0]:(c[0] + 1) * tile[0], c[1] * tile[1]:(c[1] + 1) * tile[1],
                     c[2] * tile[2]:(c[2] + 1) * tile[2]] = o
            assert np.allclose(full.reshape(N, D), got[0, h], rtol=0, atol=1e-12)


def test_partial_tiles_dense_and_blockdiag():
    rng = np.random.default_rng(32)
    video, tile = (5, 7, 4), (2, 3, 3)
    N, D = 140, 6
    q, k, v = (rng.standard_normal((1, 2, N, D)) for _ in range(3))
    got = O.sta_forward_explicit(q, k, v, video, tile, [(3, 3, 2), (9, 9, 9)], scale=0.5, partial=True)
    assert np.allclose(got, sdpa64(q, k, v, 0.5), rtol=0, atol=1e-12)
    got = O.sta_forward_explicit(q, k, v, video, tile, [(1, 1, 1)] * 2, scale=0.5, partial=True)
    coords = O.natural_coords(video)
    tid = [tuple(int(x) for x in c // np.array(tile)) for c in coords]
    for t in set(tid):
        idx = [i for i in range(N) if tid[i] == t]
        assert np.allclose(got[:, :, idx], sdpa64(q[:, :, idx], k[:, :, idx], v[:, :, idx], 0.5),
                           rtol=0, atol=1e-12)
