"""Pins of the backward oracle (oracle/sta_oracle_bwd.py) to things other
than itself (CPU only).

  * central finite differences of <O, G>, with O from the pinned forward
    oracle, on small float64 problems (every entry of dq, dk, dv),
  * special cases that reduce to a library routine: a window covering the
    grid is dense attention and a 1x1x1 window is block-diagonal attention,
    both against torch's autograd of plain float64 attention; lse against
    torch.logsumexp of the explicitly masked scores,
  * closed forms and invariants: Q = 0 gives lse = log(number of permitted
    keys); the rows of dv sum to the rows of G; the rows of dk sum to zero;
    token-order equivariance,
  * the per-tile functions used at large sizes against the explicit one,
  * planted mistakes in a copy of the oracle that the pins must catch.
"""

import math
import types

import numpy as np
import pytest
import torch

from oracle import sta_oracle as F
from oracle import sta_oracle_bwd as O


def rand_case(rng, max_tokens=72, partial=False):
    """Random video, tile and two heads' windows; with partial, at least one
    extent is not a multiple of its tile."""
    while True:
        tile = tuple(int(x) for x in rng.integers(1, 4, size=3))
        grid = tuple(int(x) for x in rng.integers(1, 5, size=3))
        video = tuple(t * g for t, g in zip(tile, grid))
        if partial:
            video = tuple(max(1, e - int(rng.integers(0, t))) for e, t in zip(video, tile))
            if all(e % t == 0 for e, t in zip(video, tile)):
                continue
        if video[0] * video[1] * video[2] <= max_tokens:
            break
    windows = [tuple(int(x) for x in rng.integers(1, 5, size=3)) for _ in range(2)]
    return video, tile, windows


def torch_attention_grads(q, k, v, g, scale):
    """Plain dense attention and its gradients by torch autograd (float64)."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.softmax(scale * (tq @ tk.transpose(-1, -2)), dim=-1) @ tv
    (o * torch.tensor(g, dtype=torch.float64)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


# ---------------------------------------------------------------------------
# The pin set, parameterised by the oracle module so that mutants can be run
# ---------------------------------------------------------------------------

def pin_finite_differences(mod, cases=3, seed=5, partial=False):
    rng = np.random.default_rng(seed)
    fails = []
    for _ in range(cases):
        video, tile, windows = rand_case(rng, partial=partial)
        N, D = video[0] * video[1] * video[2], 3
        q, k, v, g = (rng.standard_normal((1, 2, N, D)) for _ in range(4))
        scale = 0.7
        got = mod.sta_backward_explicit(q, k, v, g, video, tile, windows, scale=scale, partial=partial)

        def loss(qq, kk, vv):
            return float((F.sta_forward_explicit(qq, kk, vv, video, tile, windows, scale=scale,
                                                 partial=partial) * g).sum())

        eps = 1e-6
        for name, idx in (("dq", 0), ("dk", 1), ("dv", 2)):
            num = np.zeros_like(q)
            for pos in np.ndindex(q.shape):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[idx][pos] += eps
                args_m[idx][pos] -= eps
                num[pos] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            if not np.allclose(got[name], num, rtol=1e-6, atol=1e-7):
                fails.append((name, video, tile, windows, float(np.abs(got[name] - num).max())))
        if not np.allclose(got["o"], F.sta_forward_explicit(q, k, v, video, tile, windows, scale=scale,
                                                            partial=partial),
                           rtol=0, atol=1e-12):
            fails.append(("o", video, tile, windows))
    return fails


def pin_finite_differences_partial(mod):
    """The same finite differences on grids whose last tiles are partial."""
    return pin_finite_differences(mod, cases=3, seed=6, partial=True)


def pin_dense_blockdiag_and_lse(mod, seed=11):
    rng = np.random.default_rng(seed)
    fails = []
    video, tile = (4, 6, 4), (2, 3, 2)
    N, D = 96, 8
    q, k, v, g = (rng.standard_normal((1, 2, N, D)) for _ in range(4))
    scale = 1.0 / math.sqrt(D)
    # a window covering the grid is dense attention
    got = mod.sta_backward_explicit(q, k, v, g, video, tile, [(9, 9, 9), (2, 2, 2)], scale=scale)
    want = torch_attention_grads(q, k, v, g, scale)
    for name, w in zip(("o", "dq", "dk", "dv"), want):
        if not np.allclose(got[name], w, rtol=0, atol=1e-12):
            fails.append(("dense", name))
    lse_want = torch.logsumexp(scale * torch.tensor(q) @ torch.tensor(k).transpose(-1, -2), dim=-1).numpy()
    if not np.allclose(got["lse"], lse_want, rtol=0, atol=1e-12):
        fails.append(("dense", "lse"))
    # a 1x1x1 window is attention inside each tile
    got = mod.sta_backward_explicit(q, k, v, g, video, tile, [(1, 1, 1)] * 2, scale=scale)
    coords = F.natural_coords(video)
    tid = [tuple(int(x) for x in c // np.array(tile)) for c in coords]
    for t in sorted(set(tid)):
        idx = [i for i in range(N) if tid[i] == t]
        want = torch_attention_grads(q[:, :, idx], k[:, :, idx], v[:, :, idx], g[:, :, idx], scale)
        for name, w in zip(("o", "dq", "dk", "dv"), want):
            if not np.allclose(got[name][:, :, idx], w, rtol=0, atol=1e-12):
                fails.append(("blockdiag", name, t))
    # lse of STA rows against torch.logsumexp of the explicitly masked scores
    windows = [(3, 1, 2), (1, 2, 1)]
    got = mod.sta_backward_explicit(q, k, v, g, video, tile, windows, scale=scale)
    grid = F.tile_grid(video, tile)
    for h in range(2):
        mask = torch.tensor(F.sta_mask(coords, coords, tile, windows[h], grid))
        z = scale * torch.tensor(q[0, h]) @ torch.tensor(k[0, h]).T
        want = torch.logsumexp(z.masked_fill(~mask, -math.inf), dim=-1).numpy()
        if not np.allclose(got["lse"][0, h], want, rtol=0, atol=1e-12):
            fails.append(("lse", h))
    return fails


def pin_closed_forms_and_invariants(mod, seed=13):
    rng = np.random.default_rng(seed)
    fails = []
    video, tile = (6, 4, 6), (2, 2, 2)
    grid = F.tile_grid(video, tile)
    N, D = 144, 4
    windows = [(3, 3, 3), (1, 2, 3)]
    q, k, v, g = (rng.standard_normal((2, 2, N, D)) for _ in range(4))
    scale = 0.5
    # Q = 0: every permitted score is 0, so lse = log(prod(w') * tile volume)
    got = mod.sta_backward_explicit(np.zeros_like(q), k, v, g, video, tile, windows, scale=scale)
    for h in range(2):
        we = F.effective_window(windows[h], grid)
        count = we[0] * we[1] * we[2] * tile[0] * tile[1] * tile[2]
        if not np.allclose(got["lse"][:, h], math.log(count), rtol=0, atol=1e-12):
            fails.append(("lse q=0", h))
    got = mod.sta_backward_explicit(q, k, v, g, video, tile, windows, scale=scale)
    # probabilities of a row sum to one: sum_j dv_j = sum_i g_i
    if not np.allclose(got["dv"].sum(axis=2), g.sum(axis=2), rtol=0, atol=1e-10):
        fails.append("dv row sum")
    # softmax is shift invariant per row: sum_j dz_ij = 0, so sum_j dk_j = 0
    if not np.allclose(got["dk"].sum(axis=2), 0.0, rtol=0, atol=1e-10):
        fails.append("dk row sum")
    # token-order equivariance: the same tokens in another order
    perm = rng.permutation(N)
    coords = F.natural_coords(video)[perm]
    got_p = mod.sta_backward_explicit(q[:, :, perm], k[:, :, perm], v[:, :, perm], g[:, :, perm], video,
                                      tile, windows, scale=scale, coords=coords)
    for name in ("dq", "dk", "dv", "lse"):
        if not np.allclose(got_p[name], got[name][:, :, perm], rtol=0, atol=1e-12):
            fails.append(("order", name))
    return fails


def pin_tile_functions(mod, cases=3, seed=17, partial=False):
    rng = np.random.default_rng(seed)
    fails = []
    for _ in range(cases):
        video, tile, windows = rand_case(rng, max_tokens=120, partial=partial)
        N, D = video[0] * video[1] * video[2], 3
        q, k, v, g = (rng.standard_normal((1, 2, N, D)) for _ in range(4))
        scale = 0.9
        want = mod.sta_backward_explicit(q, k, v, g, video, tile, windows, scale=scale, partial=partial)
        grid = F.tile_grid(video, tile, partial)
        T, H, W = video
        q6, k6, v6, g6 = (x.reshape(1, 2, T, H, W, D) for x in (q, k, v, g))
        tiles = list(np.ndindex(*grid))
        for h in range(2):
            full = {n: np.zeros((T, H, W, D)) for n in ("dq", "dk", "dv")}
            lse = np.zeros((T, H, W))
            qres = mod.sta_backward_query_tiles(q6, k6, v6, g6, tile, windows[h], h, tiles, scale=scale,
                                                partial=partial)
            kres = mod.sta_backward_key_tiles(q6, k6, v6, g6, tile, windows[h], h, tiles, scale=scale,
                                              partial=partial)
            for c, (l, dq), (dk, dv) in zip(tiles, qres, kres):
                sl = tuple(slice(c[d] * tile[d], (c[d] + 1) * tile[d]) for d in range(3))
                lse[sl], full["dq"][sl], full["dk"][sl], full["dv"][sl] = l, dq, dk, dv
            if not np.allclose(lse.reshape(N), want["lse"][0, h], rtol=0, atol=1e-12):
                fails.append(("lse", video, tile, windows[h]))
            for n in ("dq", "dk", "dv"):
                if not np.allclose(full[n].reshape(N, D), want[n][0, h], rtol=0, atol=1e-12):
                    fails.append((n, video, tile, windows[h]))
    return fails


def pin_tile_functions_partial(mod):
    """The per-tile functions against the explicit one on partial grids."""
    return pin_tile_functions(mod, cases=3, seed=18, partial=True)


ALL_PINS = [pin_finite_differences, pin_finite_differences_partial, pin_dense_blockdiag_and_lse,
            pin_closed_forms_and_invariants, pin_tile_functions, pin_tile_functions_partial]


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

def test_finite_differences():
    assert pin_finite_differences(O) == []


def test_dense_blockdiag_and_lse():
    assert pin_dense_blockdiag_and_lse(O) == []


def test_closed_forms_and_invariants():
    assert pin_closed_forms_and_invariants(O) == []


def test_tile_functions_equal_explicit():
    assert pin_tile_functions(O) == []


def test_finite_differences_partial_tiles():
    assert pin_finite_differences_partial(O) == []


def test_tile_functions_equal_explicit_partial_tiles():
    assert pin_tile_functions_partial(O) == []


def test_query_tiles_seeing_is_the_inverse_of_the_window():
    rng = np.random.default_rng(3)
    for _ in range(20):
        grid = tuple(int(x) for x in rng.integers(1, 7, size=3))
        window = tuple(int(x) for x in rng.integers(1, 8, size=3))
        seen = {kc: set(O.query_tiles_seeing(kc, window, grid)) for kc in np.ndindex(*grid)}
        for c in np.ndindex(*grid):
            box = F.window_tiles(c, window, grid)
            members = set(np.ndindex(*[b[1] - b[0] for b in box]))
            members = {tuple(m[d] + box[d][0] for d in range(3)) for m in members}
            for kc in np.ndindex(*grid):
                assert (c in seen[kc]) == (kc in members)


MUTANTS = [
    ("dq scale dropped", "dq = scale * (dz @ k)", "dq = (dz @ k)"),
    ("dk scale dropped", "dk = scale * (dz.T @ q)", "dk = (dz.T @ q)"),
    ("no row correction", "dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "dz = p * dp"),
    ("row correction sign", "dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
     "dz = p * (dp + (p * dp).sum(axis=1, keepdims=True))"),
    ("dv without transpose", "dv = p.T @ g", "dv = p @ g"),
    ("dk from k", "dk = scale * (dz.T @ q)", "dk = scale * (dz.T @ k[:q.shape[0]])"),
    ("lse without max", "return m + np.log(np.exp(z - m[:, None]).sum(axis=1))",
     "return np.log(np.exp(z - m[:, None]).sum(axis=1))"),
    ("key-tile lse over the key tile", "p = np.exp(scale * (qt @ kt.T) - lse)",
     "p = np.exp(scale * (qt @ kt.T) - np.log(np.exp(scale * (qt @ kt.T)).sum(axis=1, keepdims=True)))"),
    ("key-tile delta over the key tile", "dz = p * (gt @ vt.T - delta)",
     "dz = p * (gt @ vt.T - (p * (gt @ vt.T)).sum(axis=1, keepdims=True))"),
    ("inverse strict bound", "box[d][0] <= key_tile[d] < box[d][1]", "box[d][0] <= key_tile[d] <= box[d][1]"),
    ("partial grid floored", "grid = F.tile_grid(video, tile, partial)",
     "grid = tuple(max(1, e // t) for e, t in zip(video, tile))"),
    ("partial query-tile shape", "shape = _tile_slice(q, c, tile, batch, head).shape[:3]", "shape = tuple(tile)"),
]


def _mutant(src, old, new, tag):
    assert old in src, tag
    mod = types.ModuleType("sta_oracle_bwd_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new, 1), f"<mutant {tag}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("tag,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tag, old, new):
    with open(O.__file__) as f:
        src = f.read()
    mod = _mutant(src, old, new, tag)
    assert run_pins(mod) != [], f"mutant '{tag}' survived every pin"
