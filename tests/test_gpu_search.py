"""GPU parity of the per-head window search against its CPU oracle.

Inputs: the locality calibration generator (each head attends to a
Gaussian neighbourhood of its own width), small enough for the oracle's
explicit attention.  Tolerance on each (head, candidate) error, derived
from the forward's own error: with ||dO|| / ||O|| <= 1e-3 for each of the
two outputs compared, the relative error moves by at most
2e-3 + 1e-3 * err; the bound used is 2e-3 + 1e-2 * err.  A candidate equal
to the grid runs the very same work as the full-attention reference and
must give exactly 0.  The chosen windows must equal the oracle's, except
where an oracle error lies within that tolerance of the threshold, where
the GPU's choice must be one the oracle would make for some errors inside
the tolerance.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import sta_oracle_search as OS
from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import make_local_qkv

pytestmark = pytest.mark.gpu

VIDEO, TILE, D = (6, 16, 16), (2, 4, 4), 64
GRID = (3, 4, 4)
LENGTHS = [2.0, 4.0, 8.0, 32.0]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def tol(err):
    return 2e-3 + 1e-2 * err


def _inputs(seed):
    return make_local_qkv(VIDEO, LENGTHS, D, sharpness=16.0, seed=seed)


def test_window_errors_and_choice():
    say("case window search: 6x16x16 tile 2x4x4, 4 heads (lengths 2, 4, 8, 32), d64 bf16")
    q, k, v = _inputs(11)
    cands = api.window_candidates(GRID)
    got = api.window_errors(q.cuda(), k.cuda(), v.cuda(), TILE, cands)
    N = VIDEO[0] * VIDEO[1] * VIDEO[2]
    ref = OS.window_errors(*(x.reshape(1, 4, N, D).double().numpy() for x in (q, k, v)), VIDEO, TILE,
                           cands, scale=1.0 / 8)
    d = np.abs(got - ref)
    say(f"  max |err_gpu - err_oracle| {d.max():.2e}")
    assert (d <= tol(ref)).all()
    full = cands.index(GRID)
    assert (got[:, full] == 0).all()
    for tau in (0.02, 0.1, 0.3):
        want = OS.select_windows(ref, cands, GRID, tau)
        choice = api.window_select(got, cands, GRID, tau)
        say(f"  tau {tau}: {choice}")
        for h in range(4):
            if choice[h] == want[h]:
                continue
            # allowed only when the oracle's decision sits inside the tolerance band
            lo, hi = ref[h] - tol(ref[h]), ref[h] + tol(ref[h])
            ok_lo = OS.select_windows(lo[None], cands, GRID, tau)[0]
            ok_hi = OS.select_windows(hi[None], cands, GRID, tau)[0]
            assert choice[h] in (ok_lo, ok_hi), (h, tau, choice[h], want[h])


def test_window_search_averages_samples():
    """sta_window_search over three calibration samples against the oracle's
    W1-W4 (per-sample errors, their mean, the choice from the mean)."""
    say("case window search over three calibration samples")
    samples = [_inputs(s) for s in (21, 22, 23)]
    cands = api.window_candidates(GRID)
    N = VIDEO[0] * VIDEO[1] * VIDEO[2]
    ref_samples = [tuple(x.reshape(1, 4, N, D).double().numpy() for x in s) for s in samples]
    for tau in (0.02, 0.1, 0.3):
        windows, mean, got_cands = api.window_search([tuple(x.cuda() for x in s) for s in samples], TILE, tau)
        assert got_cands == [tuple(c) for c in cands]
        want, ref = OS.search(ref_samples, VIDEO, TILE, cands, tau, scale=1.0 / 8)
        d = np.abs(mean - ref)
        say(f"  tau {tau}: max |mean_gpu - mean_oracle| {d.max():.2e}; {windows}")
        assert (d <= tol(ref)).all()
        assert (mean[:, cands.index(GRID)] == 0).all()
        for h in range(4):
            if windows[h] == want[h]:
                continue
            lo, hi = ref[h] - tol(ref[h]), ref[h] + tol(ref[h])
            ok_lo = OS.select_windows(lo[None], cands, GRID, tau)[0]
            ok_hi = OS.select_windows(hi[None], cands, GRID, tau)[0]
            assert windows[h] in (ok_lo, ok_hi), (h, tau, windows[h], want[h])
        # the library's mean is the mean of its own per-sample errors
        each = [api.window_errors(*(x.cuda() for x in s), TILE, cands) for s in samples]
        assert np.allclose(mean, (each[0] + each[1] + each[2]) / 3, rtol=1e-15, atol=0)


def test_window_search_partial_tiles():
    """Extents that are not multiples of the tile (5x15x13 with 2x4x4 tiles:
    grid 3x4x4, the last tile of every axis partial): the errors and the
    choice against the oracle with partial tiles; the grid candidate is
    again exact."""
    video = (5, 15, 13)
    grid = (3, 4, 4)
    say("case window search with partial tiles: 5x15x13 tile 2x4x4, 4 heads, d64 bf16")
    q, k, v = make_local_qkv(video, LENGTHS, D, sharpness=16.0, seed=31)
    cands = api.window_candidates(grid)
    got = api.window_errors(q.cuda(), k.cuda(), v.cuda(), TILE, cands)
    N = video[0] * video[1] * video[2]
    ref_in = tuple(x.reshape(1, 4, N, D).double().numpy() for x in (q, k, v))
    ref = OS.window_errors(*ref_in, video, TILE, cands, scale=1.0 / 8, partial=True)
    d = np.abs(got - ref)
    say(f"  max |err_gpu - err_oracle| {d.max():.2e}")
    assert (d <= tol(ref)).all()
    assert (got[:, cands.index(grid)] == 0).all()
    tau = 0.1
    windows, mean, got_cands = api.window_search([(q.cuda(), k.cuda(), v.cuda())], TILE, tau)
    assert got_cands == [tuple(c) for c in cands]
    want, _ = OS.search([ref_in], video, TILE, cands, tau, scale=1.0 / 8, partial=True)
    say(f"  tau {tau}: {windows}")
    for h in range(4):
        if windows[h] == want[h]:
            continue
        lo, hi = ref[h] - tol(ref[h]), ref[h] + tol(ref[h])
        assert windows[h] in (OS.select_windows(lo[None], cands, grid, tau)[0],
                              OS.select_windows(hi[None], cands, grid, tau)[0]), (h, windows[h], want[h])
