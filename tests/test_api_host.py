"""Argument checks of the Python binding that need no GPU: every one must
raise ValueError before anything is launched."""

import numpy as np
import pytest
import torch

from sliding_tile_attention_sta_amd import api
from sliding_tile_attention_sta_amd.synthetic import WORKLOADS


def test_video_inputs_shape_errors():
    q = torch.zeros(1, 2, 96, 64)
    with pytest.raises(ValueError, match="video"):
        api._video_inputs(q, q, q, None)
    with pytest.raises(ValueError, match="tokens"):
        api._video_inputs(q, q, q, (2, 4, 8))          # 64 tokens for a 96-token q
    with pytest.raises(ValueError, match="CUDA"):
        api._video_inputs(q, q, q, (2, 6, 8))          # right shape, host tensors
    with pytest.raises(ValueError, match="q must be"):
        api._video_inputs(torch.zeros(2, 96, 64), q, q, (2, 6, 8))
    with pytest.raises(ValueError, match="q must be"):
        api._video_inputs(None, q, q, (2, 6, 8))


def test_host_tensors_are_rejected_by_every_entry_point():
    w = WORKLOADS["tiny"]
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim)
    x = torch.zeros(w.batch, w.heads, w.tokens, w.head_dim)
    rows = torch.zeros(w.batch, w.heads, w.tokens)
    with pytest.raises(ValueError, match="CUDA"):
        api.sta_forward_plan(plan, x, x, x)
    with pytest.raises(ValueError, match="CUDA"):
        api.sta_backward_plan(plan, x, x, x, x, x, rows)
    with pytest.raises(ValueError, match="CUDA"):
        api.sta_tile_reorder(plan, x)
    with pytest.raises(ValueError, match="CUDA"):
        api.sta_forward(x, x, x, w.tile, w.windows, video=w.video)
    with pytest.raises(ValueError, match="CUDA"):
        api.window_errors(x, x, x, w.tile, [(1, 1, 1)], video=w.video)


def test_window_select_checks_its_columns():
    with pytest.raises(ValueError, match="column"):
        api.window_select(np.zeros((2, 3)), [(1, 1, 1), (2, 2, 2)], (3, 4, 4), 0.1)
