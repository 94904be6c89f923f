"""Sliding Tile Attention (STA) forward and backward for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libsta.so`` (declared in
``include/sta.h``); this package only marshals torch tensors into it.
"""

from .api import (  # noqa: F401
    Plan,
    StaError,
    sta_attention,
    sta_backward_plan,
    sta_clear_plan_cache,
    sta_forward,
    sta_forward_plan,
    sta_plan_create,
    sta_tile_reorder,
    sta_tile_unreorder,
)
