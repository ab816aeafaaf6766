"""MI355X (gfx950) In-Place TTT fast-weight MLP layer.

The layer runs in hand-written HIP kernels behind a C ABI (include/ttt_mlp.h,
built into _build/libttt_mlp.so); `ttt_mlp` is its ctypes binding and `synth`
the seeded input recipe.
"""
from . import synth  # noqa: F401
from .ttt_mlp import (TTTError, alloc_workspace, forward, forward_batched, load, make_desc,  # noqa: F401
                      ttt_fastweight_state_reset, ttt_last_error, ttt_mlp_desc_t,
                      ttt_mlp_forward, ttt_mlp_forward_batched, ttt_mlp_group_size,
                      ttt_mlp_workspace_size, ttt_profile_enable, ttt_profile_read,
                      ttt_stage_name)
