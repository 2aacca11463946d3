"""MI355X-native packed variable-length attention, forward and backward (RoPE in the kernel,
optional symmetric or causal window), built around the C-ABI library ``libvlf.so`` of
hand-written gfx950 HIP; ``tune`` picks the schedule per shape by measurement.

The binding (``variable_length_flash_amd.binding``) loads the library on first use and fails
loudly when it is missing: there is no fallback path.
"""
from .binding import (  # noqa: F401
    CAUSAL, Batch, VlfError, attend, attend_backward, attend_backward_into, attend_into,
    attend_rotated_into, backward_workspace_bytes, choose_backward, choose_backward_br, choose_br,
    choose_prerotate, choose_schedule, forward_kernel, launch_table, library_path, load_library,
    new_workspace, prepare, rotate_keys, rotate_qkv_into, schedule_rule, tile_count, tile_table,
    typical_length, visible_pairs, workspace_bytes,
)
from . import tune  # noqa: F401
