"""MI355X (gfx950) implementation of the LFM2.5-24B-A2B biased-sigmoid top-4
MoE layer: HIP kernels behind a C ABI (include/lfm_moe.h), bound with ctypes.

Importing the package loads liblfm_moe.so and fails if it has not been built.
"""

from . import _lib
from .api import (EXPERTS, FF, HIDDEN, TOP_K, abi_version, alloc_workspace,  # noqa: F401
                  block_forward, experts, experts_fp8, forward, forward_fp8, pack_down, pack_fp8_down,
                  pack_fp8_gateup, pack_fp8_gateup_stacked, pack_gateup, pack_gateup_stacked, release,
                  rmsnorm, route, route_workspace_bytes, stack_forward, stage_combine, stage_dispatch,
                  stage_down, stage_gateup, timing_enable,
                  timing_read, workspace_bytes, workspace_offset, workspace_view)

_lib.load()
