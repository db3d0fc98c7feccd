"""MI355X-native routed-expert MoE layer (HIP, gfx950): single-token and
small-batch decode, and the many-token (prefill) layer on the matrix cores.

The compute path is the C-ABI library ``libmoe_decode.so`` built from
``csrc/`` (declared in ``include/moe_decode.h`` and ``include/moe_prefill.h``);
the functions exported here only marshal torch tensors into it.  Importing the package does not load the
library; the first call does, and raises if it is missing and cannot be built.
"""
from .api import (MoeError, moe_abi_version, moe_build_id, moe_dbg_lane_map, moe_dbg_layer_stage,
                  moe_dbg_prefill_stage, moe_dbg_w13_silu, moe_dbg_w2_combine, moe_dbg_wave_sum,
                  moe_decode_fused, moe_layer_decode, moe_layer_decode_noalloc, moe_layer_launches,
                  moe_layer_prefill, moe_prefill_workspace_bytes, moe_probe_copy, moe_probe_empty,
                  moe_probe_read, moe_route, moe_status_str, moe_workspace_bytes, moe_workspace_init,
                  prefill_workspace, shared_expert, workspace)

__all__ = ["MoeError", "moe_abi_version", "moe_build_id", "moe_dbg_lane_map", "moe_dbg_layer_stage",
           "moe_dbg_prefill_stage", "moe_dbg_w13_silu", "moe_dbg_w2_combine", "moe_dbg_wave_sum",
           "moe_decode_fused", "moe_layer_decode", "moe_layer_decode_noalloc", "moe_layer_launches",
           "moe_layer_prefill", "moe_prefill_workspace_bytes", "moe_probe_copy", "moe_probe_empty",
           "moe_probe_read", "moe_route", "moe_status_str", "moe_workspace_bytes",
           "moe_workspace_init", "prefill_workspace", "shared_expert", "workspace"]
