"""MI355X (gfx950) MoE token routing: router gate -> bf16 top-k -> softmax ->
shared slot -> moe_align_block_size, in hand-written HIP kernels behind a
C ABI (include/moeroute.h).  This package is the thin Python binding."""
from ._binding import (  # noqa: F401
    MR_ECAPACITY,
    MR_EINVAL,
    MR_ELAUNCH,
    MR_EUNSUPPORTED,
    MR_OK,
    MR_STREAM_READ_OUT_WORDS,
    SIGNATURES,
    MoeRouteError,
    library_path,
    mr_abi_version,
    mr_align,
    mr_align_capacity,
    mr_debug_gate_logits,
    mr_debug_stream_read,
    mr_expert_ids_capacity,
    mr_last_error,
    mr_route,
    mr_route_align,
    mr_select_alignment,
    mr_workspace_bytes,
    mr_workspace_reset,
    new_workspace,
)
