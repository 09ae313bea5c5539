"""dgw4: W4A16 routed-expert (grouped MoE) layer for AMD Instinct MI355X.

The compute lives in libdgw4.so (hand-written HIP for gfx950, C ABI in
include/dgw4.h); this package only binds it for torch device tensors.
"""
from .binding import (  # noqa: F401
    BLOCK_M,
    Dgw4Error,
    align,
    router,
    align_capacity,
    hbm_read_probe,
    mfma_probe,
    header_functions,
    lib,
    moe_forward,
    moe_forward_routed,
    pack_tiled,
    WEIGHTS_TILED,
    ROWS_TILES,
    ROWS_CHUNKS,
    quantize_rtn,
    status_string,
    version,
    workspace_bytes,
    row_block,
    linear_row_block,
    w4a16_linear,
    sample,
    sample_noalloc,
    fused_entropy,
    moe_experts,
    gumbel_argmax_sample,
)
