"""Exact attention (FlashAttention-style tiled forward and recomputing
backward) for one AMD Instinct MI355X, as a C-ABI HIP library with a thin
ctypes binding."""
from .binding import (  # noqa: F401
    EXPORTED, FA_BWD_DQ_ATOMIC, FA_BWD_PRECISE, FlashAttnError, flash_attn_bwd, flash_attn_bwd_f32,
    flash_attn_bwd_noalloc,
    flash_attn_bwd_workspace_bytes, flash_attn_decode_fwd, flash_attn_decode_workspace_bytes,
    flash_attn_fwd, flash_attn_fwd_f32, flash_attn_status_string, library_path, load_library,
    flash_attn_fwd_dropout, flash_attn_bwd_dropout, flash_attn_dropout_mask, flash_attn_fwd_block_sparse,
    flash_attn_fwd_fp8,
)
