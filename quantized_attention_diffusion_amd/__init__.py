"""Quantized attention (INT8 Q.K^T, FP8 P.V; optional bf16 P.V; optional block-sparse key
tiles) for MI355X (gfx950).

The computation lives in the HIP library ``libsage_attn.so`` (C ABI declared in
``include/sage_attn.h``); this package is its thin ctypes binding with the same entry
point names.  There is no fallback path: if the library is not built, calls raise.
"""
from ._capi import (SageError, lib_path, load, sage_last_error, sage_kernel_info,
                    sage_padded_tokens, sage_workspace_bytes, sage_workspace_bytes_ex,
                    sage_quant_scratch_bytes, sage_quant_qk, sage_attn_fwd_prequant,
                    sage_attn_fwd, sage_attn_fwd_ex, sage_quant_qk_ex, sage_debug_qk_i32,
                    sage_debug_qk_i32_ex,
                    sage_debug_e4m3, sage_select_scratch_bytes, sage_block_select,
                    sage_workspace_bytes_sparse, sage_attn_fwd_sparse, sage_attn_fwd_noalloc,
                    sage_density_schedule, NOALLOC_SCRATCH_BYTES, EXPORTS, STATUS,
                    SAGE_PV_FP8, SAGE_PV_BF16, SAGE_QK_PER_TOKEN, SAGE_K_BLOCK_MEAN, mode_bits)

__all__ = ["SageError", "lib_path", "load", "sage_last_error", "sage_kernel_info",
           "sage_padded_tokens", "sage_workspace_bytes", "sage_workspace_bytes_ex",
           "sage_quant_scratch_bytes", "sage_quant_qk", "sage_attn_fwd_prequant",
           "sage_attn_fwd", "sage_attn_fwd_ex", "sage_quant_qk_ex", "sage_debug_qk_i32",
           "sage_debug_qk_i32_ex",
           "sage_debug_e4m3", "sage_select_scratch_bytes", "sage_block_select",
           "sage_workspace_bytes_sparse", "sage_attn_fwd_sparse", "sage_attn_fwd_noalloc",
           "sage_density_schedule", "NOALLOC_SCRATCH_BYTES", "EXPORTS", "STATUS", "SAGE_PV_FP8", "SAGE_PV_BF16",
           "SAGE_QK_PER_TOKEN", "SAGE_K_BLOCK_MEAN", "mode_bits"]
