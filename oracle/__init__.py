"""CPU oracle for SageAttention-style quantized attention.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import this
package.  The product path (the HIP library and its Python binding) never calls it,
and the oracle never imports the product: the two share no code, headers, tables or
constants.  Inputs come from the separate ``workloads`` generator module.

What the oracle computes, and where each step comes from:

* ``attention_exact`` - the plain definition softmax(Q K^T / sqrt(d)) V in fp64
  (juejin page "MiniMax H3 接入 SageAttention 实测加速", section 一; Baidu Cloud page
  "SDPA稠密注意力模式", section 三 part 1).
* ``quantize`` - K smoothing by its token mean (the "outlier smoothing" of section 一
  of the juejin page; the sd114.wiki ComfyUI-sol-attn page, "核心亮点" item 1, keeps
  that mean term in bf16), per-block INT8 codes for Q and K (INT8 for QK^T, juejin
  section 一), per-channel FP8 e4m3 codes for V (FP8 for PV, same section).
* ``attention_pipeline`` - the quantized attention: exact int32 QK^T, dequantisation,
  online softmax in base 2 over key tiles (the blockwise computation of the
  bjdmk page "GitHub榜单静默期：Attention优化从架构转向推理加速", section 2.2), P rounded
  to FP8 e4m3, PV accumulated, normalised at the end.  By default every step is fp64
  (the plain reading); ``arith="fp32"`` decides the P codes in fp32, the precision
  the method gives its softmax.
* ``select_tiles`` (module ``sparse``) - block-sparse attention: the key tiles each
  query block keeps for a density tau (the sd114.wiki ComfyUI-sol-attn page, 核心亮点
  item 4, names tau and its sparse-to-dense schedule; the selection rule is a reading).

Points the pages leave open are fixed by readings that are listed in the module
docstrings.  Everything is numpy; floating point is fp64 except where the method's
own precision (fp32 scales, and in the ``arith="fp32"`` reading the fp32 softmax)
decides a quantised code, where the oracle computes in fp32 as the method does.
"""
from .fp8 import e4m3_decode, e4m3_encode, e4m3_table, E4M3_MAX
from .quant import (QUANT_BLOCK, bf16_round, k_token_mean, quantize_int8_blocks,
                    quantize_v_fp8, quantize)
from .attention import (LOG2E, P_SCALE, attention_exact, qk_int32, pipeline_logits,
                        attention_pipeline, bf16_round64, default_sm_scale, rel_l2)
from .sparse import SPARSE_TILE, keep_count, block_code_sums, tile_importance, select_tiles

__all__ = [
    "e4m3_decode", "e4m3_encode", "e4m3_table", "E4M3_MAX",
    "QUANT_BLOCK", "bf16_round", "k_token_mean", "quantize_int8_blocks",
    "quantize_v_fp8", "quantize",
    "LOG2E", "P_SCALE", "attention_exact", "qk_int32", "pipeline_logits",
    "attention_pipeline", "bf16_round64", "default_sm_scale", "rel_l2",
    "SPARSE_TILE", "keep_count", "block_code_sums", "tile_importance", "select_tiles",
]
