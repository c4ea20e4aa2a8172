"""Quantisation steps of the method: K smoothing, INT8 Q/K codes, FP8 V codes.

Sources (pages):
* Low-bit quantisation of the attention products with outlier smoothing, INT8 for
  QK^T and FP8 for PV: juejin page "MiniMax H3 接入 SageAttention 实测加速", section 一.
* The K mean term is kept in bf16 and only the remainder is quantised: sd114.wiki
  page on ComfyUI-sol-attn, "核心亮点" item 1.
* Quantising attention matrices from FP16 to INT8: bjdmk page
  "GitHub榜单静默期：Attention优化从架构转向推理加速", section 2.2.

Readings of what the pages leave open:
* K smoothing subtracts the per-(batch, head, channel) mean over the N valid tokens.
  The mean is summed in fp64, divided by N in fp64, rounded to fp32 and then to bf16
  (round to nearest even), and is stored in bf16.  K' = fp32(K) - fp32(mean), one fp32
  subtraction per element.  Q and V are not smoothed.
* INT8 granularity: one scale per (batch, head, block of 64 consecutive tokens), the
  same for Q and K.  A finer option gives every token its own scale (block = 1), the
  per-token granularity that quality-first settings use (bjdmk page
  "GitHub榜单静默期：Attention优化从架构转向推理加速", section 4.3).  For a block, amax = max |x| over its valid rows;
  scale = fp32(amax / 127); inv = fp32(127 / amax); code = clamp(rint(fp32(x * inv)),
  -127, 127) with rint rounding half to even.  The range is symmetric (-128 is never
  produced).  amax = 0 gives scale 0 and all-zero codes.  Scales do not contain the
  softmax scale.
* Block-residual K (the Sol-Attn variant of the sd114.wiki page, "核心亮点" item 1:
  only the residual inside each K block is quantised, the mean term stays bf16): the
  mean of each 64-token block, computed like the token mean, replaces the token mean
  in the subtraction.
* FP8 V: one scale per (batch, head, channel) over the valid tokens:
  scale = fp32(vamax / 448); code = e4m3(fp32(v * fp32(448 / vamax))); vamax = 0 gives
  scale 0 and zero codes.

Array conventions: inputs are float32 arrays holding bf16 values in the [B, N, H, d]
layout; outputs use [B, H, N, d] for codes, [B, H, ceil(N/64)] for Q/K scales and
[B, H, d] for the K mean and the V scales (no padding: the oracle knows no tiling).
"""
from __future__ import annotations

import numpy as np

from .fp8 import e4m3_encode, E4M3_MAX

QUANT_BLOCK = 64

__all__ = ["QUANT_BLOCK", "bf16_round", "k_token_mean", "k_block_means", "quantize_int8_blocks",
           "quantize_v_fp8", "quantize"]

F32 = np.float32


def bf16_round(x) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returned as float32.

    bf16 keeps the top 16 bits of the fp32 pattern; adding 0x7FFF plus the lowest
    kept bit before truncating rounds to nearest with ties to the even pattern."""
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(F32)


def k_token_mean(k) -> np.ndarray:
    """Per-(b, h, channel) mean of K over tokens -> bf16 values as float32 [B, H, d]."""
    k = np.asarray(k, dtype=F32)
    n = k.shape[1]
    s = k.astype(np.float64).sum(axis=1)               # [B, H, d], fp64
    mean = (s / n).astype(F32)                         # fp64 divide, one fp32 rounding
    return bf16_round(mean)


def k_block_means(k, block: int = QUANT_BLOCK) -> np.ndarray:
    """Per-(b, h, block of `block` tokens, channel) mean of K over the block's valid
    tokens -> bf16 values as float32 [B, H, nblk, d] (fp64 sum, fp64 divide, fp32 then
    bf16 rounding, as for the token mean)."""
    k = np.asarray(k, dtype=F32)
    B, N, H, d = k.shape
    nblk = -(-N // block)
    out = np.zeros((B, H, nblk, d), dtype=F32)
    for j in range(nblk):
        r0, r1 = j * block, min(N, (j + 1) * block)
        s = k[:, r0:r1].astype(np.float64).sum(axis=1)           # [B, H, d]
        out[:, :, j] = bf16_round((s / (r1 - r0)).astype(F32))
    return out


def quantize_int8_blocks(x, block: int = QUANT_BLOCK):
    """Per-block symmetric INT8 codes.  x: float32 [B, H, N, d] (already in the
    per-head layout).  Returns (codes int8 [B, H, N, d], scales float32 [B, H, nblk])."""
    x = np.asarray(x, dtype=F32)
    B, H, N, d = x.shape
    nblk = -(-N // block)
    codes = np.zeros((B, H, N, d), dtype=np.int8)
    scales = np.zeros((B, H, nblk), dtype=F32)
    for j in range(nblk):
        r0, r1 = j * block, min(N, (j + 1) * block)
        xb = x[:, :, r0:r1, :]
        amax = np.abs(xb).max(axis=(2, 3)).astype(F32)            # exact
        nz = amax > 0
        safe = np.where(nz, amax, F32(1))
        scale = np.where(nz, safe / F32(127), F32(0)).astype(F32)  # fp32 IEEE divide
        inv = (F32(127) / safe).astype(F32)
        y = (xb * inv[:, :, None, None]).astype(F32)              # fp32 multiply
        c = np.clip(np.rint(y), -127, 127)
        c = np.where(nz[:, :, None, None], c, 0)
        codes[:, :, r0:r1, :] = c.astype(np.int8)
        scales[:, :, j] = scale
    return codes, scales


def quantize_v_fp8(v):
    """Per-channel FP8 codes of V.  v: float32 [B, N, H, d].
    Returns (codes uint8 [B, H, N, d], scales float32 [B, H, d])."""
    v = np.asarray(v, dtype=F32)
    B, N, H, d = v.shape
    codes = np.zeros((B, H, N, d), dtype=np.uint8)
    scales = np.zeros((B, H, d), dtype=F32)
    for b in range(B):
        for h in range(H):
            vh = v[b, :, h, :]                                   # [N, d]
            vamax = np.abs(vh).max(axis=0).astype(F32)           # [d], exact
            nz = vamax > 0
            safe = np.where(nz, vamax, F32(1))
            scales[b, h] = np.where(nz, safe / F32(E4M3_MAX), F32(0))
            inv = (F32(E4M3_MAX) / safe).astype(F32)
            y = (vh * inv[None, :]).astype(F32)                  # fp32 multiply
            c = e4m3_encode(y)
            codes[b, h] = np.where(nz[None, :], c, np.uint8(0))
    return codes, scales


def quantize(q, k, v, smooth_k: bool = True, block: int = QUANT_BLOCK,
             k_block_mean: bool = False) -> dict:
    """All quantised operands of one attention call.  q, k, v: float32 [B, N, H, d]
    holding bf16 values.  ``smooth_k=False`` skips the K mean subtraction (used only to
    measure what smoothing buys).  ``block``: tokens per Q/K scale (64, or 1 for one
    scale per token); it is returned with the operands.  ``k_block_mean``: K keeps a
    bf16 mean per 64-token block (returned as k_bmean [B, H, nblk, d]) and only the
    residual is quantised; k_mean is still the token mean."""
    q = np.asarray(q, dtype=F32)
    k = np.asarray(k, dtype=F32)
    qh = q.transpose(0, 2, 1, 3)
    kh = k.transpose(0, 2, 1, 3)
    N = k.shape[1]
    kbm = None
    if k_block_mean:
        mu = k_token_mean(k)
        kbm = k_block_means(k)                                   # [B, H, nblk, d]
        rep = np.repeat(kbm, QUANT_BLOCK, axis=2)[:, :, :N]      # mean of each token's block
        kr = (kh - rep).astype(F32)                              # fp32 subtraction
    elif smooth_k:
        mu = k_token_mean(k)                                     # [B, H, d]
        kr = (kh - mu[:, :, None, :]).astype(F32)                # fp32 subtraction
    else:
        mu = np.zeros((k.shape[0], k.shape[2], k.shape[3]), dtype=F32)
        kr = kh
    q_i8, q_scale = quantize_int8_blocks(qh, block)
    k_i8, k_scale = quantize_int8_blocks(kr, block)
    v_f8, v_scale = quantize_v_fp8(v)
    out = dict(q_i8=q_i8, q_scale=q_scale, k_i8=k_i8, k_scale=k_scale, k_mean=mu,
               v_f8=v_f8, v_scale=v_scale, block=block)
    if kbm is not None:
        out["k_bmean"] = kbm
    return out
