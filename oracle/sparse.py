"""Block-sparse key tiles chosen by a density.  TEST INFRASTRUCTURE ONLY: only the tests,
the smoke check and the bench's CPU-baseline leg may import this module.

Source: the sd114.wiki page "ComfyUI-sol-attn" (核心亮点, item 4, 智能调度与回退).  Its
sparse attention takes a value tau that changes over the sampling steps: sparse early,
dense late.  The page gives no rule for which blocks to skip, so this module fixes one.
Readings:

* Granularity.  Queries are taken in blocks of BQ = 128 and keys in tiles of BK = 128,
  the attention kernel's own tiles, so a skipped tile is skipped whole.
* Density.  tau (0 < tau) is the fraction of key tiles each query block keeps:
  k = max(1, min(T, ceil(tau * T))) of its T tiles.  tau >= 1 keeps every tile, which
  is the dense pipeline.
* Importance.  The importance of tile J for query block I is the mean, over the
  block's valid (query, key) pairs, of the dequantised product q_scale * k_scale * S of
  the INT8 codes (the softmax scale is a positive constant and does not change the
  order).  The 64-token scale blocks a of I and b of J each share one scale, so the
  mean follows from the per-channel code sums A_a and B_b of those blocks (exact
  integers).  Decision arithmetic, fp64, every operation correctly rounded:
      t_ab = (qs_a * ks_b) * <A_a, B_b>           (qs_a * ks_b is exact in fp64)
      imp  = ((t_00 + t_01) + (t_10 + t_11)) / (n_I * n_J)
  with a = 0, 1 the first and second scale block of I, b likewise for J, n_I and n_J
  the valid queries and keys.  A scale block that lies past the last token contributes
  t = 0.
* Selection.  The k tiles of largest importance; between equal importances the lower
  tile index wins.  The kept tiles are visited in ascending order by the same online
  softmax as the dense pipeline (``attention_pipeline(..., tiles=...)``); skipped tiles
  contribute nothing.
"""
from __future__ import annotations

import math

import numpy as np

from .quant import QUANT_BLOCK

__all__ = ["SPARSE_TILE", "keep_count", "block_code_sums", "tile_importance", "select_tiles"]

SPARSE_TILE = 128      # queries per block and keys per tile


def keep_count(density: float, n_tiles: int) -> int:
    """Tiles each query block keeps: max(1, min(T, ceil(tau * T))), tau an fp32 value."""
    tau = float(np.float32(density))
    if not tau > 0.0 or math.isnan(tau):
        raise ValueError("density must be positive")
    return max(1, min(n_tiles, math.ceil(tau * n_tiles)))


def block_code_sums(codes) -> np.ndarray:
    """Per-(b, h, 64-token block, channel) sums of INT8 codes: codes int8 [B, H, N, d]
    -> int64 [B, H, ceil(N/64), d] (exact)."""
    c = np.asarray(codes).astype(np.int64)
    B, H, N, d = c.shape
    nblk = -(-N // QUANT_BLOCK)
    out = np.zeros((B, H, nblk, d), dtype=np.int64)
    for j in range(nblk):
        out[:, :, j] = c[:, :, j * QUANT_BLOCK:(j + 1) * QUANT_BLOCK].sum(axis=2)
    return out


def tile_importance(quant: dict) -> np.ndarray:
    """Importance of every (query block, key tile) pair: fp64 [B, H, nqb, T] with
    nqb = T = ceil(N / 128), by the decision arithmetic of the module docstring."""
    if int(quant.get("block", QUANT_BLOCK)) != QUANT_BLOCK:
        raise ValueError("tile importance is defined for 64-token scale blocks")
    q8, k8 = quant["q_i8"], quant["k_i8"]
    qs, ks = quant["q_scale"], quant["k_scale"]                   # [B, H, nblk] fp32
    B, H, N, d = q8.shape
    A, Bs = block_code_sums(q8), block_code_sums(k8)              # [B, H, nblk, d]
    nblk = A.shape[2]
    nt = -(-N // SPARSE_TILE)
    per = SPARSE_TILE // QUANT_BLOCK                              # scale blocks per tile (2)
    valid = [min(N, (i + 1) * SPARSE_TILE) - i * SPARSE_TILE for i in range(nt)]
    imp = np.zeros((B, H, nt, nt), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            dots = A[b, h] @ Bs[b, h].T                           # int64 [nblk, nblk], exact
            for I in range(nt):
                for J in range(nt):
                    t = [[0.0, 0.0], [0.0, 0.0]]
                    for x in range(per):
                        a = per * I + x
                        for y in range(per):
                            c = per * J + y
                            if a < nblk and c < nblk:
                                w = float(qs[b, h, a]) * float(ks[b, h, c])   # exact
                                t[x][y] = w * float(dots[a, c])
                    imp[b, h, I, J] = ((t[0][0] + t[0][1]) + (t[1][0] + t[1][1])) / float(valid[I] * valid[J])
    return imp


def select_tiles(quant: dict, density: float):
    """Kept key tiles per query block.  Returns (counts int64 [B, H, nqb], tiles: nested
    lists [b][h][I] of ascending tile indices)."""
    imp = tile_importance(quant)
    B, H, nqb, nt = imp.shape
    k = keep_count(density, nt)
    counts = np.full((B, H, nqb), k, dtype=np.int64)
    tiles = [[[None] * nqb for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for I in range(nqb):
                order = sorted(range(nt), key=lambda J: (-imp[b, h, I, J], J))
                tiles[b][h][I] = sorted(order[:k])
    return counts, tiles
