"""Exact attention and the quantised attention pipeline.

EXACT (the plain definition): O = softmax(Q K^T * sm_scale) V with sm_scale = 1/sqrt(d),
evaluated in fp64 with the row maximum subtracted before exp (juejin page
"MiniMax H3 接入 SageAttention 实测加速", section 一; Baidu Cloud page
"SDPA稠密注意力模式", section 三 part 1, whose three-line PyTorch function is the
same definition).

PIPE (the quantised method): INT8 Q.K'^T with exact int32 sums, dequantised by
q_scale * k_scale * sm_scale, online softmax in fp32 and base 2 over key tiles of T
keys, P rounded to FP8 e4m3, P.V8 accumulated, normalised at the end, V scales applied
(juejin section 一 for INT8-QK/FP8-PV; bjdmk page
"GitHub榜单静默期：Attention优化从架构转向推理加速", section 2.2, for computing attention
block by block without writing the score matrix).

Readings (the pages give none of these details):
* Keys are visited in ascending tiles of T keys; the running maximum, and therefore
  each FP8 rounding of P, depends on T, so T is an argument and must equal the tile
  of the implementation under test.
* fp32 softmax arithmetic, in this order, for query i and key j (c.f. the
  correctly rounded fp32 operations written as fp32(.)):
    L    = fp32(sm_scale * log2(e))             (product formed in fp64)
    qf_i = fp32(q_scale_i * L)
    c_ij = fp32(qf_i * k_scale_j)
    s_ij = fp32(S_ij * c_ij)                     (base-2 logit, S_ij the int32 sum)
    m    = max(m_prev, max_j s_ij)               (m_prev = -inf before the first tile)
    nb   = fp32(log2(448)_fp32 - m)
    p_ij = exp2(fp32(S_ij * c_ij + nb))          (one rounding: a fused multiply-add)
    alpha= exp2(fp32(m_prev - m))
  so p_ij = 448 * 2^(s_ij - m): P is mapped onto the full e4m3 range with a static
  scale of 448, and p8_ij = e4m3(p_ij).  exp2 is evaluated to fp32 (correctly
  rounded here; an implementation's exp2 may differ by one unit in the last place).
* l accumulates the unrounded p_ij: l = alpha * l + sum_j p_ij, acc = alpha * acc +
  sum_j p8_ij * v8_j; O = acc * v_scale / l.  (The 448 cancels between acc and l.)
  acc and l are kept in fp64 here; they decide no code.
* Keys at or beyond N do not exist (no padding in the oracle).

Per-token scales (``quantize(..., block=1)``): every query and key token has its own
INT8 scale, so the key factor varies within a tile.  Reading of the arithmetic: the
key scale is applied first, y_ij = fp32(S_ij * k_scale_j); the row maximum is over
fp32(y_ij * qf_i), and p_ij = exp2(fp32(y_ij * qf_i + nb)) with one rounding (a fused
multiply-add).  qf_i and nb are as above.

Block-residual K (``quantize(..., k_block_mean=True)``): the key of token j is
mu_b + K''_j with mu_b the bf16 mean of its 64-token block.  The logit adds the query's
product with that mean: D_ib = fp32(sum_c q8_ic * mu_bc) (exact sum, one rounding),
e_ib = fp32(D_ib * qf_i); s_ij = fp32(s'_ij + e_ib) where s'_ij is the logit above,
and p_ij = exp2(fma(., ., fp32(e_ib + nb))) with the fma operands of the scale mode.

Quality mode (``bf16_p=True, fp8_p=False, fp8_v=False``): the pages mention that
quantised attention schemes offer a quality-first setting next to the speed-first one
(bjdmk page "GitHub榜单静默期：Attention优化从架构转向推理加速", section 4.3) and that
critical work should keep 16-bit attention for P.V (apatero page
"TeaCache和SageAttention优化实现更快的AI图像生成", section on when quality differences
appear).  Reading: Q.K^T stays INT8 exactly as above; the same fp32 p (including the
static 448) is rounded to bf16 (nearest, ties to even) instead of e4m3; V is not
quantised (its bf16 values are used as they are, scale 1); l still accumulates the
unrounded p.
"""
from __future__ import annotations

import math

import numpy as np

from .fp8 import e4m3_encode, e4m3_decode
from .quant import quantize, QUANT_BLOCK, bf16_round

__all__ = ["LOG2E", "default_sm_scale", "attention_exact", "qk_int32",
           "attention_pipeline", "rel_l2"]

F32 = np.float32
LOG2E = math.log2(math.e)
LOG2_448_F32 = F32(math.log2(448.0))


def default_sm_scale(d: int) -> float:
    """fp32(1/sqrt(d)), returned as a Python float holding that fp32 value."""
    return float(F32(1.0 / math.sqrt(d)))


def _rows(n: int, rows):
    return np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)


def attention_exact(q, k, v, sm_scale=None, rows=None) -> np.ndarray:
    """fp64 softmax(Q K^T * sm_scale) V.  q, k, v: float32 [B, N, H, d].
    ``rows`` selects query tokens.  Returns fp64 [B, R, H, d]."""
    q = np.asarray(q, dtype=F32)
    k = np.asarray(k, dtype=F32)
    v = np.asarray(v, dtype=F32)
    B, N, H, d = q.shape
    sm = default_sm_scale(d) if sm_scale is None else float(sm_scale)
    r = _rows(N, rows)
    out = np.empty((B, len(r), H, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kh = k[b, :, h, :].astype(np.float64)
            vh = v[b, :, h, :].astype(np.float64)
            for c0 in range(0, len(r), 512):
                qh = q[b, r[c0:c0 + 512], h, :].astype(np.float64)
                s = (qh @ kh.T) * sm
                s -= s.max(axis=1, keepdims=True)
                p = np.exp(s)
                out[b, c0:c0 + 512, h, :] = (p @ vh) / p.sum(axis=1, keepdims=True)
    return out


def qk_int32(q_codes, k_codes) -> np.ndarray:
    """Exact S = Q8 K8^T for one head.  q_codes [R, d], k_codes [M, d] int8.

    Formed as an fp64 matrix product of integer-valued operands: every product and
    partial sum is an integer of magnitude below 2^53 (|S| <= d * 127^2), so the fp64
    result is exact.  Returns int64."""
    a = np.asarray(q_codes, dtype=np.float64)
    bm = np.asarray(k_codes, dtype=np.float64)
    return (a @ bm.T).astype(np.int64)


def _fma_f32(x, c, b):
    """fp32(x * c + b) with one rounding (round to nearest even), for x and c fp32
    values (or integers below 2^24) and b fp32.  The product is exact in fp64 (at most
    48 significant bits); the fp64 sum s carries an error e that the error-free
    two-sum recovers exactly (s + e is the exact sum).  Rounding s to fp32 is then the
    correct rounding of s + e except when s sits exactly halfway between two fp32
    values and e is not zero: then the exact sum lies on e's side of the halfway
    point."""
    a = np.asarray(x, dtype=np.float64) * np.asarray(c, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    s = a + b
    bb = s - a
    e = (a - (s - bb)) + (b - bb)
    r = s.astype(F32)
    r64 = r.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        other = np.nextafter(r, np.where(s > r64, F32(np.inf), F32(-np.inf)).astype(F32))
        half = (r64 + other.astype(np.float64)) / 2
        tie = (s != r64) & (s == half) & (e != 0) & np.isfinite(s)
        toward_other = np.sign(e) == np.sign(s - r64)
    return np.where(tie & toward_other, other, r).astype(F32)


def _exp2_f32(x):
    return np.exp2(np.asarray(x, dtype=F32).astype(np.float64)).astype(F32)


def attention_pipeline(q, k, v, sm_scale=None, kv_tile: int = 128, rows=None,
                       quant=None, int8_qk: bool = True, fp8_p: bool = True,
                       fp8_v: bool = True, smooth_k: bool = True,
                       bf16_p: bool = False, block: int = QUANT_BLOCK,
                       k_block_mean: bool = False, tiles=None) -> np.ndarray:
    """Quantised attention.  q, k, v: float32 [B, N, H, d] holding bf16 values.

    ``quant``: the dict of :func:`oracle.quantize` if already computed.  ``rows``:
    query tokens to evaluate (rows are independent given the quantised K and V).
    The switches ``int8_qk``, ``fp8_p`` and ``fp8_v`` replace a quantised operand by
    its exact value; with all three off the pipeline is exact online softmax.
    ``bf16_p`` (with ``fp8_p`` off) rounds P to bf16 instead: together with
    ``fp8_v=False`` this is the quality mode (INT8 QK^T, bf16 P.V).  ``block``: tokens
    per Q/K scale when ``quant`` is not given (``quant`` carries its own); 1 selects
    per-token scales and their decision arithmetic.
    ``tiles``: block-sparse attention (``oracle.sparse``); tiles[b][h][I] lists, in
    ascending order, the key tiles of ``kv_tile`` keys that query block I (rows
    I*kv_tile ...) visits.  None visits every tile.
    The keys are those of ``quant`` (their count may differ from the queries').
    Returns fp64 [B, R, H, d]."""
    if fp8_p and bf16_p:
        raise ValueError("P is rounded either to e4m3 or to bf16, not both")
    q = np.asarray(q, dtype=F32)
    k = np.asarray(k, dtype=F32)
    v = np.asarray(v, dtype=F32)
    B, N, H, d = q.shape
    sm = default_sm_scale(d) if sm_scale is None else float(sm_scale)
    if quant is None:
        quant = quantize(q, k, v, smooth_k=smooth_k, block=block, k_block_mean=k_block_mean)
    qb = int(quant.get("block", QUANT_BLOCK))
    kbm = quant.get("k_bmean")                       # [B, H, nblk, d] or None
    r = _rows(N, rows)
    Nk = int(quant["k_i8"].shape[2]) if int8_qk else k.shape[1]
    L = F32(sm * LOG2E)
    out = np.empty((B, len(r), H, d), dtype=np.float64)
    T = int(kv_tile)
    for b in range(B):
        for h in range(H):
            if fp8_v:
                vv = e4m3_decode(quant["v_f8"][b, h]).astype(np.float64)      # [N, d]
                vs = quant["v_scale"][b, h].astype(np.float64)
            else:
                vv = v[b, :, h, :].astype(np.float64)
                vs = np.ones(d)
            if int8_qk:
                kq = quant["k_i8"][b, h]
                ks = quant["k_scale"][b, h][np.arange(Nk) // qb]                # [Nk]
            else:
                kf = k[b, :, h, :].astype(np.float64)
            if tiles is None:
                chunks = [np.arange(c0, min(len(r), c0 + 256)) for c0 in range(0, len(r), 256)]
            else:
                qblk = r // T
                chunks = [np.nonzero(qblk == I)[0] for I in np.unique(qblk)]
            for pos in chunks:
                rr = r[pos]
                R = len(rr)
                if int8_qk:
                    S = qk_int32(quant["q_i8"][b, h][rr], kq)                 # [R, N]
                    qs = quant["q_scale"][b, h][rr // qb]
                    qf = (qs * L).astype(F32)                                 # [R]
                    if kbm is not None:
                        # q8 . mean of each key block, exact then rounded to fp32; times qf
                        Dq = (quant["q_i8"][b, h][rr].astype(np.float64) @
                              kbm[b, h].astype(np.float64).T).astype(F32)      # [R, nblk]
                        E = (Dq.astype(np.float64) * qf[:, None]).astype(F32)
                        ek = E[:, np.arange(Nk) // QUANT_BLOCK]               # [R, Nk]
                    else:
                        ek = None
                else:
                    S = (q[b, rr, h, :].astype(np.float64) @ kf.T) * (sm * LOG2E)
                m = np.full(R, -np.inf, dtype=F32)
                l = np.zeros(R)
                acc = np.zeros((R, d))
                starts = (range(0, Nk, T) if tiles is None
                          else [int(J) * T for J in tiles[b][h][int(rr[0]) // T]])
                for t0 in starts:
                    t1 = min(Nk, t0 + T)
                    if int8_qk and qb > 1:
                        x = S[:, t0:t1]
                        c = (qf[:, None] * ks[None, t0:t1]).astype(F32)       # [R, t]
                        s = (x.astype(np.float64) * c).astype(F32)
                    elif int8_qk:
                        # per-token scales: the key scale first, the query factor last
                        y = (S[:, t0:t1] * ks[None, t0:t1].astype(np.float64)).astype(F32)
                        s = (y.astype(np.float64) * qf[:, None]).astype(F32)
                    else:
                        s = S[:, t0:t1].astype(F32)
                    if int8_qk and ek is not None:
                        e = ek[:, t0:t1]
                        s = (s.astype(np.float64) + e).astype(F32)            # + block-mean term
                    m_new = np.maximum(m, s.max(axis=1))
                    nb = (LOG2_448_F32 - m_new).astype(F32)
                    nbe = np.broadcast_to(nb[:, None], (len(rr), t1 - t0)).astype(F32)
                    if int8_qk and ek is not None:
                        nbe = (e.astype(np.float64) + nbe).astype(F32)
                    if int8_qk and qb > 1:
                        arg = _fma_f32(x, c, nbe)
                    elif int8_qk:
                        arg = _fma_f32(y, np.broadcast_to(qf[:, None], y.shape), nbe)
                    else:
                        arg = (s.astype(np.float64) + nb[:, None]).astype(F32)
                    p = _exp2_f32(arg)                                        # [R, t]
                    with np.errstate(invalid="ignore"):
                        alpha = _exp2_f32((m - m_new).astype(F32)).astype(np.float64)
                    alpha = np.where(np.isneginf(m), 0.0, alpha)
                    if fp8_p:
                        pq = e4m3_decode(e4m3_encode(p))
                    elif bf16_p:
                        pq = bf16_round(p).astype(np.float64)
                    else:
                        pq = p.astype(np.float64)
                    l = alpha * l + p.astype(np.float64).sum(axis=1)
                    acc = alpha[:, None] * acc + pq @ vv[t0:t1]
                    m = m_new
                out[b, pos, h, :] = acc * vs[None, :] / l[:, None]
    return out


def rel_l2(a, b) -> float:
    """||a - b||_2 / ||b||_2 in fp64."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))
