// Fused quantised attention for gfx950 (MI355X): INT8 Q.K^T on matrix cores with
// int32 accumulation, dequantisation, fp32 online softmax in base 2, P rounded to
// FP8 e4m3, P.V on FP8 matrix cores, bf16 output (juejin page "MiniMax H3 接入
// SageAttention 实测加速", section 一: INT8 for QK, FP8 for PV; bjdmk page
// "GitHub榜单静默期：Attention优化从架构转向推理加速", section 2.2: blockwise computation
// that never writes the score matrix out).  A quality mode keeps P.V in bf16 (P rounded
// to bf16, V unquantised) on bf16 matrix cores (the quality-first setting of the same
// bjdmk page, section 4.3).
//
// Options (template parameters, chosen by the mode bits of the C ABI): PV = FP8 or bf16
// P.V; TOK = one Q/K scale per token (the tile's key scales are staged in LDS with the
// K tile); KBM = block-residual K (sd114.wiki ComfyUI-sol-attn page, "核心亮点" item 1:
// the tile's two bf16 block means are staged with the K tile, and their products with
// the query codes, on bf16 matrix cores, enter the logits); PAIR = the issue priorities
// that even out the two workgroups sharing a CU, chosen by the host for grids of at most
// two rounds (IssuePriority).  The block-sparse kernels (k_attn32_sparse at d = 128,
// k_attn_sparse at d = 64) are the FP8 bodies visiting only the key tiles their query
// block keeps (sd114.wiki ComfyUI-sol-attn page, "核心亮点" item 4; the selection is in
// sage_select.hip).
//
// Two bodies.  The default path at d = 128 (FP8 P.V, 64-token scales, token-mean K,
// dense and block-sparse) runs on 32x32 matrix-core tiles, one 32-query group per wave
// (k_attn32, described at attn32_body below); every other combination runs on the
// 16x16 tiles described here (k_attn).  Both share the workgroup shape, the LDS DMA
// staging, the per-element softmax arithmetic and the epilogue.
//
// Work decomposition
//   workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 32 queries (16x16
//   body: 2 groups of 16); 2 workgroups per CU (2 waves per SIMD).  Keys are visited in
//   tiles of 128.
//   K tiles (128 x d int8) and V tiles (d x 128, channel-major) are copied HBM -> LDS
//   by LDS DMA (buffer_load_dwordx4 ... lds: no data registers, and the per-tile
//   address advance is a scalar offset, so no vector instruction) and shared by the 4
//   waves: speed mode double-buffers (K, V) stages, one tile ahead of use; quality mode
//   double-buffers K and refills a single bf16 V buffer during the softmax of the same
//   tile.  The copies of the next tile are issued after the K operand reads of the
//   current one (the compiler makes an LDS read wait for every LDS copy issued before
//   it), so they overlap the softmax.  Waits are counted (s_waitcnt vmcnt(n) +
//   s_barrier), so a wave only waits for the copies it needs.
//
// Register layouts (16x16 matrix-core tiles; lane l, r = l % 16, g = l / 16)
//   S^T = K . Q^T with v_mfma_i32_16x16x64_i8: the row operand is 16 keys, the column
//   operand 16 queries.  Output element (row 4g+i, column r) sits in lane l, register i.
//   Row j of key sub-tile kt is mapped to tile key 32*(j/4) + 4*kt + j%4, so lane l ends
//   up holding, for its query r, the 32 consecutive tile keys 32g .. 32g+31 (register i
//   of sub-tile kt = key 32g + 4kt + i).  Those 32 keys lie in one 64-key scale block.
//   The int32 accumulators start at 0x4B400000 (s_to_f32 recovers fp32(S) with one
//   exact subtraction).
//   O^T = V^T . P^T with v_mfma_f32_16x16x128_f8f6f4 (speed): the column operand of
//   lane l is 32 bytes of P for query r over keys 32g .. 32g+31, exactly the values the
//   lane already holds, so P never leaves its registers; the row operand is 32 bytes of
//   channel-major V (channel 16*dt + r, the same 32 keys).  Quality mode uses
//   v_mfma_f32_16x16x32_bf16 four times per channel tile: step s takes the lane's keys
//   32g + 8s .. +7 from both operands (any key order common to both operands sums the
//   same products).  Output: lane l holds O[query r][channel 16*dt + 4g + i].
//   Every per-query quantity (running max m, partial row sum, accumulators) is thus
//   lane-local; only the tile maximum and the final row sum combine the 4 lanes
//   r, r+16, r+32, r+48.
#include <atomic>
#include "sage_internal.h"
#include "sage_device.h"
#include "sage_tiles.h"

namespace sage {

constexpr int G = kGroupsPerWave;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Per-lane LDS byte offsets of the matrix-core operand reads (sage_tiles.h): the
// offset of K sub-tile kt is koff[kk] + kt * 4 * D and that of V channel tile dt is
// voff[half] + dt * 16 * 128.
template <int D>
struct LaneOffsets {
  int koff[D / 64];
  int voff[2];
  __device__ __forceinline__ explicit LaneOffsets(int lane) {
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) koff[kk] = k_read_offset<D>(lane, kk);
#pragma unroll
    for (int h = 0; h < 2; ++h) voff[h] = v_read_offset(lane, h);
  }
};

// Buffer resource of `bytes` bytes at p (raw buffer, no stride; gfx9 descriptor word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Per-lane source offsets of the LDS DMA copies (computed once per kernel, sage_tiles.h):
// the K tile copy of wave w, instruction j reads K + koff0 + 1024 j (the K swizzle
// leaves key bits 3 and 4, which j changes, alone: k_dma_src is affine in j, so one
// register serves, the 1024 j going into the scalar offset, which moves the global
// address only; the instruction's immediate offset would move the LDS address too),
// the V tile copy V + voff[j] (bytes, relative to the tile's first key); copy j lands at
// LDS offset dma_lds_offset(w, j, PW, lane).
template <int D>
struct DmaOffsets {
  static constexpr int KPW = DmaShape<D>::KPW;
  static constexpr int VPW = DmaShape<D>::VPW;
  static constexpr int PER_TILE = KPW + VPW;     // DMA instructions per wave per tile
  uint32_t koff0;
  uint32_t voff[VPW];
  __device__ __forceinline__ DmaOffsets(int wave, int lane, int64_t npad) {
    koff0 = k_dma_src<D>(wave, 0, lane);
#pragma unroll
    for (int j = 0; j < VPW; ++j) voff[j] = v_dma_src<D>(wave, j, lane, npad);
  }
  // tile_off: byte offset of the tile inside the buffer (a scalar operand)
  __device__ __forceinline__ void issue_k(__amdgpu_buffer_rsrc_t kbufr, int tile_off, uint8_t* klds, int wave) const {
#pragma unroll
    for (int j = 0; j < KPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kbufr, (lds_ptr_t)(klds + (wave * KPW + j) * 1024), 16, koff0,
                                               tile_off + 1024 * j, 0, 0);
  }
  __device__ __forceinline__ void issue_v(__amdgpu_buffer_rsrc_t vbufr, int tile_off, uint8_t* vlds, int wave) const {
#pragma unroll
    for (int j = 0; j < VPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vbufr, (lds_ptr_t)(vlds + (wave * VPW + j) * 1024), 16, voff[j],
                                               tile_off, 0, 0);
  }
};

// Quality mode: per-lane LDS offsets of the bf16 V reads (step s of channel tile dt is
// voff[s] + dt * 16 * 256) and source offsets of the bf16 V tile copies.
template <int D>
struct LaneOffsets16 {
  int voff[4];
  __device__ __forceinline__ explicit LaneOffsets16(int lane) {
#pragma unroll
    for (int s = 0; s < 4; ++s) voff[s] = v16_read_offset(lane, s);
  }
};

template <int D>
struct DmaOffsets16 {
  static constexpr int VPW = DmaShape<D>::V16PW;
  uint32_t voff[VPW];
  __device__ __forceinline__ DmaOffsets16(int wave, int lane, int64_t npad) {
#pragma unroll
    for (int j = 0; j < VPW; ++j) voff[j] = v16_dma_src<D>(wave, j, lane, npad);
  }
  __device__ __forceinline__ void issue_v(__amdgpu_buffer_rsrc_t vbufr, int tile_off, uint8_t* vlds, int wave) const {
#pragma unroll
    for (int j = 0; j < VPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vbufr, (lds_ptr_t)(vlds + (wave * VPW + j) * 1024), 16, voff[j],
                                               tile_off, 0, 0);
  }
};

// Column operands (queries) of S^T for this wave: lane l holds query row `qrow0 + 16*gq
// + r`, bytes 64*kk + 16*g .. +15.
template <int D>
__device__ __forceinline__ void load_q(const int8_t* __restrict__ qh, int qrow0, int lane,
                                       v4i (&qf)[G][D / 64]) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int gq = 0; gq < G; ++gq)
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk)
      qf[gq][kk] = *(const v4i*)(qh + (int64_t)(qrow0 + 16 * gq + r) * D + 64 * kk + 16 * g);
}

// K operand of S^T sub-tile kt = q / (D/64), 64-byte slice kk = q % (D/64).
template <int D>
__device__ __forceinline__ v4i load_kfrag(const uint8_t* kbuf, int q, const LaneOffsets<D>& lo) {
  const int kt = q / (D / 64), kk = q % (D / 64);
  return *(const v4i*)(kbuf + lo.koff[kk] + kt * 4 * D);
}

// V operand of O^T channel tile dt.
template <int D>
__device__ __forceinline__ v8i load_vfrag(const uint8_t* vbuf, int dt, const LaneOffsets<D>& lo) {
  const v4i a = *(const v4i*)(vbuf + lo.voff[0] + dt * 16 * kKvTile);
  const v4i b = *(const v4i*)(vbuf + lo.voff[1] + dt * 16 * kKvTile);
  return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// The attention kernel starts its int32 S accumulators at kSBiasBits instead of 0.  The
// products are bounded, |S| <= d * 127^2 < 2^21, so S + kSBiasBits is the bit pattern of
// the float S + 1.5 * 2^23, which lies in [2^23, 2^24) where floats are the integers;
// subtracting 1.5 * 2^23 then yields fp32(S) exactly.  One full-rate add replaces the
// int-to-float conversion, which issues at a quarter of the VALU rate.  The biased
// values keep the order of the integers, so maxima may still be taken on them.
constexpr int kSBiasBits = 0x4B400000;
constexpr float kSBias = 12582912.0f;                // 1.5 * 2^23
static_assert(128 * 127 * 127 < (1 << 21), "S + 1.5 * 2^23 must stay in [2^23, 2^24)");

__device__ __forceinline__ float s_to_f32(int biased) { return __builtin_bit_cast(float, biased) - kSBias; }

// int32 S^T of both query groups for a staged key tile, plus s0 (each K operand feeds
// both groups): S[gq][kt] register i = s0 + S(query r of group gq, tile key 32g + 4kt + i).
template <int D>
__device__ __forceinline__ void qk_tile(const uint8_t* kbuf, const v4i (&qfr)[G][D / 64],
                                        const LaneOffsets<D>& lo, v4i (&S)[G][8], int s0) {
#pragma unroll
  for (int q = 0; q < 8 * (D / 64); ++q) {
    const int kt = q / (D / 64), kk = q % (D / 64);
    const v4i a = load_kfrag<D>(kbuf, q, lo);
#pragma unroll
    for (int gq = 0; gq < G; ++gq)
      S[gq][kt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qfr[gq][kk], kk == 0 ? v4i{s0, s0, s0, s0} : S[gq][kt], 0, 0, 0);
  }
}

// The P operand of one query group: e4m3 (word kt = keys 32g + 4kt .. +3), or bf16
// (words 2kt and 2kt+1 = keys 32g + 4kt .. +3, in w[kt / 4]).
template <int PV> struct PTile;
template <> struct PTile<kPvFp8> { v8i w; };
template <> struct PTile<kPvBf16> { v8i w[2]; };

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Two fp32 values -> two bf16 (round to nearest even), first value in the low half.
__device__ __forceinline__ int pk_bf16(float a, float b) {
  return __builtin_bit_cast(int, __builtin_convertvector((v2f){a, b}, v2bf));
}

// Saturation of the FP8 P codes.  p = 448 * 2^(s - m) is at most 448 up to the fp32
// roundings of the running maximum m, of log2(448) - m and (block-residual K) of the
// block-mean term e, each at most half an ulp of a value below 2^17 when |m| and |e|
// stay below 2^16: together less than 2^-5 in the exponent, so p < 448 * 2^(2^-5) <
// 464, which v_cvt_pk_fp8_f32 rounds to 448 (it gives the NaN code 0x7F from 464 up).
// Tiles whose |m| or |e| reach 2^16 (base-2 logits of 65536: only for inputs far
// outside attention's usual range) replace every 0x7F code of P by 0x7E (448) after
// the conversion, as an e4m3 encoder that saturates does; l sums the unclamped p.
constexpr float kSatLimit = 65536.0f;

// Four e4m3 codes of non-negative values (bytes 0x00 .. 0x7F): 0x7F -> 0x7E.  A byte
// is 0x7F exactly when adding 1 sets its top bit, with no carry into the next byte.
__device__ __forceinline__ int e4m3x4_saturate(int w) {
  const uint32_t u = (uint32_t)w;
  return (int)(u - (((u + 0x01010101u) & 0x80808080u) >> 7));
}

__device__ __forceinline__ bool wave_any(bool c) { return __ballot(c) != 0ull; }

template <bool BM>
__device__ __forceinline__ bool saturate_tile(const float (&m)[kGroupsPerWave], const float (&e)[kGroupsPerWave]) {
  bool big = false;
#pragma unroll
  for (int gq = 0; gq < kGroupsPerWave; ++gq)
    big = big || fabsf(m[gq]) >= kSatLimit || (BM && fabsf(e[gq]) >= kSatLimit);
  return wave_any(big);
}

template <int PV>
__device__ __forceinline__ void saturate_p(PTile<PV>& P) {
  if constexpr (PV == kPvFp8) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) P.w[kt] = e4m3x4_saturate(P.w[kt]);
  }
}

// Rounds the p of keys 32g + 4kt .. +3 into P.  The e4m3 conversions overwrite both
// halves of the word, so its previous contents only serve as the operand they replace.
template <int PV>
__device__ __forceinline__ void store_p(PTile<PV>& P, int kt, const float (&p)[4]) {
  if constexpr (PV == kPvFp8) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], P.w[kt], false);
    P.w[kt] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
  } else {
    P.w[kt >> 2][2 * (kt & 3)] = pk_bf16(p[0], p[1]);
    P.w[kt >> 2][2 * (kt & 3) + 1] = pk_bf16(p[2], p[3]);
  }
}

// acc[gq][dt] += V^T(channels 16dt..16dt+15) . P[gq]^T for both groups.
template <int D>
__device__ __forceinline__ void pv_tile(const uint8_t* vbuf, const PTile<kPvFp8> (&P)[G],
                                        const LaneOffsets<D>& lo, v4f (&acc)[G][D / 16]) {
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const v8i vf = load_vfrag<D>(vbuf, dt, lo);
#pragma unroll
    for (int gq = 0; gq < G; ++gq)
      acc[gq][dt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vf, P[gq].w, acc[gq][dt], 0, 0, 0, 0, 0, 0);
  }
}

// Quality mode: the same product with bf16 P and bf16 V, four 32-key steps per channel
// tile; step s uses the lane's keys 32g + 8s .. +7 of both operands.
template <int D>
__device__ __forceinline__ void pv_tile16(const uint8_t* vbuf, const PTile<kPvBf16> (&P)[G],
                                          const LaneOffsets16<D>& lo, v4f (&acc)[G][D / 16]) {
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v8bf vf = __builtin_bit_cast(v8bf, *(const v4i*)(vbuf + lo.voff[s] + dt * 16 * 256));
#pragma unroll
      for (int gq = 0; gq < G; ++gq) {
        const v4i pw = (s & 1) ? __builtin_shufflevector(P[gq].w[s >> 1], P[gq].w[s >> 1], 4, 5, 6, 7)
                               : __builtin_shufflevector(P[gq].w[s >> 1], P[gq].w[s >> 1], 0, 1, 2, 3);
        acc[gq][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(v8bf, pw), acc[gq][dt], 0, 0, 0);
      }
    }
  }
}

// Online-softmax update of one 16-query group for one tile, not interleaved (used at the
// ends of the pipeline and for the ragged last tile).  S holds biased accumulators
// (s_to_f32 recovers fp32(S) exactly); c = fp32(q factor * k_scale) of this lane's keys.  Produces the
// P operand, updates the running max m and this lane's partial row sum, and
// returns alpha = 2^(m_old - m_new), the factor the accumulators need.  When MASKED,
// keys at tile index >= nvalid are removed by giving them the logit -inf; a lane whose
// c is 0 then uses x = 0 and c = 1 for its valid keys, which yields the same s = 0 and
// p = 448 * 2^-m without forming -inf * 0.
template <bool MASKED, int PV, bool BM = false>
__device__ __forceinline__ float softmax_group(v4i (&S)[8], float c, int nvalid, float log2_pscale,
                                               float& m, float& lpart, PTile<PV>& P, int g, float e = 0.0f) {
  float xf[8][4];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) xf[kt][i] = s_to_f32(S[kt][i]);
  if constexpr (MASKED) {
    const int nv = nvalid - 32 * g;                // valid keys among this lane's 32
    const bool zero_c = (c == 0.0f);
    c = zero_c ? 1.0f : c;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xf[kt][i] = ((4 * kt + i) < nv) ? (zero_c ? 0.0f : xf[kt][i]) : -INFINITY;
  }
  float xm = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) xm = fmaxf(xm, xf[kt][i]);
  // c >= 0 and rounding is monotone, so this is the max of fp32(x * c) over the keys
  float sl = (xm == -INFINITY) ? -INFINITY : (BM ? xm * c + e : xm * c);
  sl = max_over_lane_groups(sl);
  const float m_new = fmaxf(m, sl);
  const float nb = BM ? e + (log2_pscale - m_new) : log2_pscale - m_new;
  const float alpha = __builtin_amdgcn_exp2f(m - m_new);
  float lsum = 0.0f;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(xf[kt][i], c, nb));
      lsum += p[i];
    }
    store_p<PV>(P, kt, p);
  }
  if (PV == kPvFp8 && wave_any(fabsf(m_new) >= kSatLimit || (BM && fabsf(e) >= kSatLimit))) saturate_p<PV>(P);
  lpart = alpha * lpart + lsum;
  m = m_new;
  return alpha;
}

// acc *= alpha, skipped when no lane's maximum moved (multiplying by exactly 1).
template <int D>
__device__ __forceinline__ void rescale(v4f (&acc)[D / 16], float alpha) {
  if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] *= alpha;
  }
}

// Online-softmax update of both query groups for one full tile (no masking): integer
// row max of the biased S (exact, no NaN handling), exact fp32 S by s_to_f32, exp2 of the
// fused multiply-add, rounding into P, independent partial row sums.  Same
// arithmetic as softmax_group<false>; the two groups' work is interleaved for ILP.
template <int PV, bool BM = false>
__device__ __forceinline__ void softmax_tile(v4i (&S)[G][8], const float (&c)[G], float log2_pscale,
                                             float (&m)[G], float (&lpart)[G], PTile<PV> (&P)[G],
                                             float (&alpha)[G], const float (&e)[G]) {
  // integer row maximum: two chains of three-input maxima (16 per group)
  int xmi[G];
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    int a0 = max(S[gq][0][0], S[gq][0][1]);
    int a1 = max(S[gq][1][0], S[gq][1][1]);
    a0 = max(max(a0, S[gq][0][2]), S[gq][0][3]);
    a1 = max(max(a1, S[gq][1][2]), S[gq][1][3]);
#pragma unroll
    for (int kt = 2; kt < 8; kt += 2)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        a0 = max(max(a0, S[gq][kt][i]), S[gq][kt][i + 1]);
        a1 = max(max(a1, S[gq][kt + 1][i]), S[gq][kt + 1][i + 1]);
      }
    xmi[gq] = max(a0, a1);
  }
  float nb[G], m_new[G], sl[G];
  static_assert(G == 2, "the lane-group reduction below pairs the two query groups");
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    // c >= 0 and rounding is monotone: this is the max of fp32(x * c) (+ e) over the keys
    const float xs = s_to_f32(xmi[gq]) * c[gq];
    sl[gq] = BM ? xs + e[gq] : xs;
  }
  max_over_lane_groups_pair(sl[0], sl[1]);
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    m_new[gq] = max2_nan_free(m[gq], sl[gq]);
    nb[gq] = BM ? e[gq] + (log2_pscale - m_new[gq]) : log2_pscale - m_new[gq];
    alpha[gq] = __builtin_amdgcn_exp2f(m[gq] - m_new[gq]);
  }
  float ls[G][4];   // partial row sums, started from the first sub-tile's p (p >= 0, so 0 + p = p)
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
    for (int gq = 0; gq < G; ++gq) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_to_f32(S[gq][kt][i]), c[gq], nb[gq]));
#pragma unroll
      for (int i = 0; i < 4; ++i) ls[gq][i] = kt == 0 ? p[i] : ls[gq][i] + p[i];
      store_p<PV>(P[gq], kt, p);
    }
  }
  if (PV == kPvFp8 && saturate_tile<BM>(m_new, e)) {
#pragma unroll
    for (int gq = 0; gq < G; ++gq) saturate_p<PV>(P[gq]);
  }
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    lpart[gq] = alpha[gq] * lpart[gq] + ((ls[gq][0] + ls[gq][1]) + (ls[gq][2] + ls[gq][3]));
    m[gq] = m_new[gq];
  }
}

// With BM (block-residual K) the logits gain e = fp32(qf * q8.mean_block), constant over
// the lane's 32 keys: the maximum is taken over fp32(. + e) and e is added to nb.
//
// Online-softmax update of both query groups with per-token scales: ks_lds holds the
// tile's 128 key scales (fp32, in key order), so the scale of tile key 32g + 4kt + i is
// at byte 128g + 16kt + 4i, and qf is the query factor fp32(q_scale * sm_scale * log2 e).
// y = fp32(S * ks) per key (S from the biased accumulators by s_to_f32); the row
// maximum is the max of fp32(y * qf) (qf >= 0 and rounding is monotone, so it is
// fp32(max y * qf)); p = exp2(fma(y, qf, nb)).  When MASKED, keys at tile index >=
// nvalid get p = 0 and take no part in the maximum.
template <int PV, bool MASKED, bool BM = false>
__device__ __forceinline__ void softmax_tile_tok(v4i (&S)[G][8], const uint8_t* ks_lds, const float (&qf)[G],
                                                 int nvalid, int g, float log2_pscale, float (&m)[G],
                                                 float (&lpart)[G], PTile<PV> (&P)[G], float (&alpha)[G],
                                                 const float (&e)[G]) {
  float y[G][8][4];
  float ym[G];
  // Without BM all 32 scales are read up front.  With BM (32 more registers hold the
  // query codes as bf16) each key sub-tile's four scales are read just before their
  // products with both groups, so that only a few are live next to the S registers
  // (measured at 16K keys: 20% faster than the up-front reads, which spill; without BM
  // the up-front reads are 1-3% faster).
  v4f ks_all[BM ? 1 : 8];
  if constexpr (!BM) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) ks_all[kt] = *(const v4f*)(ks_lds + 128 * g + 16 * kt);
  }
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    const v4f ks = BM ? *(const v4f*)(ks_lds + 128 * g + 16 * kt) : ks_all[BM ? 0 : kt];
#pragma unroll
    for (int gq = 0; gq < G; ++gq)
#pragma unroll
      for (int i = 0; i < 4; ++i) y[gq][kt][i] = s_to_f32(S[gq][kt][i]) * ks[i];
  }
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    float a0 = -INFINITY, a1 = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 8; kt += 2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v0 = !MASKED || (4 * kt + i) < nvalid - 32 * g;
        const bool v1 = !MASKED || (4 * kt + 4 + i) < nvalid - 32 * g;
        a0 = fmaxf(a0, v0 ? y[gq][kt][i] : -INFINITY);
        a1 = fmaxf(a1, v1 ? y[gq][kt + 1][i] : -INFINITY);
      }
    ym[gq] = fmaxf(a0, a1);
  }
  float nb[G], m_new[G], sl[G];
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    const float ys = ym[gq] * qf[gq];
    sl[gq] = ym[gq] == -INFINITY ? -INFINITY : (BM ? ys + e[gq] : ys);
  }
  max_over_lane_groups_pair(sl[0], sl[1]);
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    m_new[gq] = max2_nan_free(m[gq], sl[gq]);
    nb[gq] = BM ? e[gq] + (log2_pscale - m_new[gq]) : log2_pscale - m_new[gq];
    alpha[gq] = __builtin_amdgcn_exp2f(m[gq] - m_new[gq]);
  }
  float ls[G][4];   // partial row sums, started from the first sub-tile's p (p >= 0, so 0 + p = p)
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
    for (int gq = 0; gq < G; ++gq) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(y[gq][kt][i], qf[gq], nb[gq]));
        if constexpr (MASKED) p[i] = (4 * kt + i) < nvalid - 32 * g ? p[i] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) ls[gq][i] = kt == 0 ? p[i] : ls[gq][i] + p[i];
      store_p<PV>(P[gq], kt, p);
    }
  }
  if (PV == kPvFp8 && saturate_tile<BM>(m_new, e)) {
#pragma unroll
    for (int gq = 0; gq < G; ++gq) saturate_p<PV>(P[gq]);
  }
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    lpart[gq] = alpha[gq] * lpart[gq] + ((ls[gq][0] + ls[gq][1]) + (ls[gq][2] + ls[gq][3]));
    m[gq] = m_new[gq];
  }
}

// Per-token key scales of one tile, staged in LDS next to the K tile: each wave copies
// 128 of the 512 bytes with 8 lanes (one DMA instruction per wave).
__device__ __forceinline__ void issue_kscale(__amdgpu_buffer_rsrc_t ksr, int tile_off, uint8_t* lds, int wave, int lane) {
  if (lane < 8)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ksr, (lds_ptr_t)(lds + 128 * wave), 16, 128 * wave + 16 * lane,
                                             tile_off, 0, 0);
}


// Block-residual K: the bf16 means of the tile's two 64-key blocks (2 x D values) are
// staged in LDS next to the K tile, D bytes per wave (D/16 lanes of one DMA instruction).
template <int D>
__device__ __forceinline__ void issue_kbmean(__amdgpu_buffer_rsrc_t r, int tile_off, uint8_t* lds, int wave, int lane) {
  if (lane < D / 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds + D * wave), 16, D * wave + 16 * lane,
                                             tile_off, 0, 0);
}

// The query's INT8 codes as bf16 (exact), in the operand order of the mean products:
// qb[gq][kk][h] = channels 64kk + 16g + 8h .. +7 of query r, from qfr[gq][kk].
template <int D>
__device__ __forceinline__ void q_codes_bf16(const v4i (&qfr)[G][D / 64], v4i (&qb)[G][D / 64][2]) {
#pragma unroll
  for (int gq = 0; gq < G; ++gq)
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int word = qfr[gq][kk][2 * h + (w >> 1)];
          const int sh = 16 * (w & 1);
          const float lo = (float)(int8_t)(word >> sh), hi = (float)(int8_t)(word >> (sh + 8));
          qb[gq][kk][h][w] = pk_bf16(lo, hi);
        }
}

// e[gq] = fp32(qf * D) with D = q8 . mean of this lane's key block (bf16 matrix cores,
// fp32 accumulation): rows of the row operand are the two block means (rows 0-7 block
// 0, 8-15 block 1), columns the queries, so lane (r, g) finds D for query r and block
// g/2 in register 0.
template <int D>
__device__ __forceinline__ void block_mean_terms(const uint8_t* kbm_lds, const v4i (&qb)[G][D / 64][2],
                                                 const float (&qf)[G], int r, int g, float (&e)[G]) {
  v4f acc[G] = {};
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4i mf = *(const v4i*)(kbm_lds + (r >> 3) * 2 * D + 128 * kk + 32 * g + 16 * h);
#pragma unroll
      for (int gq = 0; gq < G; ++gq)
        acc[gq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, mf),
                                                          __builtin_bit_cast(v8bf, qb[gq][kk][h]), acc[gq], 0, 0, 0);
    }
#pragma unroll
  for (int gq = 0; gq < G; ++gq) e[gq] = acc[gq][0] * qf[gq];
}

// Wave issue priorities.
// - A wave raises its priority while it issues a run of matrix-core instructions, so
//   that on a SIMD shared with a wave in its softmax the matrix core is fed first and the
//   softmax's VALU work fills the cycles the products take (measured: +3% at 4.6K and
//   16K keys, neutral at 64K).
// - PAIR (chosen by the host when the grid is at most two rounds of two workgroups per
//   CU): the base priority also evens out the two workgroups that share a CU.
//   Workgroups are dispatched in id order, about one per CU for each group of cu_count
//   consecutive ids, so in the first rounds a CU's two workgroups come from neighbouring
//   groups and the later one is the younger. When waves of both are ready, a SIMD issues
//   the older wave first; the younger workgroup then lags and runs its last tiles alone,
//   at a lower rate, which in the last round leaves the CU's other slot idle. With PAIR,
//   workgroups of odd groups take base priority 1, the others 0, and the matrix-core
//   runs priority 2 (measured: +3% at 4.6K keys and 24 heads). The per-workgroup choice
//   costs a branch at each switch, which measured 1-5% slower on long grids, where the
//   pairs are no longer neighbours in id; those use the plain form.
template <bool PAIR>
struct IssuePriority {
  int raised = 0;   // workgroup-uniform (scalar register)
  __device__ __forceinline__ explicit IssuePriority(int cu_count) {
    if constexpr (PAIR)
      raised = __builtin_amdgcn_readfirstlane(((blockIdx.x / (unsigned)cu_count) & 1u) ? 1 : 0);
  }
  __device__ __forceinline__ void mfma() const { __builtin_amdgcn_s_setprio(PAIR ? 2 : 1); }
  __device__ __forceinline__ void base() const {
    if constexpr (PAIR) {
      if (raised) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    } else {
      __builtin_amdgcn_s_setprio(0);
    }
  }
};

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Barrier that orders LDS use between the waves of the workgroup.  Each wave first waits
// for its own LDS reads and scalar loads (lgkmcnt 0) and for its DMA copies older than
// the newest `KEEP` ones (they complete in order), so after the barrier every copy but
// the newest KEEP per wave has landed and no wave still reads a buffer about to be
// refilled.
template <int KEEP>
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(KEEP));
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// LDS stages (each a K tile and a V tile): copies run kStages-1 tiles ahead of use.
template <int D>
struct Ring {
  static constexpr int STAGE = Lds<D>::KBYTES + Lds<D>::VBYTES;
  uint8_t* smem;
  __device__ __forceinline__ uint8_t* kbuf(int t) const { return smem + (t % kStages) * STAGE; }
  __device__ __forceinline__ uint8_t* vbuf(int t) const { return smem + (t % kStages) * STAGE + Lds<D>::KBYTES; }
};

template <int D, int PV, bool TOK, bool KBM>
struct AttnSmem {
  static constexpr int MAIN = PV == kPvFp8 ? kStages * Ring<D>::STAGE
                                           : 2 * Lds<D>::KBYTES + Lds<D>::V16BYTES;
  static constexpr int KSCALE = TOK ? 2 * 512 : 0;   // per-token key scales, 2 buffers
  static constexpr int KBMEAN = KBM ? 2 * 4 * D : 0; // two block means per tile, 2 buffers
  static constexpr int BYTES = MAIN + KSCALE + KBMEAN;
};

// TOK: per-token Q/K scales (q_scale, k_scale [B][H][Npad]); the key scales of each
// tile are staged in LDS with the K tile.  KBM: block-residual K; the block means of
// each tile are staged likewise and their products with the query codes are added to
// the logits.  SPARSE: the workgroup visits only the key tiles its query block keeps
// (a.tile_list, ascending), with the same per-tile arithmetic; the masked last tile
// is visited only if it is kept.
template <int D, int PV, bool TOK, bool KBM, bool SPARSE, bool PAIR>
__device__ __forceinline__ void attn_body(const AttnArgs& a) {
  static_assert(!SPARSE || (PV == kPvFp8 && !TOK && !KBM), "block-sparse visits: FP8 P.V, 64-token scales");
  using Smem = AttnSmem<D, PV, TOK, KBM>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Smem::BYTES];
  uint8_t* const ksmem = smem + Smem::MAIN;
  auto ksbuf = [&](int t) { return ksmem + (t & 1) * 512; };
  uint8_t* const kbmem = smem + Smem::MAIN + Smem::KSCALE;
  auto kbmbuf = [&](int t) { return kbmem + (t & 1) * 4 * D; };

  // workgroup-uniform indices kept in scalar registers (readfirstlane), so that the
  // per-tile k_scale reads are scalar loads and never wait on the vector-memory counter
  const IssuePriority<PAIR> prio(a.cu_count);
  if constexpr (PAIR) prio.base();
  const int nqb = (int)(a.npad / kBlockM);
  const int total = nqb * a.B * a.H;
  const int work = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, total));
  const int64_t bh = __builtin_amdgcn_readfirstlane(work / nqb);
  const int qb = __builtin_amdgcn_readfirstlane(work % nqb);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int r = lane & 15, g = lane >> 4;
  // After the main loop the lane-derived indices are derived again from the lane id
  // computed anew (mbcnt counts the lanes below this one), so that the compiler
  // recomputes what the masked last tile and the epilogue need instead of keeping it in
  // registers across the loop (the per-token block-residual instances would otherwise
  // spill it).
  auto refresh_lane = [&]() {
    int l2 = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(l2));
    r = l2 & 15;
    g = l2 >> 4;
  };
  const int qrow0 = qb * kBlockM + wave * (G * 16);
  const int64_t nblk = a.npad / kQuantBlock;

  const LaneOffsets<D> lo(lane);
  const DmaOffsets<D> dma(wave, lane, a.npad);
  const int8_t* kh = a.k_i8 + bh * a.npad * D;
  // buffer resources of this head's operands (byte ranges; reads past them return 0)
  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(kh, a.npad * D);
  typedef const __attribute__((address_space(4))) float* const_f32_ptr;
  // k_scale through the constant address space: scalar loads (counted by lgkmcnt)
  const const_f32_ptr ksh = (const_f32_ptr)(a.k_scale + bh * nblk);
  const int ntiles = (a.N + kKvTile - 1) / kKvTile;
  const int tail = a.N - (ntiles - 1) * kKvTile;     // keys in the last tile (1..128)
  const int nfull = (tail == kKvTile) ? ntiles : ntiles - 1;   // tiles without masking

  float qf[G], m[G], lpart[G], alpha[G], c[G];
  v4f acc[G][D / 16];
  v4i qfr[G][D / 64];
  v4i S[G][8];
  PTile<PV> P[G];
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef const __attribute__((address_space(4))) f32x2* const_f32x2_ptr;
  auto scale_products = [&](int t) {
    // both halves' scales with one scalar load, then a per-lane select
    const f32x2 k01 = *(const_f32x2_ptr)(ksh + 2 * t);
    const float ks = (g >> 1) ? k01[1] : k01[0];
#pragma unroll
    for (int gq = 0; gq < G; ++gq) c[gq] = qf[gq] * ks;
  };
  const __amdgpu_buffer_rsrc_t ks_rsrc = make_rsrc(a.k_scale + bh * a.npad, TOK ? a.npad * 4 : 0);
  const __amdgpu_buffer_rsrc_t kbm_rsrc = make_rsrc(KBM ? a.k_bmean + bh * nblk * D : a.k_bmean,
                                                    KBM ? nblk * D * 2 : 0);
  // the per-tile side copies that go with the K tile (key scales, block means)
  auto copy_ks = [&](int t) {
    if constexpr (TOK) {
      if (t < ntiles) issue_kscale(ks_rsrc, t * kKvTile * 4, ksbuf(t), wave, lane);
    }
    if constexpr (KBM) {
      if (t < ntiles) issue_kbmean<D>(kbm_rsrc, t * 4 * D, kbmbuf(t), wave, lane);
    }
  };
  constexpr int SIDE = (TOK ? 1 : 0) + (KBM ? 1 : 0);   // side copies per wave and tile
  v4i qcb[G][D / 64][2];                               // query codes as bf16 (KBM)
  float e[G] = {};
  // softmax of tile t, masked to `tail` keys or not
  auto softmax_step = [&](int t, bool masked) {
    if constexpr (KBM) block_mean_terms<D>(kbmbuf(t), qcb, qf, r, g, e);
    if constexpr (TOK) {
      if (!masked) softmax_tile_tok<PV, false, KBM>(S, ksbuf(t), qf, kKvTile, g, a.log2_pscale, m, lpart, P, alpha, e);
      else softmax_tile_tok<PV, true, KBM>(S, ksbuf(t), qf, tail, g, a.log2_pscale, m, lpart, P, alpha, e);
    } else {
      scale_products(t);
      if (!masked) {
        softmax_tile<PV, KBM>(S, c, a.log2_pscale, m, lpart, P, alpha, e);
      } else {
#pragma unroll
        for (int gq = 0; gq < G; ++gq)
          alpha[gq] = softmax_group<true, PV, KBM>(S[gq], c[gq], tail, a.log2_pscale, m[gq], lpart[gq], P[gq],
                                                   g, e[gq]);
      }
    }
  };
  auto init_state = [&]() {
#pragma unroll
    for (int gq = 0; gq < G; ++gq) {
      qf[gq] = (TOK ? a.q_scale[bh * a.npad + qrow0 + 16 * gq + r]
                    : a.q_scale[bh * nblk + (qrow0 + 16 * gq) / kQuantBlock]) * a.log2e_scale;
      m[gq] = -INFINITY;
      lpart[gq] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[gq][dt] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (KBM) q_codes_bf16<D>(qfr, qcb);
  };

  if constexpr (PV == kPvFp8) {
    // visit i (LDS stage i % kStages) processes key tile tile_at(i): every tile in
    // order, or the query block's kept tiles
    int nvis = ntiles;
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const_i32_ptr kept = nullptr;
    if constexpr (SPARSE) {
      const int64_t row = bh * nqb + qb;
      nvis = __builtin_amdgcn_readfirstlane(((const_i32_ptr)a.tile_count)[row]);
      kept = (const_i32_ptr)a.tile_list + row * a.tiles_max;
    }
    auto tile_at = [&](int i) -> int {
      if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane(kept[i]);
      else return i;
    };
    const bool last_masked = nfull < ntiles && tile_at(nvis - 1) == ntiles - 1;
    const int nfull_vis = last_masked ? nvis - 1 : nvis;   // visits without masking
    const Ring<D> ring{smem};
    const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(a.v_f8 + bh * D * a.npad, (int64_t)D * a.npad);
    auto copy_tile = [&](int i) {
      if (i < nvis) {
        const int t = tile_at(i);
        dma.issue_k(k_rsrc, t * kKvTile * D, ring.kbuf(i), wave);
        dma.issue_v(v_rsrc, t * kKvTile, ring.vbuf(i), wave);
        copy_ks(t);
      }
    };
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i) copy_tile(i);
    load_q<D>(a.q_i8 + bh * a.npad * D, qrow0, lane, qfr);
    init_state();
    static_assert(kStages == 2, "visit i copies visit i + 1 into the other stage");
    for (int i = 0; i < nfull_vis; ++i) {
      // visit i has landed, and every wave is done with the other stage (visit i-1)
      tile_barrier<0>();
      prio.mfma();
      qk_tile<D>(ring.kbuf(i), qfr, lo, S, kSBiasBits);
      prio.base();
      // The compiler makes every LDS read that follows an LDS copy wait for that copy,
      // so the next visit's copy is issued after the K reads: it overlaps the softmax.
      copy_tile(i + 1);
      softmax_step(tile_at(i), false);
#pragma unroll
      for (int gq = 0; gq < G; ++gq) rescale<D>(acc[gq], alpha[gq]);
      prio.mfma();
      pv_tile<D>(ring.vbuf(i), P, lo, acc);
      prio.base();
    }
    refresh_lane();
    if (last_masked) {                   // last tile: keys >= N masked
      const int i = nvis - 1;
      tile_barrier<0>();
      qk_tile<D>(ring.kbuf(i), qfr, lo, S, kSBiasBits);
      softmax_step(ntiles - 1, true);
#pragma unroll
      for (int gq = 0; gq < G; ++gq) rescale<D>(acc[gq], alpha[gq]);
      pv_tile<D>(ring.vbuf(i), P, lo, acc);
    }
  } else {
    // K double-buffered, one bf16 V buffer.  Step t: barrier (K(t) landed, every wave
    // done with step t-1), S of tile t, copy V(t) and K(t+1), softmax of tile t, barrier
    // (V(t) landed; K(t+1) may still be in flight), P.V of tile t.
    uint8_t* vbuf = smem + 2 * Lds<D>::KBYTES;
    auto kbuf = [&](int t) { return smem + (t & 1) * Lds<D>::KBYTES; };
    const LaneOffsets16<D> lo16(lane);
    const DmaOffsets16<D> dma16(wave, lane, a.npad);
    const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(a.v16 + bh * D * a.npad, (int64_t)D * a.npad * 2);
    auto copy_k = [&](int t) {
      if (t < ntiles) {
        dma.issue_k(k_rsrc, t * kKvTile * D, kbuf(t), wave);
        copy_ks(t);
      }
    };
    copy_k(0);
    load_q<D>(a.q_i8 + bh * a.npad * D, qrow0, lane, qfr);
    init_state();
    auto step = [&](int t, bool masked) {
      tile_barrier<0>();
      prio.mfma();
      qk_tile<D>(kbuf(t), qfr, lo, S, kSBiasBits);
      prio.base();
      // copies issued after the K reads (see the FP8 loop): V(t) and K(t+1) overlap the softmax
      dma16.issue_v(v_rsrc, t * kKvTile * 2, vbuf, wave);
      copy_k(t + 1);
      softmax_step(t, masked);
#pragma unroll
      for (int gq = 0; gq < G; ++gq) rescale<D>(acc[gq], alpha[gq]);
      // V(t) must have landed; the copies of tile t+1 (K and key scales) may be in flight
      if (t + 1 < ntiles) tile_barrier<DmaOffsets<D>::KPW + SIDE>();
      else tile_barrier<0>();
      prio.mfma();
      pv_tile16<D>(vbuf, P, lo16, acc);
      prio.base();
    };
    for (int t = 0; t < nfull; ++t) step(t, false);
    refresh_lane();
    if (nfull < ntiles) step(nfull, true);
  }

  // epilogue: total row sum over the 4 lanes of each query, normalise, V scale, bf16
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  uint16_t* ob = a.out + (int64_t)b * a.so.b + (int64_t)h * a.so.h;
  const float* vsh = a.v_scale + bh * D;
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    const float l = sum_over_lane_groups(lpart[gq]);
    const float rl = 1.0f / l;
    const int qrow = qrow0 + 16 * gq + r;
    if (qrow < a.N) {
      uint16_t* orow = ob + (int64_t)qrow * a.so.n;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int c0 = 16 * dt + 4 * g;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = PV == kPvFp8 ? acc[gq][dt][i] * vsh[c0 + i] * rl : acc[gq][dt][i] * rl;
        *(uint2*)(orow + c0) = make_uint2(f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16),
                                          f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16));
      }
    }
  }
}

template <int D, int PV, bool TOK, bool KBM, bool PAIR>
__global__ __launch_bounds__(kThreads, kMinWavesPerSimd) void k_attn(AttnArgs a) {
  attn_body<D, PV, TOK, KBM, false, PAIR>(a);
}

template <int D, bool PAIR>
__global__ __launch_bounds__(kThreads, kMinWavesPerSimd) void k_attn_sparse(AttnArgs a) {
  attn_body<D, kPvFp8, false, false, true, PAIR>(a);
}


// =====================================================================================
// 32x32 matrix-core body (d = 128, FP8 P.V, 64-token scales; dense and block-sparse).
// One group of 32 queries per wave: S^T on v_mfma_i32_32x32x32_i8 (four 32-key
// sub-tiles x four 32-channel slices), O^T on v_mfma_scale_f32_32x32x64_f8f6f4 (four
// 32-channel tiles x two 64-key halves).  Lane (n, h) holds, for its query n, the 64
// keys 64ps + 32h + 0 .. 31 (ps = 0, 1) of every tile (k32_row_key): 32 keys in each
// 64-key scale block, so two key scales per lane; the row maximum combines the lane
// pair n, n + 32 with one v_permlane32_swap.  The larger shapes spend fewer VALU issue
// cycles next to the softmax of the other wave on the SIMD, and one query per lane
// halves the per-tile bookkeeping (maximum, rescale test, partial row sum).
// The per-element arithmetic is that of softmax_tile.
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

struct LaneOffsets32 {
  int koff[4];            // K slice kk (sub-tile kt adds k32_subtile_offset(kt))
  int voff[2][2];         // V half ps, 16-byte part (channel tile dt adds dt * 32 * 128)
  __device__ __forceinline__ explicit LaneOffsets32(int lane) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) koff[kk] = k32_read_offset(lane, kk);
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
      for (int x = 0; x < 2; ++x) voff[ps][x] = v32_read_offset(lane, ps, x);
  }
};

struct DmaOffsets32 {
  static constexpr int KPW = DmaShape<128>::KPW;
  static constexpr int VPW = DmaShape<128>::VPW;
  static constexpr int PER_TILE = KPW + VPW;
  uint32_t koff[KPW];
  uint32_t voff[VPW];
  __device__ __forceinline__ DmaOffsets32(int wave, int lane, int64_t npad) {
#pragma unroll
    for (int j = 0; j < KPW; ++j) koff[j] = k32_dma_src(wave, j, lane);
#pragma unroll
    for (int j = 0; j < VPW; ++j) voff[j] = v32_dma_src(wave, j, lane, npad);
  }
  __device__ __forceinline__ void issue_k(__amdgpu_buffer_rsrc_t r, int tile_off, uint8_t* klds, int wave) const {
#pragma unroll
    for (int j = 0; j < KPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(klds + (wave * KPW + j) * 1024), 16, koff[j],
                                               tile_off, 0, 0);
  }
  __device__ __forceinline__ void issue_v(__amdgpu_buffer_rsrc_t r, int tile_off, uint8_t* vlds, int wave) const {
#pragma unroll
    for (int j = 0; j < VPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(vlds + (wave * VPW + j) * 1024), 16, voff[j],
                                               tile_off, 0, 0);
  }
};

// Q operand of S^T: lane (n, h) holds bytes 32kk + 16h .. +15 of query row qrow0 + n.
__device__ __forceinline__ void load_q32(const int8_t* __restrict__ qh, int qrow0, int lane, v4i (&qf)[4]) {
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = *(const v4i*)(qh + (int64_t)(qrow0 + n) * 128 + 32 * kk + 16 * h);
}

// int32 S^T of the staged key tile: S[kt] register i = s0 + S(query n, key 64(kt/2) +
// 32h + 16(kt%2) + i).  Consecutive products go to different accumulators.
__device__ __forceinline__ void qk_tile32(const uint8_t* kbuf, const v4i (&qf)[4], const LaneOffsets32& lo,
                                          v16i (&S)[4], const v16i& s0) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const v4i a = *(const v4i*)(kbuf + lo.koff[kk] + k32_subtile_offset(kt));
      S[kt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[kk], kk == 0 ? s0 : S[kt], 0, 0, 0);
    }
}

// acc[dt] += V^T(channels 32dt .. +31) . P^T over the tile's two 64-key halves
// (consecutive products go to different accumulators).
__device__ __forceinline__ void pv_tile32(const uint8_t* vbuf, const v8i (&P)[2], const LaneOffsets32& lo,
                                          v16f (&acc)[4]) {
#pragma unroll
  for (int ps = 0; ps < 2; ++ps)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const v4i a = *(const v4i*)(vbuf + lo.voff[ps][0] + dt * 32 * kKvTile);
      const v4i b = *(const v4i*)(vbuf + lo.voff[ps][1] + dt * 32 * kKvTile);
      const v8i vf = v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, P[ps], acc[dt], 0, 0, 0, 0, 0, 0);
    }
}

// Online-softmax update of the lane's query for one tile.  c[ps] = fp32(q factor *
// k_scale of block ps).  When MASKED, keys at tile index >= nvalid get the logit -inf
// (a lane whose c is 0 then uses x = 0, c = 1 for its valid keys, as softmax_group
// does).  Produces P, updates m and the partial row sum, returns alpha.
template <bool MASKED>
__device__ __forceinline__ float softmax32(v16i (&S)[4], const float (&c_in)[2], int nvalid, int h,
                                           float log2_pscale, float& m, float& lpart, v8i (&P)[2]) {
  float c[2] = {c_in[0], c_in[1]};
  float sl;
  if constexpr (!MASKED) {
    int xm[2];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      int a0 = max(S[2 * ps][0], S[2 * ps][1]);
      int a1 = max(S[2 * ps + 1][0], S[2 * ps + 1][1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) {
        a0 = max(max(a0, S[2 * ps][i]), S[2 * ps][i + 1]);
        a1 = max(max(a1, S[2 * ps + 1][i]), S[2 * ps + 1][i + 1]);
      }
      xm[ps] = max(a0, a1);
    }
    // c >= 0 and rounding is monotone: the block's maximum logit is fp32(max S * c)
    sl = fmaxf(s_to_f32(xm[0]) * c[0], s_to_f32(xm[1]) * c[1]);
  } else {
    sl = -INFINITY;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const bool zero_c = (c[ps] == 0.0f);
      c[ps] = zero_c ? 1.0f : c[ps];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool valid = 64 * ps + 32 * h + 16 * u + i < nvalid;
          const float x = valid ? (zero_c ? 0.0f : s_to_f32(S[2 * ps + u][i])) : -INFINITY;
          S[2 * ps + u][i] = __builtin_bit_cast(int, x);     // S now holds the fp32 logit factor
          sl = fmaxf(sl, x == -INFINITY ? -INFINITY : x * c[ps]);
        }
    }
  }
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sl), __float_as_uint(sl), false, false);
    sl = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  const float m_new = fmaxf(m, sl);
  const float nb = log2_pscale - m_new;
  const float alpha = __builtin_amdgcn_exp2f(m - m_new);
  float ls[4];      // partial row sums, started from the first p (p >= 0, so 0 + p = p)
#pragma unroll
  for (int ps = 0; ps < 2; ++ps)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int v = S[2 * ps + u][4 * i4 + t];
          const float x = MASKED ? __builtin_bit_cast(float, v) : s_to_f32(v);
          p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c[ps], nb));
          ls[t] = (ps == 0 && u == 0 && i4 == 0) ? p[t] : ls[t] + p[t];
        }
        const int w = 4 * u + i4;          // P word: keys 4w .. 4w+3 of the half
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], P[ps][w], false);
        P[ps][w] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], x, true);
      }
  if (wave_any(fabsf(m_new) >= kSatLimit)) {
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
      for (int w = 0; w < 8; ++w) P[ps][w] = e4m3x4_saturate(P[ps][w]);
  }
  lpart = alpha * lpart + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
  m = m_new;
  return alpha;
}

template <bool SPARSE, bool PAIR>
__device__ __forceinline__ void attn32_body(const AttnArgs& a) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * Ring<D>::STAGE];
  const IssuePriority<PAIR> prio(a.cu_count);
  if constexpr (PAIR) prio.base();
  const int nqb = (int)(a.npad / kBlockM);
  const int total = nqb * a.B * a.H;
  const int work = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, total));
  const int64_t bh = __builtin_amdgcn_readfirstlane(work / nqb);
  const int qb = __builtin_amdgcn_readfirstlane(work % nqb);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int qrow0 = qb * kBlockM + wave * 32;
  const int64_t nblk = a.npad / kQuantBlock;

  const LaneOffsets32 lo(lane);
  const DmaOffsets32 dma(wave, lane, a.npad);
  const int8_t* kh = a.k_i8 + bh * a.npad * D;
  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(kh, a.npad * D);
  const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(a.v_f8 + bh * D * a.npad, (int64_t)D * a.npad);
  typedef const __attribute__((address_space(4))) float* const_f32_ptr;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef const __attribute__((address_space(4))) f32x2* const_f32x2_ptr;
  const const_f32_ptr ksh = (const_f32_ptr)(a.k_scale + bh * nblk);
  const int ntiles = (a.N + kKvTile - 1) / kKvTile;
  const int tail = a.N - (ntiles - 1) * kKvTile;

  int nvis = ntiles;
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const_i32_ptr kept = nullptr;
  if constexpr (SPARSE) {
    const int64_t row = bh * nqb + qb;
    nvis = __builtin_amdgcn_readfirstlane(((const_i32_ptr)a.tile_count)[row]);
    kept = (const_i32_ptr)a.tile_list + row * a.tiles_max;
  }
  auto tile_at = [&](int i) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane(kept[i]);
    else return i;
  };
  const bool last_masked = tail < kKvTile && tile_at(nvis - 1) == ntiles - 1;
  const int nfull_vis = last_masked ? nvis - 1 : nvis;
  static_assert(kStages == 2, "visit i uses stage i % 2 and copies visit i + 1 into the other");
  const Ring<D> ring{smem};
  auto copy_tile = [&](int i) {
    if (i < nvis) {
      const int t = tile_at(i);
      dma.issue_k(k_rsrc, t * kKvTile * D, ring.kbuf(i), wave);
      dma.issue_v(v_rsrc, t * kKvTile, ring.vbuf(i), wave);
    }
  };
  copy_tile(0);

  v4i qfr[4];
  load_q32(a.q_i8 + bh * a.npad * D, qrow0, lane, qfr);
  const float qf = a.q_scale[bh * nblk + qrow0 / kQuantBlock] * a.log2e_scale;
  float m = -INFINITY, lpart = 0.0f;
  v16f acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;
  v16i s0;
#pragma unroll
  for (int i = 0; i < 16; ++i) s0[i] = kSBiasBits;
  v16i S[4];
  v8i P[2] = {};
  auto scales = [&](int t, float (&c)[2]) {
    const f32x2 k01 = *(const_f32x2_ptr)(ksh + 2 * t);
    c[0] = qf * k01[0];
    c[1] = qf * k01[1];
  };
  auto rescale32 = [&](float alpha) {
    if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
    }
  };
  // One visit: the barrier (its copies have landed; every wave is done with the other
  // stage), the K operand reads and QK^T, then the next visit's copy into the other
  // stage, the softmax, and P.V.  The compiler makes every LDS read that follows an LDS
  // copy wait for that copy (it cannot tell the stages apart), so the copy is issued
  // after the K reads: it overlaps the softmax, and the P.V reads' wait finds it done.
  auto visit = [&](int i, bool masked) {
    tile_barrier<0>();
    prio.mfma();
    qk_tile32(ring.kbuf(i), qfr, lo, S, s0);
    prio.base();
    copy_tile(i + 1);
    float c[2];
    scales(tile_at(i), c);
    const float alpha = masked ? softmax32<true>(S, c, tail, h, a.log2_pscale, m, lpart, P)
                               : softmax32<false>(S, c, kKvTile, h, a.log2_pscale, m, lpart, P);
    rescale32(alpha);
    prio.mfma();
    pv_tile32(ring.vbuf(i), P, lo, acc);
    prio.base();
  };
  for (int i = 0; i < nfull_vis; ++i) visit(i, false);
  if (last_masked) visit(nvis - 1, true);

  // epilogue: the row sum over the lane pair, normalise, V scale, bf16
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lpart), __float_as_uint(lpart), false, false);
  const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  const float rl = 1.0f / l;
  const int b = (int)(bh / a.H), hh = (int)(bh % a.H);
  const int qrow = qrow0 + n;
  if (qrow < a.N) {
    uint16_t* orow = a.out + (int64_t)b * a.so.b + (int64_t)hh * a.so.h + (int64_t)qrow * a.so.n;
    const float* vsh = a.v_scale + bh * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int c0 = 32 * dt + 8 * jj + 4 * h;
        float o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = acc[dt][4 * jj + t] * vsh[c0 + t] * rl;
        *(uint2*)(orow + c0) = make_uint2(f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16),
                                          f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16));
      }
  }
}

template <bool PAIR>
__global__ __launch_bounds__(kThreads, kMinWavesPerSimd) void k_attn32(AttnArgs a) {
  attn32_body<false, PAIR>(a);
}

template <bool PAIR>
__global__ __launch_bounds__(kThreads, kMinWavesPerSimd) void k_attn32_sparse(AttnArgs a) {
  attn32_body<true, PAIR>(a);
}

// Int32 S tiles through the 32x32 body's staging, swizzle, matrix-core code and biased
// accumulator start (d = 128).
__global__ __launch_bounds__(kThreads) void k_debug_qk32(const int8_t* __restrict__ q_i8,
                                                    const int8_t* __restrict__ k_i8, int64_t npad,
                                                    int64_t bh, int q_block, int kv_tile,
                                                    int n_kv_tiles, int32_t* __restrict__ s_out) {
  __shared__ __attribute__((aligned(1024))) uint8_t klds[Lds<128>::KBYTES];
  const int qb = q_block + blockIdx.y, kvt = kv_tile + blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int qrow0 = qb * kBlockM + wave * 32;
  const DmaOffsets32 dma(wave, lane, npad);
  dma.issue_k(make_rsrc(k_i8 + bh * npad * 128, npad * 128), kvt * kKvTile * 128, klds, wave);
  v4i qfr[4];
  load_q32(q_i8 + bh * npad * 128, qrow0, lane, qfr);
  __syncthreads();
  v16i s0;
#pragma unroll
  for (int i = 0; i < 16; ++i) s0[i] = kSBiasBits;
  v16i S[4];
  qk_tile32(klds, qfr, LaneOffsets32(lane), S, s0);
  const int64_t ld = (int64_t)n_kv_tiles * kKvTile;
  const int64_t row = (int64_t)blockIdx.y * kBlockM + wave * 32 + n;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      s_out[row * ld + (int64_t)blockIdx.x * kKvTile + 64 * (kt >> 1) + 32 * h + 16 * (kt & 1) + i] =
          S[kt][i] - kSBiasBits;
}

// Int32 S tiles through the same staging (LDS DMA, swizzle), matrix-core code and
// biased accumulator start as k_attn; the bias is subtracted on the way out.
template <int D>
__global__ __launch_bounds__(kThreads) void k_debug_qk(const int8_t* __restrict__ q_i8,
                                                  const int8_t* __restrict__ k_i8, int64_t npad,
                                                  int64_t bh, int q_block, int kv_tile,
                                                  int n_kv_tiles, int32_t* __restrict__ s_out) {
  __shared__ __attribute__((aligned(1024))) uint8_t klds[Lds<D>::KBYTES];
  const int qb = q_block + blockIdx.y, kvt = kv_tile + blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int qrow0 = qb * kBlockM + wave * (G * 16);
  const DmaOffsets<D> dma(wave, lane, npad);
  dma.issue_k(make_rsrc(k_i8 + bh * npad * D, npad * D), kvt * kKvTile * D, klds, wave);
  v4i qfr[G][D / 64];
  load_q<D>(q_i8 + bh * npad * D, qrow0, lane, qfr);
  __syncthreads();
  v4i S[G][8];
  qk_tile<D>(klds, qfr, LaneOffsets<D>(lane), S, kSBiasBits);   // the attention kernel's accumulator start
  const int64_t ld = (int64_t)n_kv_tiles * kKvTile;
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    const int64_t row = (int64_t)blockIdx.y * kBlockM + wave * (G * 16) + 16 * gq + r;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_out[row * ld + (int64_t)blockIdx.x * kKvTile + 32 * g + 4 * kt + i] = S[gq][kt][i] - kSBiasBits;
  }
}

// Workgroup-pair issue priorities for grids of at most two rounds of two workgroups per
// compute unit.
static bool pair_priorities(const AttnArgs& a, unsigned grid) {
  return grid <= 4u * (unsigned)a.cu_count;
}

template <int D, int PV, bool TOK, bool KBM>
static void launch_attn_pair(const AttnArgs& a, unsigned grid, hipStream_t s) {
  if (pair_priorities(a, grid))
    hipLaunchKernelGGL((k_attn<D, PV, TOK, KBM, true>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn<D, PV, TOK, KBM, false>), dim3(grid), dim3(kThreads), 0, s, a);
}

template <int D, int PV, bool TOK>
static void launch_attn_kbm(const AttnArgs& a, unsigned grid, hipStream_t s) {
  if constexpr (PV == kPvFp8 && D == 128 && !TOK) {
    // FP8 P.V with 64-token scales and the token mean runs the 32x32 body
    // (launch_attn_d); of this mode only the block-residual form comes here
    launch_attn_pair<D, PV, TOK, true>(a, grid, s);
  } else {
    if constexpr (PV == kPvFp8) {
      if (a.k_bmean) {
        launch_attn_pair<D, PV, TOK, true>(a, grid, s);
        return;
      }
    }
    launch_attn_pair<D, PV, TOK, false>(a, grid, s);
  }
}

template <int D, int PV>
static void launch_attn_tok(const AttnArgs& a, unsigned grid, hipStream_t s) {
  if (a.tok) launch_attn_kbm<D, PV, true>(a, grid, s);
  else launch_attn_kbm<D, PV, false>(a, grid, s);
}

template <int D>
static void launch_attn_d(const AttnArgs& a, unsigned grid, hipStream_t s) {
  if constexpr (D == 128) {
    // the 32x32 body: FP8 P.V with 64-token scales, dense or block-sparse
    if (a.pv == kPvFp8 && !a.tok && !a.k_bmean) {
      const bool pair = pair_priorities(a, grid);
      if (a.tile_list) {
        if (pair) hipLaunchKernelGGL((k_attn32_sparse<true>), dim3(grid), dim3(kThreads), 0, s, a);
        else hipLaunchKernelGGL((k_attn32_sparse<false>), dim3(grid), dim3(kThreads), 0, s, a);
      } else {
        if (pair) hipLaunchKernelGGL((k_attn32<true>), dim3(grid), dim3(kThreads), 0, s, a);
        else hipLaunchKernelGGL((k_attn32<false>), dim3(grid), dim3(kThreads), 0, s, a);
      }
      return;
    }
  }
  if constexpr (D == 64) {
    // block-sparse steps always take mode 0, which at d = 128 is the 32x32 body
    if (a.tile_list) {
      if (pair_priorities(a, grid))
        hipLaunchKernelGGL((k_attn_sparse<D, true>), dim3(grid), dim3(kThreads), 0, s, a);
      else
        hipLaunchKernelGGL((k_attn_sparse<D, false>), dim3(grid), dim3(kThreads), 0, s, a);
      return;
    }
  }
  if (a.pv == kPvBf16) launch_attn_tok<D, kPvBf16>(a, grid, s);
  else launch_attn_tok<D, kPvFp8>(a, grid, s);
}

// Compute units of the current device, read once per device (the period of the
// workgroup-pair priorities; any positive value gives the same results).
static int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_attn(const AttnArgs& args, hipStream_t s) {
  AttnArgs a = args;
  a.cu_count = device_cu_count();
  const int nqb = (int)(a.npad / kBlockM);
  const unsigned grid = (unsigned)((int64_t)nqb * a.B * a.H);
  if (a.d == 64) launch_attn_d<64>(a, grid, s);
  else launch_attn_d<128>(a, grid, s);
  return hipGetLastError();
}

hipError_t launch_debug_qk(const int8_t* q_i8, const int8_t* k_i8, int d, bool body32, int64_t npad,
                           int64_t bh, int q_block, int kv_tile, int n_q_blocks,
                           int n_kv_tiles, int32_t* s_out, hipStream_t s) {
  const dim3 grid(n_kv_tiles, n_q_blocks);
  if (d == 128 && body32) {
    hipLaunchKernelGGL(k_debug_qk32, grid, dim3(kThreads), 0, s, q_i8, k_i8, npad, bh, q_block, kv_tile,
                       n_kv_tiles, s_out);
    return hipGetLastError();
  }
  if (d == 64)
    hipLaunchKernelGGL(k_debug_qk<64>, grid, dim3(kThreads), 0, s, q_i8, k_i8, npad, bh, q_block,
                       kv_tile, n_kv_tiles, s_out);
  else
    hipLaunchKernelGGL(k_debug_qk<128>, grid, dim3(kThreads), 0, s, q_i8, k_i8, npad, bh, q_block,
                       kv_tile, n_kv_tiles, s_out);
  return hipGetLastError();
}

// explicit instantiations: the host pass does not always emit launch stubs for kernel
// templates that are only named inside hipLaunchKernelGGL
template __global__ void k_attn<64, kPvFp8, false, false, false>(AttnArgs);
template __global__ void k_attn<64, kPvFp8, false, false, true>(AttnArgs);
template __global__ void k_attn<64, kPvFp8, true, false, false>(AttnArgs);
template __global__ void k_attn<64, kPvFp8, true, false, true>(AttnArgs);
template __global__ void k_attn<64, kPvFp8, false, true, false>(AttnArgs);
template __global__ void k_attn<64, kPvFp8, false, true, true>(AttnArgs);
template __global__ void k_attn<64, kPvFp8, true, true, false>(AttnArgs);
template __global__ void k_attn<64, kPvFp8, true, true, true>(AttnArgs);
template __global__ void k_attn<64, kPvBf16, false, false, false>(AttnArgs);
template __global__ void k_attn<64, kPvBf16, false, false, true>(AttnArgs);
template __global__ void k_attn<64, kPvBf16, true, false, false>(AttnArgs);
template __global__ void k_attn<64, kPvBf16, true, false, true>(AttnArgs);
template __global__ void k_attn<128, kPvFp8, true, false, false>(AttnArgs);
template __global__ void k_attn<128, kPvFp8, true, false, true>(AttnArgs);
template __global__ void k_attn<128, kPvFp8, false, true, false>(AttnArgs);
template __global__ void k_attn<128, kPvFp8, false, true, true>(AttnArgs);
template __global__ void k_attn<128, kPvFp8, true, true, false>(AttnArgs);
template __global__ void k_attn<128, kPvFp8, true, true, true>(AttnArgs);
template __global__ void k_attn<128, kPvBf16, false, false, false>(AttnArgs);
template __global__ void k_attn<128, kPvBf16, false, false, true>(AttnArgs);
template __global__ void k_attn<128, kPvBf16, true, false, false>(AttnArgs);
template __global__ void k_attn<128, kPvBf16, true, false, true>(AttnArgs);
template __global__ void k_attn32<false>(AttnArgs);
template __global__ void k_attn32<true>(AttnArgs);
template __global__ void k_attn32_sparse<false>(AttnArgs);
template __global__ void k_attn32_sparse<true>(AttnArgs);
template __global__ void k_attn_sparse<64, false>(AttnArgs);
template __global__ void k_attn_sparse<64, true>(AttnArgs);
template __global__ void k_debug_qk<64>(const int8_t* __restrict__, const int8_t* __restrict__, int64_t,
                                        int64_t, int, int, int, int32_t* __restrict__);
template __global__ void k_debug_qk<128>(const int8_t* __restrict__, const int8_t* __restrict__, int64_t,
                                         int64_t, int, int, int, int32_t* __restrict__);

}  // namespace sage
