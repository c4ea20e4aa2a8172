// Quantisation pass for gfx950: K token mean (smoothing), per-block INT8 codes of Q
// and K - mean, per-channel FP8 e4m3 codes of V (juejin page "MiniMax H3 接入
// SageAttention 实测加速", section 一; the bf16 mean term of the sd114.wiki
// ComfyUI-sol-attn page, "核心亮点" item 1).
//
// Three launches, all HBM-bound (Q/K scales per 64-token block, or per token):
//   1. q+stats  grid (chunks, H, B): each workgroup walks a run of 64-token blocks; it
//               writes the final INT8 codes and scales of Q (they need only the block
//               itself) and one row of fp64 partial sums of K and partial max |V| per
//               channel.  The run length grows with N so a head never has more than
//               kMaxStatsChunks partial rows.
//   2. finalize grid (B*H): sums the partial rows -> k_mean (bf16), v_scale =
//               vamax/448 and 448/vamax.
//   3. k+v      grid (Npad/64, H, B): one 64-token block of K and V per workgroup
//               (both read again, in the reverse order of pass 1 so that the most
//               recently read blocks come first, while still cached); block max-abs
//               reduced across the workgroup, K codes written with 8-byte stores; V
//               codes transposed through LDS into the channel-major layout the
//               attention kernel stages directly.
// Every workgroup issues all of its row loads before the first reduction, so each
// thread keeps 8 to 12 16-byte loads in flight.
#include "sage_internal.h"
#include "sage_device.h"

namespace sage {

// INT8 codes of one 64-token block held as x[RPT][8] per thread; returns the scale.
template <int RPT>
__device__ __forceinline__ float int8_block(const float (&x)[RPT][8], uint2 (&codes)[RPT], float* red) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[i][j]));
  amax = block256_max(amax, red);
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float y = rintf(x[i][j] * inv);                // round half to even
      y = fminf(fmaxf(y, -127.0f), 127.0f);
      w[j >> 2] |= ((uint32_t)((int)y & 0xff)) << (8 * (j & 3));
    }
    codes[i] = make_uint2(w[0], w[1]);
  }
  return amax / 127.0f;
}

// Per-token INT8 codes: row i of x is one token, held by the TPR consecutive lanes that
// share it (8 channels each); its max |x| is reduced over those lanes.  Returns the
// scales of the thread's RPT rows.
template <int RPT, int TPR>
__device__ __forceinline__ void int8_rows(const float (&x)[RPT][8], uint2 (&codes)[RPT], float (&scale)[RPT]) {
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[i][j]));
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float y = rintf(x[i][j] * inv);                // round half to even
      y = fminf(fmaxf(y, -127.0f), 127.0f);
      w[j >> 2] |= ((uint32_t)((int)y & 0xff)) << (8 * (j & 3));
    }
    codes[i] = make_uint2(w[0], w[1]);
    scale[i] = amax / 127.0f;
  }
}

// Loads the 16-byte words (8 channels) of rows row0 + r + RPI*i of one 64-token block;
// rows at or past N read as zero.
template <int RPT, int RPI>
__device__ __forceinline__ void load_block(const uint16_t* base, int64_t stride_n, int row0, int r,
                                           int N, uint4 (&w)[RPT]) {
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int n = row0 + r + RPI * i;
    w[i] = make_uint4(0u, 0u, 0u, 0u);
    if (n < N) w[i] = *(const uint4*)(base + (int64_t)n * stride_n);
  }
}

// NEED_V: the speed mode also needs the per-channel max |V| (e4m3 V scales); the
// quality mode keeps V in bf16 and skips it.
// TOK: one INT8 scale per token (q_scale [B][H][Npad]) instead of per 64-token block.
// NEED_KSUM: the token mean of K is needed (not with block-residual K).
template <int D, bool NEED_V, bool TOK, bool NEED_KSUM>
__global__ __launch_bounds__(256) void k_quant_q_stats(
    const uint16_t* __restrict__ q, Strides sq, const uint16_t* __restrict__ k, Strides sk,
    const uint16_t* __restrict__ v, Strides sv, int N, int64_t npad, int blocks_per_chunk,
    int8_t* __restrict__ q_i8, float* __restrict__ q_scale,
    double* __restrict__ ksum_part, float* __restrict__ vmax_part) {
  constexpr int TPR = D / 8;        // threads per token row, 8 channels each
  constexpr int RPI = 256 / TPR;    // token rows per sweep of the workgroup
  constexpr int RPT = kQuantBlock / RPI;
  // heads fastest in the workgroup order: the workgroups that run together read all
  // heads of the same token rows, which lie together in a [B, N, H, d] tensor
  // (measured 1-3% off the pass)
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int chunk = lin / gridDim.y, h = lin % gridDim.y, b = blockIdx.z;
  const int t = threadIdx.x, r = t / TPR, cg = t % TPR;
  const int64_t bh = (int64_t)b * gridDim.y + h;
  const int64_t nblk = npad / kQuantBlock;
  const int blk0 = chunk * blocks_per_chunk;
  const int blk1 = (int)min((int64_t)blk0 + blocks_per_chunk, nblk);
  const uint16_t* qb = q + (int64_t)b * sq.b + (int64_t)h * sq.h + 8 * cg;
  const uint16_t* kb = k + (int64_t)b * sk.b + (int64_t)h * sk.h + 8 * cg;
  const uint16_t* vb = v + (int64_t)b * sv.b + (int64_t)h * sv.h + 8 * cg;
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) double red_s[RPI][D];
  __shared__ float red_v[RPI][D];

  double s[8];
  float vm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { s[j] = 0.0; vm[j] = 0.0f; }
  for (int blk = blk0; blk < blk1; ++blk) {
    const int row0 = blk * kQuantBlock;
    uint4 qw[RPT], kw[RPT], vw[RPT];
    load_block<RPT, RPI>(qb, sq.n, row0, r, N, qw);
    if constexpr (NEED_KSUM) load_block<RPT, RPI>(kb, sk.n, row0, r, N, kw);
    if constexpr (NEED_V) load_block<RPT, RPI>(vb, sv.n, row0, r, N, vw);
    float x[RPT][8];
    uint2 codes[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) bf16x8_to_f32(qw[i], x[i]);
    if constexpr (TOK) {
      float sc[RPT];
      int8_rows<RPT, TPR>(x, codes, sc);
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        if (cg == 0) q_scale[bh * npad + row0 + r + RPI * i] = sc[i];
    } else {
      const float scale = int8_block<RPT>(x, codes, red);
      if (t == 0) q_scale[bh * nblk + blk] = scale;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *(uint2*)(q_i8 + (bh * npad + row0 + r + RPI * i) * D + 8 * cg) = codes[i];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      if constexpr (NEED_KSUM) {
        float kx[8];
        bf16x8_to_f32(kw[i], kx);
#pragma unroll
        for (int j = 0; j < 8; ++j) s[j] += (double)kx[j];
      }
      if constexpr (NEED_V) {
        float vx[8];
        bf16x8_to_f32(vw[i], vx);
#pragma unroll
        for (int j = 0; j < 8; ++j) vm[j] = fmaxf(vm[j], fabsf(vx[j]));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) { red_s[r][8 * cg + j] = s[j]; red_v[r][8 * cg + j] = vm[j]; }
  __syncthreads();
  if (t < D) {
    double acc = 0.0;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < RPI; ++i) { acc += red_s[i][t]; m = fmaxf(m, red_v[i][t]); }
    const int64_t o = (bh * gridDim.x + chunk) * D + t;
    ksum_part[o] = acc;
    vmax_part[o] = m;
  }
}

// One workgroup per (b, h): 1024 threads = D channels x (1024 / D) slices of the
// partial rows, combined through LDS in slice order.
constexpr int kFinalizeThreads = 1024;
template <int D, bool NEED_V, bool NEED_K>
__global__ __launch_bounds__(kFinalizeThreads) void k_quant_finalize(
    const double* __restrict__ ksum_part, const float* __restrict__ vmax_part, int chunks, int N,
    uint16_t* __restrict__ k_mean, float* __restrict__ v_scale, float* __restrict__ v_inv) {
  constexpr int SL = kFinalizeThreads / D;
  const int64_t bh = blockIdx.x;
  const int c = threadIdx.x % D, sl = threadIdx.x / D;
  __shared__ double ps[SL][D];
  __shared__ float pv[SL][D];
  double s = 0.0;
  float vm = 0.0f;
#pragma unroll 4
  for (int i = sl; i < chunks; i += SL) {
    if constexpr (NEED_K) s += ksum_part[(bh * chunks + i) * D + c];
    if constexpr (NEED_V) vm = fmaxf(vm, vmax_part[(bh * chunks + i) * D + c]);
  }
  ps[sl][c] = s;
  pv[sl][c] = vm;
  __syncthreads();
  if (sl == 0) {
#pragma unroll
    for (int i = 1; i < SL; ++i) { s += ps[i][c]; vm = fmaxf(vm, pv[i][c]); }
    if constexpr (NEED_K) {
      const float mean = (float)(s / (double)N);      // fp64 divide, one rounding to fp32
      k_mean[bh * D + c] = (uint16_t)f32_to_bf16_rne(mean);
    }
    if constexpr (NEED_V) {
      v_scale[bh * D + c] = vm / kPScale;             // IEEE division (0 when vm = 0)
      v_inv[bh * D + c] = vm > 0.0f ? kPScale / vm : 0.0f;
    }
  }
}

// K - mean codes and V codes of one 64-token block.  Here thread (r, cg) holds the RPT
// consecutive tokens RPT*r .. RPT*r + RPT-1 (8 channels each), so for every channel it
// owns RPT adjacent bytes of the channel-major V block: they go to LDS as one word
// (RPT = 4) or half word (RPT = 2), in rows of VW words whose odd pitch spreads the
// 16 channel groups of a wave over distinct banks (at most 2 lanes per bank).
//
// V16 (quality mode): V keeps its bf16 values and is only transposed: each thread's
// RPT tokens of a channel (2*RPT bytes) go to LDS as RPT/2 words in rows of 33 words.
//
// KBM (block-residual K): the mean subtracted from K is that of the block's own valid
// tokens (fp64 sums reduced through LDS, then fp32 and bf16 rounding like the token
// mean), written to k_mean [B][H][Npad/64][d].
// Work item of k+v workgroup `lin` of `total`: the grid is walked backwards in steps of
// the 8 XCDs (workgroup ids x, x+8, x+16, ... go to XCD x), so the pass first re-reads
// the K and V blocks that the q+stats pass read last, while they are still cached
// (measured 4-9% off the whole quantisation pass).  Identity when total is not a
// multiple of 8.
__device__ __forceinline__ int64_t kv_work_item(int64_t lin, int64_t total) {
  constexpr int kXcds = 8;
  return total % kXcds == 0 ? total - kXcds - kXcds * (lin / kXcds) + lin % kXcds : lin;
}

template <int D, bool V16, bool TOK, bool KBM>
__global__ __launch_bounds__(256) void k_quant_kv(
    const uint16_t* __restrict__ k, Strides sk, const uint16_t* __restrict__ v, Strides sv,
    int N, int64_t npad, uint16_t* __restrict__ k_mean, const float* __restrict__ v_inv,
    int8_t* __restrict__ k_i8, float* __restrict__ k_scale, uint8_t* __restrict__ v_f8,
    uint16_t* __restrict__ v16) {
  constexpr int TPR = D / 8;
  constexpr int RPI = 256 / TPR;
  constexpr int RPT = kQuantBlock / RPI;   // consecutive tokens per thread (4 or 2)
  constexpr int VW = kQuantBlock / 4 + 1;  // LDS words per channel row (odd pitch)
  const int64_t work = kv_work_item(blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z),
                                    (int64_t)gridDim.x * gridDim.y * gridDim.z);
  const int h = (int)(work % gridDim.y);                     // heads fastest, as in pass 1
  const int blk = (int)((work / gridDim.y) % gridDim.x);
  const int b = (int)(work / ((int64_t)gridDim.x * gridDim.y));
  const int t = threadIdx.x, r = t / TPR, cg = t % TPR;
  const int64_t bh = (int64_t)b * gridDim.y + h;
  const int row0 = blk * kQuantBlock;
  const int tok0 = row0 + RPT * r;           // this thread's first token
  const int64_t nblk = npad / kQuantBlock;
  constexpr int VW16 = kQuantBlock / 2 + 1;  // LDS words per channel row, bf16 (odd pitch)
  __shared__ float red[4];
  __shared__ uint32_t vt[D * (V16 ? VW16 : VW)];

  uint4 kw[RPT], vw[RPT];
  load_block<RPT, 1>(k + (int64_t)b * sk.b + (int64_t)h * sk.h + 8 * cg, sk.n, tok0, 0, N, kw);
  load_block<RPT, 1>(v + (int64_t)b * sv.b + (int64_t)h * sv.h + 8 * cg, sv.n, tok0, 0, N, vw);
  float mu[8], inv[8];
  if constexpr (KBM) {
    __shared__ double bsum[RPI][D];
    __shared__ __attribute__((aligned(16))) uint16_t bmean[D];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        acc += (double)bf16_bits_to_f32(((const uint16_t*)&kw[i])[j]);   // rows >= N read as 0
      bsum[r][8 * cg + j] = acc;
    }
    __syncthreads();
    if (t < D) {
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < RPI; ++i) acc += bsum[i][t];
      const int nvalid = min(kQuantBlock, N - row0);    // <= 0 for an all-padding block
      const uint16_t m16 = nvalid > 0 ? (uint16_t)f32_to_bf16_rne((float)(acc / (double)nvalid)) : 0;
      bmean[t] = m16;
      k_mean[(bh * nblk + blk) * D + t] = m16;
    }
    __syncthreads();
    bf16x8_to_f32(*(const uint4*)(bmean + 8 * cg), mu);
  } else {
    bf16x8_to_f32(*(const uint4*)(k_mean + bh * D + 8 * cg), mu);
  }
  if constexpr (!V16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) inv[j] = v_inv[bh * D + 8 * cg + j];
  }

  // ---- K - mean -> INT8 ----
  {
    float x[RPT][8];
    uint2 codes[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const bool valid = tok0 + i < N;
      bf16x8_to_f32(kw[i], x[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[i][j] = valid ? x[i][j] - mu[j] : 0.0f;
    }
    if constexpr (TOK) {
      float sc[RPT];
      int8_rows<RPT, TPR>(x, codes, sc);
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        if (cg == 0) k_scale[bh * npad + tok0 + i] = sc[i];
    } else {
      const float scale = int8_block<RPT>(x, codes, red);
      if (t == 0) k_scale[bh * nblk + blk] = scale;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *(uint2*)(k_i8 + (bh * npad + tok0 + i) * D + 8 * cg) = codes[i];
  }
  if constexpr (V16) {
    // ---- V (bf16) transposed to [channel][token] ----
    // word w of channel j: tokens tok0 + 2w, tok0 + 2w + 1 (RPT/2 words per channel)
#pragma unroll
    for (int w = 0; w < RPT / 2; ++w) {
      const uint4 a = vw[2 * w], b = vw[2 * w + 1];
      const uint32_t ea[4] = {a.x, a.y, a.z, a.w}, eb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t lo = (ea[j >> 1] >> (16 * (j & 1))) & 0xffffu;
        const uint32_t hi = (eb[j >> 1] >> (16 * (j & 1))) & 0xffffu;
        vt[(8 * cg + j) * VW16 + (RPT / 2) * r + w] = lo | (hi << 16);
      }
    }
    __syncthreads();
    constexpr int CPR = kQuantBlock * 2 / 16;        // 16-byte chunks per channel row
#pragma unroll
    for (int cid = t; cid < D * CPR; cid += 256) {
      const int c = cid / CPR, part = cid % CPR;
      const uint32_t* src = vt + c * VW16 + 4 * part;
      *(uint4*)(v16 + (bh * D + c) * npad + row0 + 8 * part) = make_uint4(src[0], src[1], src[2], src[3]);
    }
    return;
  }
  // ---- V -> e4m3, transposed to [channel][token] ----
  {
    uint32_t packed[8];                    // channel j: codes of tokens tok0 .. tok0+RPT-1
#pragma unroll
    for (int j = 0; j < 8; ++j) packed[j] = 0u;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float x[8];
      bf16x8_to_f32(vw[i], x);
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const uint32_t c2 = e4m3x2_sat(x[j] * inv[j], x[j + 1] * inv[j + 1]);
        packed[j] |= (c2 & 0xffu) << (8 * i);
        packed[j + 1] |= (c2 >> 8) << (8 * i);
      }
    }
    if constexpr (RPT == 4) {
#pragma unroll
      for (int j = 0; j < 8; ++j) vt[(8 * cg + j) * VW + r] = packed[j];
    } else {
      uint16_t* vt16 = (uint16_t*)vt;
#pragma unroll
      for (int j = 0; j < 8; ++j) vt16[(8 * cg + j) * 2 * VW + r] = (uint16_t)packed[j];
    }
    __syncthreads();
    constexpr int NCH = D * (kQuantBlock / 16);      // 16-byte chunks of the block
#pragma unroll
    for (int cid = t; cid < NCH; cid += 256) {
      const int c = cid / (kQuantBlock / 16), part = cid % (kQuantBlock / 16);
      const uint32_t* src = vt + c * VW + 4 * part;
      *(uint4*)(v_f8 + (bh * D + c) * npad + row0 + 16 * part) = make_uint4(src[0], src[1], src[2], src[3]);
    }
  }
}

__global__ void k_debug_e4m3(const float* __restrict__ x, uint8_t* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t j = 2 * i;
  if (j + 1 < n) {
    const uint32_t c = e4m3x2_sat(x[j], x[j + 1]);
    y[j] = (uint8_t)(c & 0xff);
    y[j + 1] = (uint8_t)(c >> 8);
  } else if (j < n) {
    y[j] = (uint8_t)(e4m3x2_sat(x[j], 0.0f) & 0xff);
  }
}

template <int D, bool V16, bool TOK, bool KBM>
static hipError_t launch_quant_d(const QuantArgs& a, hipStream_t s) {
  const int per = stats_blocks_per_chunk(a.npad);
  const int chunks = stats_chunks(a.N);
  hipLaunchKernelGGL((k_quant_q_stats<D, !V16, TOK, !KBM>), dim3(chunks, a.H, a.B), dim3(256), 0, s,
                     a.q, a.sq, a.k, a.sk, a.v, a.sv, a.N, a.npad, per,
                     a.q_i8, a.q_scale, a.ksum_part, a.vmax_part);
  if constexpr (!V16 || !KBM)
    hipLaunchKernelGGL((k_quant_finalize<D, !V16, !KBM>), dim3(a.B * a.H), dim3(kFinalizeThreads), 0, s,
                       a.ksum_part, a.vmax_part, chunks, a.N, a.k_mean, a.v_scale, a.v_inv);
  hipLaunchKernelGGL((k_quant_kv<D, V16, TOK, KBM>), dim3((unsigned)(a.npad / kQuantBlock), a.H, a.B), dim3(256), 0, s,
                     a.k, a.sk, a.v, a.sv, a.N, a.npad, a.k_mean, a.v_inv,
                     a.k_i8, a.k_scale, a.v_f8, a.v16);
  return hipGetLastError();
}

template <int D, bool V16, bool TOK>
static hipError_t launch_quant_kbm(const QuantArgs& a, hipStream_t s) {
  if constexpr (!V16) {
    if (a.kbm) return launch_quant_d<D, V16, TOK, true>(a, s);
  }
  return launch_quant_d<D, V16, TOK, false>(a, s);
}

template <int D>
static hipError_t launch_quant_mode(const QuantArgs& a, hipStream_t s) {
  if (a.pv == kPvBf16) return a.tok ? launch_quant_kbm<D, true, true>(a, s) : launch_quant_kbm<D, true, false>(a, s);
  return a.tok ? launch_quant_kbm<D, false, true>(a, s) : launch_quant_kbm<D, false, false>(a, s);
}

hipError_t launch_quant(const QuantArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_quant_mode<64>(a, s) : launch_quant_mode<128>(a, s);
}

hipError_t launch_debug_e4m3(const float* x, uint8_t* y, int64_t n, hipStream_t s) {
  const int64_t pairs = (n + 1) / 2;
  const unsigned blocks = (unsigned)((pairs + 255) / 256);
  hipLaunchKernelGGL(k_debug_e4m3, dim3(blocks), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}

}  // namespace sage
