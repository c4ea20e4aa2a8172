// Quantisation pass for gfx950: K token mean (smoothing), per-block INT8 codes of Q
// and K - mean, per-channel FP8 e4m3 codes of V (juejin page "MiniMax H3 接入
// SageAttention 实测加速", section 一; the bf16 mean term of the sd114.wiki
// ComfyUI-sol-attn page, "核心亮点" item 1).
//
// Three launches, all HBM-bound:
//   1. stats    grid (chunks of 256 tokens, H, B): fp64 partial sums of K and partial
//               max |V| per channel, read with 16-byte loads along the channel axis.
//   2. finalize grid (B*H): sums the partials in chunk order -> k_mean (bf16),
//               v_scale = vamax/448 and 448/vamax.
//   3. codes    grid (Npad/64, H, B): one 64-token block of Q, K and V per workgroup;
//               block max-abs reduced across the workgroup, codes written with 8-byte
//               stores; V codes are transposed through LDS into the channel-major
//               layout the attention kernel stages directly.
#include "sage_internal.h"
#include "sage_device.h"

namespace sage {

template <int D>
__global__ __launch_bounds__(256) void k_quant_stats(
    const uint16_t* __restrict__ k, Strides sk, const uint16_t* __restrict__ v, Strides sv,
    int H, int N, int chunks, double* __restrict__ ksum_part, float* __restrict__ vmax_part) {
  constexpr int TPR = D / 8;        // threads per token row, 8 channels each
  constexpr int RPI = 256 / TPR;    // token rows per iteration
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, r = t / TPR, cg = t % TPR;
  const int n0 = chunk * kStatsChunk;
  const int n1 = min(N, n0 + kStatsChunk);
  const uint16_t* kb = k + (int64_t)b * sk.b + (int64_t)h * sk.h + 8 * cg;
  const uint16_t* vb = v + (int64_t)b * sv.b + (int64_t)h * sv.h + 8 * cg;
  double s[8];
  float vm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { s[j] = 0.0; vm[j] = 0.0f; }
#pragma unroll 4
  for (int n = n0 + r; n < n1; n += RPI) {
    const uint4 kw = *(const uint4*)(kb + (int64_t)n * sk.n);
    const uint4 vw = *(const uint4*)(vb + (int64_t)n * sv.n);
    float kx[8], vx[8];
    bf16x8_to_f32(kw, kx);
    bf16x8_to_f32(vw, vx);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s[j] += (double)kx[j];
      vm[j] = fmaxf(vm[j], fabsf(vx[j]));
    }
  }
  __shared__ __attribute__((aligned(16))) double red_s[RPI][D];
  __shared__ float red_v[RPI][D];
#pragma unroll
  for (int j = 0; j < 8; ++j) { red_s[r][8 * cg + j] = s[j]; red_v[r][8 * cg + j] = vm[j]; }
  __syncthreads();
  if (t < D) {
    double acc = 0.0;
    float m = 0.0f;
    for (int i = 0; i < RPI; ++i) { acc += red_s[i][t]; m = fmaxf(m, red_v[i][t]); }
    const int64_t o = ((int64_t)(b * H + h) * chunks + chunk) * D + t;
    ksum_part[o] = acc;
    vmax_part[o] = m;
  }
}

template <int D>
__global__ __launch_bounds__(D) void k_quant_finalize(
    const double* __restrict__ ksum_part, const float* __restrict__ vmax_part, int chunks, int N,
    uint16_t* __restrict__ k_mean, float* __restrict__ v_scale, float* __restrict__ v_inv) {
  const int64_t bh = blockIdx.x;
  const int c = threadIdx.x;
  double s = 0.0;
  float vm = 0.0f;
  for (int i = 0; i < chunks; ++i) {
    s += ksum_part[(bh * chunks + i) * D + c];
    vm = fmaxf(vm, vmax_part[(bh * chunks + i) * D + c]);
  }
  const float mean = (float)(s / (double)N);        // fp64 divide, one rounding to fp32
  k_mean[bh * D + c] = (uint16_t)f32_to_bf16_rne(mean);
  v_scale[bh * D + c] = vm / kPScale;               // IEEE division (0 when vm = 0)
  v_inv[bh * D + c] = vm > 0.0f ? kPScale / vm : 0.0f;
}

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

template <int D>
__global__ __launch_bounds__(256) void k_quant_codes(
    const uint16_t* __restrict__ q, Strides sq, const uint16_t* __restrict__ k, Strides sk,
    const uint16_t* __restrict__ v, Strides sv, int H, int N, int64_t npad,
    const uint16_t* __restrict__ k_mean, const float* __restrict__ v_inv,
    int8_t* __restrict__ q_i8, float* __restrict__ q_scale, int8_t* __restrict__ k_i8,
    float* __restrict__ k_scale, uint8_t* __restrict__ v_f8) {
  constexpr int TPR = D / 8;
  constexpr int RPI = 256 / TPR;
  constexpr int RPT = kQuantBlock / RPI;   // token rows per thread
  constexpr int VLD = kQuantBlock + 16;    // LDS row pitch of the transposed V block
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, r = t / TPR, cg = t % TPR;
  const int64_t bh = (int64_t)b * gridDim.y + h;
  const int row0 = blk * kQuantBlock;
  const int64_t nblk = npad / kQuantBlock;
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t vt[D][VLD];

  float x[RPT][8];
  uint2 codes[RPT];

  // ---- Q ----
  {
    const uint16_t* base = q + (int64_t)b * sq.b + (int64_t)h * sq.h + 8 * cg;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int n = row0 + r + RPI * i;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (n < N) w = *(const uint4*)(base + (int64_t)n * sq.n);
      bf16x8_to_f32(w, x[i]);
    }
    const float scale = int8_block<RPT>(x, codes, red);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int n = row0 + r + RPI * i;
      *(uint2*)(q_i8 + (bh * npad + n) * D + 8 * cg) = codes[i];
    }
    if (t == 0) q_scale[bh * nblk + blk] = scale;
  }
  // ---- K - mean ----
  {
    float mu[8];
    const uint4 mw = *(const uint4*)(k_mean + bh * D + 8 * cg);
    bf16x8_to_f32(mw, mu);
    const uint16_t* base = k + (int64_t)b * sk.b + (int64_t)h * sk.h + 8 * cg;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int n = row0 + r + RPI * i;
      if (n < N) {
        const uint4 w = *(const uint4*)(base + (int64_t)n * sk.n);
        bf16x8_to_f32(w, x[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[i][j] = x[i][j] - mu[j];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[i][j] = 0.0f;
      }
    }
    const float scale = int8_block<RPT>(x, codes, red);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int n = row0 + r + RPI * i;
      *(uint2*)(k_i8 + (bh * npad + n) * D + 8 * cg) = codes[i];
    }
    if (t == 0) k_scale[bh * nblk + blk] = scale;
  }
  // ---- V -> e4m3, transposed to [channel][token] ----
  {
    float inv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) inv[j] = v_inv[bh * D + 8 * cg + j];
    const uint16_t* base = v + (int64_t)b * sv.b + (int64_t)h * sv.h + 8 * cg;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int n = row0 + r + RPI * i;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (n < N) w = *(const uint4*)(base + (int64_t)n * sv.n);
      bf16x8_to_f32(w, x[i]);
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const uint32_t c2 = e4m3x2_sat(x[i][j] * inv[j], x[i][j + 1] * inv[j + 1]);
        vt[8 * cg + j][r + RPI * i] = (uint8_t)(c2 & 0xff);
        vt[8 * cg + j + 1][r + RPI * i] = (uint8_t)(c2 >> 8);
      }
    }
    __syncthreads();
    constexpr int NCH = D * (kQuantBlock / 16);      // 16-byte chunks of the block
#pragma unroll
    for (int cid = t; cid < NCH; cid += 256) {
      const int c = cid / (kQuantBlock / 16), part = cid % (kQuantBlock / 16);
      const uint4 w = *(const uint4*)(&vt[c][16 * part]);
      *(uint4*)(v_f8 + (bh * D + c) * npad + row0 + 16 * part) = w;
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

template <int D>
static hipError_t launch_quant_d(const QuantArgs& a, hipStream_t s) {
  const int chunks = stats_chunks(a.N);
  hipLaunchKernelGGL(k_quant_stats<D>, dim3(chunks, a.H, a.B), dim3(256), 0, s,
                     a.k, a.sk, a.v, a.sv, a.H, a.N, chunks, a.ksum_part, a.vmax_part);
  hipLaunchKernelGGL(k_quant_finalize<D>, dim3(a.B * a.H), dim3(D), 0, s,
                     a.ksum_part, a.vmax_part, chunks, a.N, a.k_mean, a.v_scale, a.v_inv);
  hipLaunchKernelGGL(k_quant_codes<D>, dim3((unsigned)(a.npad / kQuantBlock), a.H, a.B), dim3(256), 0, s,
                     a.q, a.sq, a.k, a.sk, a.v, a.sv, a.H, a.N, a.npad, a.k_mean, a.v_inv,
                     a.q_i8, a.q_scale, a.k_i8, a.k_scale, a.v_f8);
  return hipGetLastError();
}

hipError_t launch_quant(const QuantArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_quant_d<64>(a, s) : launch_quant_d<128>(a, s);
}

hipError_t launch_debug_e4m3(const float* x, uint8_t* y, int64_t n, hipStream_t s) {
  const int64_t pairs = (n + 1) / 2;
  const unsigned blocks = (unsigned)((pairs + 255) / 256);
  hipLaunchKernelGGL(k_debug_e4m3, dim3(blocks), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}

}  // namespace sage
