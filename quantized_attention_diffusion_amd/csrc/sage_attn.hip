// Fused quantised attention for gfx950 (MI355X): INT8 Q.K^T on matrix cores with
// int32 accumulation, dequantisation, fp32 online softmax in base 2, P rounded to
// FP8 e4m3, P.V on FP8 matrix cores, bf16 output (juejin page "MiniMax H3 接入
// SageAttention 实测加速", section 一: INT8 for QK, FP8 for PV; bjdmk page
// "GitHub榜单静默期：Attention优化从架构转向推理加速", section 2.2: blockwise computation
// that never writes the score matrix out).
//
// Work decomposition
//   workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 2 groups of 16
//   queries.  Keys are visited in tiles of 128; K (128 x d int8) and V (d x 128 e4m3,
//   channel-major) tiles are staged in LDS and shared by the 4 waves.
//
// Register layouts (16x16 matrix-core tiles; lane l, r = l % 16, g = l / 16)
//   S^T = K . Q^T with v_mfma_i32_16x16x64_i8: the row operand is 16 keys, the column
//   operand 16 queries.  Output element (row 4g+i, column r) sits in lane l, register i.
//   Row j of key sub-tile kt is mapped to tile key 32*(j/4) + 4*kt + j%4, so lane l ends
//   up holding, for its query r, the 32 consecutive tile keys 32g .. 32g+31 (register i
//   of sub-tile kt = key 32g + 4kt + i).  Those 32 keys lie in one 64-key scale block.
//   O^T = V^T . P^T with v_mfma_f32_16x16x128_f8f6f4: the column operand of lane l is
//   32 bytes of P for query r over keys 32g .. 32g+31, exactly the values the lane
//   already holds, so P never leaves its registers; the row operand is 32 bytes of
//   channel-major V (channel 16*dt + r, the same 32 keys).  Output: lane l holds
//   O[query r][channel 16*dt + 4g + i].
//   Every per-query quantity (running max m, partial row sum, accumulators) is thus
//   lane-local; only the tile maximum and the final row sum combine the 4 lanes
//   r, r+16, r+32, r+48.
#include "sage_internal.h"
#include "sage_device.h"

namespace sage {

constexpr int G = kGroupsPerWave;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS tiles are unpadded and XOR-swizzled at 16-byte granularity so that the 16 lanes
// served together by a 128-bit LDS read hit 16 distinct bank groups:
//   K tile [128 keys][D bytes]:   physical chunk = chunk ^ kswz(key)
//   V tile [D channels][128 keys]: physical chunk = chunk ^ vswz(channel)
// (the matrix-core operand reads below touch keys 32*(r/4) + 4*kt + r%4 and channels
// 16*dt + r for r = 0..15).
template <int D>
__device__ __forceinline__ int kswz(int key) {
  if constexpr (D == 128) return ((key >> 5) & 3) | (((key >> 1) & 1) << 2);
  else return (key >> 5) & 3;
}
__device__ __forceinline__ int vswz(int ch) { return (ch >> 1) & 7; }

template <int D>
struct Lds {
  static constexpr int KBYTES = kKvTile * D;   // one K tile
  static constexpr int VBYTES = D * kKvTile;   // one V tile
  static constexpr int STAGE = KBYTES + VBYTES;
};

// Asynchronous copies of one K tile (128 x D int8, rows of D bytes at kg) and one V tile
// (D channel rows of 128 e4m3 bytes at vg, row pitch npad) straight into LDS with
// global_load_lds_dwordx4: each wave instruction fills 1 KB of LDS, lane i the 16 bytes
// at offset 16*i, so the swizzle is applied by choosing which global chunk lane i reads.
// Completion is awaited by the s_waitcnt vmcnt(0) that precedes the next barrier.
template <int D>
__device__ __forceinline__ void issue_k(const int8_t* __restrict__ kg, uint8_t* klds) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int PW = Lds<D>::KBYTES / 1024 / kWaves;   // 1 KB blocks per wave
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    const int blk = wave * PW + j;
    const int pos = blk * 1024 + lane * 16;
    const int key = pos / D, pc = (pos % D) / 16;
    const int c = pc ^ kswz<D>(key);
    __builtin_amdgcn_global_load_lds(kg + key * D + c * 16, (lds_ptr_t)(klds + blk * 1024), 16, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void issue_v(const uint8_t* __restrict__ vg, int64_t npad, uint8_t* vlds) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int PW = Lds<D>::VBYTES / 1024 / kWaves;
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    const int blk = wave * PW + j;
    const int pos = blk * 1024 + lane * 16;
    const int ch = pos / kKvTile, pc = (pos % kKvTile) / 16;
    const int c = pc ^ vswz(ch);
    __builtin_amdgcn_global_load_lds(vg + (int64_t)ch * npad + c * 16, (lds_ptr_t)(vlds + blk * 1024), 16, 0, 0);
  }
}

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

// Exact int32 S^T for the staged key tile: S[gq][kt] register i = S(query r of group gq,
// tile key 32g + 4kt + i).
template <int D>
__device__ __forceinline__ void qk_tile(const int8_t* klds, const v4i (&qf)[G][D / 64], int lane,
                                        v4i (&S)[G][8]) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    const int key = 32 * (r >> 2) + 4 * kt + (r & 3);
#pragma unroll
    for (int gq = 0; gq < G; ++gq) S[gq][kt] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
      const v4i a = *(const v4i*)(klds + key * D + 16 * ((4 * kk + g) ^ kswz<D>(key)));
#pragma unroll
      for (int gq = 0; gq < G; ++gq)
        S[gq][kt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qf[gq][kk], S[gq][kt], 0, 0, 0);
    }
  }
}

// Online-softmax update and P.V for one staged tile.  S is consumed: it is
// converted to fp32 in place (|S| < 2^24, so exactly).  When MASKED, keys at tile
// index >= nvalid are removed by setting their logit to -inf; a lane whose scale
// product is 0 then takes x = 0 and c = 1 for its valid keys, which gives the same
// values (s = 0, p = 448 * 2^-m) without forming -inf * 0.
template <int D, bool MASKED>
__device__ __forceinline__ void softmax_pv(v4i (&S)[G][8], const uint8_t* vlds, int lane,
                                           float kscale, int nvalid,
                                           const float (&qf)[G], float log2_pscale,
                                           float (&m)[G], float (&lpart)[G],
                                           v4f (&acc)[G][D / 16]) {
  const int r = lane & 15, g = lane >> 4;
  float xf[G][8][4];
  float c[G];
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    c[gq] = qf[gq] * kscale;                       // fp32(qf * k_scale)
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) xf[gq][kt][i] = (float)S[gq][kt][i];
  }
  if constexpr (MASKED) {
    const int nv = nvalid - 32 * g;                // valid keys among this lane's 32
#pragma unroll
    for (int gq = 0; gq < G; ++gq) {
      const bool zero_c = (c[gq] == 0.0f);
      if (zero_c) c[gq] = 1.0f;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = (4 * kt + i) < nv;
          xf[gq][kt][i] = ok ? (zero_c ? 0.0f : xf[gq][kt][i]) : -INFINITY;
        }
    }
  }
  v8i P[G];
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    float xm = xf[gq][0][0];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) xm = fmaxf(xm, xf[gq][kt][i]);
    // c >= 0 and rounding is monotone, so this is the max of fp32(x * c) over the keys
    float sl = (xm == -INFINITY) ? -INFINITY : xm * c[gq];
    sl = max_over_lane_groups(sl);
    const float m_new = fmaxf(m[gq], sl);
    const float nb = log2_pscale - m_new;
    const float alpha = __builtin_amdgcn_exp2f(m[gq] - m_new);
    float lsum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(xf[gq][kt][i], c[gq], nb));
        lsum += p[i];
      }
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
      P[gq][kt] = w;
    }
    lpart[gq] = alpha * lpart[gq] + lsum;
    m[gq] = m_new;
    // multiplying by exactly 1 changes nothing: skip when no lane's max moved
    if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[gq][dt] *= alpha;
    }
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int ch = 16 * dt + r;
    const uint8_t* vp = vlds + ch * kKvTile;
    const v4i lo = *(const v4i*)(vp + 16 * ((2 * g) ^ vswz(ch)));
    const v4i hi = *(const v4i*)(vp + 16 * ((2 * g + 1) ^ vswz(ch)));
    const v8i vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int gq = 0; gq < G; ++gq)
      acc[gq][dt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vf, P[gq], acc[gq][dt],
                                                                      0, 0, 0, 0, 0, 0);
  }
}

// Maps the linear workgroup id to (head, query block) so that the workgroups one XCD
// receives (ids x, x+8, x+16, ... go to XCD x) are consecutive query blocks of the same
// heads and share that head's K/V tiles in the XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  constexpr int kXcds = 8;
  const int per = total / kXcds, rem = total % kXcds;
  const int x = id % kXcds, idx = id / kXcds;
  return (x < rem) ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

// One key tile from an LDS stage: exact int32 S^T, then softmax and P.V.
template <int D, bool MASKED>
__device__ __forceinline__ void tile_step(const uint8_t* stage, const v4i (&qfr)[G][D / 64], int lane,
                                          float ksc, int nvalid, const float (&qf)[G],
                                          float log2_pscale, float (&m)[G], float (&lpart)[G],
                                          v4f (&acc)[G][D / 16]) {
  v4i S[G][8];
  qk_tile<D>((const int8_t*)stage, qfr, lane, S);
  softmax_pv<D, MASKED>(S, stage + Lds<D>::KBYTES, lane, ksc, nvalid, qf, log2_pscale, m, lpart, acc);
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn(AttnArgs a) {
  // two LDS stages of (K tile, V tile): the copy of tile it+1 overlaps the compute of tile it
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * Lds<D>::STAGE];

  const int nqb = (int)(a.npad / kBlockM);
  const int total = nqb * a.B * a.H;
  const int work = xcd_remap(blockIdx.x, total);
  const int64_t bh = work / nqb;
  const int qb = work % nqb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int qrow0 = qb * kBlockM + wave * (G * 16);
  const int64_t nblk = a.npad / kQuantBlock;

  const int8_t* kh = a.k_i8 + bh * a.npad * D;
  const uint8_t* vh = a.v_f8 + bh * D * a.npad;
  const float* ksh = a.k_scale + bh * nblk + (g >> 1);   // this lane's 64-key half of a tile
  const int ntiles = (a.N + kKvTile - 1) / kKvTile;
  const int tail = a.N - (ntiles - 1) * kKvTile;     // keys in the last tile (1..128)
  const int nfull = (tail == kKvTile) ? ntiles : ntiles - 1;

  issue_k<D>(kh, smem);
  issue_v<D>(vh, a.npad, smem + Lds<D>::KBYTES);

  v4i qfr[G][D / 64];
  load_q<D>(a.q_i8 + bh * a.npad * D, qrow0, lane, qfr);
  float qf[G], m[G], lpart[G];
  v4f acc[G][D / 16];
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    qf[gq] = a.q_scale[bh * nblk + (qrow0 + 16 * gq) / kQuantBlock] * a.log2e_scale;
    m[gq] = -INFINITY;
    lpart[gq] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[gq][dt] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  float ksc = ksh[0];
  __syncthreads();

  for (int it = 0; it < nfull; ++it) {
    const uint8_t* cur = smem + (it & 1) * Lds<D>::STAGE;
    float ksc_next = 0.0f;
    if (it + 1 < ntiles) {
      uint8_t* nxt = smem + ((it + 1) & 1) * Lds<D>::STAGE;
      issue_k<D>(kh + (int64_t)(it + 1) * kKvTile * D, nxt);
      issue_v<D>(vh + (int64_t)(it + 1) * kKvTile, a.npad, nxt + Lds<D>::KBYTES);
      ksc_next = ksh[2 * (it + 1)];
    }
    tile_step<D, false>(cur, qfr, lane, ksc, kKvTile, qf, a.log2_pscale, m, lpart, acc);
    ksc = ksc_next;
    __syncthreads();
  }
  if (nfull < ntiles)   // last tile with keys beyond N: already staged in stage nfull & 1
    tile_step<D, true>(smem + (nfull & 1) * Lds<D>::STAGE, qfr, lane, ksc, tail, qf,
                       a.log2_pscale, m, lpart, acc);

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
        uint32_t h0 = f32_to_bf16_rne(acc[gq][dt][0] * vsh[c0 + 0] * rl);
        uint32_t h1 = f32_to_bf16_rne(acc[gq][dt][1] * vsh[c0 + 1] * rl);
        uint32_t h2 = f32_to_bf16_rne(acc[gq][dt][2] * vsh[c0 + 2] * rl);
        uint32_t h3 = f32_to_bf16_rne(acc[gq][dt][3] * vsh[c0 + 3] * rl);
        *(uint2*)(orow + c0) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
      }
    }
  }
}

// Int32 S tiles through the same staging and matrix-core code as k_attn.
template <int D>
__global__ __launch_bounds__(256) void k_debug_qk(const int8_t* __restrict__ q_i8,
                                                  const int8_t* __restrict__ k_i8, int64_t npad,
                                                  int64_t bh, int q_block, int kv_tile,
                                                  int n_kv_tiles, int32_t* __restrict__ s_out) {
  __shared__ __attribute__((aligned(1024))) uint8_t klds[Lds<D>::KBYTES];
  const int qb = q_block + blockIdx.y, kvt = kv_tile + blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int qrow0 = qb * kBlockM + wave * (G * 16);
  issue_k<D>(k_i8 + bh * npad * D + (int64_t)kvt * kKvTile * D, klds);
  v4i qfr[G][D / 64];
  load_q<D>(q_i8 + bh * npad * D, qrow0, lane, qfr);
  __syncthreads();
  v4i S[G][8];
  qk_tile<D>((const int8_t*)klds, qfr, lane, S);
  const int64_t ld = (int64_t)n_kv_tiles * kKvTile;
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    const int64_t row = (int64_t)blockIdx.y * kBlockM + wave * (G * 16) + 16 * gq + r;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_out[row * ld + (int64_t)blockIdx.x * kKvTile + 32 * g + 4 * kt + i] = S[gq][kt][i];
  }
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int nqb = (int)(a.npad / kBlockM);
  const unsigned grid = (unsigned)((int64_t)nqb * a.B * a.H);
  if (a.d == 64)
    hipLaunchKernelGGL(k_attn<64>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_attn<128>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_debug_qk(const int8_t* q_i8, const int8_t* k_i8, int d, int64_t npad,
                           int64_t bh, int q_block, int kv_tile, int n_q_blocks,
                           int n_kv_tiles, int32_t* s_out, hipStream_t s) {
  const dim3 grid(n_kv_tiles, n_q_blocks);
  if (d == 64)
    hipLaunchKernelGGL(k_debug_qk<64>, grid, dim3(256), 0, s, q_i8, k_i8, npad, bh, q_block,
                       kv_tile, n_kv_tiles, s_out);
  else
    hipLaunchKernelGGL(k_debug_qk<128>, grid, dim3(256), 0, s, q_i8, k_i8, npad, bh, q_block,
                       kv_tile, n_kv_tiles, s_out);
  return hipGetLastError();
}

}  // namespace sage
