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

// LDS tiles are unpadded and XOR-swizzled at 16-byte granularity so that the 128-bit
// operand reads below run without bank conflicts:
//   K tile [128 keys][D bytes]:    physical chunk = chunk ^ kswz(key)
//   V tile [D channels][128 keys]: physical chunk = chunk ^ vswz(channel)
// A K read touches keys 32*(r/4) + 4*kt + r%4 (r = lane % 16), i.e. varies key bits
// 0, 1, 5, 6 across the wave; a V read touches channels 16*dt + r.  The K swizzle is a
// linear map of those four key bits onto the three chunk bits; gfx950's bank grouping
// for 128-bit reads is not documented, so it was chosen by timing all 4096 such maps on
// the exact K read pattern (about a third run at the conflict-free rate; the obvious
// maps for 16- or 32-lane passes do not).  The V swizzle runs at the contiguous rate.
template <int D>
__device__ __forceinline__ int kswz(int key) {
  if constexpr (D == 128)
    return ((key ^ (key >> 1) ^ (key >> 6)) & 1) | (((key ^ (key >> 5)) & 1) << 1) | (((key >> 6) & 1) << 2);
  else
    return (key >> 5) & 3;
}
__device__ __forceinline__ int vswz(int ch) { return ((ch ^ (ch >> 3)) & 1) | (ch & 6); }

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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
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

// Per-lane source offsets of the LDS DMA copies (computed once per kernel): the K tile
// copy of wave w, instruction j reads K + koff[j], the V tile copy V + voff[j] (bytes,
// relative to the tile's first key), which lands at LDS offset (w*PW + j)*1024 + 16*lane.
template <int D>
struct DmaOffsets {
  static constexpr int KPW = Lds<D>::KBYTES / 1024 / kWaves;
  static constexpr int VPW = Lds<D>::VBYTES / 1024 / kWaves;
  uint32_t koff[KPW];
  uint32_t voff[VPW];
  __device__ __forceinline__ DmaOffsets(int wave, int lane, int64_t npad) {
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int pos = (wave * KPW + j) * 1024 + lane * 16;
      const int key = pos / D, pc = (pos % D) / 16;
      koff[j] = (uint32_t)(key * D + (pc ^ kswz<D>(key)) * 16);
    }
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
      const int pos = (wave * VPW + j) * 1024 + lane * 16;
      const int ch = pos / kKvTile, pc = (pos % kKvTile) / 16;
      voff[j] = (uint32_t)(ch * npad + (pc ^ vswz(ch)) * 16);
    }
  }
  __device__ __forceinline__ void issue_k(const int8_t* __restrict__ ktile, uint8_t* klds, int wave) const {
#pragma unroll
    for (int j = 0; j < KPW; ++j)
      __builtin_amdgcn_global_load_lds(ktile + koff[j], (lds_ptr_t)(klds + (wave * KPW + j) * 1024), 16, 0, 0);
  }
  __device__ __forceinline__ void issue_v(const uint8_t* __restrict__ vtile, uint8_t* vlds, int wave) const {
#pragma unroll
    for (int j = 0; j < VPW; ++j)
      __builtin_amdgcn_global_load_lds(vtile + voff[j], (lds_ptr_t)(vlds + (wave * VPW + j) * 1024), 16, 0, 0);
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

// Exact int32 S^T of one 16-query group for a staged key tile: S[kt] register i =
// S(query r, tile key 32g + 4kt + i).
template <int D>
__device__ __forceinline__ void qk_group(const uint8_t* kbuf, const v4i (&qg)[D / 64], int lane,
                                         v4i (&S)[8]) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    const int key = 32 * (r >> 2) + 4 * kt + (r & 3);
    S[kt] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
      const v4i a = *(const v4i*)(kbuf + key * D + 16 * ((4 * kk + g) ^ kswz<D>(key)));
      S[kt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qg[kk], S[kt], 0, 0, 0);
    }
  }
}

// acc[dt] += V^T(channels 16dt..16dt+15) . P^T for one 16-query group.
template <int D>
__device__ __forceinline__ void pv_group(const uint8_t* vbuf, const v8i& P, int lane,
                                         v4f (&acc)[D / 16]) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int ch = 16 * dt + r;
    const uint8_t* vp = vbuf + ch * kKvTile;
    const v4i lo = *(const v4i*)(vp + 16 * ((2 * g) ^ vswz(ch)));
    const v4i hi = *(const v4i*)(vp + 16 * ((2 * g + 1) ^ vswz(ch)));
    const v8i vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    acc[dt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vf, P, acc[dt], 0, 0, 0, 0, 0, 0);
  }
}

// Online-softmax update of one 16-query group for one tile.  S is consumed (converted
// to fp32 exactly: |S| < 2^24); c = fp32(q factor * k_scale) of this lane's keys.
// Produces the e4m3 P operand, updates the running max m and this lane's partial row
// sum, and returns alpha = 2^(m_old - m_new), the factor the accumulators need.
// When MASKED, keys at tile index >= nvalid are removed by giving them the logit -inf;
// a lane whose c is 0 then uses x = 0 and c = 1 for its valid keys, which yields the
// same s = 0 and p = 448 * 2^-m without forming -inf * 0.
template <bool MASKED>
__device__ __forceinline__ float softmax_group(v4i (&S)[8], float c, int nvalid, float log2_pscale,
                                               float& m, float& lpart, v8i& P, int g) {
  float xf[8][4];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) xf[kt][i] = (float)S[kt][i];
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
  float xm = xf[0][0];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) xm = fmaxf(xm, xf[kt][i]);
  // c >= 0 and rounding is monotone, so this is the max of fp32(x * c) over the keys
  float sl = (xm == -INFINITY) ? -INFINITY : xm * c;
  sl = max_over_lane_groups(sl);
  const float m_new = fmaxf(m, sl);
  const float nb = log2_pscale - m_new;
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
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
    P[kt] = w;
  }
  lpart = alpha * lpart + lsum;
  m = m_new;
  return alpha;
}

// Marks P (and the row-sum state) as used at this point, so that the compiler keeps the
// softmax work that produces it inside the phase it was interleaved with instead of
// sinking it past the barrier into the next phase.
__device__ __forceinline__ void materialize(const v8i& P, float l) {
  asm volatile("" : : "v"(P[0]), "v"(P[1]), "v"(P[2]), "v"(P[3]), "v"(P[4]), "v"(P[5]),
               "v"(P[6]), "v"(P[7]), "v"(l));
}

// acc *= alpha, skipped when no lane's maximum moved (multiplying by exactly 1).
template <int D>
__device__ __forceinline__ void rescale(v4f (&acc)[D / 16], float alpha) {
  if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] *= alpha;
  }
}

// ---------------------------------------------------------------------------------
// Explicitly scheduled phase: the softmax of one query group (17 VALU chunks) with the
// matrix-core work of the other group placed between the chunks.  Each chunk ends in a
// scheduling fence, so the issue order is exactly the one written here: matrix-core
// instructions (16-32 cycles each) are spread over the VALU stream, and their LDS
// operands are loaded PF instructions ahead.
template <int D>
struct PhaseShape {
  static constexpr int NQ = 8 * (D / 64);   // S^T matrix-core instructions (8 key sub-tiles)
  static constexpr int NP = D / 16;         // O^T matrix-core instructions (channel tiles)
  static constexpr int NM = NQ + NP;
  static constexpr int PF = 4;              // operand loads in flight
  static constexpr int CHUNKS = 17;         // 8 convert/max, 1 reduce, 8 exp/pack
  // matrix-core instructions issued before VALU chunk ch (none in the reduce chunk)
  static constexpr int ops_before(int ch) {
    const int a = ch < 8 ? ch : 8, b = ch > 9 ? ch - 9 : 0;
    return D == 128 ? a + 2 * b : (a + 1) / 2 + b;
  }
};

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f.template operator()<B>();
    static_for<B + 1, E>(f);
  }
}

// Per-lane LDS byte offsets of the matrix-core operand reads.  The swizzles depend only
// on key bits 0, 1, 5, 6 and channel bits 0-3, so the offset of K sub-tile kt is
// koff[kk] + kt * 4 * D and that of V channel tile dt is voff[half] + dt * 16 * 128.
template <int D>
struct LaneOffsets {
  int koff[D / 64];
  int voff[2];
  __device__ __forceinline__ explicit LaneOffsets(int lane) {
    const int r = lane & 15, g = lane >> 4;
    const int key = 32 * (r >> 2) + (r & 3);
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) koff[kk] = key * D + 16 * ((4 * kk + g) ^ kswz<D>(key));
#pragma unroll
    for (int h = 0; h < 2; ++h) voff[h] = r * kKvTile + 16 * ((2 * g + h) ^ vswz(r));
  }
};

template <int D>
__device__ __forceinline__ v4i load_kfrag(const uint8_t* kbuf, int q, const LaneOffsets<D>& lo) {
  const int kt = q / (D / 64), kk = q % (D / 64);
  return *(const v4i*)(kbuf + lo.koff[kk] + kt * 4 * D);
}

template <int D>
__device__ __forceinline__ v8i load_vfrag(const uint8_t* vbuf, int dt, const LaneOffsets<D>& lo) {
  const v4i a = *(const v4i*)(vbuf + lo.voff[0] + dt * 16 * kKvTile);
  const v4i b = *(const v4i*)(vbuf + lo.voff[1] + dt * 16 * kKvTile);
  return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Matrix cores: Sout = K . qg^T (S^T of the other group, from kbuf) and acc += V^T . Pin^T
// (from vbuf), in the order QK then PV when QK_FIRST, else PV then QK.
// VALU: online-softmax update of this group from Sin with scale product c -> Pout, m,
// lpart (same arithmetic and masking as softmax_group).  Returns alpha.
template <int D, bool MASKED, bool QK_FIRST>
__device__ __forceinline__ float phase(const uint8_t* kbuf, const v4i (&qg)[D / 64], v4i (&Sout)[8],
                                       const uint8_t* vbuf, const v8i& Pin, v4f (&acc)[D / 16],
                                       v4i (&Sin)[8], float c, int nvalid, float log2_pscale,
                                       float& m, float& lpart, v8i& Pout, int lane,
                                       const LaneOffsets<D>& lo) {
  using PS = PhaseShape<D>;
  const int g = lane >> 4;
  v4i kf[PS::NQ];
  v8i vf[PS::NP];
  auto load = [&]<int I>() {
    constexpr bool qk = QK_FIRST ? (I < PS::NQ) : (I >= PS::NP);
    constexpr int j = QK_FIRST ? (I < PS::NQ ? I : I - PS::NQ) : (I < PS::NP ? I : I - PS::NP);
    if constexpr (qk) kf[j] = load_kfrag<D>(kbuf, j, lo);
    else vf[j] = load_vfrag<D>(vbuf, j, lo);
  };
  auto issue = [&]<int I>() {
    constexpr bool qk = QK_FIRST ? (I < PS::NQ) : (I >= PS::NP);
    constexpr int j = QK_FIRST ? (I < PS::NQ ? I : I - PS::NQ) : (I < PS::NP ? I : I - PS::NP);
    if constexpr (qk) {
      constexpr int kt = j / (D / 64), kk = j % (D / 64);
      Sout[kt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf[j], qg[kk], kk == 0 ? v4i{0, 0, 0, 0} : Sout[kt], 0, 0, 0);
    } else {
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vf[j], Pin, acc[j], 0, 0, 0, 0, 0, 0);
    }
    if constexpr (I + PS::PF < PS::NM) load.template operator()<I + PS::PF>();
  };

  float xf[8][4];
  float xm = -INFINITY, cc = c, nb = 0.0f, m_new = m, alpha = 1.0f;
  float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};          // partial row sums (independent chains)
  int xmi = INT_MIN;
  const int nv = nvalid - 32 * g;                  // valid keys among this lane's 32
  bool zero_c = false;
  if constexpr (MASKED) {
    zero_c = (c == 0.0f);
    cc = zero_c ? 1.0f : c;
  }
  auto valu = [&]<int CH>() {
    if constexpr (CH < 8) {
      if constexpr (MASKED) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = (float)Sin[CH][i];
          xf[CH][i] = ((4 * CH + i) < nv) ? (zero_c ? 0.0f : x) : -INFINITY;
        }
        xm = fmaxf(xm, fmaxf(fmaxf(xf[CH][0], xf[CH][1]), fmaxf(xf[CH][2], xf[CH][3])));
      } else {
        // integer max (exact, no NaN handling); the conversion is exact since |S| < 2^24
        xmi = max(xmi, max(max(Sin[CH][0], Sin[CH][1]), max(Sin[CH][2], Sin[CH][3])));
#pragma unroll
        for (int i = 0; i < 4; ++i) xf[CH][i] = (float)Sin[CH][i];
      }
    } else if constexpr (CH == 8) {
      // c >= 0 and rounding is monotone: this is the max of fp32(x * c) over the keys
      float sl;
      if constexpr (MASKED) sl = (xm == -INFINITY) ? -INFINITY : xm * cc;
      else sl = (float)xmi * cc;
      sl = max_over_lane_groups(sl);
      m_new = fmaxf(m, sl);
      nb = log2_pscale - m_new;
      alpha = __builtin_amdgcn_exp2f(m - m_new);
    } else {
      constexpr int kt = CH - 9;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(xf[kt][i], cc, nb));
#pragma unroll
      for (int i = 0; i < 4; ++i) ls[i] += p[i];
      // the previous contents of Pout[kt] are overwritten by the two conversions
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], Pout[kt], false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
      Pout[kt] = w;
    }
  };
  auto chunk = [&]<int CH>() {
    static_for<PS::ops_before(CH), PS::ops_before(CH + 1)>(issue);
    valu.template operator()<CH>();
    __builtin_amdgcn_sched_barrier(0);
  };

  static_for<0, PS::PF>(load);
  static_for<0, PS::CHUNKS>(chunk);
  lpart = alpha * lpart + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
  m = m_new;
  return alpha;
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

// Interleaving hint for one phase (24 matrix-core instructions, 32 LDS operand reads,
// the softmax VALU work of one query group): LDS reads run 4 ahead of the matrix-core
// instruction that consumes them, and each matrix-core instruction is followed by VALU
// work, so the softmax of one group runs while the matrix cores work on the other.
__device__ __forceinline__ void interleave_phase() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // LDS reads
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
  }
}

struct AttnState {
  float qf[G], m[G], lpart[G];
};

// Per-workgroup pointers and sizes.
template <int D>
struct AttnCtx {
  LaneOffsets<D> lo;      // per-lane LDS operand offsets
  DmaOffsets<D> dma;      // per-lane DMA source offsets
  int wave;               // wave index (uniform)
  const int8_t* kh;       // K codes of this head
  const uint8_t* vh;      // V codes of this head (channel-major)
  const float* ksh;       // k_scale of this head, offset to this lane's 64-key half
  int64_t npad;
  int ntiles;
  float log2_pscale;
};

// One tile `it` of the software pipeline.  On entry S0 holds group 0's S for tile it
// and P1 group 1's P of tile it-1 (not yet applied).  LDS: K tiles alternate between
// two buffers (tile t in K buffer t & 1), V tiles likewise.
//   phase A: matrix cores: S1 = QK(group 1, tile it); acc1 += P1(it-1) V(it-1)
//            VALU:          softmax of group 0, tile it -> P0
//   barrier: K(it+1), V(it) have landed; K(it), V(it-1) are no longer read
//            -> copies of K(it+2) and V(it+1) into the buffers just freed
//   phase B: matrix cores: acc0 += P0 V(it); S0 = QK(group 0, tile it+1)
//            VALU:          softmax of group 1, tile it -> P1
// For it = 0 the "previous" V buffer is zero-filled and P1 = 0, so phase A adds 0.
// For the last tile the QK of "tile it+1" reads a stale K buffer; its result is unused.
template <int D, bool MASKED>
__device__ __forceinline__ void pipeline_step(int it, const AttnCtx<D>& cx, uint8_t* smem, int lane,
                                              const v4i (&qfr)[G][D / 64], AttnState& st,
                                              float& ksc, int nvalid, v4i (&S0)[8], v4i (&S1)[8],
                                              v8i& P0, v8i& P1, v4f (&acc0)[D / 16],
                                              v4f (&acc1)[D / 16]) {
  // buffer t & 1 of K / V (plain offsets keep the LDS address space visible)
  uint8_t* const kcur = smem + (it & 1) * Lds<D>::KBYTES;
  uint8_t* const knxt = smem + ((it + 1) & 1) * Lds<D>::KBYTES;
  uint8_t* const vcur = smem + 2 * Lds<D>::KBYTES + (it & 1) * Lds<D>::VBYTES;
  uint8_t* const vprv = smem + 2 * Lds<D>::KBYTES + ((it + 1) & 1) * Lds<D>::VBYTES;
  const bool has_next = it + 1 < cx.ntiles;
  const float ksc_next = cx.ksh[2 * (has_next ? it + 1 : it)];

  // ---- phase A
  const float alpha0 = phase<D, MASKED, true>(kcur, qfr[1], S1, vprv, P1, acc1, S0, st.qf[0] * ksc,
                                              nvalid, cx.log2_pscale, st.m[0], st.lpart[0], P0, lane, cx.lo);
  materialize(P0, st.lpart[0]);
  rescale<D>(acc0, alpha0);

  __syncthreads();
  if (it + 2 < cx.ntiles) cx.dma.issue_k(cx.kh + (int64_t)(it + 2) * kKvTile * D, kcur, cx.wave);
  if (has_next) cx.dma.issue_v(cx.vh + (int64_t)(it + 1) * kKvTile, vprv, cx.wave);

  // ---- phase B
  const float alpha1 = phase<D, MASKED, false>(knxt, qfr[0], S0, vcur, P0, acc0, S1, st.qf[1] * ksc,
                                               nvalid, cx.log2_pscale, st.m[1], st.lpart[1], P1, lane, cx.lo);
  materialize(P1, st.lpart[1]);
  rescale<D>(acc1, alpha1);
  ksc = ksc_next;
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn(AttnArgs a) {
  // K tiles in two LDS buffers, V tiles in two more
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

  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  AttnCtx<D> cx{LaneOffsets<D>(lane), DmaOffsets<D>(uwave, lane, a.npad), uwave};
  cx.kh = a.k_i8 + bh * a.npad * D;
  cx.vh = a.v_f8 + bh * D * a.npad;
  cx.ksh = a.k_scale + bh * nblk + (g >> 1);
  cx.npad = a.npad;
  cx.ntiles = (a.N + kKvTile - 1) / kKvTile;
  cx.log2_pscale = a.log2_pscale;
  const int tail = a.N - (cx.ntiles - 1) * kKvTile;     // keys in the last tile (1..128)

  cx.dma.issue_k(cx.kh, smem, cx.wave);
  if (cx.ntiles > 1) cx.dma.issue_k(cx.kh + kKvTile * D, smem + Lds<D>::KBYTES, cx.wave);
  cx.dma.issue_v(cx.vh, smem + 2 * Lds<D>::KBYTES, cx.wave);
  {
    // zero the second V buffer: the first phase A multiplies it by P1 = 0
    v4i* z = (v4i*)(smem + 2 * Lds<D>::KBYTES + Lds<D>::VBYTES);
#pragma unroll
    for (int i = 0; i < Lds<D>::VBYTES / 16 / 256; ++i) z[threadIdx.x + 256 * i] = v4i{0, 0, 0, 0};
  }

  v4i qfr[G][D / 64];
  load_q<D>(a.q_i8 + bh * a.npad * D, qrow0, lane, qfr);
  AttnState st;
  v4f acc0[D / 16], acc1[D / 16];
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    st.qf[gq] = a.q_scale[bh * nblk + (qrow0 + 16 * gq) / kQuantBlock] * a.log2e_scale;
    st.m[gq] = -INFINITY;
    st.lpart[gq] = 0.0f;
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    acc0[dt] = v4f{0.f, 0.f, 0.f, 0.f};
    acc1[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  float ksc = cx.ksh[0];
  __syncthreads();

  v4i S0[8], S1[8];
  v8i P0, P1 = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  qk_group<D>(smem, qfr[0], lane, S0);
  const int nfull = (tail == kKvTile) ? cx.ntiles : cx.ntiles - 1;   // tiles without masking
  for (int it = 0; it < nfull; ++it)
    pipeline_step<D, false>(it, cx, smem, lane, qfr, st, ksc, kKvTile, S0, S1, P0, P1, acc0, acc1);
  if (nfull < cx.ntiles)
    pipeline_step<D, true>(nfull, cx, smem, lane, qfr, st, ksc, tail, S0, S1, P0, P1, acc0, acc1);
  // group 1's P of the last tile
  pv_group<D>(smem + 2 * Lds<D>::KBYTES + ((cx.ntiles - 1) & 1) * Lds<D>::VBYTES, P1, lane, acc1);

  // epilogue: total row sum over the 4 lanes of each query, normalise, V scale, bf16
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  uint16_t* ob = a.out + (int64_t)b * a.so.b + (int64_t)h * a.so.h;
  const float* vsh = a.v_scale + bh * D;
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    const float l = sum_over_lane_groups(st.lpart[gq]);
    const float rl = 1.0f / l;
    const int qrow = qrow0 + 16 * gq + r;
    v4f (&acc)[D / 16] = gq == 0 ? acc0 : acc1;
    if (qrow < a.N) {
      uint16_t* orow = ob + (int64_t)qrow * a.so.n;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int c0 = 16 * dt + 4 * g;
        uint32_t h0 = f32_to_bf16_rne(acc[dt][0] * vsh[c0 + 0] * rl);
        uint32_t h1 = f32_to_bf16_rne(acc[dt][1] * vsh[c0 + 1] * rl);
        uint32_t h2 = f32_to_bf16_rne(acc[dt][2] * vsh[c0 + 2] * rl);
        uint32_t h3 = f32_to_bf16_rne(acc[dt][3] * vsh[c0 + 3] * rl);
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
  const int64_t ld = (int64_t)n_kv_tiles * kKvTile;
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    v4i S[8];
    qk_group<D>(klds, qfr[gq], lane, S);
    const int64_t row = (int64_t)blockIdx.y * kBlockM + wave * (G * 16) + 16 * gq + r;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_out[row * ld + (int64_t)blockIdx.x * kKvTile + 32 * g + 4 * kt + i] = S[kt][i];
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
