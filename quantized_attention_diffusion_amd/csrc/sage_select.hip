// Block-sparse key tiles for gfx950: which key tiles each query block visits.
//
// The sd114.wiki page "ComfyUI-sol-attn" (核心亮点, item 4) describes a sparse attention
// whose value tau moves over the sampling steps, sparse early and dense late, without a
// selection rule.  The rule used here: tau is the density, each block of 128 queries
// keeps the k = max(1, min(T, ceil(tau * T))) key tiles of largest importance, the
// importance of tile J for query block I being the mean over their valid (query, key)
// pairs of the dequantised product q_scale * k_scale * S.  The 64-token scale blocks a
// of I and b of J share one scale each, so that mean follows exactly from per-channel
// sums A_a, B_b of the INT8 codes:
//     t_ab = (qs_a * ks_b) * <A_a, B_b>,  imp = ((t_00 + t_01) + (t_10 + t_11)) / (n_I * n_J)
// in fp64 with every operation rounded once (the products of fp32 scales are exact,
// the integer dot products are exact in int64), so any implementation that follows
// the formula takes the same decisions.  Ties go to the lower tile index.
//
// Three kernels: code sums per 64-token block (reads the INT8 operands once; each sum
// stored as two int8 digits); the importance matrix of each head (32 query blocks x 32
// key tiles per workgroup, the dot products of the digits on INT8 matrix cores); and
// the selection of each query block, on order-preserving 64-bit keys of the
// importances: exact ranks up to 128 tiles, above that an MSB-first radix select of
// the k-th largest key, then the tiles above it and the first tiles equal to it; the
// kept tiles are compacted in ascending order with a workgroup prefix sum.  (A bitonic
// sort in LDS measured slower.)
#include "sage_internal.h"

namespace sage {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kSelThreads = 256;
constexpr int kImpTiles = 32;   // query and key tiles per importance workgroup
constexpr int kRankMaxTiles = 128;           // selection by ranks up to this many tiles
static_assert(kRankMaxTiles <= kSelThreads, "one tile per thread in the rank selection");
constexpr int kTilesPerBlock = kKvTile / kQuantBlock;   // scale blocks per tile (2)
static_assert(kBlockM == kKvTile, "query blocks and key tiles have the same size");
constexpr int kImpRows = kImpTiles * kTilesPerBlock;   // scale blocks a side (64)

// The sum s of the codes of channel c over the 64 rows of block blk (rows past N are zero
// in the padded operands), stored as its two int8 digits: |s| <= 64*127 < 64*128, so
// s = 128*h + l exactly with h = s >> 7 in [-64, 63] and l = s & 127 in [0, 127];
// digits[z][bh][blk][0][c] = h, digits[z][bh][blk][1][c] = l, z = 0 for Q, 1 for K.
template <int D>
__global__ __launch_bounds__(kSelThreads) void k_block_sums(const int8_t* __restrict__ q_i8,
                                                           const int8_t* __restrict__ k_i8, int64_t npad,
                                                           int64_t n_bh, int8_t* __restrict__ digits) {
  static_assert(kQuantBlock * 127 < 64 * 128, "a code sum splits into two int8 digits");
  constexpr int TPR = D / 16;                  // threads per row, 16 codes each
  constexpr int RPI = kSelThreads / TPR;       // rows per pass
  constexpr int PASSES = kQuantBlock / RPI;
  __shared__ int part[RPI][D + 1];
  const int blk = blockIdx.x, z = blockIdx.z;
  const int64_t bh = blockIdx.y, nblk = npad / kQuantBlock;
  const int8_t* src = (z == 0 ? q_i8 : k_i8) + (bh * npad + (int64_t)blk * kQuantBlock) * D;
  const int t = threadIdx.x, cg = t % TPR, r = t / TPR;
  int acc[16] = {};
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int4 w = *(const int4*)(src + (int64_t)(p * RPI + r) * D + cg * 16);
    const int words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[4 * j + b] += (words[j] << (24 - 8 * b)) >> 24;   // sign-extended byte b
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) part[r][cg * 16 + i] = acc[i];
  __syncthreads();
  if (t < D) {
    int s = 0;
    for (int i = 0; i < RPI; ++i) s += part[i][t];
    int8_t* dst = digits + (((int64_t)z * n_bh + bh) * nblk + blk) * 2 * D;
    dst[t] = (int8_t)(s >> 7);
    dst[D + t] = (int8_t)(s & 127);
  }
}

// imp[bh][I][J] for the tiles I in [32*blockIdx.y, +32) and J in [32*blockIdx.x, +32).
// The dot products G[a][b] = <A_a, B_b> of the workgroup's 64 query and 64 key scale
// blocks run on the INT8 matrix cores on the digits of the code sums (s = 128*h + l):
// G = 16384*<h,h'> + 128*(<h,l'> + <l,h'>) + <l,l'>, four INT8 products, each an exact
// int32 sum (at most 128*127*127 in magnitude), combined in int64.
// Wave w computes the 16 query blocks 16w.. against the 64 key blocks (four 16x16
// tiles); lane l then holds G[16w + 4g + i][16c + r] (g = l/16, r = l%16) and pairs
// with lane l^1, which holds the other key block of the same tile, for the fp64 sum.
template <int D>
__global__ __launch_bounds__(kSelThreads) void k_tile_importance(const int8_t* __restrict__ digits,
                                                                const float* __restrict__ q_scale,
                                                                const float* __restrict__ k_scale,
                                                                int N, int64_t npad, int64_t n_bh,
                                                                double* __restrict__ imp) {
  constexpr int CH = D / 16;                   // 16-byte chunks per staged row
  static_assert(kSelThreads == 4 * 64 && kImpRows == 64, "four waves of 16 query blocks, 64 key blocks");
  // [operand: Q, K][digit: h, l][row][D bytes]; chunks XOR-swizzled by row
  __shared__ __attribute__((aligned(16))) int8_t parts[2][2][kImpRows][D];
  auto swz = [](int row, int ch) { return ch ^ (row & (CH - 1)); };
  const int64_t bh = blockIdx.z, nblk = npad / kQuantBlock;
  const int nt = (int)(npad / kKvTile);
  const int I0 = blockIdx.y * kImpTiles, J0 = blockIdx.x * kImpTiles;
  // staging: one 16-byte chunk of one digit row per step
  static_assert((2 * 2 * kImpRows * CH) % kSelThreads == 0, "whole staging passes");
#pragma unroll
  for (int e = threadIdx.x; e < 2 * 2 * kImpRows * CH; e += kSelThreads) {
    const int op = e / (2 * kImpRows * CH), dg = (e / (kImpRows * CH)) % 2, row = (e / CH) % kImpRows, ch = e % CH;
    const int64_t blk = (int64_t)(op == 0 ? I0 : J0) * kTilesPerBlock + row;
    i32x4 x = {0, 0, 0, 0};
    if (blk < nblk) x = *(const i32x4*)(digits + ((((int64_t)op * n_bh + bh) * nblk + blk) * 2 + dg) * D + 16 * ch);
    *(i32x4*)&parts[op][dg][row][16 * swz(row, ch)] = x;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
  i32x4 acc[4][4];                               // [key tile c][product hh, hl, lh, ll]
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[c][p] = i32x4{0, 0, 0, 0};
  const int arow = 16 * wave + r;
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk) {
    const int ch = 4 * kk + g;                 // channels 64kk + 16g .. +15
    const i32x4 ah = *(const i32x4*)&parts[0][0][arow][16 * swz(arow, ch)];
    const i32x4 al = *(const i32x4*)&parts[0][1][arow][16 * swz(arow, ch)];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int brow = 16 * c + r;
      const i32x4 bhv = *(const i32x4*)&parts[1][0][brow][16 * swz(brow, ch)];
      const i32x4 blv = *(const i32x4*)&parts[1][1][brow][16 * swz(brow, ch)];
      acc[c][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah, bhv, acc[c][0], 0, 0, 0);
      acc[c][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah, blv, acc[c][1], 0, 0, 0);
      acc[c][2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al, bhv, acc[c][2], 0, 0, 0);
      acc[c][3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al, blv, acc[c][3], 0, 0, 0);
    }
  }
  // tile (I, J): query blocks 2I + a (registers 2rp + a), key blocks 2J + b (b = r & 1)
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int J = J0 + (16 * c + r) / 2, b = r & 1;
#pragma unroll
    for (int rp = 0; rp < 2; ++rp) {
      const int I = I0 + 8 * wave + 2 * g + rp;
      const bool valid = I < nt && J < nt;     // the same for both lanes of a pair
      double t[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int i = 2 * rp + a;
        const int64_t G = 16384 * (int64_t)acc[c][0][i] + 128 * ((int64_t)acc[c][1][i] + (int64_t)acc[c][2][i]) +
                          (int64_t)acc[c][3][i];
        const int64_t ablk = (int64_t)I * kTilesPerBlock + a, bblk = (int64_t)J * kTilesPerBlock + b;
        t[a] = valid ? ((double)q_scale[bh * nblk + ablk] * (double)k_scale[bh * nblk + bblk]) * (double)G : 0.0;
      }
      // the partner lane holds t[a] for the other key block of the tile
      const double o0 = __shfl_xor(t[0], 1), o1 = __shfl_xor(t[1], 1);
      if (valid && b == 0) {
        const int nI = min(N, (I + 1) * kBlockM) - I * kBlockM;
        const int nJ = min(N, (J + 1) * kKvTile) - J * kKvTile;
        imp[(bh * nt + I) * nt + J] = ((t[0] + o0) + (t[1] + o1)) / (double)(nI * nJ);
      }
    }
  }
}

// Order-preserving unsigned image of an fp64 value: a larger value gives a larger key,
// and both zeros give the key of +0.0, as they compare equal in fp64.  (Importances are
// finite: no NaN occurs.)
__device__ __forceinline__ uint64_t order_key(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x == 0.0 ? 0.0 : x);
  return (b >> 63) ? ~b : (b | (1ull << 63));
}

// Exclusive prefix sum over the workgroup of one value per thread: shuffles within each
// wave, then the totals of the preceding waves.
__device__ __forceinline__ int workgroup_exclusive_sum(int x, int* wave_tot) {
  constexpr int kWaves = kSelThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) before += w < wave ? wave_tot[w] : 0;
  return before + inc - x;
}

// Kept tiles of query block blockIdx.x of head blockIdx.y: tile_list row = the keep
// most important tiles, equal importances taken in ascending tile order, listed
// ascending; tile_count = keep.  Two exact methods, by the number of tiles:
// - up to kRankMaxTiles: ranks.  Thread t holds tile t; its rank is the number of tiles
//   with a larger key, or an equal key and a lower index; it is kept iff rank < keep.
// - more: the keep-th largest order key is found by an MSB-first radix select, 8 bits
//   a pass: a histogram of the current byte over the keys that match the bytes fixed
//   so far, then the byte whose bin holds the keep-th largest of them.  The tiles whose
//   key is larger are kept, and of those equal to it the first `need` in tile order.
// (Measured, one query block per workgroup, 24 heads: ranks 4.9 / 20.6 / 456 us and the
// radix select 8.1 / 22.7 / 102 us at 36 / 128 / 512 tiles.)
__global__ __launch_bounds__(kSelThreads) void k_tile_select(const double* __restrict__ imp, int nt, int keep,
                                                            int32_t* __restrict__ tile_count,
                                                            int32_t* __restrict__ tile_list) {
  static_assert(kSelThreads == 256, "one histogram bin per thread");
  extern __shared__ uint64_t key[];            // nt keys (dynamic LDS: more workgroups per CU at small nt)
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel[2];                  // chosen byte, candidates above its bin
  __shared__ int wave_tot[kSelThreads / 64];
  const int t = threadIdx.x, lane = t & 63;
  const int64_t row = (int64_t)blockIdx.y * nt + blockIdx.x;
  const double* src = imp + row * nt;
  for (int j = t; j < nt; j += kSelThreads) key[j] = order_key(src[j]);
  int32_t* dst = tile_list + row * nt;
  if (t == 0) tile_count[row] = keep;
  if (nt <= kRankMaxTiles) {
    __syncthreads();
    bool kept = false;
    if (t < nt) {
      const uint64_t x = key[t];
      int rank = 0;
      for (int jj = 0; jj < nt; ++jj) {
        const uint64_t y = key[jj];
        rank += (y > x || (y == x && jj < t)) ? 1 : 0;
      }
      kept = rank < keep;
    }
    const int pos = workgroup_exclusive_sum(kept ? 1 : 0, wave_tot);
    if (kept) dst[pos] = t;
    return;
  }
  uint64_t prefix = 0, mask = 0;
  int need = keep;                             // 1 <= need <= number of candidates
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[t] = 0;
    __syncthreads();                           // keys stored, last pass's sel read
    for (int j = t; j < nt; j += kSelThreads) {
      const uint64_t k = key[j];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1u);
    }
    __syncthreads();
    if (t < 64) {
      // lane l holds bins 4l .. 4l+3; ge_b = candidates with byte >= b.  The chosen
      // byte b has ge_b >= need > ge_b - hist[b].
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      const uint32_t own = h0 + h1 + h2 + h3;
      uint32_t suf = own;                      // sum over lanes >= lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(suf, off);
        if (lane + off < 64) suf += o;
      }
      const uint32_t above = suf - own;
      const uint32_t ge3 = above + h3, ge2 = ge3 + h2, ge1 = ge2 + h1, ge0 = ge1 + h0;
      const uint32_t n = (uint32_t)need;
      if (ge3 >= n && above < n) { sel[0] = 4 * lane + 3; sel[1] = above; }
      else if (ge2 >= n && ge3 < n) { sel[0] = 4 * lane + 2; sel[1] = ge3; }
      else if (ge1 >= n && ge2 < n) { sel[0] = 4 * lane + 1; sel[1] = ge2; }
      else if (ge0 >= n && ge1 < n) { sel[0] = 4 * lane; sel[1] = ge1; }
    }
    __syncthreads();
    need -= (int)sel[1];
    prefix |= (uint64_t)sel[0] << shift;
    mask |= 255ull << shift;
  }
  // prefix is the keep-th largest key; keep the larger keys and the first `need` equal ones
  const int per = (nt + kSelThreads - 1) / kSelThreads;
  const int j0 = t * per, j1 = min(nt, j0 + per);
  int gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    gt += key[j] > prefix ? 1 : 0;
    eq += key[j] == prefix ? 1 : 0;
  }
  const int packed = workgroup_exclusive_sum(gt | (eq << 16), wave_tot);   // counts < 2^13
  const int gt_before = packed & 0xffff;
  int eq_seen = packed >> 16;
  int pos = gt_before + min(eq_seen, need);
  for (int j = j0; j < j1; ++j) {
    const uint64_t k = key[j];
    if (k > prefix) {
      dst[pos++] = j;
    } else if (k == prefix) {
      if (eq_seen < need) dst[pos++] = j;
      ++eq_seen;
    }
  }
}

template <int D>
static void launch_select_d(const SelectArgs& a, hipStream_t s) {
  const int64_t nblk = a.npad / kQuantBlock, n_bh = (int64_t)a.B * a.H;
  const int nt = (int)(a.npad / kKvTile);
  hipLaunchKernelGGL(k_block_sums<D>, dim3((unsigned)nblk, (unsigned)n_bh, 2), dim3(kSelThreads), 0, s,
                     a.q_i8, a.k_i8, a.npad, n_bh, a.digits);
  hipLaunchKernelGGL(k_tile_importance<D>,
                     dim3((nt + kImpTiles - 1) / kImpTiles, (nt + kImpTiles - 1) / kImpTiles, (unsigned)n_bh),
                     dim3(kSelThreads), 0, s, a.digits, a.q_scale, a.k_scale, a.N, a.npad, n_bh, a.imp);
  hipLaunchKernelGGL(k_tile_select, dim3(nt, (unsigned)n_bh), dim3(kSelThreads), (unsigned)(nt * sizeof(uint64_t)), s,
                     a.imp, nt, a.keep, a.tile_count, a.tile_list);
}

hipError_t launch_block_select(const SelectArgs& a, hipStream_t s) {
  if (a.d == 64) launch_select_d<64>(a, s);
  else launch_select_d<128>(a, s);
  return hipGetLastError();
}

template __global__ void k_block_sums<64>(const int8_t* __restrict__, const int8_t* __restrict__, int64_t,
                                          int64_t, int8_t* __restrict__);
template __global__ void k_block_sums<128>(const int8_t* __restrict__, const int8_t* __restrict__, int64_t,
                                           int64_t, int8_t* __restrict__);
template __global__ void k_tile_importance<64>(const int8_t* __restrict__, const float* __restrict__,
                                               const float* __restrict__, int, int64_t, int64_t,
                                               double* __restrict__);
template __global__ void k_tile_importance<128>(const int8_t* __restrict__, const float* __restrict__,
                                                const float* __restrict__, int, int64_t, int64_t,
                                                double* __restrict__);

}  // namespace sage
