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
// Three kernels: code sums per 64-token block (reads the INT8 operands once); the
// importance matrix of each head (8 query blocks x 32 key tiles per workgroup, code
// sums staged in LDS as int16 pairs for v_dot2_i32_i16); and the selection of each
// query block by exact ranks (rank of J = tiles more important than J, or as important
// with a lower index; kept iff rank < k), compacted in ascending tile order with a
// workgroup prefix sum.  (A bitonic sort in LDS measured slower: its barrier per stage
// costs more than the independent rank loops at 36 and 512 tiles.)
#include "sage_internal.h"

namespace sage {

constexpr int kSelThreads = 256;
constexpr int kImpQb = 8;       // query blocks per importance workgroup
constexpr int kImpKt = 32;      // key tiles per importance workgroup
constexpr int kTilesPerBlock = kKvTile / kQuantBlock;   // scale blocks per tile (2)
static_assert(kBlockM == kKvTile, "query blocks and key tiles have the same size");
static_assert(kImpQb * kImpKt == kSelThreads, "one importance per thread");

// sums[z][bh][blk][c] = sum over the 64 rows of block blk of the codes of channel c,
// z = 0 for Q, 1 for K.  Rows past N are zero in the padded operands.
template <int D>
__global__ __launch_bounds__(kSelThreads) void k_block_sums(const int8_t* __restrict__ q_i8,
                                                           const int8_t* __restrict__ k_i8, int64_t npad,
                                                           int64_t n_bh, int32_t* __restrict__ sums) {
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
    sums[(((int64_t)z * n_bh + bh) * nblk + blk) * D + t] = s;
  }
}

// imp[bh][I][J] for I in [8*blockIdx.y, +8) and J in [32*blockIdx.x, +32): thread
// (i = t / 32, j = t % 32).  A code sum is at most 64 * 127 = 8128 in magnitude, so the
// sums are staged as int16 channel pairs and the dot products run on v_dot2_i32_i16:
// 16 products (each below 2^26) per int32 partial, the partials summed in int64.
template <int D>
__global__ __launch_bounds__(kSelThreads) void k_tile_importance(const int32_t* __restrict__ sums,
                                                                const float* __restrict__ q_scale,
                                                                const float* __restrict__ k_scale,
                                                                int N, int64_t npad, int64_t n_bh,
                                                                double* __restrict__ imp) {
  constexpr int W = D / 2;                     // int16 pairs per row
  constexpr int P = W + 4;                     // LDS row pitch of the query rows (16-byte aligned)
  constexpr int CH = W / 4;                    // 16-byte chunks per key row
  // Key rows are unpadded and their 16-byte chunks XOR-swizzled by key tile, so the 32
  // tiles a wave reads at once spread over the banks (at most 2 lanes per bank group).
  auto ksw = [](int row) { return (row / kTilesPerBlock) & (CH - 1); };
  static_assert(kQuantBlock * 127 < 32768, "code sums fit int16");
  __shared__ __attribute__((aligned(16))) int qa[kImpQb * kTilesPerBlock][P];
  __shared__ __attribute__((aligned(16))) int kb[kImpKt * kTilesPerBlock][W];
  const int64_t bh = blockIdx.z, nblk = npad / kQuantBlock;
  const int nt = (int)(npad / kKvTile);
  const int I0 = blockIdx.y * kImpQb, J0 = blockIdx.x * kImpKt;
  const int32_t* qs_sums = sums + bh * nblk * D;
  const int32_t* ks_sums = sums + (n_bh + bh) * nblk * D;
  auto pack = [](int2 x) { return (x.x & 0xffff) | (x.y << 16); };
  // stage the code sums of the 16 query and 64 key scale blocks (zeros past the end);
  // the trip counts are constants, so every load is issued before the first store
  static_assert((kImpQb * kTilesPerBlock * W) % kSelThreads == 0 && (kImpKt * kTilesPerBlock * W) % kSelThreads == 0,
                "whole staging passes");
#pragma unroll
  for (int e = threadIdx.x; e < kImpQb * kTilesPerBlock * W; e += kSelThreads) {
    const int row = e / W, w = e % W;
    const int64_t blk = (int64_t)I0 * kTilesPerBlock + row;
    qa[row][w] = blk < nblk ? pack(*(const int2*)(qs_sums + blk * D + 2 * w)) : 0;
  }
#pragma unroll
  for (int e = threadIdx.x; e < kImpKt * kTilesPerBlock * W; e += kSelThreads) {
    const int row = e / W, w = e % W;
    const int64_t blk = (int64_t)J0 * kTilesPerBlock + row;
    kb[row][4 * ((w / 4) ^ ksw(row)) + w % 4] = blk < nblk ? pack(*(const int2*)(ks_sums + blk * D + 2 * w)) : 0;
  }
  __syncthreads();
  const int i = threadIdx.x / kImpKt, j = threadIdx.x % kImpKt;
  const int I = I0 + i, J = J0 + j;
  if (I >= nt || J >= nt) return;
  typedef short v2s __attribute__((ext_vector_type(2)));
  double tab[kTilesPerBlock][kTilesPerBlock];
#pragma unroll
  for (int a = 0; a < kTilesPerBlock; ++a) {
#pragma unroll
    for (int b = 0; b < kTilesPerBlock; ++b) {
      const int64_t ablk = (int64_t)I * kTilesPerBlock + a, bblk = (int64_t)J * kTilesPerBlock + b;
      const int* x = qa[i * kTilesPerBlock + a];
      const int yrow = j * kTilesPerBlock + b;
      const int* y = kb[yrow];
      int64_t dot = 0;
#pragma unroll
      for (int w0 = 0; w0 < W; w0 += 8) {
        const int4 x0 = *(const int4*)(x + w0), x1 = *(const int4*)(x + w0 + 4);
        const int4 y0 = *(const int4*)(y + 4 * ((w0 / 4) ^ ksw(yrow)));
        const int4 y1 = *(const int4*)(y + 4 * ((w0 / 4 + 1) ^ ksw(yrow)));
        const int xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        const int ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
        int part = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          part = __builtin_amdgcn_sdot2(__builtin_bit_cast(v2s, xs[u]), __builtin_bit_cast(v2s, ys[u]), part, false);
        dot += part;
      }
      tab[a][b] = (ablk < nblk && bblk < nblk)
                      ? ((double)q_scale[bh * nblk + ablk] * (double)k_scale[bh * nblk + bblk]) * (double)dot
                      : 0.0;
    }
  }
  const int nI = min(N, (I + 1) * kBlockM) - I * kBlockM;
  const int nJ = min(N, (J + 1) * kKvTile) - J * kKvTile;
  imp[(bh * nt + I) * nt + J] = ((tab[0][0] + tab[0][1]) + (tab[1][0] + tab[1][1])) / (double)(nI * nJ);
}

// Kept tiles of query block blockIdx.x of head blockIdx.y: tile_list row = the keep
// tiles of lowest rank, ascending; tile_count = keep.
__global__ __launch_bounds__(kSelThreads) void k_tile_select(const double* __restrict__ imp, int nt, int keep,
                                                            int32_t* __restrict__ tile_count,
                                                            int32_t* __restrict__ tile_list) {
  __shared__ double v[kMaxSparseTiles];
  __shared__ int scan[kSelThreads];
  const int64_t row = (int64_t)blockIdx.y * nt + blockIdx.x;
  const double* src = imp + row * nt;
  for (int j = threadIdx.x; j < nt; j += kSelThreads) v[j] = src[j];
  __syncthreads();
  // thread t owns the contiguous tiles [t*per, t*per + per)
  const int per = (nt + kSelThreads - 1) / kSelThreads;
  const int j0 = threadIdx.x * per, j1 = min(nt, j0 + per);
  uint32_t kept = 0;                           // bit (j - j0) set when tile j is kept
  for (int j = j0; j < j1; ++j) {
    const double x = v[j];
    int rank = 0;
    for (int jj = 0; jj < nt; ++jj) {
      const double y = v[jj];
      rank += (y > x || (y == x && jj < j)) ? 1 : 0;
    }
    if (rank < keep) kept |= 1u << (j - j0);
  }
  // exclusive prefix sum of the kept counts over the threads
  const int cnt = __popc(kept);
  scan[threadIdx.x] = cnt;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {
    const int add = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
    __syncthreads();
    scan[threadIdx.x] += add;
    __syncthreads();
  }
  int pos = scan[threadIdx.x] - cnt;
  int32_t* dst = tile_list + row * nt;
  for (int j = j0; j < j1; ++j)
    if (kept & (1u << (j - j0))) dst[pos++] = j;
  if (threadIdx.x == 0) tile_count[row] = keep;
}

template <int D>
static void launch_select_d(const SelectArgs& a, hipStream_t s) {
  const int64_t nblk = a.npad / kQuantBlock, n_bh = (int64_t)a.B * a.H;
  const int nt = (int)(a.npad / kKvTile);
  hipLaunchKernelGGL(k_block_sums<D>, dim3((unsigned)nblk, (unsigned)n_bh, 2), dim3(kSelThreads), 0, s,
                     a.q_i8, a.k_i8, a.npad, n_bh, a.sums);
  hipLaunchKernelGGL(k_tile_importance<D>,
                     dim3((nt + kImpKt - 1) / kImpKt, (nt + kImpQb - 1) / kImpQb, (unsigned)n_bh),
                     dim3(kSelThreads), 0, s, a.sums, a.q_scale, a.k_scale, a.N, a.npad, n_bh, a.imp);
  hipLaunchKernelGGL(k_tile_select, dim3(nt, (unsigned)n_bh), dim3(kSelThreads), 0, s, a.imp, nt, a.keep,
                     a.tile_count, a.tile_list);
}

hipError_t launch_block_select(const SelectArgs& a, hipStream_t s) {
  if (a.d == 64) launch_select_d<64>(a, s);
  else launch_select_d<128>(a, s);
  return hipGetLastError();
}

template __global__ void k_block_sums<64>(const int8_t* __restrict__, const int8_t* __restrict__, int64_t,
                                          int64_t, int32_t* __restrict__);
template __global__ void k_block_sums<128>(const int8_t* __restrict__, const int8_t* __restrict__, int64_t,
                                           int64_t, int32_t* __restrict__);
template __global__ void k_tile_importance<64>(const int32_t* __restrict__, const float* __restrict__,
                                               const float* __restrict__, int, int64_t, int64_t,
                                               double* __restrict__);
template __global__ void k_tile_importance<128>(const int32_t* __restrict__, const float* __restrict__,
                                                const float* __restrict__, int, int64_t, int64_t,
                                                double* __restrict__);

}  // namespace sage
