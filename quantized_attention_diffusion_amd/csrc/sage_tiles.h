// Index maps of the attention kernel's LDS tiles: the XOR swizzles, the per-lane
// operand read offsets and the per-lane LDS DMA source offsets, plus the workgroup
// remap.  Plain integer functions for host and device, so that the host can check
// that every copy stays inside its tile, every LDS byte is written once and every
// operand read returns the keys and channels the matrix-core layouts need.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sage_internal.h"

namespace sage {

// LDS tiles are unpadded and XOR-swizzled at 16-byte granularity so that the 128-bit
// operand reads run without bank conflicts:
//   K tile [128 keys][D bytes]:    physical chunk = chunk ^ kswz(key)
//   V tile [D channels][128 keys]: physical chunk = chunk ^ vswz(channel)
// A K read touches keys 32*(r/4) + 4*kt + r%4 (r = lane % 16), i.e. varies key bits
// 0, 1, 5, 6 across the wave; a V read touches channels 16*dt + r.  The K swizzle is a
// linear map of those four key bits onto the three chunk bits; gfx950's bank grouping
// for 128-bit reads is not documented, so it was chosen by timing all 4096 such maps on
// the exact K read pattern (about a third run at the conflict-free rate; the obvious
// maps for 16- or 32-lane passes do not).  The V swizzle runs at the contiguous rate.
template <int D>
__host__ __device__ __forceinline__ int kswz(int key) {
  if constexpr (D == 128)
    return ((key ^ (key >> 1) ^ (key >> 6)) & 1) | (((key ^ (key >> 5)) & 1) << 1) | (((key >> 6) & 1) << 2);
  else
    return (key >> 5) & 3;
}
__host__ __device__ __forceinline__ int vswz(int ch) { return ((ch ^ (ch >> 3)) & 1) | (ch & 6); }
// bf16 V tile [D channels][128 keys], 256 bytes per channel: physical chunk = chunk ^
// v16swz(channel).  A read touches channels 16*dt + r and chunks 4g + s; the map is
// linear in channel bits 0-3 and was chosen by timing all 2^16 such maps on this
// pattern (about 30% run at the conflict-free rate, the plain XOR with the channel at
// half of it).
__host__ __device__ __forceinline__ int v16swz(int ch) {
  const int b0 = ch & 1, b1 = (ch >> 1) & 1, b2 = (ch >> 2) & 1, b3 = (ch >> 3) & 1;
  return b1 | ((b1 ^ b2 ^ b3) << 1) | ((b1 ^ b3) << 2) | ((b0 ^ b1 ^ b2 ^ b3) << 3);
}

template <int D>
struct Lds {
  static constexpr int KBYTES = kKvTile * D;       // one K tile
  static constexpr int VBYTES = D * kKvTile;       // one e4m3 V tile
  static constexpr int V16BYTES = D * kKvTile * 2; // one bf16 V tile
};

// The tile key that row j of K sub-tile kt (a 16-row matrix-core operand) holds.  With
// it, lane (r, g) of the S^T = K.Q^T product finds in register i of sub-tile kt the
// key 32g + 4kt + i of its query r: 32 consecutive keys, all in one 64-key scale block.
__host__ __device__ __forceinline__ int k_row_key(int kt, int j) { return 32 * (j >> 2) + 4 * kt + (j & 3); }

// LDS byte offset of lane `lane`'s 16-byte K operand read of sub-tile 0, 64-byte
// channel slice kk (sub-tile kt adds kt * 4 * D): row r = lane % 16 of the operand,
// channel bytes 64kk + 16g .. +15 (g = lane / 16).  The swizzle depends only on key
// bits 0, 1, 5 and 6, which the sub-tile offset leaves alone.
template <int D>
__host__ __device__ __forceinline__ int k_read_offset(int lane, int kk) {
  const int r = lane & 15, g = lane >> 4;
  const int key = k_row_key(0, r);
  return key * D + 16 * ((4 * kk + g) ^ kswz<D>(key));
}

// LDS byte offset of lane `lane`'s V operand read, half h, channel tile 0 (channel
// tile dt adds dt * 16 * 128): channel r, keys 32g + 16h .. +15.
__host__ __device__ __forceinline__ int v_read_offset(int lane, int h) {
  const int r = lane & 15, g = lane >> 4;
  return r * kKvTile + 16 * ((2 * g + h) ^ vswz(r));
}

// bf16 V: step s of channel tile 0 (tile dt adds dt * 16 * 256): channel r, keys
// 32g + 8s .. +7.
__host__ __device__ __forceinline__ int v16_read_offset(int lane, int s) {
  const int r = lane & 15, g = lane >> 4;
  return r * 256 + 16 * ((4 * g + s) ^ v16swz(r));
}

// LDS DMA copies (buffer_load_dwordx4 ... lds): instruction j of wave w writes lane
// i's 16 bytes at LDS byte (w * PER_WAVE + j) * 1024 + 16 * i of the tile, so the
// swizzle is applied by choosing which global chunk lane i reads.
template <int D> struct DmaShape {
  static constexpr int KPW = Lds<D>::KBYTES / 1024 / kWaves;     // K copies per wave
  static constexpr int VPW = Lds<D>::VBYTES / 1024 / kWaves;     // e4m3 V copies per wave
  static constexpr int V16PW = Lds<D>::V16BYTES / 1024 / kWaves; // bf16 V copies per wave
};
__host__ __device__ __forceinline__ int dma_lds_offset(int wave, int j, int per_wave, int lane) {
  return (wave * per_wave + j) * 1024 + 16 * lane;
}

// Source byte offset, relative to the tile's first key, of K copy j of wave w, lane i
// (K rows of D bytes).
template <int D>
__host__ __device__ __forceinline__ uint32_t k_dma_src(int wave, int j, int lane) {
  const int pos = dma_lds_offset(wave, j, DmaShape<D>::KPW, lane);
  const int key = pos / D, pc = (pos % D) / 16;
  return (uint32_t)(key * D + (pc ^ kswz<D>(key)) * 16);
}
// e4m3 V (channel-major rows of npad bytes): relative to the tile's first key column.
template <int D>
__host__ __device__ __forceinline__ uint32_t v_dma_src(int wave, int j, int lane, int64_t npad) {
  const int pos = dma_lds_offset(wave, j, DmaShape<D>::VPW, lane);
  const int ch = pos / kKvTile, pc = (pos % kKvTile) / 16;
  return (uint32_t)(ch * npad + (pc ^ vswz(ch)) * 16);
}
// bf16 V (channel-major rows of 2 * npad bytes).
template <int D>
__host__ __device__ __forceinline__ uint32_t v16_dma_src(int wave, int j, int lane, int64_t npad) {
  const int pos = dma_lds_offset(wave, j, DmaShape<D>::V16PW, lane);
  const int ch = pos / 256, pc = (pos % 256) / 16;
  return (uint32_t)(ch * npad * 2 + (pc ^ v16swz(ch & 15)) * 16);
}

// ---- 32x32 matrix-core layout (d = 128): one group of 32 queries per wave ----
// S^T = K.Q^T on v_mfma_i32_32x32x32_i8 over four 32-key sub-tiles kt: lane l holds
// query n = l % 32 and, in register i = 4jj + t of sub-tile kt, output row
// 8jj + 4h + t (h = l / 32).  Row j of sub-tile kt is mapped to the tile key
// k32_row_key(kt, j), so lane (n, h) holds in sub-tiles 2ps and 2ps + 1 the 32
// consecutive keys 64ps + 32h .. +31 (ps = 0, 1: the tile's two 64-key scale blocks),
// register i of sub-tile 2ps + u being key 64ps + 32h + 16u + i: exactly the k bytes
// 0 .. 31 of lane (n, h)'s P operand of O^T = V^T.P^T on
// v_mfma_scale_f32_32x32x64_f8f6f4 over the same 64 keys.
__host__ __device__ __forceinline__ int k32_row_key(int kt, int j) {
  return 64 * (kt >> 1) + 32 * ((j >> 2) & 1) + 16 * (kt & 1) + 4 * (j >> 3) + (j & 3);
}
// Swizzles of the 32x32 operand reads (K tile [128 keys][128 B], V tile [128 channels]
// [128 B]): a K read touches keys k32_row_key(kt, 0 .. 31), which vary key bits 0-3 and
// 5, at chunk 2kk + h; a V read touches channels 32dt + 0 .. 31 at chunk 4ps + 2h +
// half.  Both maps were chosen by timing all 2^15 linear maps of those five row bits
// onto the three chunk bits on these read patterns (about one in eight runs at the
// conflict-free rate); these are among the fastest.
__host__ __device__ __forceinline__ int kswz32(int key) {
  return ((key >> 5) & 1) | ((((key >> 1) ^ (key >> 3)) & 1) << 1) | (((key >> 2) & 1) << 2);
}
__host__ __device__ __forceinline__ int vswz32(int ch) {
  return ((ch >> 3) & 1) | ((((ch >> 1) ^ (ch >> 3)) & 1) << 1) | ((((ch >> 2) ^ (ch >> 3)) & 1) << 2);
}
// LDS byte offset of lane `lane`'s 16-byte K operand read of sub-tile kt, 32-channel
// slice kk: row n = lane % 32 of the operand, channel bytes 32kk + 16h .. +15.  The
// swizzle reads key bits 1, 2, 3 and 5, which the sub-tile leaves alone, so sub-tile kt
// adds (k32_row_key(kt, 0)) * 128.
__host__ __device__ __forceinline__ int k32_read_offset(int lane, int kk) {
  const int n = lane & 31, h = lane >> 5;
  const int key = k32_row_key(0, n);
  return key * 128 + 16 * ((2 * kk + h) ^ kswz32(key));
}
__host__ __device__ __forceinline__ int k32_subtile_offset(int kt) { return k32_row_key(kt, 0) * 128; }
// LDS byte offset of the V operand read (channel tile 0, key half ps, 16-byte half
// `half`): channel n, keys 64ps + 32h + 16half .. +15.  Channel tile dt adds dt * 32 * 128
// (the swizzle reads channel bits 1-3 only).
__host__ __device__ __forceinline__ int v32_read_offset(int lane, int ps, int half) {
  const int n = lane & 31, h = lane >> 5;
  return n * kKvTile + 16 * ((4 * ps + 2 * h + half) ^ vswz32(n));
}
// LDS DMA sources of the 32x32 layout (same instruction shape as DmaShape<128>).
__host__ __device__ __forceinline__ uint32_t k32_dma_src(int wave, int j, int lane) {
  const int pos = dma_lds_offset(wave, j, DmaShape<128>::KPW, lane);
  const int key = pos / 128, pc = (pos % 128) / 16;
  return (uint32_t)(key * 128 + (pc ^ kswz32(key)) * 16);
}
__host__ __device__ __forceinline__ uint32_t v32_dma_src(int wave, int j, int lane, int64_t npad) {
  const int pos = dma_lds_offset(wave, j, DmaShape<128>::VPW, lane);
  const int ch = pos / kKvTile, pc = (pos % kKvTile) / 16;
  return (uint32_t)(ch * npad + (pc ^ vswz32(ch)) * 16);
}

// Maps the linear workgroup id to (head, query block) so that the workgroups one XCD
// receives (ids x, x+8, x+16, ... go to XCD x) are consecutive query blocks of the same
// heads and share that head's K/V tiles in the XCD's L2.  A permutation of [0, total).
__host__ __device__ __forceinline__ int xcd_remap(int id, int total) {
  constexpr int kXcds = 8;
  const int per = total / kXcds, rem = total % kXcds;
  const int x = id % kXcds, idx = id / kXcds;
  return (x < rem) ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

}  // namespace sage
