// Internal declarations shared by the gfx950 kernels and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

constexpr int kQuantBlock = 64;     // tokens per Q/K scale block
constexpr int kTokenAlign = 128;    // Npad alignment (one key tile)
constexpr int kKvTile = 128;        // keys per online-softmax step
constexpr int kWaves = 4;           // waves per attention workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kGroupsPerWave = 2;   // 16-query groups per wave
constexpr int kBlockM = kWaves * kGroupsPerWave * 16;   // query rows per workgroup
constexpr int kStages = 2;          // LDS stages (K tile + V tile) of the attention kernel
constexpr int kMinWavesPerSimd = 2; // occupancy the attention kernel is compiled for
constexpr float kPScale = 448.0f;   // static scale of P before e4m3 rounding
constexpr int kMaxStatsChunks = 128; // partial-statistics rows per (b, h) in the quantisation pass
constexpr int kMaxSparseTiles = 4096; // key tiles per head of the block-sparse path (LDS of the selection)

// Precision of the P.V product: P in e4m3 with per-channel e4m3 V (speed), or P in
// bf16 with the unquantised bf16 V (quality).
enum PvMode { kPvFp8 = 0, kPvBf16 = 1 };

struct Strides { int64_t b, h, n; };

inline int64_t padded_tokens(int n) {
  return n <= 0 ? 0 : ((int64_t)n + kTokenAlign - 1) / kTokenAlign * kTokenAlign;
}
// 64-token blocks per first-pass workgroup: the fewest that keep the number of partial
// rows per (b, h) within kMaxStatsChunks.
inline int stats_blocks_per_chunk(int64_t npad) {
  const int64_t nblk = npad / kQuantBlock;
  return (int)((nblk + kMaxStatsChunks - 1) / kMaxStatsChunks);
}
inline int stats_chunks(int n) {
  const int64_t nblk = padded_tokens(n) / kQuantBlock;
  const int per = stats_blocks_per_chunk(padded_tokens(n));
  return (int)((nblk + per - 1) / per);
}

// Operands of the quantisation pass.
struct QuantArgs {
  const uint16_t *q, *k, *v;
  Strides sq, sk, sv;
  int B, H, N, d;
  int64_t npad;
  int8_t* q_i8;
  float* q_scale;
  int8_t* k_i8;
  float* k_scale;
  uint16_t* k_mean;
  uint8_t* v_f8;       // kPvFp8: e4m3 codes [B][H][d][Npad]
  float* v_scale;
  uint16_t* v16;       // kPvBf16: bf16 V [B][H][d][Npad]
  int pv;              // PvMode
  int tok;             // 1: Q/K scales per token [B][H][Npad], 0: per 64-token block
  int kbm;             // 1: block-residual K, k_mean holds [B][H][Npad/64][d] block means
  double* ksum_part;   // [B*H][chunks][d]
  float* vmax_part;    // [B*H][chunks][d]
  float* v_inv;        // [B*H][d]
};

// Operands of the fused attention kernel.
struct AttnArgs {
  const int8_t* q_i8;
  const float* q_scale;
  const int8_t* k_i8;
  const float* k_scale;
  const uint8_t* v_f8;
  const float* v_scale;
  const uint16_t* v16;
  int pv;              // PvMode
  int tok;             // Q/K scales per token
  const uint16_t* k_bmean;  // block-residual K: bf16 block means [B][H][Npad/64][d], or null
  uint16_t* out;
  Strides so;
  int B, H, N, d;
  int64_t npad;
  float log2e_scale;   // fp32(sm_scale * log2(e))
  float log2_pscale;   // fp32(log2(448))
  // block-sparse: kept key tiles per (b, h, query block) and their ascending indices
  // [B][H][Npad/128][tiles_max]; null for the dense kernel
  const int32_t* tile_count = nullptr;
  const int32_t* tile_list = nullptr;
  int tiles_max = 0;
  // compute units of the device: the period of the workgroup-pair issue priorities
  int cu_count = 256;
};

// Operands of the block-sparse tile selection.
struct SelectArgs {
  const int8_t *q_i8, *k_i8;
  const float *q_scale, *k_scale;   // [B][H][Npad/64]
  int B, H, N, d;
  int64_t npad;
  int keep;                         // tiles kept per query block
  int8_t* digits;                   // scratch [2][B*H][Npad/64][2][d]: per-block code sums of Q, K
                                    // as int8 digits (sum = 128 * digit 0 + digit 1)
  double* imp;                      // scratch [B*H][Npad/128][Npad/128]: tile importance
  int32_t* tile_count;              // [B*H][Npad/128]
  int32_t* tile_list;               // [B*H][Npad/128][Npad/128]
};

hipError_t launch_quant(const QuantArgs& a, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
hipError_t launch_block_select(const SelectArgs& a, hipStream_t s);
// body32: the 32x32 matrix-core body (d = 128 only), else the 16x16 one
hipError_t launch_debug_qk(const int8_t* q_i8, const int8_t* k_i8, int d, bool body32, int64_t npad,
                           int64_t bh, int q_block, int kv_tile, int n_q_blocks,
                           int n_kv_tiles, int32_t* s_out, hipStream_t s);
hipError_t launch_debug_e4m3(const float* x, uint8_t* y, int64_t n, hipStream_t s);

}  // namespace sage
