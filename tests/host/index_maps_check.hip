// Host check of the attention kernel's LDS index maps (sage_tiles.h), run by
// tests/test_index_maps.py.  No GPU call: the maps are plain integer functions, and
// this program simulates the LDS DMA of one tile into a byte array and then every
// lane's operand reads.  It checks, for d = 64 and 128:
//   - every DMA source offset stays inside its tile (and its buffer for every tile of
//     every padded length), every LDS byte of a stage is written exactly once and every
//     source chunk is read exactly once;
//   - every operand read stays inside its tile and returns the keys and channels the
//     matrix-core operand layout assigns to the lane (K rows per k_row_key, V rows per
//     channel), covering each tile byte exactly once per wave;
//   - the block-mean operands and the query-code operands name the same channels;
//   - the side copies (key scales, block means) fill their LDS slots exactly once;
//   - the epilogue writes each output channel once per query row, the masked-tile
//     predicate keeps exactly the keys below N, and xcd_remap is a permutation;
//   - the same for the 32x32 layout of d = 128 (one 32-query group per wave: every K
//     and V byte of a tile is read once per wave).
// Prints "ok" and exits 0, or prints the first failure and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../quantized_attention_diffusion_amd/csrc/sage_tiles.h"

using namespace sage;

static int g_fail = 0;
#define CHECK(cond, ...)                              \
  do {                                                \
    if (!(cond)) {                                    \
      printf("FAIL %s:%d: ", __FILE__, __LINE__);     \
      printf(__VA_ARGS__);                            \
      printf("\n");                                   \
      exit(1);                                        \
    }                                                 \
  } while (0)

// A tag for each source byte: its byte index in the source buffer + 1 (0 = unwritten).
typedef std::vector<int64_t> Tags;

template <int D>
static void check_k() {
  const int KB = Lds<D>::KBYTES;
  Tags lds(KB, 0), src_seen(KB, 0);
  for (int w = 0; w < kWaves; ++w)
    for (int j = 0; j < DmaShape<D>::KPW; ++j)
      for (int i = 0; i < 64; ++i) {
        const int dst = dma_lds_offset(w, j, DmaShape<D>::KPW, i);
        const uint32_t src = k_dma_src<D>(w, j, i);
        // the kernel issues copy j from k_dma_src(w, 0, lane) + 1024 j
        CHECK(src == k_dma_src<D>(w, 0, i) + 1024u * j, "d=%d K DMA source not affine in j", D);
        CHECK(src % 16 == 0 && src + 16 <= (uint32_t)KB, "d=%d K DMA source %u outside the tile", D, src);
        CHECK(dst >= 0 && dst + 16 <= KB, "d=%d K DMA destination %d outside the stage", D, dst);
        for (int b = 0; b < 16; ++b) {
          CHECK(lds[dst + b] == 0, "d=%d K LDS byte %d written twice", D, dst + b);
          CHECK(src_seen[src + b] == 0, "d=%d K source byte %u copied twice", D, src + b);
          lds[dst + b] = (int64_t)src + b + 1;
          src_seen[src + b] = 1;
        }
      }
  for (int x = 0; x < KB; ++x) CHECK(lds[x] != 0, "d=%d K LDS byte %d never written", D, x);
  // operand reads: lane (r, g), sub-tile kt, slice kk must read K[k_row_key(kt, r)][64kk + 16g ..]
  Tags read_count(KB, 0);
  for (int lane = 0; lane < 64; ++lane) {
    const int r = lane & 15, g = lane >> 4;
    for (int kt = 0; kt < 8; ++kt)
      for (int kk = 0; kk < D / 64; ++kk) {
        const int off = k_read_offset<D>(lane, kk) + kt * 4 * D;
        CHECK(off % 16 == 0 && off >= 0 && off + 16 <= KB, "d=%d K read %d outside the tile", D, off);
        const int key = k_row_key(kt, r);
        for (int b = 0; b < 16; ++b) {
          const int64_t want = (int64_t)key * D + 64 * kk + 16 * g + b + 1;
          CHECK(lds[off + b] == want, "d=%d K read lane %d kt %d kk %d byte %d: got source %lld, want %lld",
                D, lane, kt, kk, b, (long long)lds[off + b] - 1, (long long)want - 1);
          read_count[off + b] += 1;
        }
      }
  }
  for (int x = 0; x < KB; ++x) CHECK(read_count[x] == 1, "d=%d K LDS byte %d read %lld times per wave", D, x, (long long)read_count[x]);
  // the S^T output layout: register i of sub-tile kt in lane group g holds row 4g + i,
  // which must be tile key 32g + 4kt + i, inside the 64-key scale block g / 2
  for (int g = 0; g < 4; ++g)
    for (int kt = 0; kt < 8; ++kt)
      for (int i = 0; i < 4; ++i) {
        CHECK(k_row_key(kt, 4 * g + i) == 32 * g + 4 * kt + i, "S layout: g %d kt %d i %d", g, kt, i);
        CHECK((32 * g + 4 * kt + i) / 64 == g / 2, "S keys of a lane span two scale blocks");
      }
}

template <int D>
static void check_v(int64_t npad) {
  const int VB = Lds<D>::VBYTES;
  // source: channel-major rows of npad bytes; the tile's first key column is 0
  Tags lds(VB, 0);
  std::vector<char> seen((size_t)D * kKvTile, 0);
  for (int w = 0; w < kWaves; ++w)
    for (int j = 0; j < DmaShape<D>::VPW; ++j)
      for (int i = 0; i < 64; ++i) {
        const int dst = dma_lds_offset(w, j, DmaShape<D>::VPW, i);
        const uint32_t src = v_dma_src<D>(w, j, i, npad);
        const int64_t ch = src / npad, key = src % npad;
        CHECK(src % 16 == 0 && ch < D && key + 16 <= kKvTile, "d=%d V DMA source ch %lld key %lld outside the tile",
              D, (long long)ch, (long long)key);
        // every tile t adds t * 128 to the key: the last byte of the last tile is in the buffer
        CHECK((int64_t)src + (npad - kKvTile) + 16 <= (int64_t)D * npad, "d=%d V DMA past the buffer", D);
        CHECK(dst >= 0 && dst + 16 <= VB, "d=%d V DMA destination outside the stage", D);
        for (int b = 0; b < 16; ++b) {
          CHECK(lds[dst + b] == 0, "d=%d V LDS byte written twice", D);
          CHECK(!seen[ch * kKvTile + key + b], "d=%d V source byte copied twice", D);
          seen[ch * kKvTile + key + b] = 1;
          lds[dst + b] = ch * kKvTile + key + b + 1;      // tag: channel * 128 + key
        }
      }
  for (int x = 0; x < VB; ++x) CHECK(lds[x] != 0, "d=%d V LDS byte %d never written", D, x);
  Tags read_count(VB, 0);
  for (int lane = 0; lane < 64; ++lane) {
    const int r = lane & 15, g = lane >> 4;
    for (int dt = 0; dt < D / 16; ++dt)
      for (int h = 0; h < 2; ++h) {
        const int off = v_read_offset(lane, h) + dt * 16 * kKvTile;
        CHECK(off % 16 == 0 && off >= 0 && off + 16 <= VB, "d=%d V read outside the tile", D);
        for (int b = 0; b < 16; ++b) {
          const int64_t want = (int64_t)(16 * dt + r) * kKvTile + 32 * g + 16 * h + b + 1;
          CHECK(lds[off + b] == want, "d=%d V read lane %d dt %d h %d byte %d", D, lane, dt, h, b);
          read_count[off + b] += 1;
        }
      }
  }
  for (int x = 0; x < VB; ++x) CHECK(read_count[x] == 1, "d=%d V LDS byte %d read %lld times per wave", D, x, (long long)read_count[x]);
}

template <int D>
static void check_v16(int64_t npad) {
  const int VB = Lds<D>::V16BYTES;
  Tags lds(VB, 0);
  std::vector<char> seen((size_t)D * 256, 0);
  for (int w = 0; w < kWaves; ++w)
    for (int j = 0; j < DmaShape<D>::V16PW; ++j)
      for (int i = 0; i < 64; ++i) {
        const int dst = dma_lds_offset(w, j, DmaShape<D>::V16PW, i);
        const uint32_t src = v16_dma_src<D>(w, j, i, npad);
        const int64_t ch = src / (2 * npad), kb = src % (2 * npad);   // key byte within the row
        CHECK(src % 16 == 0 && ch < D && kb + 16 <= 256, "d=%d bf16 V DMA source outside the tile", D);
        CHECK((int64_t)src + 2 * (npad - kKvTile) + 16 <= (int64_t)D * npad * 2, "d=%d bf16 V DMA past the buffer", D);
        CHECK(dst >= 0 && dst + 16 <= VB, "d=%d bf16 V DMA destination outside the stage", D);
        for (int b = 0; b < 16; ++b) {
          CHECK(lds[dst + b] == 0, "d=%d bf16 V LDS byte written twice", D);
          CHECK(!seen[ch * 256 + kb + b], "d=%d bf16 V source byte copied twice", D);
          seen[ch * 256 + kb + b] = 1;
          lds[dst + b] = ch * 256 + kb + b + 1;
        }
      }
  for (int x = 0; x < VB; ++x) CHECK(lds[x] != 0, "d=%d bf16 V LDS byte %d never written", D, x);
  Tags read_count(VB, 0);
  for (int lane = 0; lane < 64; ++lane) {
    const int r = lane & 15, g = lane >> 4;
    for (int dt = 0; dt < D / 16; ++dt)
      for (int s = 0; s < 4; ++s) {
        const int off = v16_read_offset(lane, s) + dt * 16 * 256;
        CHECK(off % 16 == 0 && off >= 0 && off + 16 <= VB, "d=%d bf16 V read outside the tile", D);
        for (int b = 0; b < 16; ++b) {
          // keys 32g + 8s .. +7 of channel 16dt + r, two bytes each
          const int64_t want = (int64_t)(16 * dt + r) * 256 + 2 * (32 * g + 8 * s) + b + 1;
          CHECK(lds[off + b] == want, "d=%d bf16 V read lane %d dt %d s %d byte %d", D, lane, dt, s, b);
          read_count[off + b] += 1;
        }
      }
  }
  for (int x = 0; x < VB; ++x) CHECK(read_count[x] == 1, "d=%d bf16 V LDS byte read %lld times per wave", D, (long long)read_count[x]);
}

template <int D>
static void check_side_copies_and_epilogue() {
  // key scales: lanes < 8 of each wave copy 16 bytes at 128 * wave + 16 * lane of 512
  std::vector<int> ks(512, 0);
  for (int w = 0; w < kWaves; ++w)
    for (int lane = 0; lane < 8; ++lane)
      for (int b = 0; b < 16; ++b) ks[128 * w + 16 * lane + b]++;
  for (int x = 0; x < 512; ++x) CHECK(ks[x] == 1, "key-scale slot byte %d copied %d times", x, ks[x]);
  // block means: lanes < D/16 copy 16 bytes at D * wave + 16 * lane of 4 * D (two bf16 rows of D)
  std::vector<int> bm(4 * D, 0);
  for (int w = 0; w < kWaves; ++w)
    for (int lane = 0; lane < D / 16; ++lane)
      for (int b = 0; b < 16; ++b) bm[D * w + 16 * lane + b]++;
  for (int x = 0; x < 4 * D; ++x) CHECK(bm[x] == 1, "block-mean slot byte %d copied %d times", x, bm[x]);
  // block-mean products: for step (kk, h) lane (r, g) reads the mean of block r / 8 at
  // bf16 channels (byte 128kk + 32g + 16h) / 2 .. +7 and supplies the query codes of
  // channels 64kk + 16g + 8h .. +7: the same channels, each channel once per block
  std::vector<int> chan(2 * D, 0);
  for (int lane = 0; lane < 64; ++lane) {
    const int r = lane & 15, g = lane >> 4;
    for (int kk = 0; kk < D / 64; ++kk)
      for (int h = 0; h < 2; ++h) {
        const int byte = (r >> 3) * 2 * D + 128 * kk + 32 * g + 16 * h;
        CHECK(byte + 16 <= 4 * D, "block-mean read outside its slot");
        const int blk = byte / (2 * D), c0 = (byte % (2 * D)) / 2;
        CHECK(blk == (r >> 3) && c0 == 64 * kk + 16 * g + 8 * h, "block-mean operand channels differ from the query codes'");
        if ((r & 7) == 0)
          for (int c = 0; c < 8; ++c) chan[blk * D + c0 + c]++;
      }
  }
  for (int x = 0; x < 2 * D; ++x) CHECK(chan[x] == 1, "block-mean channel %d used %d times", x, chan[x]);
  // epilogue: lane (r, g) writes channels 16dt + 4g + i of query r
  std::vector<int> oc(D, 0);
  for (int g = 0; g < 4; ++g)
    for (int dt = 0; dt < D / 16; ++dt)
      for (int i = 0; i < 4; ++i) oc[16 * dt + 4 * g + i]++;
  for (int c = 0; c < D; ++c) CHECK(oc[c] == 1, "output channel %d written %d times", c, oc[c]);
}

// The 32x32 layout (d = 128): DMA with the 32x32 swizzles, K operand reads (row n of
// sub-tile kt = key k32_row_key(kt, n), channel bytes 32kk + 16h ..), V operand reads
// (channel 32dt + n, keys 64ps + 32h + 16half ..), and the S / P key correspondence.
static void check_32x32(int64_t npad) {
  const int KB = Lds<128>::KBYTES, VB = Lds<128>::VBYTES;
  Tags kl(KB, 0), vl(VB, 0);
  std::vector<char> kseen(KB, 0), vseen(VB, 0);
  for (int w = 0; w < kWaves; ++w)
    for (int i = 0; i < 64; ++i) {
      for (int j = 0; j < DmaShape<128>::KPW; ++j) {
        const int dst = dma_lds_offset(w, j, DmaShape<128>::KPW, i);
        const uint32_t src = k32_dma_src(w, j, i);
        CHECK(src % 16 == 0 && src + 16 <= (uint32_t)KB && dst + 16 <= KB, "32x32 K DMA out of the tile");
        for (int b = 0; b < 16; ++b) {
          CHECK(kl[dst + b] == 0 && !kseen[src + b], "32x32 K DMA byte copied twice");
          kl[dst + b] = (int64_t)src + b + 1;
          kseen[src + b] = 1;
        }
      }
      for (int j = 0; j < DmaShape<128>::VPW; ++j) {
        const int dst = dma_lds_offset(w, j, DmaShape<128>::VPW, i);
        const uint32_t src = v32_dma_src(w, j, i, npad);
        const int64_t ch = src / npad, key = src % npad;
        CHECK(src % 16 == 0 && ch < 128 && key + 16 <= kKvTile && dst + 16 <= VB, "32x32 V DMA out of the tile");
        CHECK((int64_t)src + (npad - kKvTile) + 16 <= (int64_t)128 * npad, "32x32 V DMA past the buffer");
        for (int b = 0; b < 16; ++b) {
          CHECK(vl[dst + b] == 0 && !vseen[ch * kKvTile + key + b], "32x32 V DMA byte copied twice");
          vl[dst + b] = ch * kKvTile + key + b + 1;
          vseen[ch * kKvTile + key + b] = 1;
        }
      }
    }
  for (int x = 0; x < KB; ++x) CHECK(kl[x] != 0, "32x32 K LDS byte %d never written", x);
  for (int x = 0; x < VB; ++x) CHECK(vl[x] != 0, "32x32 V LDS byte %d never written", x);
  Tags kr(KB, 0), vr(VB, 0);
  for (int lane = 0; lane < 64; ++lane) {
    const int n = lane & 31, h = lane >> 5;
    for (int kt = 0; kt < 4; ++kt)
      for (int kk = 0; kk < 4; ++kk) {
        const int off = k32_read_offset(lane, kk) + k32_subtile_offset(kt);
        CHECK(off % 16 == 0 && off >= 0 && off + 16 <= KB, "32x32 K read outside the tile");
        const int key = k32_row_key(kt, n);
        for (int b = 0; b < 16; ++b) {
          CHECK(kl[off + b] == (int64_t)key * 128 + 32 * kk + 16 * h + b + 1,
                "32x32 K read lane %d kt %d kk %d byte %d", lane, kt, kk, b);
          kr[off + b]++;
        }
      }
    for (int dt = 0; dt < 4; ++dt)
      for (int ps = 0; ps < 2; ++ps)
        for (int x = 0; x < 2; ++x) {
          const int off = v32_read_offset(lane, ps, x) + dt * 32 * kKvTile;
          CHECK(off % 16 == 0 && off >= 0 && off + 16 <= VB, "32x32 V read outside the tile");
          for (int b = 0; b < 16; ++b) {
            CHECK(vl[off + b] == (int64_t)(32 * dt + n) * kKvTile + 64 * ps + 32 * h + 16 * x + b + 1,
                  "32x32 V read lane %d dt %d ps %d", lane, dt, ps);
            vr[off + b]++;
          }
        }
  }
  for (int x = 0; x < KB; ++x) CHECK(kr[x] == 1, "32x32 K LDS byte %d read %lld times per wave", x, (long long)kr[x]);
  for (int x = 0; x < VB; ++x) CHECK(vr[x] == 1, "32x32 V LDS byte %d read %lld times per wave", x, (long long)vr[x]);
  // S^T output: register i = 4jj + t of sub-tile kt in lane half h is row 8jj + 4h + t,
  // which must be key 64(kt/2) + 32h + 16(kt%2) + i: byte 16(kt%2) + i of the P operand
  // of half kt/2, whose lane half h covers keys 64ps + 32h .. +31
  for (int h = 0; h < 2; ++h)
    for (int kt = 0; kt < 4; ++kt)
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * h + (i & 3);
        CHECK(k32_row_key(kt, row) == 64 * (kt >> 1) + 32 * h + 16 * (kt & 1) + i, "32x32 S layout h %d kt %d i %d", h, kt, i);
      }
  // each sub-tile's 32 rows are 32 distinct keys, and the four sub-tiles cover the tile
  std::vector<int> cover(128, 0);
  for (int kt = 0; kt < 4; ++kt)
    for (int j = 0; j < 32; ++j) cover[k32_row_key(kt, j)]++;
  for (int key = 0; key < 128; ++key) CHECK(cover[key] == 1, "32x32 key %d covered %d times", key, cover[key]);
  // epilogue: lane half h writes channels 32dt + 8jj + 4h + t
  std::vector<int> oc(128, 0);
  for (int h = 0; h < 2; ++h)
    for (int dt = 0; dt < 4; ++dt)
      for (int jj = 0; jj < 4; ++jj)
        for (int t = 0; t < 4; ++t) oc[32 * dt + 8 * jj + 4 * h + t]++;
  for (int c = 0; c < 128; ++c) CHECK(oc[c] == 1, "32x32 output channel %d written %d times", c, oc[c]);
}

static void check_tails_rows_and_remap() {
  for (int N = 1; N <= 1100; ++N) {
    const int ntiles = (N + kKvTile - 1) / kKvTile;
    const int tail = N - (ntiles - 1) * kKvTile;
    CHECK(tail >= 1 && tail <= kKvTile, "tail %d for N %d", tail, N);
    const int64_t npad = padded_tokens(N);
    CHECK(npad % kBlockM == 0 && npad % kKvTile == 0 && npad >= N && npad - N < kKvTile, "Npad for N %d", N);
    // masked last tile: lane group g, register i of sub-tile kt holds key 32g + 4kt + i,
    // kept iff 4kt + i < tail - 32g (the kernel's predicate), i.e. iff the key < tail
    for (int g = 0; g < 4; ++g)
      for (int kt = 0; kt < 8; ++kt)
        for (int i = 0; i < 4; ++i) {
          const bool kept = (4 * kt + i) < tail - 32 * g;
          CHECK(kept == (32 * g + 4 * kt + i < tail), "mask predicate N %d g %d kt %d i %d", N, g, kt, i);
        }
    // query rows: workgroup qb, wave w, group gq, lane r -> row qb*128 + 32w + 16gq + r
    std::vector<int> rows(npad, 0);
    for (int qb = 0; qb < npad / kBlockM; ++qb)
      for (int w = 0; w < kWaves; ++w)
        for (int gq = 0; gq < kGroupsPerWave; ++gq)
          for (int r = 0; r < 16; ++r) rows[qb * kBlockM + w * (kGroupsPerWave * 16) + 16 * gq + r]++;
    for (int64_t x = 0; x < npad; ++x) CHECK(rows[x] == 1, "query row %lld covered %d times", (long long)x, rows[x]);
  }
  for (int total = 1; total <= 5000; total += (total < 300 ? 1 : 37)) {
    std::vector<int> hit(total, 0);
    for (int id = 0; id < total; ++id) {
      const int w = xcd_remap(id, total);
      CHECK(w >= 0 && w < total, "xcd_remap(%d, %d) = %d out of range", id, total, w);
      hit[w]++;
    }
    for (int x = 0; x < total; ++x) CHECK(hit[x] == 1, "xcd_remap(., %d) hits %d %d times", total, x, hit[x]);
  }
}

int main() {
  check_k<64>();
  check_k<128>();
  for (int64_t npad : {128LL, 256LL, 4608LL, 32768LL, 65536LL}) {
    check_v<64>(npad);
    check_v<128>(npad);
    check_v16<64>(npad);
    check_v16<128>(npad);
    check_32x32(npad);
  }
  check_side_copies_and_epilogue<64>();
  check_side_copies_and_epilogue<128>();
  check_tails_rows_and_remap();
  printf("ok\n");
  return g_fail;
}
