// C ABI of the quantized-attention library: host-side validation, workspace carving
// and kernel launches.  Every argument check runs before the first HIP call, so error
// paths never touch the GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/sage_attn.h"
#include "sage_internal.h"

#define SAGE_EXPORT extern "C" __attribute__((visibility("default")))

static_assert(SAGE_MAX_SPARSE_TILES == sage::kMaxSparseTiles, "header and kernel limits agree");

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SAGE_OK;
}

constexpr size_t kAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return fail(SAGE_EINVAL, "B, H and N must be >= 1 (got B=%d H=%d N=%d)", B, H, N);
  if (d != 64 && d != 128) return fail(SAGE_EUNSUPPORTED, "head dim d=%d is not supported (64 or 128)", d);
  if (N > SAGE_MAX_TOKENS) return fail(SAGE_EUNSUPPORTED, "N=%d exceeds SAGE_MAX_TOKENS=%d", N, SAGE_MAX_TOKENS);
  if (B > 65535 || H > 65535) return fail(SAGE_EUNSUPPORTED, "B=%d or H=%d exceeds 65535", B, H);
  const int64_t nqb = sage::padded_tokens(N) / sage::kBlockM;
  if (nqb * B * H > 0x7fffffffLL) return fail(SAGE_EUNSUPPORTED, "B*H*Npad/%d exceeds the launch grid", sage::kBlockM);
  return SAGE_OK;
}

// Byte extent [lo, hi) of a bf16 [B][H][N][d] view.
struct Extent { uintptr_t lo, hi; };

Extent extent(const void* p, const sage_strides& s, int B, int H, int N, int d) {
  int64_t lo = 0, hi = 0;
  const int64_t st[3] = {s.b, s.h, s.n};
  const int64_t ex[3] = {B, H, N};
  for (int i = 0; i < 3; ++i) {
    const int64_t span = st[i] * (ex[i] - 1);
    if (span < 0) lo += span; else hi += span;
  }
  hi += d;
  return Extent{(uintptr_t)p + (uintptr_t)(lo * 2), (uintptr_t)p + (uintptr_t)(hi * 2)};
}

bool overlaps(const Extent& a, const Extent& b) { return a.lo < b.hi && b.lo < a.hi; }

int check_view(const char* name, const void* p, const sage_strides* s) {
  if (!p) return fail(SAGE_EINVAL, "%s is NULL", name);
  if (!s) return fail(SAGE_EINVAL, "strides of %s are NULL", name);
  if (!aligned(p, 16)) return fail(SAGE_EALIGN, "%s is not 16-byte aligned", name);
  if (s->b % 8 || s->h % 8 || s->n % 8)
    return fail(SAGE_EALIGN, "strides of %s (b=%lld h=%lld n=%lld) must be multiples of 8 elements",
                name, (long long)s->b, (long long)s->h, (long long)s->n);
  return SAGE_OK;
}

// A written view must not map two (b, h, n) rows onto overlapping memory.
int check_no_self_overlap(const char* name, const sage_strides& s, int B, int H, int N, int d) {
  int64_t st[3] = {s.b, s.h, s.n}, ex[3] = {B, H, N};
  int64_t vs[3], ve[3];
  int m = 0;
  for (int i = 0; i < 3; ++i)
    if (ex[i] > 1) { vs[m] = st[i] < 0 ? -st[i] : st[i]; ve[m] = ex[i]; ++m; }
  for (int i = 0; i < m; ++i)
    for (int j = i + 1; j < m; ++j)
      if (vs[j] < vs[i]) { std::swap(vs[i], vs[j]); std::swap(ve[i], ve[j]); }
  int64_t span = d;   // bytes/2 covered by the dims so far
  for (int i = 0; i < m; ++i) {
    if (vs[i] < span) return fail(SAGE_EINVAL, "%s: strides make distinct rows overlap", name);
    span = vs[i] * (ve[i] - 1) + span;
  }
  return SAGE_OK;
}

struct QuantLayout {
  int64_t npad;
  size_t q_i8, k_i8, v_f8, q_scale, k_scale, k_mean, v_scale;   // sizes in bytes
  size_t ksum, vmax, vinv;
};

// mode: SAGE_* bits.  With SAGE_PV_BF16 the V region holds bf16 values (2 bytes
// each); with SAGE_QK_PER_TOKEN the Q/K scale arrays have one entry per token.
QuantLayout layout(int B, int H, int N, int d, int mode = 0) {
  QuantLayout L;
  L.npad = sage::padded_tokens(N);
  const size_t bh = (size_t)B * H;
  L.q_i8 = L.k_i8 = bh * L.npad * d;
  L.v_f8 = bh * L.npad * d * ((mode & SAGE_PV_BF16) ? 2 : 1);
  L.q_scale = L.k_scale =
      bh * ((mode & SAGE_QK_PER_TOKEN) ? L.npad : L.npad / sage::kQuantBlock) * sizeof(float);
  L.k_mean = bh * d * sizeof(uint16_t) * ((mode & SAGE_K_BLOCK_MEAN) ? L.npad / sage::kQuantBlock : 1);
  L.v_scale = bh * d * sizeof(float);
  const size_t chunks = sage::stats_chunks(N);
  L.ksum = bh * chunks * d * sizeof(double);
  L.vmax = bh * chunks * d * sizeof(float);
  L.vinv = bh * d * sizeof(float);
  return L;
}

size_t scratch_size(const QuantLayout& L) {
  return round_up(L.ksum, kAlign) + round_up(L.vmax, kAlign) + round_up(L.vinv, kAlign);
}

size_t workspace_size(const QuantLayout& L) {
  return round_up(L.q_i8, kAlign) + round_up(L.k_i8, kAlign) + round_up(L.v_f8, kAlign) +
         round_up(L.q_scale, kAlign) + round_up(L.k_scale, kAlign) + round_up(L.k_mean, kAlign) +
         round_up(L.v_scale, kAlign) + scratch_size(L);
}

void carve_scratch(char*& p, const QuantLayout& L, sage::QuantArgs& a) {
  a.ksum_part = (double*)p; p += round_up(L.ksum, kAlign);
  a.vmax_part = (float*)p;  p += round_up(L.vmax, kAlign);
  a.v_inv = (float*)p;      p += round_up(L.vinv, kAlign);
}

// Block-sparse selection: code sums, importance matrix, and the kept-tile lists.
struct SelectLayout {
  int nt;                              // key tiles (= query blocks) per head
  size_t sums, imp, count, list;       // sizes in bytes
};

SelectLayout select_layout(int B, int H, int N, int d) {
  SelectLayout S;
  const int64_t npad = sage::padded_tokens(N);
  const size_t bh = (size_t)B * H;
  S.nt = (int)(npad / sage::kKvTile);
  S.sums = 2 * bh * (npad / sage::kQuantBlock) * 2 * d;   // two int8 digits per code sum
  S.imp = bh * S.nt * S.nt * sizeof(double);
  S.count = bh * S.nt * sizeof(int32_t);
  S.list = bh * S.nt * S.nt * sizeof(int32_t);
  return S;
}

size_t select_scratch_size(const SelectLayout& S) { return round_up(S.sums, kAlign) + round_up(S.imp, kAlign); }

int check_sparse(int B, int H, int N, int d, float density) {
  if (int rc = check_shape(B, H, N, d)) return rc;
  if (isnan(density) || !(density > 0.0f)) return fail(SAGE_EINVAL, "density must be > 0 (got %g)", (double)density);
  if ((int64_t)B * H > 65535) return fail(SAGE_EUNSUPPORTED, "block-sparse attention needs B*H <= 65535");
  if (sage::padded_tokens(N) / sage::kKvTile > sage::kMaxSparseTiles)
    return fail(SAGE_EUNSUPPORTED, "block-sparse attention supports at most %d key tiles (N=%d)",
                sage::kMaxSparseTiles, N);
  return SAGE_OK;
}

// k = max(1, min(T, ceil(density * T))), exact in fp64 for an fp32 density.
int keep_count(float density, int nt) {
  const double k = ceil((double)density * (double)nt);
  return (int)std::max(1.0, std::min((double)nt, k));
}

sage::Strides to_internal(const sage_strides& s) { return sage::Strides{s.b, s.h, s.n}; }

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SAGE_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

float log2e_scale(float sm_scale) { return (float)((double)sm_scale * 1.4426950408889634); }

// sm_scale 0 selects the definition's 1/sqrt(d) (rounded once to fp32); anything else
// must be finite and positive.
int resolve_sm_scale(float& sm_scale, int d) {
  if (sm_scale == 0.0f) {
    sm_scale = (float)(1.0 / sqrt((double)d));
    return SAGE_OK;
  }
  if (!(sm_scale > 0.0f) || !isfinite(sm_scale))
    return fail(SAGE_EINVAL, "sm_scale must be 0 (default 1/sqrt(d)) or finite and > 0 (got %g)", (double)sm_scale);
  return SAGE_OK;
}
float log2_pscale() { return (float)log2(448.0); }

}  // namespace

SAGE_EXPORT const char* sage_last_error(void) { return g_err; }

SAGE_EXPORT int sage_kernel_info(sage_info* info) {
  if (!info) return fail(SAGE_EINVAL, "info is NULL");
  memset(info, 0, sizeof(*info));
  info->block_m = sage::kBlockM;
  info->kv_tile = sage::kKvTile;
  info->quant_block = sage::kQuantBlock;
  info->token_align = sage::kTokenAlign;
  info->p_scale = sage::kPScale;
  info->d_supported_mask = (1 << 0) | (1 << 1);
  strncpy(info->arch, "gfx950", sizeof(info->arch) - 1);
  return ok();
}

SAGE_EXPORT int64_t sage_padded_tokens(int N) { return sage::padded_tokens(N); }

SAGE_EXPORT int sage_quant_scratch_bytes(int B, int H, int N, int d, size_t* bytes) {
  if (!bytes) return fail(SAGE_EINVAL, "bytes is NULL");
  if (int rc = check_shape(B, H, N, d)) return rc;
  *bytes = scratch_size(layout(B, H, N, d));
  return ok();
}

static int check_mode(int mode) {
  if (mode & ~(SAGE_PV_BF16 | SAGE_QK_PER_TOKEN | SAGE_K_BLOCK_MEAN))
    return fail(SAGE_EINVAL, "mode %#x has bits other than SAGE_PV_BF16 | SAGE_QK_PER_TOKEN | SAGE_K_BLOCK_MEAN",
                mode);
  if ((mode & SAGE_PV_BF16) && (mode & SAGE_K_BLOCK_MEAN))
    return fail(SAGE_EUNSUPPORTED, "SAGE_K_BLOCK_MEAN is implemented with FP8 P.V only");
  return SAGE_OK;
}

SAGE_EXPORT int sage_workspace_bytes_ex(int B, int H, int N, int d, int mode, size_t* bytes) {
  if (!bytes) return fail(SAGE_EINVAL, "bytes is NULL");
  if (int rc = check_mode(mode)) return rc;
  if (int rc = check_shape(B, H, N, d)) return rc;
  *bytes = workspace_size(layout(B, H, N, d, mode));
  return ok();
}

SAGE_EXPORT int sage_workspace_bytes(int B, int H, int N, int d, size_t* bytes) {
  return sage_workspace_bytes_ex(B, H, N, d, 0, bytes);
}

static int validate_quant_inputs(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const sage_strides* sq, const sage_strides* sk,
                                 const sage_strides* sv, int B, int H, int N, int d) {
  if (int rc = check_shape(B, H, N, d)) return rc;
  if (int rc = check_view("q", q, sq)) return rc;
  if (int rc = check_view("k", k, sk)) return rc;
  if (int rc = check_view("v", v, sv)) return rc;
  return SAGE_OK;
}

SAGE_EXPORT int sage_quant_qk_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const sage_strides* sq, const sage_strides* sk, const sage_strides* sv,
                                 int B, int H, int N, int d, int mode,
                                 int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                 uint16_t* k_mean, uint8_t* v_f8, float* v_scale,
                                 void* scratch, size_t scratch_bytes, void* stream) {
  if (int rc = check_mode(mode)) return rc;
  if (int rc = validate_quant_inputs(q, k, v, sq, sk, sv, B, H, N, d)) return rc;
  const void* outs[7] = {q_i8, q_scale, k_i8, k_scale, k_mean, v_f8, v_scale};
  const char* names[7] = {"q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "v_f8", "v_scale"};
  const QuantLayout L = layout(B, H, N, d, mode);
  const size_t sizes[7] = {L.q_i8, L.q_scale, L.k_i8, L.k_scale, L.k_mean, L.v_f8, L.v_scale};
  const Extent in[3] = {extent(q, *sq, B, H, N, d), extent(k, *sk, B, H, N, d), extent(v, *sv, B, H, N, d)};
  for (int i = 0; i < 7; ++i) {
    if (!outs[i]) return fail(SAGE_EINVAL, "%s is NULL", names[i]);
    if (!aligned(outs[i], kAlign)) return fail(SAGE_EALIGN, "%s is not 256-byte aligned", names[i]);
    const Extent e{(uintptr_t)outs[i], (uintptr_t)outs[i] + sizes[i]};
    for (int j = 0; j < 3; ++j)
      if (overlaps(e, in[j])) return fail(SAGE_EINVAL, "%s overlaps an input", names[i]);
    for (int j = 0; j < i; ++j) {
      const Extent f{(uintptr_t)outs[j], (uintptr_t)outs[j] + sizes[j]};
      if (overlaps(e, f)) return fail(SAGE_EINVAL, "%s overlaps %s", names[i], names[j]);
    }
  }
  if (!scratch) return fail(SAGE_EWORKSPACE, "scratch is NULL");
  if (!aligned(scratch, kAlign)) return fail(SAGE_EWORKSPACE, "scratch is not 256-byte aligned");
  if (scratch_bytes < scratch_size(L))
    return fail(SAGE_EWORKSPACE, "scratch has %zu bytes, %zu needed", scratch_bytes, scratch_size(L));

  sage::QuantArgs a;
  a.q = q; a.k = k; a.v = v;
  a.sq = to_internal(*sq); a.sk = to_internal(*sk); a.sv = to_internal(*sv);
  a.B = B; a.H = H; a.N = N; a.d = d; a.npad = L.npad;
  a.q_i8 = q_i8; a.q_scale = q_scale; a.k_i8 = k_i8; a.k_scale = k_scale;
  a.k_mean = k_mean; a.v_f8 = v_f8; a.v_scale = v_scale;
  a.pv = (mode & SAGE_PV_BF16) ? sage::kPvBf16 : sage::kPvFp8;
  a.v16 = (mode & SAGE_PV_BF16) ? (uint16_t*)v_f8 : nullptr;
  a.tok = (mode & SAGE_QK_PER_TOKEN) ? 1 : 0;
  a.kbm = (mode & SAGE_K_BLOCK_MEAN) ? 1 : 0;
  char* p = (char*)scratch;
  carve_scratch(p, L, a);
  return launch_status(sage::launch_quant(a, (hipStream_t)stream), "quantisation");
}

SAGE_EXPORT int sage_quant_qk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const sage_strides* sq, const sage_strides* sk, const sage_strides* sv,
                              int B, int H, int N, int d,
                              int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                              uint16_t* k_mean, uint8_t* v_f8, float* v_scale,
                              void* scratch, size_t scratch_bytes, void* stream) {
  return sage_quant_qk_ex(q, k, v, sq, sk, sv, B, H, N, d, 0, q_i8, q_scale, k_i8, k_scale, k_mean,
                          v_f8, v_scale, scratch, scratch_bytes, stream);
}

SAGE_EXPORT int sage_attn_fwd_prequant(const int8_t* q_i8, const float* q_scale,
                                       const int8_t* k_i8, const float* k_scale,
                                       const uint8_t* v_f8, const float* v_scale,
                                       uint16_t* out, const sage_strides* so,
                                       int B, int H, int N, int d, float sm_scale, void* stream) {
  if (int rc = check_shape(B, H, N, d)) return rc;
  const void* ins[6] = {q_i8, q_scale, k_i8, k_scale, v_f8, v_scale};
  const char* names[6] = {"q_i8", "q_scale", "k_i8", "k_scale", "v_f8", "v_scale"};
  const QuantLayout L = layout(B, H, N, d);
  const size_t sizes[6] = {L.q_i8, L.q_scale, L.k_i8, L.k_scale, L.v_f8, L.v_scale};
  for (int i = 0; i < 6; ++i) {
    if (!ins[i]) return fail(SAGE_EINVAL, "%s is NULL", names[i]);
    if (!aligned(ins[i], kAlign)) return fail(SAGE_EALIGN, "%s is not 256-byte aligned", names[i]);
  }
  if (int rc = check_view("out", out, so)) return rc;
  if (int rc = check_no_self_overlap("out", *so, B, H, N, d)) return rc;
  const Extent eo = extent(out, *so, B, H, N, d);
  for (int i = 0; i < 6; ++i)
    if (overlaps(eo, Extent{(uintptr_t)ins[i], (uintptr_t)ins[i] + sizes[i]}))
      return fail(SAGE_EINVAL, "out overlaps %s", names[i]);
  if (int rc = resolve_sm_scale(sm_scale, d)) return rc;

  sage::AttnArgs a;
  a.q_i8 = q_i8; a.q_scale = q_scale; a.k_i8 = k_i8; a.k_scale = k_scale;
  a.v_f8 = v_f8; a.v_scale = v_scale; a.v16 = nullptr; a.pv = sage::kPvFp8; a.tok = 0;
  a.k_bmean = nullptr;
  a.out = out; a.so = to_internal(*so);
  a.B = B; a.H = H; a.N = N; a.d = d; a.npad = L.npad;
  a.log2e_scale = log2e_scale(sm_scale);
  a.log2_pscale = log2_pscale();
  return launch_status(sage::launch_attn(a, (hipStream_t)stream), "attention");
}

// The whole path; with `sparse` the tile selection runs between the quantisation and
// the attention, on the selection region that follows the mode-0 layout.
// Every check of the whole path that does not concern the workspace.
static int validate_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                        int B, int H, int N, int d, float sm_scale,
                        const sage_strides strides[4], int mode, bool sparse, float density) {
  if (int rc = check_mode(mode)) return rc;
  if (sparse) {
    if (int rc = check_sparse(B, H, N, d, density)) return rc;
  }
  if (!strides) return fail(SAGE_EINVAL, "strides is NULL");
  if (int rc = validate_quant_inputs(q, k, v, &strides[0], &strides[1], &strides[2], B, H, N, d)) return rc;
  if (int rc = check_view("out", out, &strides[3])) return rc;
  if (int rc = check_no_self_overlap("out", strides[3], B, H, N, d)) return rc;
  const Extent eo = extent(out, strides[3], B, H, N, d);
  const void* ins[3] = {q, k, v};
  const char* names[3] = {"q", "k", "v"};
  for (int i = 0; i < 3; ++i)
    if (overlaps(eo, extent(ins[i], strides[i], B, H, N, d)))
      return fail(SAGE_EINVAL, "out overlaps %s", names[i]);
  return resolve_sm_scale(sm_scale, d);
}

static int attn_fwd_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                         int B, int H, int N, int d, float sm_scale,
                         const sage_strides strides[4], int mode, bool sparse, float density,
                         void* stream, void* workspace, size_t workspace_bytes) {
  if (int rc = validate_fwd(q, k, v, out, B, H, N, d, sm_scale, strides, mode, sparse, density)) return rc;
  if (int rc = resolve_sm_scale(sm_scale, d)) return rc;
  const void* ins[3] = {q, k, v};
  const char* names[3] = {"q", "k", "v"};
  const Extent eo = extent(out, strides[3], B, H, N, d);
  const QuantLayout L = layout(B, H, N, d, mode);
  const SelectLayout SL = select_layout(B, H, N, d);
  const size_t need = workspace_size(L) +
      (sparse ? select_scratch_size(SL) + round_up(SL.count, kAlign) + round_up(SL.list, kAlign) : 0);
  if (!workspace) return fail(SAGE_EWORKSPACE, "workspace is NULL");
  if (!aligned(workspace, kAlign)) return fail(SAGE_EWORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(SAGE_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const Extent ew{(uintptr_t)workspace, (uintptr_t)workspace + need};
  if (overlaps(ew, eo)) return fail(SAGE_EINVAL, "workspace overlaps out");
  for (int i = 0; i < 3; ++i)
    if (overlaps(ew, extent(ins[i], strides[i], B, H, N, d)))
      return fail(SAGE_EINVAL, "workspace overlaps %s", names[i]);

  sage::QuantArgs qa;
  qa.q = q; qa.k = k; qa.v = v;
  qa.sq = to_internal(strides[0]); qa.sk = to_internal(strides[1]); qa.sv = to_internal(strides[2]);
  qa.B = B; qa.H = H; qa.N = N; qa.d = d; qa.npad = L.npad;
  char* p = (char*)workspace;
  qa.q_i8 = (int8_t*)p;    p += round_up(L.q_i8, kAlign);
  qa.k_i8 = (int8_t*)p;    p += round_up(L.k_i8, kAlign);
  qa.v_f8 = (uint8_t*)p;   p += round_up(L.v_f8, kAlign);
  qa.q_scale = (float*)p;  p += round_up(L.q_scale, kAlign);
  qa.k_scale = (float*)p;  p += round_up(L.k_scale, kAlign);
  qa.k_mean = (uint16_t*)p; p += round_up(L.k_mean, kAlign);
  qa.v_scale = (float*)p;  p += round_up(L.v_scale, kAlign);
  qa.pv = (mode & SAGE_PV_BF16) ? sage::kPvBf16 : sage::kPvFp8;
  qa.v16 = (mode & SAGE_PV_BF16) ? (uint16_t*)qa.v_f8 : nullptr;
  qa.tok = (mode & SAGE_QK_PER_TOKEN) ? 1 : 0;
  qa.kbm = (mode & SAGE_K_BLOCK_MEAN) ? 1 : 0;
  carve_scratch(p, L, qa);
  hipStream_t s = (hipStream_t)stream;
  if (int rc = launch_status(sage::launch_quant(qa, s), "quantisation")) return rc;

  sage::AttnArgs a;
  a.q_i8 = qa.q_i8; a.q_scale = qa.q_scale; a.k_i8 = qa.k_i8; a.k_scale = qa.k_scale;
  a.v_f8 = qa.v_f8; a.v_scale = qa.v_scale; a.v16 = qa.v16; a.pv = qa.pv; a.tok = qa.tok;
  a.k_bmean = qa.kbm ? qa.k_mean : nullptr;
  a.out = out; a.so = to_internal(strides[3]);
  a.B = B; a.H = H; a.N = N; a.d = d; a.npad = L.npad;
  a.log2e_scale = log2e_scale(sm_scale);
  a.log2_pscale = log2_pscale();
  if (sparse) {
    sage::SelectArgs sa;
    sa.q_i8 = qa.q_i8; sa.k_i8 = qa.k_i8; sa.q_scale = qa.q_scale; sa.k_scale = qa.k_scale;
    sa.B = B; sa.H = H; sa.N = N; sa.d = d; sa.npad = L.npad;
    sa.keep = keep_count(density, SL.nt);
    sa.digits = (int8_t*)p;      p += round_up(SL.sums, kAlign);
    sa.imp = (double*)p;        p += round_up(SL.imp, kAlign);
    sa.tile_count = (int32_t*)p; p += round_up(SL.count, kAlign);
    sa.tile_list = (int32_t*)p;  p += round_up(SL.list, kAlign);
    if (int rc = launch_status(sage::launch_block_select(sa, s), "tile selection")) return rc;
    a.tile_count = sa.tile_count;
    a.tile_list = sa.tile_list;
    a.tiles_max = SL.nt;
  }
  return launch_status(sage::launch_attn(a, s), "attention");
}

SAGE_EXPORT int sage_attn_fwd_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                                 int B, int H, int N, int d, float sm_scale,
                                 const sage_strides strides[4], int mode, void* stream,
                                 void* workspace, size_t workspace_bytes) {
  return attn_fwd_impl(q, k, v, out, B, H, N, d, sm_scale, strides, mode, false, 1.0f, stream,
                       workspace, workspace_bytes);
}

SAGE_EXPORT int sage_workspace_bytes_sparse(int B, int H, int N, int d, size_t* bytes) {
  if (!bytes) return fail(SAGE_EINVAL, "bytes is NULL");
  if (int rc = check_sparse(B, H, N, d, 1.0f)) return rc;
  const SelectLayout SL = select_layout(B, H, N, d);
  *bytes = workspace_size(layout(B, H, N, d)) + select_scratch_size(SL) + round_up(SL.count, kAlign) +
           round_up(SL.list, kAlign);
  return ok();
}

SAGE_EXPORT int sage_density_schedule(int step, int n_steps, float tau_start, float tau_end, float* tau) {
  if (!tau) return fail(SAGE_EINVAL, "tau is NULL");
  if (n_steps < 1 || step < 0 || step >= n_steps)
    return fail(SAGE_EINVAL, "step %d outside [0, %d)", step, n_steps);
  if (!(isfinite(tau_start) && tau_start > 0.0f) || !(isfinite(tau_end) && tau_end > 0.0f))
    return fail(SAGE_EINVAL, "tau_start and tau_end must be finite and > 0");
  const double t = n_steps == 1 ? 1.0 : (double)step / (double)(n_steps - 1);
  *tau = (float)((double)tau_start + ((double)tau_end - (double)tau_start) * t);
  return ok();
}

SAGE_EXPORT int sage_attn_fwd_sparse(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                                     int B, int H, int N, int d, float sm_scale,
                                     const sage_strides strides[4], float density, void* stream,
                                     void* workspace, size_t workspace_bytes) {
  return attn_fwd_impl(q, k, v, out, B, H, N, d, sm_scale, strides, 0, true, density, stream,
                       workspace, workspace_bytes);
}

SAGE_EXPORT int sage_select_scratch_bytes(int B, int H, int N, int d, size_t* bytes) {
  if (!bytes) return fail(SAGE_EINVAL, "bytes is NULL");
  if (int rc = check_sparse(B, H, N, d, 1.0f)) return rc;
  *bytes = select_scratch_size(select_layout(B, H, N, d));
  return ok();
}

SAGE_EXPORT int sage_block_select(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                  const float* k_scale, int B, int H, int N, int d, float density,
                                  int32_t* tile_count, int32_t* tile_list, void* scratch,
                                  size_t scratch_bytes, void* stream) {
  if (int rc = check_sparse(B, H, N, d, density)) return rc;
  const QuantLayout L = layout(B, H, N, d);
  const SelectLayout SL = select_layout(B, H, N, d);
  const void* ins[4] = {q_i8, q_scale, k_i8, k_scale};
  const char* in_names[4] = {"q_i8", "q_scale", "k_i8", "k_scale"};
  const size_t in_sizes[4] = {L.q_i8, L.q_scale, L.k_i8, L.k_scale};
  for (int i = 0; i < 4; ++i) {
    if (!ins[i]) return fail(SAGE_EINVAL, "%s is NULL", in_names[i]);
    if (!aligned(ins[i], kAlign)) return fail(SAGE_EALIGN, "%s is not 256-byte aligned", in_names[i]);
  }
  if (!tile_count || !tile_list) return fail(SAGE_EINVAL, "tile_count and tile_list must not be NULL");
  if (!aligned(tile_count, 4) || !aligned(tile_list, 4)) return fail(SAGE_EALIGN, "tile_count/tile_list not 4-byte aligned");
  const Extent outs[2] = {{(uintptr_t)tile_count, (uintptr_t)tile_count + SL.count},
                          {(uintptr_t)tile_list, (uintptr_t)tile_list + SL.list}};
  if (overlaps(outs[0], outs[1])) return fail(SAGE_EINVAL, "tile_count overlaps tile_list");
  const size_t need = select_scratch_size(SL);
  if (!scratch) return fail(SAGE_EWORKSPACE, "scratch is NULL");
  if (!aligned(scratch, kAlign)) return fail(SAGE_EWORKSPACE, "scratch is not 256-byte aligned");
  if (scratch_bytes < need) return fail(SAGE_EWORKSPACE, "scratch has %zu bytes, %zu needed", scratch_bytes, need);
  const Extent es{(uintptr_t)scratch, (uintptr_t)scratch + need};
  for (int i = 0; i < 2; ++i) {
    if (overlaps(outs[i], es)) return fail(SAGE_EINVAL, "tile lists overlap the scratch");
    for (int j = 0; j < 4; ++j)
      if (overlaps(outs[i], Extent{(uintptr_t)ins[j], (uintptr_t)ins[j] + in_sizes[j]}))
        return fail(SAGE_EINVAL, "tile lists overlap %s", in_names[j]);
  }
  sage::SelectArgs sa;
  sa.q_i8 = q_i8; sa.k_i8 = k_i8; sa.q_scale = q_scale; sa.k_scale = k_scale;
  sa.B = B; sa.H = H; sa.N = N; sa.d = d; sa.npad = L.npad;
  sa.keep = keep_count(density, SL.nt);
  char* p = (char*)scratch;
  sa.digits = (int8_t*)p; p += round_up(SL.sums, kAlign);
  sa.imp = (double*)p;
  sa.tile_count = tile_count;
  sa.tile_list = tile_list;
  return launch_status(sage::launch_block_select(sa, (hipStream_t)stream), "tile selection");
}

SAGE_EXPORT int sage_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                              int B, int H, int N, int d, float sm_scale,
                              const sage_strides strides[4], void* stream,
                              void* workspace, size_t workspace_bytes) {
  return sage_attn_fwd_ex(q, k, v, out, B, H, N, d, sm_scale, strides, 0, stream,
                          workspace, workspace_bytes);
}

SAGE_EXPORT int sage_debug_qk_i32_ex(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d,
                                     int b, int h, int q_block, int kv_tile, int n_q_blocks, int n_kv_tiles,
                                     int mode, int32_t* s_out, void* stream) {
  if (int rc = check_shape(B, H, N, d)) return rc;
  if (int rc = check_mode(mode)) return rc;
  if (!q_i8 || !k_i8 || !s_out) return fail(SAGE_EINVAL, "q_i8, k_i8 and s_out must not be NULL");
  if (!aligned(q_i8, kAlign) || !aligned(k_i8, kAlign)) return fail(SAGE_EALIGN, "q_i8/k_i8 not 256-byte aligned");
  if (!aligned(s_out, 16)) return fail(SAGE_EALIGN, "s_out is not 16-byte aligned");
  if (b < 0 || b >= B || h < 0 || h >= H) return fail(SAGE_EINVAL, "head (%d, %d) out of range", b, h);
  const int64_t npad = sage::padded_tokens(N);
  const int64_t nqb = npad / sage::kBlockM, nkt = npad / sage::kKvTile;
  if (n_q_blocks < 1 || n_kv_tiles < 1 || q_block < 0 || kv_tile < 0 ||
      q_block + (int64_t)n_q_blocks > nqb || kv_tile + (int64_t)n_kv_tiles > nkt)
    return fail(SAGE_EINVAL, "tile range outside the padded operands");
  // the body sage_attn_fwd_ex launches for this mode: 32x32 for the FP8, 64-token,
  // token-mean mode at d = 128, 16x16 otherwise
  const bool body32 = d == 128 && mode == 0;
  return launch_status(sage::launch_debug_qk(q_i8, k_i8, d, body32, npad, (int64_t)b * H + h, q_block,
                                             kv_tile, n_q_blocks, n_kv_tiles, s_out, (hipStream_t)stream),
                       "debug_qk");
}

SAGE_EXPORT int sage_debug_qk_i32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d,
                                  int b, int h, int q_block, int kv_tile, int n_q_blocks, int n_kv_tiles,
                                  int32_t* s_out, void* stream) {
  return sage_debug_qk_i32_ex(q_i8, k_i8, B, H, N, d, b, h, q_block, kv_tile, n_q_blocks, n_kv_tiles, 0,
                              s_out, stream);
}

SAGE_EXPORT int sage_debug_e4m3(const float* x, uint8_t* codes, int64_t n, void* stream) {
  if (n < 0) return fail(SAGE_EINVAL, "n < 0");
  if (n == 0) return ok();
  if (!x || !codes) return fail(SAGE_EINVAL, "x and codes must not be NULL");
  if (n > ((int64_t)1 << 40)) return fail(SAGE_EUNSUPPORTED, "n too large");
  return launch_status(sage::launch_debug_e4m3(x, codes, n, (hipStream_t)stream), "debug_e4m3");
}

// ---------------------------------------------------------------------------------------
// sage_attn_fwd_noalloc: sage_attn_fwd with the workspace in a file-scope device array,
// for callers that cannot allocate.  Each device holds its own copy of `scratch` (from
// the first load of the library on it until the process ends); host code uses only the
// device address hipGetSymbolAddress returns for the current device, resolved once per
// device on the first call there.  Every call on a device shares its copy: calls that
// can run concurrently on one device race.  No kernel of the path needs the workspace to
// start zeroed (each writes every byte it later reads), so nothing is cleared.
namespace {
constexpr size_t kNoAllocBytes = (size_t)SAGE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

static int device_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SAGE_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(SAGE_EUNSUPPORTED, "device %d is beyond the %d the no-allocation entry point tracks", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SAGE_EHIP, "hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SAGE_OK;
}

SAGE_EXPORT int sage_attn_fwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                                      int B, int H, int N, int d, float sm_scale,
                                      const sage_strides strides[4], void* stream) {
  if (int rc = validate_fwd(q, k, v, out, B, H, N, d, sm_scale, strides, 0, false, 1.0f)) return rc;
  const size_t need = workspace_size(layout(B, H, N, d));
  if (need > kNoAllocBytes)
    return fail(SAGE_EWORKSPACE,
                "B=%d H=%d N=%d d=%d needs %zu bytes of workspace; the no-allocation entry point holds %zu "
                "(use sage_attn_fwd with a caller-owned workspace)", B, H, N, d, need, kNoAllocBytes);
  void* ws = nullptr;
  if (int rc = device_scratch(&ws)) return rc;
  return attn_fwd_impl(q, k, v, out, B, H, N, d, sm_scale, strides, 0, false, 1.0f, stream, ws, kNoAllocBytes);
}
