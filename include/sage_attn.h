/*
 * sage_attn.h - C ABI of the gfx950 (MI355X) quantized-attention library.
 *
 * Computes O = softmax(Q K^T * sm_scale) V, sm_scale normally 1/sqrt(d), with the
 * low-bit scheme of SageAttention as the pages describe it: Q.K^T in INT8 after the
 * K "outlier smoothing", P.V in FP8 (juejin page "MiniMax H3 接入 SageAttention 实测加速",
 * section 一), the K mean term kept in bf16 and only the remainder quantised
 * (sd114.wiki page on ComfyUI-sol-attn, "核心亮点" item 1), computed block by block
 * without materialising the N x N score matrix (bjdmk page
 * "GitHub榜单静默期：Attention优化从架构转向推理加速", section 2.2).  Options: bf16 P.V,
 * per-token scales and block-residual K (sage_attn_fwd_ex), and block-sparse key tiles
 * chosen by a density (sage_attn_fwd_sparse; sd114.wiki page, "核心亮点" item 4).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers of the calling process's current HIP
 *   device.  bf16 tensors are passed as their 16-bit patterns (uint16_t).
 * - Q, K, V and O are addressed as logical [B][H][N][d] views through sage_strides
 *   (element strides of the b, h and n dimensions; the channel dimension must be
 *   contiguous).  This covers [B, N, H, d] tensors, [B, H, N, d] tensors and the
 *   strided q/k/v slices of a fused qkv projection without copies (the zero-copy
 *   reading of fused qkv on the sd114.wiki page, "核心亮点" item 2).
 * - Quantised operands use fixed layouts, padded to Npad = sage_padded_tokens(N)
 *   tokens; padding rows hold zero codes and padding scale blocks hold 0:
 *     q_i8, k_i8   int8    [B][H][Npad][d]
 *     v_f8         uint8   [B][H][d][Npad]   (channel-major: row c holds V[:, c])
 *     q_scale, k_scale float [B][H][Npad/64]  (one per block of 64 tokens)
 *     k_mean       bf16    [B][H][d]
 *     v_scale      float   [B][H][d]
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null stream).
 *   They never synchronise and never allocate: scratch memory is passed in by the
 *   caller.  Inputs are read-only; outputs must not overlap inputs.  One workspace
 *   must not be used by two calls that can run concurrently.
 * - Every argument is validated on the host before any HIP call.  A non-zero status
 *   leaves every output untouched (except SAGE_EHIP, returned when a launch fails);
 *   sage_last_error() then returns a description (thread-local, valid until the
 *   calling thread's next call).  There is no fallback path inside the library.
 * - Supported: d in {64, 128}; 1 <= N <= SAGE_MAX_TOKENS; B, H >= 1; non-causal
 *   attention without a mask (diffusion transformers attend bidirectionally).
 *   Base pointers of bf16 views must be 16-byte aligned and their strides multiples
 *   of 8 elements (128-bit loads); quantised buffers, scratch and workspace must be
 *   256-byte aligned.
 */
#ifndef SAGE_ATTN_H
#define SAGE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_QUANT_BLOCK 64    /* tokens per Q/K scale block */
#define SAGE_TOKEN_ALIGN 128   /* Npad is N rounded up to this */
#define SAGE_MAX_TOKENS (1 << 22)

typedef struct sage_strides {
    int64_t b, h, n;           /* element strides; channel stride is 1 */
} sage_strides;

enum {
    SAGE_OK = 0,
    SAGE_EINVAL = -1,          /* null pointer, bad size, overlap, bad sm_scale */
    SAGE_EUNSUPPORTED = -2,    /* d not in {64,128}, N too large, grid too large */
    SAGE_EALIGN = -3,          /* misaligned pointer or stride */
    SAGE_EWORKSPACE = -4,      /* workspace/scratch missing, short or misaligned */
    SAGE_EHIP = -5             /* a kernel launch failed (HIP error text in sage_last_error) */
};

/* Mode bits of the _ex entry points; 0 is the default path of the others. */
enum {
    SAGE_PV_FP8 = 0,           /* P and V in FP8 e4m3 (speed; the default) */
    SAGE_PV_BF16 = 1,          /* P rounded to bf16, V unquantised bf16 (quality) */
    SAGE_QK_PER_TOKEN = 2,     /* one INT8 scale per Q and K token instead of per 64 */
    SAGE_K_BLOCK_MEAN = 4      /* block-residual K: bf16 mean per 64-key block (FP8 P.V only) */
};

typedef struct sage_info {
    int block_m;               /* query rows per attention workgroup */
    int kv_tile;               /* keys per online-softmax step (the tile T) */
    int quant_block;           /* tokens per Q/K scale block */
    int token_align;           /* Npad alignment */
    float p_scale;             /* static scale of P before its e4m3 rounding (448) */
    int d_supported_mask;      /* bit (d/64 - 1) set for each supported head dim */
    char arch[16];             /* "gfx950" */
} sage_info;

/* Description of the last failing call on this thread ("" if none). */
const char* sage_last_error(void);

/* Compile-time parameters of the kernels.  Returns SAGE_OK (SAGE_EINVAL on NULL). */
int sage_kernel_info(sage_info* info);

/* Npad: N rounded up to SAGE_TOKEN_ALIGN (0 for N <= 0). */
int64_t sage_padded_tokens(int N);

/* Bytes of scratch sage_quant_qk needs (fp64 partial sums of K, V max partials,
 * 1/scale factors of V), and bytes of workspace sage_attn_fwd needs (all quantised
 * operands plus that scratch).  Status as for the calls they size. */
int sage_quant_scratch_bytes(int B, int H, int N, int d, size_t* bytes);
int sage_workspace_bytes(int B, int H, int N, int d, size_t* bytes);
/* Workspace bytes of sage_attn_fwd_ex for `mode` (SAGE_EINVAL for unknown bits). */
int sage_workspace_bytes_ex(int B, int H, int N, int d, int mode, size_t* bytes);

/*
 * sage_quant_qk - the quantisation pass.
 *   k_mean[b,h,c] = bf16(fp32(sum_t K[b,h,t,c] / N))  (sum over the N valid tokens, fp64)
 *   Q, and K' = fp32(K) - fp32(k_mean), are coded per block of 64 tokens:
 *     scale = amax/127, code = clamp(rint(x * (127/amax)), -127, 127) (rint: half to even)
 *   V is coded per (b, h, channel): v_scale = vamax/448, code = e4m3(v * (448/vamax)),
 *     e4m3 rounding to nearest even, saturating.
 *   amax = 0 gives scale 0 and zero codes.
 * Inputs q, k, v: bf16 [B][H][N][d] views (strides sq, sk, sv).
 * Outputs: the quantised layouts above, all allocated by the caller.
 * scratch: >= sage_quant_scratch_bytes() bytes, 256-byte aligned.
 * Sources: K smoothing and INT8 for QK^T, FP8 for PV (juejin page section 一);
 * mean term kept in bf16 (sd114.wiki page "核心亮点" item 1).
 */
int sage_quant_qk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const sage_strides* sq, const sage_strides* sk, const sage_strides* sv,
                  int B, int H, int N, int d,
                  int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                  uint16_t* k_mean, uint8_t* v_f8, float* v_scale,
                  void* scratch, size_t scratch_bytes, void* stream);

/* sage_quant_qk with mode bits (see sage_attn_fwd_ex): SAGE_QK_PER_TOKEN gives per-token
 * q_scale/k_scale [B][H][Npad]; SAGE_PV_BF16 writes bf16 V [B][H][d][Npad] into v_f8
 * (sized 2 bytes per element) and leaves v_scale unwritten; SAGE_K_BLOCK_MEAN writes
 * the block means [B][H][Npad/64][d] into k_mean (zero for all-padding blocks). */
int sage_quant_qk_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const sage_strides* sq, const sage_strides* sk, const sage_strides* sv,
                     int B, int H, int N, int d, int mode,
                     int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                     uint16_t* k_mean, uint8_t* v_f8, float* v_scale,
                     void* scratch, size_t scratch_bytes, void* stream);

/*
 * sage_attn_fwd_prequant - fused attention on quantised operands (mode 0 layouts).
 * Sources: Q.K^T on INT8 and P.V on FP8 (juejin page "MiniMax H3 接入 SageAttention
 * 实测加速", section 一); the result is softmax(Q K^T * sm_scale) V (Baidu Cloud page
 * "SDPA稠密注意力模式", section 三 part 1), computed block by block, the score matrix
 * never written out (bjdmk page "GitHub榜单静默期：Attention优化从架构转向推理加速",
 * section 2.2).
 * For each query i, keys are visited in tiles of kv_tile (sage_kernel_info) keys:
 *   S = q_i8 . k_i8^T exactly in int32 (INT8 matrix cores),
 *   base-2 logits s = S * fp32(fp32(q_scale*fp32(sm_scale*log2 e)) * k_scale),
 *   fp32 online softmax with exp2 (running max m, p = 448 * 2^(s - m)),
 *   P rounded to e4m3 (nearest even, saturating at 448), acc += P8 . V8 (FP8 matrix
 *   cores, fp32 accumulation), l accumulates the unrounded p; O = acc * v_scale / l,
 *   written as bf16 (RNE) through the [B][H][N][d] view `out` (strides so).
 * Keys and queries at index >= N are never read as data: keys are masked, rows
 * beyond N are not written.  sm_scale: 0 selects 1/sqrt(d) (rounded once to fp32);
 * otherwise it must be finite and > 0 (else SAGE_EINVAL).
 * Buffers: the quantised operands (device, 256-byte aligned, owned by the caller,
 * read only); `out` must not overlap them.
 */
int sage_attn_fwd_prequant(const int8_t* q_i8, const float* q_scale,
                           const int8_t* k_i8, const float* k_scale,
                           const uint8_t* v_f8, const float* v_scale,
                           uint16_t* out, const sage_strides* so,
                           int B, int H, int N, int d, float sm_scale, void* stream);

/*
 * sage_attn_fwd - the whole hot path, O = softmax(Q K^T * sm_scale) V (Baidu Cloud page
 * "SDPA稠密注意力模式", section 三 part 1) by the quantised method: K smoothing, INT8
 * Q.K^T and FP8 P.V (juejin page "MiniMax H3 接入 SageAttention 实测加速", section 一),
 * i.e. sage_quant_qk into the workspace, then sage_attn_fwd_prequant on it.
 * q, k, v, out: bf16 device views; strides[0..3] describe q, k, v and out; out must
 * not overlap q, k, v or the workspace.  sm_scale as for sage_attn_fwd_prequant.
 * workspace: >= sage_workspace_bytes() bytes, 256-byte aligned, owned by the caller.
 * After the call the workspace holds the quantised operands in this order, each
 * region starting on a 256-byte boundary: q_i8, k_i8, v_f8, q_scale, k_scale, k_mean,
 * v_scale.
 */
int sage_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                  int B, int H, int N, int d, float sm_scale,
                  const sage_strides strides[4], void* stream,
                  void* workspace, size_t workspace_bytes);

/*
 * sage_attn_fwd_noalloc - sage_attn_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace in a device array of
 * SAGE_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on until
 * the process ends.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  Shapes whose sage_workspace_bytes() exceed that size return
 * SAGE_EWORKSPACE.  Every call on one device shares the array: calls that can run
 * concurrently on the same device (different streams, or several host threads) race
 * and must be serialised by the caller.  Other arguments and status codes as for
 * sage_attn_fwd; the first call on a device also resolves the array's address there
 * (SAGE_EHIP if that fails).
 */
#define SAGE_NOALLOC_SCRATCH_BYTES (64u << 20)
int sage_attn_fwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                          int B, int H, int N, int d, float sm_scale,
                          const sage_strides strides[4], void* stream);

/*
 * sage_attn_fwd_ex - sage_attn_fwd with quality options.  The pages note that
 * quantised attention schemes offer a quality-first setting beside the speed-first
 * one (bjdmk page "GitHub榜单静默期：Attention优化从架构转向推理加速", section 4.3) and
 * advise 16-bit attention for critical work (apatero page
 * "TeaCache和SageAttention优化实现更快的AI图像生成", section on when quality differences
 * appear).  `mode` is a combination of:
 *   SAGE_PV_BF16: p (same p = 448 * 2^(s - m)) is rounded to bf16 (nearest even)
 *     instead of e4m3 and V is not quantised (its bf16 values, transposed to
 *     channel-major in the workspace); acc += P16 . V16 on bf16 matrix cores with fp32
 *     accumulation, O = acc / l.  The workspace then holds bf16 V [B][H][d][Npad] in
 *     place of v_f8; v_scale is not written.
 *   SAGE_QK_PER_TOKEN: Q and K' are coded with one scale per token (amax over the
 *     token's d channels; same rounding), q_scale/k_scale become [B][H][Npad].  The
 *     logit arithmetic applies the key scale first: y = fp32(S * k_scale_j), the row
 *     maximum is over fp32(y * qf), p = 448 * 2^(s - m) = exp2(fma(y, qf, log2(448) - m)).
 *   SAGE_K_BLOCK_MEAN: block-residual K (sd114.wiki ComfyUI-sol-attn page, "核心亮点"
 *     item 1: only the residual inside each K block is quantised, the mean term stays
 *     bf16).  k_mean becomes [B][H][Npad/64][d]: the bf16 mean of each 64-token block's
 *     valid tokens (fp64 sum, fp32 then bf16 rounding); K' = fp32(K) - fp32(block mean)
 *     is coded as usual.  The logits gain e = fp32(qf * D), D = q8 . block mean (bf16
 *     matrix cores, fp32 accumulation): s = fp32(fp32(S * c) + e) for the maximum (with
 *     per-token scales fp32(fp32(y * qf) + e)) and p = exp2(fma(., ., fp32(e + nb))).
 *     Only with SAGE_PV_FP8 (with SAGE_PV_BF16: SAGE_EUNSUPPORTED).
 * mode 0 is identical to sage_attn_fwd.  Unknown bits return SAGE_EINVAL.  The
 * workspace size comes from sage_workspace_bytes_ex with the same mode.
 */
int sage_attn_fwd_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                     int B, int H, int N, int d, float sm_scale,
                     const sage_strides strides[4], int mode, void* stream,
                     void* workspace, size_t workspace_bytes);

/*
 * Block-sparse attention over key tiles.  The sd114.wiki page "ComfyUI-sol-attn"
 * (核心亮点, item 4) runs its sparse attention with a value tau that moves over the
 * sampling steps, sparse early and dense late, and gives no rule for which blocks to
 * skip.  Here tau is the density: each block of 128 queries keeps
 * k = max(1, min(T, ceil(tau * T))) of the T key tiles of 128 keys, those of largest
 * importance, the lower tile index winning ties.  The importance of tile J for query
 * block I is the mean, over their valid (query, key) pairs, of q_scale * k_scale * S,
 * computed exactly from the per-channel sums A_a, B_b of the INT8 codes of each
 * 64-token scale block a of I and b of J, in fp64 with every operation rounded once:
 * t_ab = (qs_a * ks_b) * <A_a, B_b>, importance = ((t_00 + t_01) + (t_10 + t_11)) /
 * (n_I * n_J) (a scale block past the last token gives t = 0).  The kept tiles are
 * visited in ascending order with the arithmetic of sage_attn_fwd_prequant; tau >= 1
 * gives exactly the dense result.  Limits: Npad/128 <= SAGE_MAX_SPARSE_TILES and
 * B*H <= 65535 (else SAGE_EUNSUPPORTED); tau must be > 0 (else SAGE_EINVAL).
 *
 * sage_select_scratch_bytes - scratch size of sage_block_select.  After the call the
 *   scratch holds the code sums as two int8 digits, [2][B][H][Npad/64][2][d] (Q then K;
 *   each sum s = 128 * digit0 + digit1, digit0 = s >> 7, digit1 = s & 127), and from
 *   the next 256-byte boundary the fp64 importance matrix [B][H][Npad/128][Npad/128].
 * sage_block_select - the kept tiles from the quantised operands of sage_quant_qk
 *   (mode 0, device pointers, 256-byte aligned): tile_count [B][H][Npad/128] int32
 *   (k in every entry) and tile_list [B][H][Npad/128][Npad/128] int32, whose rows
 *   start with the k kept tile indices in ascending order (the rest of each row is
 *   not written).  Asynchronous on `stream`; the outputs must not overlap the inputs
 *   or the scratch.
 * sage_workspace_bytes_sparse / sage_attn_fwd_sparse - sage_attn_fwd with the tile
 *   selection between the quantisation and the attention.  The workspace holds the
 *   mode-0 layout of sage_attn_fwd, then the selection scratch, tile_count and
 *   tile_list, each region starting on a 256-byte boundary.
 */
#define SAGE_MAX_SPARSE_TILES 4096
int sage_select_scratch_bytes(int B, int H, int N, int d, size_t* bytes);
int sage_block_select(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                      const float* k_scale, int B, int H, int N, int d, float density,
                      int32_t* tile_count, int32_t* tile_list, void* scratch,
                      size_t scratch_bytes, void* stream);
int sage_workspace_bytes_sparse(int B, int H, int N, int d, size_t* bytes);
int sage_attn_fwd_sparse(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                         int B, int H, int N, int d, float sm_scale,
                         const sage_strides strides[4], float density, void* stream,
                         void* workspace, size_t workspace_bytes);

/*
 * sage_density_schedule - the density of sampling step `step` of `n_steps` for
 * sage_attn_fwd_sparse when it moves from sparse early to dense late over a sampling
 * run (sd114.wiki page "ComfyUI-sol-attn", 核心亮点 item 4; the page gives no curve).
 * Reading: linear in the step index, tau = fp32(tau_start + (tau_end - tau_start) *
 * step / (n_steps - 1)) evaluated in fp64, so step 0 gets tau_start and the last step
 * tau_end; a run of one step gets tau_end.  Host only (no GPU call).  Requires
 * 0 <= step < n_steps, finite tau_start and tau_end > 0, tau non-NULL (else
 * SAGE_EINVAL; *tau is then left unchanged).
 */
int sage_density_schedule(int step, int n_steps, float tau_start, float tau_end, float* tau);

/*
 * sage_debug_qk_i32 - diagnostic: the exact int32 S = Q8.K8^T tiles of head (b, h),
 * computed by the same staging, LDS layout, matrix-core code and accumulator start as
 * the attention kernel of mode 0.  Covers query rows [q_block*block_m,
 * (q_block+n_q_blocks)*block_m) and keys [kv_tile*T, (kv_tile+n_kv_tiles)*T) of the
 * padded operands; s_out is int32, row-major [n_q_blocks*block_m][n_kv_tiles*T].
 * Tiles must lie inside Npad.  q_i8/k_i8: device, 256-byte aligned, the layout of
 * sage_quant_qk; s_out: device, 16-byte aligned, caller-owned.
 * sage_debug_qk_i32_ex - the same through the attention body that sage_attn_fwd_ex
 * launches for `mode` (SAGE_* bits): at d = 128 the 32x32 matrix-core body for mode 0
 * and the 16x16 body for every other mode; at d = 64 the 16x16 body.
 */
int sage_debug_qk_i32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d,
                      int b, int h, int q_block, int kv_tile, int n_q_blocks, int n_kv_tiles,
                      int32_t* s_out, void* stream);
int sage_debug_qk_i32_ex(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d,
                         int b, int h, int q_block, int kv_tile, int n_q_blocks, int n_kv_tiles,
                         int mode, int32_t* s_out, void* stream);

/*
 * sage_debug_e4m3 - diagnostic: the device fp32 -> e4m3 conversion the quantisation
 * kernel uses for V (round to nearest even, saturating to +-448), on n values.
 */
int sage_debug_e4m3(const float* x, uint8_t* codes, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_ATTN_H */
