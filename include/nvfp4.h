/*
 * nvfp4.h -- C ABI of the NVFP4 hot path on AMD Instinct MI355X (gfx950).
 *
 * NVFP4 (techwalker.com LongLive-2.0 report summary, section 一): 4-bit E2M1
 * values; every 16 consecutive values along a row share one FP8 (E4M3) block
 * scale; the whole tensor shares one FP32 scale.  Weights, activations and
 * the KV cache all use it, and the linear layers multiply in 4 bits
 * (zuobiaodaohang LongLive blog, section "NVFP4：数据体积砍到 1/4"; techwalker
 * summary, section 四).
 *
 * Numerics (every rounding is one round-to-nearest-even of the exact value):
 *   amax    = max |x| over the tensor
 *   s_g     = RN_fp32(amax / 2688)            (2688 = 6 * 448; s_g = 1 if amax == 0)
 *   s_b     = RN_e4m3(b / (6 s_g)), saturating at 448, b = max |x| over the block
 *   code    = sign(x) | RN_e2m1(|x| / (s_b s_g)), saturating at 6; 0 magnitude if s_b == 0
 *   x^      = q * s_b * s_g
 * E2M1: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0; magnitudes
 * 0, .5, 1, 1.5, 2, 3, 4, 6.  E4M3: OCP E4M3FN (bias 7, max 448).
 *
 * Byte layouts (part of the contract):
 *   codes   [rows][cols/2] bytes; byte j holds code 2j in bits 3:0 and
 *           code 2j+1 in bits 7:4.
 *   scales  NVFP4_SCALES_ROWMAJOR: [rows][cols/16] bytes.
 *           NVFP4_SCALES_TILED: byte of (row r, block kb) at
 *             ((r/128) * (cols/64) + kb/4) * 512 + (r%128) * 4 + kb%4
 *           (rows % 128 == 0 and cols % 64 == 0 required).
 *
 * Conventions of every call:
 *   - All pointers are device pointers unless marked (host).  The caller
 *     owns every buffer; the library allocates nothing.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise the host.  Outputs are valid once the
 *     stream has reached the call.
 *   - Return value: NVFP4_OK or a negative nvfp4_status_t.  Arguments are
 *     checked before anything is launched; on an error nothing is launched
 *     and no output is touched, except NVFP4_EHIP (a launch failed).
 *   - Quantized buffers are opaque bytes: never cast them to another dtype
 *     (LongLive 2.0 README copy on news.ainew.jp, section "NVFP4": a dtype
 *     cast of the quantized buffers corrupts them).
 *   - Non-finite inputs and amax < 2688 * 2^-126 are outside the contract:
 *     the outputs are unspecified, but no call reads or writes out of bounds.
 *   - Thread safety: the library state is a once-per-device flag per kernel
 *     recording that its dynamic-LDS limit was raised (set atomically) and the
 *     per-device address of nvfp4_quantize_noalloc's scratch array (looked up
 *     once under a lock); concurrent calls on different streams are safe when
 *     their buffers do not overlap (nvfp4_quantize_noalloc: see there).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 1

typedef enum {
  NVFP4_OK = 0,
  NVFP4_EINVAL = -1,      /* null pointer, bad enum, negative size            */
  NVFP4_ESHAPE = -2,      /* cols % 16, alignment, layout divisibility, ranges */
  NVFP4_EWORKSPACE = -3,  /* workspace missing or smaller than required       */
  NVFP4_EHIP = -4         /* a HIP launch failed (hipGetLastError)            */
} nvfp4_status_t;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype_t;

typedef enum { NVFP4_SCALES_ROWMAJOR = 0, NVFP4_SCALES_TILED = 1 } nvfp4_scale_layout_t;

/* An NVFP4 tensor [rows x cols] (cols % 16 == 0, cols <= 65535 * 128,
 * rows <= 2^28; larger sizes give ESHAPE).  The struct itself is a host
 * object; its pointers are device pointers. */
typedef struct {
  uint8_t* codes;        /* rows * cols / 2 bytes                               */
  uint8_t* scales;       /* rows * cols / 16 bytes, in `scale_layout`           */
  float* global_scale;   /* one float: s_g                                      */
  int64_t rows;
  int64_t cols;
  int32_t scale_layout;  /* nvfp4_scale_layout_t                                */
} nvfp4_tensor_t;

/* Operation ids for nvfp4_workspace_bytes. */
typedef enum {
  NVFP4_OP_QUANTIZE = 0,
  NVFP4_OP_KV_QUANTIZE = 1,
  NVFP4_OP_KV_ATTENTION = 2,
  NVFP4_OP_ADALN_QUANTIZE = 3
} nvfp4_op_t;

/* Workspace (device bytes) a call needs.
 *   NVFP4_OP_QUANTIZE:     a = rows, b = cols, c = 1 if the caller passes amax, else 0
 *   NVFP4_OP_KV_QUANTIZE:  a = T (tokens), b = n_heads, c = head_dim
 *   NVFP4_OP_KV_ATTENTION: a = n_q, b = n_heads, c = n_pages * page_tokens
 *                          (0 when the window is not split over workgroups)
 *   NVFP4_OP_ADALN_QUANTIZE: a = rows, b = cols, c unused
 * Returns 0 for a bad op id.  The workspace must be 256-byte aligned. */
size_t nvfp4_workspace_bytes(int32_t op, int64_t a, int64_t b, int64_t c);

/* Quantize X [rows x cols] (fp32 or bf16, row stride ld_x elements) to NVFP4
 * (techwalker summary, section 一: two-level scaling; the scale and the
 * quantization are one fused pass per block).
 *   x          rows x cols input, dtype x_dtype; 16-byte aligned, ld_x * elem % 16 == 0
 *   amax       NULL: the call computes max|x| (two reads of X);
 *              else a device float that already holds max|x| (e.g. from
 *              nvfp4_gemm_w4a4's y_amax) and X is read once.
 *   out        (host struct) destination: codes, scales in out->scale_layout,
 *              *out->global_scale = s_g.  out->rows/cols must equal rows/cols.
 *   workspace  nvfp4_workspace_bytes(NVFP4_OP_QUANTIZE, rows, cols, amax != NULL)
 * rows == 0 is a no-op (s_g is still written: 1.0).
 * Errors: EINVAL (nulls, dtype), ESHAPE (cols % 16, alignment, tiled layout
 * with rows % 128 or cols % 64, ld_x < cols or ld_x > 2^40), EWORKSPACE. */
int nvfp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                   const float* amax, const nvfp4_tensor_t* out, void* workspace,
                   size_t ws_bytes, void* stream);

/* nvfp4_quantize without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that forbid allocation).
 * Arguments and results are those of nvfp4_quantize.  The amax pass's partial
 * maxima go to a 4096-byte array that the library holds in device memory on
 * each GPU it runs on (until the process ends); its address is looked up once
 * per device, and the call itself allocates nothing.  Every call on one GPU
 * shares that array and rewrites it completely before reading it, so calls
 * that overlap on one GPU (concurrent streams) race and must not be issued;
 * calls ordered on a stream, or across synchronised streams, are fine.
 * Errors: those of nvfp4_quantize; EWORKSPACE if a call needs more than the
 * array holds (none does at present: the partials are 4096 bytes for every
 * shape); EHIP if the array's address cannot be looked up. */
int nvfp4_quantize_noalloc(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                           int64_t ld_x, const float* amax, const nvfp4_tensor_t* out,
                           void* stream);

/* Transposed quantize: out = NVFP4 of X^T, i.e. output row k holds column k of
 * X [rows x cols] and the blocks of 16 run along X's rows.  This is the operand
 * layout of NVFP4 training's backward GEMMs (techwalker summary, sections 一
 * and 五: NVFP4 training and distillation), which contract over the other axis
 * of a forward operand; with it both run on nvfp4_gemm_w4a4 (Y = A B^T):
 *   dgrad  dX = dY W     A = nvfp4_quantize(dY),  B = nvfp4_quantize_transposed(W)
 *   wgrad  dW = dY^T X   A = nvfp4_quantize_transposed(dY),
 *                        B = nvfp4_quantize_transposed(X)
 * Same quantizer as nvfp4_quantize (round to nearest even, one s_g from the
 * tensor amax, which a transposition leaves unchanged).
 *   x          rows x cols, fp32 or bf16, row stride ld_x elements;
 *              16-byte aligned, ld_x * elem % 16 == 0
 *   amax       NULL, or a device float holding max|x| (X is then read once)
 *   out        (host struct) out->rows == cols, out->cols == rows
 *              (so rows % 16 == 0; tiled scales need cols % 128 and rows % 64;
 *              cols <= 65535 * 128)
 *   workspace  nvfp4_workspace_bytes(NVFP4_OP_QUANTIZE, rows, cols, amax != NULL)
 * rows == 0 or cols == 0: only s_g (1.0, or from amax) is written.
 * Errors: EINVAL (nulls, dtype), ESHAPE (cols % 16, out dims, alignment,
 * ld_x < cols or ld_x > 2^40), EWORKSPACE. */
int nvfp4_quantize_transposed(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                              int64_t ld_x, const float* amax, const nvfp4_tensor_t* out,
                              void* workspace, size_t ws_bytes, void* stream);

/* Fused producer of a DiT block's W4A4 activations: LayerNorm of each row of
 * the residual X (no affine parameters), adaLN modulation, then NVFP4 -- one
 * kernel pair instead of a normalisation kernel, a modulation kernel and a
 * quantize (zuobiaodaohang LongLive blog, section "NVFP4：数据体积砍到 1/4":
 * adaLN fused into one kernel; ai-manual.ru LongLive-2.0 article, section
 * "Как это работает под капотом": scaling fused with quantization).
 *   mu_r   = mean of row r,  var_r = mean of (x - mu_r)^2 (biased),
 *   rstd_r = 1 / sqrt(var_r + eps)  -- evaluated in fp64, stored as fp32;
 *   x'     = RN32(RN32(n * RN32(1 + scale[g][c])) + shift[g][c]),
 *   n      = RN32(RN32(x - mu_r) * rstd_r),  g = r / rows_per_group
 * (fp32, one rounding per operation, no fused multiply-add), and x' is
 * quantized as nvfp4_quantize does with amax = max|x'|.  X is read twice
 * (statistics + amax, then encode); x' never goes to memory.
 *   x               rows x cols, fp32 or bf16, row stride ld_x elements;
 *                   16-byte aligned, ld_x * elem % 16 == 0
 *   shift, scale    fp32 [ceil(rows / rows_per_group)][cols], 16-byte aligned
 *                   (one modulation pair per group of rows, e.g. a latent frame)
 *   rows_per_group  >= 1
 *   eps             finite, > 0
 *   row_stats       out: fp32 [rows][2] = (mu_r, rstd_r), 8-byte aligned
 *   out             (host struct) as for nvfp4_quantize
 *   workspace       nvfp4_workspace_bytes(NVFP4_OP_ADALN_QUANTIZE, rows, cols, 0)
 * rows == 0 or cols == 0: only s_g (1.0) is written.
 * Errors: EINVAL (nulls, dtype, rows_per_group, eps), ESHAPE (as
 * nvfp4_quantize), EWORKSPACE. */
int nvfp4_adaln_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                         int64_t ld_x, const float* shift, const float* scale,
                         int64_t rows_per_group, float eps, float* row_stats,
                         const nvfp4_tensor_t* out, void* workspace, size_t ws_bytes,
                         void* stream);

/* Dequantize: y = RN(q * s_b * s_g) in y_dtype (fp32, or bf16 with one
 * rounding of the exact product).  y: rows x cols, row stride ld_y elements,
 * 16-byte aligned with ld_y * elem % 16 == 0.  Parallel dequantization is the
 * read side of the NVFP4 format (techwalker summary, section 四).
 * Errors: EINVAL, ESHAPE. */
int nvfp4_dequantize(const nvfp4_tensor_t* in, void* y, int32_t y_dtype, int64_t ld_y,
                     void* stream);

/* W4A4 GEMM: Y[M x N] = X[M x K] * W[N x K]^T with both operands NVFP4
 * (techwalker summary, section 四: every matrix multiplication in 4 bits).
 * Y = s_gx * s_gw * sum_k (q_x s_bx)(q_w s_bw): the block products are exact
 * and accumulate in fp32; the result is stored as y_dtype (fp32 or bf16, RNE).
 *   x, w    (host structs) K = x->cols = w->cols (any multiple of 16; K == 0
 *           gives Y = 0); any scale layout
 *   y       M x N, row stride ld_y elements (ld_y >= N), 4-byte aligned rows
 *   y_amax  NULL, or a device float that the call max-folds max|Y as stored|
 *           into (atomic max; initialise it to 0 before the first GEMM whose
 *           amax it should hold).  Lets the next quantize read Y once.
 * M == 0 or N == 0 is a no-op.
 * Errors: EINVAL, ESHAPE (K mismatch, ld_y < N or ld_y > 2^40). */
int nvfp4_gemm_w4a4(const nvfp4_tensor_t* x, const nvfp4_tensor_t* w, void* y, int32_t y_dtype,
                    int64_t ld_y, float* y_amax, void* stream);

/* Paged NVFP4 KV cache (techwalker summary, section 四, second key: K gets a
 * simple mean subtraction, then K and V are stored in NVFP4; the cache is
 * read as many blocks of a window at once; zuobiaodaohang blog: the quantized
 * cache is updated in place).
 *
 * Page byte layout (page_bytes = 2 * n_heads * page_tokens * head_dim * 9/16):
 *   K codes  [n_heads][page_tokens][head_dim/2]
 *   K scales [n_heads][page_tokens][head_dim/16]   (E4M3, blocks of 16 along head_dim)
 *   V codes  [n_heads][page_tokens][head_dim/2]
 *   V scales [n_heads][page_tokens][head_dim/16]
 * Token position p of a layer lives in logical page p / page_tokens, slot
 * p % page_tokens, physical page page_table[layer][p / page_tokens].
 * Each written chunk c of a layer has its own K mean mu[h][d] (fp32) and
 * global scales s_gK, s_gV.  page_chunk[layer][lp] = {c_first, split}: slots
 * [0, split) belong to chunk c_first, slots [split, page_tokens) to c_first+1. */
typedef struct {
  uint8_t* pool;              /* n_phys_pages * page_bytes                        */
  int64_t n_phys_pages;
  int32_t n_layers;
  int32_t n_heads;
  int32_t head_dim;           /* % 16 == 0, <= 256                                */
  int32_t page_tokens;        /* > 0                                              */
  int32_t max_pages;          /* logical pages per layer                          */
  int32_t max_chunks;         /* chunks per layer                                 */
  const int32_t* page_table;  /* [n_layers][max_pages] -> physical page            */
  int32_t* page_chunk;        /* [n_layers][max_pages][2], written by kv_quantize  */
  float* k_mean;              /* [n_layers][max_chunks][n_heads][head_dim]         */
  float* k_gscale;            /* [n_layers][max_chunks]                            */
  float* v_gscale;            /* [n_layers][max_chunks]                            */
} nvfp4_kv_cache_t;

/* Bytes of one page. */
int64_t nvfp4_kv_page_bytes(int32_t n_heads, int32_t head_dim, int32_t page_tokens);

/* Write chunk `chunk_id` of `layer`: tokens [start_token, start_token + T)
 * from K, V bf16 [T][n_heads][head_dim] (contiguous, 16-byte aligned).
 *   mu[h][d] = RN32(exact mean over the T tokens of K[.][h][d]),
 *   K' = RN32(K - mu), s_gK from max|K'|, s_gV from max|V|,
 *   K', V quantized along head_dim and stored in place in their pages;
 *   k_mean / k_gscale / v_gscale / page_chunk updated.
 * Chunks of a layer are written in order, chunk c + 1 starting where chunk
 * c ended (so a page holds at most two chunks); chunk 0 starts on a page
 * boundary.  A chunk c > 0 that starts inside a page records that page's
 * earlier slots as chunk c - 1's.  The page table entries for
 * the touched pages must be valid physical pages.  The mean is exact for every
 * finite bf16 input: a channel is summed in fp64 when its values' range keeps
 * every partial sum within fp64's 53 bits, else as an exact integer (a channel
 * that needs it costs the call some 50 us).
 * Errors: EINVAL, ESHAPE (T < page_tokens unless it is chunk 0, chunk 0 not
 * starting on a page boundary, T >= 2^30, head_dim, token range past
 * max_pages, chunk_id >= max_chunks), EWORKSPACE. */
int nvfp4_kv_quantize(const nvfp4_kv_cache_t* cache, int32_t layer, int32_t chunk_id,
                      const void* k_bf16, const void* v_bf16, int64_t T, int64_t start_token,
                      void* workspace, size_t ws_bytes, void* stream);

/* Dequantize the pages of a window in one launch (techwalker summary,
 * section 四: one parallel kernel decompresses many cache blocks of a time
 * window).  For each listed logical page, in list order:
 *   K^ = RN_bf16(q s_b s_gK + mu),  V^ = RN_bf16(q s_b s_gV)   (one rounding each)
 * using the chunk of every slot (page_chunk).
 *   logical_pages  device int32[n_pages]; an entry outside [0, max_pages), or
 *                  one whose page-table entry is outside the pool, gives zero rows
 *   k_out, v_out   bf16 [n_pages * page_tokens][n_heads][head_dim], 16-byte aligned
 * Errors: EINVAL, ESHAPE (also ceil(page_tokens / 8) * n_pages >= 2^32). */
int nvfp4_kv_dequant_blocks(const nvfp4_kv_cache_t* cache, int32_t layer,
                            const int32_t* logical_pages, int32_t n_pages, void* k_out,
                            void* v_out, void* stream);

/* Attention of new queries over a window of the cache, reading the NVFP4
 * pages directly: no bf16 K or V is written to memory (techwalker summary,
 * section 四: the cache is decompressed block by block for the time window;
 * here each block is decompressed into on-chip memory and consumed at once).
 * For every query row n and head h:
 *   O[n][h] = sum_j softmax_j(softmax_scale * q[n][h] . K^[j][h]) V^[j][h]
 * over the valid keys j of the window, with K^, V^ exactly the values
 * nvfp4_kv_dequant_blocks produces.  Valid keys: every slot of every listed
 * logical page, except the last listed page, which contributes its first
 * last_page_tokens slots; a listed page that is not mapped (logical index or
 * page table entry out of range) contributes none.  Every query sees every
 * valid key (no causal mask).  Accumulation in fp32, the softmax weights
 * enter the P V product rounded to bf16, O is rounded once to bf16; rows
 * with no valid key are 0.
 *   logical_pages  device int32[n_pages]
 *   q_bf16         device bf16 [n_q][n_heads][head_dim], 16-byte aligned
 *   out_bf16       device bf16 [n_q][n_heads][head_dim], 8-byte aligned
 *   workspace      nvfp4_workspace_bytes(NVFP4_OP_KV_ATTENTION, n_q, n_heads,
 *                  n_pages * page_tokens) bytes, 256-byte aligned: when few
 *                  (query block, head) pairs exist the window is split over
 *                  workgroups and their partial results meet there
 * Requires head_dim 64 or 128 and page_tokens % 64 == 0.
 * Errors: EINVAL (nulls, negative sizes, last_page_tokens outside
 * [0, page_tokens] when n_pages > 0), ESHAPE (head_dim, page_tokens, layer,
 * alignment, n_heads > 65535), EWORKSPACE. */
int nvfp4_kv_attention(const nvfp4_kv_cache_t* cache, int32_t layer,
                       const int32_t* logical_pages, int32_t n_pages, int32_t last_page_tokens,
                       const void* q_bf16, int64_t n_q, float softmax_scale, void* out_bf16,
                       void* workspace, size_t ws_bytes, void* stream);

/* Logical page list of a multi-shot sink window (techwalker summary,
 * section 六: a global sink on the first frames, a shot sink re-bound to the
 * start of the current shot and kept as two pointers (start, length), both
 * laid over a sliding window).  The list holds every logical page with at
 * least one token of
 *   [0, global_sink_tokens) U [shot_start, shot_start + shot_sink_tokens)
 *   U [total_tokens - window_tokens, total_tokens),
 * each range clipped to [0, total_tokens), in increasing order, each page
 * once (ranges round outward to whole pages).  The count and the valid
 * tokens of the last listed page, min(page_tokens, total_tokens -
 * page_tokens * last_page), are computed on the host and returned at once
 * (0 and 0 for an empty list); the list is written to device memory by a
 * kernel on `stream`, ready for nvfp4_kv_dequant_blocks / nvfp4_kv_attention.
 *   pages_dev         device int32[max_pages] (may be NULL when the list is empty)
 *   n_pages           host out
 *   last_page_tokens  host out
 * Errors: EINVAL (null outputs, negative sizes or lengths, page_tokens <= 0),
 * ESHAPE (list longer than max_pages, or pages past 2^31 - 1). */
int nvfp4_kv_window_pages(int64_t total_tokens, int32_t page_tokens, int64_t global_sink_tokens,
                          int64_t shot_start, int64_t shot_sink_tokens, int64_t window_tokens,
                          int32_t* pages_dev, int32_t max_pages, int32_t* n_pages,
                          int32_t* last_page_tokens, void* stream);

/* Library version and messages.  nvfp4_source_hash: sha256 (hex) of the
 * sources the library was built from, as computed by the build script. */
int nvfp4_abi_version(void);
const char* nvfp4_status_string(int status);
const char* nvfp4_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
