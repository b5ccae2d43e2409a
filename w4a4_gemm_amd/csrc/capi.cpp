// C ABI of the NVFP4 library (declared in include/nvfp4.h): argument checks,
// status codes and dispatch to the gfx950 kernels.  No allocation and no host
// synchronisation.  Library state: the per-device flags of launch.hpp and the
// per-device address of the allocation-free quantize's scratch array.

#include "nvfp4.h"
#include <climits>
#include <cmath>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Launch errors are sticky per thread in HIP; clear any stale error first so
// that a failure is attributed to this call.
inline int finish() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

inline hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// Tensor size limits from the launch grids: columns go on grid.y (at most
// 65535 workgroups of 128 input columns in the transposed quantize), rows on
// grid.x, where quantize/dequantize/adaLN run one 256-thread workgroup per 32
// rows and one grid dimension holds fewer than 2^32 work-items.
constexpr int64_t kMaxCols = int64_t(65535) * 128;
constexpr int64_t kMaxRows = int64_t(1) << 28;
// Row strides (elements) beyond any addressable tensor are rejected before they
// are multiplied by an element size.
constexpr int64_t kMaxLd = int64_t(1) << 40;

// A row stride: at least `cols`, at most kMaxLd, rows 16-byte aligned.
inline bool stride_ok(int64_t ld, int64_t cols, int64_t elem) {
  return ld >= cols && ld <= kMaxLd && (ld * elem) % 16 == 0;
}

int check_tensor(const nvfp4_tensor_t* t) {
  if (!t) return NVFP4_EINVAL;
  if (t->rows < 0 || t->cols < 0) return NVFP4_EINVAL;
  if (t->scale_layout != NVFP4_SCALES_ROWMAJOR && t->scale_layout != NVFP4_SCALES_TILED)
    return NVFP4_EINVAL;
  if (t->cols % 16) return NVFP4_ESHAPE;
  if (t->cols > kMaxCols || t->rows > kMaxRows) return NVFP4_ESHAPE;
  if (!t->global_scale) return NVFP4_EINVAL;
  if (t->rows > 0 && t->cols > 0 && (!t->codes || !t->scales)) return NVFP4_EINVAL;
  if (t->scale_layout == NVFP4_SCALES_TILED && (t->rows % 128 || t->cols % 64))
    return NVFP4_ESHAPE;
  if (!aligned(t->codes, 16) || !aligned(t->scales, 4) || !aligned(t->global_scale, 4))
    return NVFP4_ESHAPE;
  return NVFP4_OK;
}

// Arguments of a quantize call other than its workspace.
int check_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                   const float* amax, const nvfp4_tensor_t* out) {
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (rows < 0 || cols < 0) return NVFP4_EINVAL;
  int st = check_tensor(out);
  if (st) return st;
  if (out->rows != rows || out->cols != cols) return NVFP4_ESHAPE;
  const int64_t elem = x_dtype == NVFP4_BF16 ? 2 : 4;
  if (!stride_ok(ld_x, cols, elem)) return NVFP4_ESHAPE;
  if (rows > 0 && cols > 0 && !x) return NVFP4_EINVAL;
  if (!aligned(x, 16)) return NVFP4_ESHAPE;
  if (amax && !aligned(amax, 4)) return NVFP4_ESHAPE;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

#ifndef NVFP4_SOURCE_HASH
#define NVFP4_SOURCE_HASH "unknown"
#endif
const char* nvfp4_source_hash(void) { return NVFP4_SOURCE_HASH; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_EINVAL: return "invalid argument (null pointer, bad enum or negative size)";
    case NVFP4_ESHAPE: return "unsupported shape, stride or alignment";
    case NVFP4_EWORKSPACE: return "workspace missing or too small";
    case NVFP4_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

size_t nvfp4_workspace_bytes(int32_t op, int64_t a, int64_t b, int64_t c) {
  switch (op) {
    case NVFP4_OP_QUANTIZE: return nvfp4::quantize_workspace_bytes(a, b, c != 0);
    case NVFP4_OP_KV_QUANTIZE: return nvfp4::kv_quantize_workspace_bytes(a, b, c);
    case NVFP4_OP_ADALN_QUANTIZE: return nvfp4::adaln_quantize_workspace_bytes(a, b);
    case NVFP4_OP_KV_ATTENTION:
      return a < 0 || b <= 0 || c < 0 ? 0 : nvfp4::kv_attention_workspace_bytes(a, b, c);
    default: return 0;
  }
}

int nvfp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                   const float* amax, const nvfp4_tensor_t* out, void* workspace,
                   size_t ws_bytes, void* stream) {
  const int st = check_quantize(x, x_dtype, rows, cols, ld_x, amax, out);
  if (st) return st;
  const size_t need = nvfp4::quantize_workspace_bytes(rows, cols, amax != nullptr);
  if (need && (!workspace || ws_bytes < need || !aligned(workspace, 256))) return NVFP4_EWORKSPACE;
  (void)hipGetLastError();
  nvfp4::launch_quantize(x, x_dtype == NVFP4_BF16, rows, cols, ld_x, amax, out->codes,
                         out->scales, out->scale_layout == NVFP4_SCALES_TILED,
                         out->global_scale, workspace, as_stream(stream));
  return finish();
}

int nvfp4_quantize_noalloc(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                           int64_t ld_x, const float* amax, const nvfp4_tensor_t* out,
                           void* stream) {
  const int st = check_quantize(x, x_dtype, rows, cols, ld_x, amax, out);
  if (st) return st;
  // the library's scratch array stands in for the workspace
  const size_t need = nvfp4::quantize_workspace_bytes(rows, cols, amax != nullptr);
  if (need > nvfp4::kQuantizeScratchBytes) return NVFP4_EWORKSPACE;
  void* scratch = nullptr;
  if (need && nvfp4::quantize_scratch(&scratch) != hipSuccess) return NVFP4_EHIP;
  (void)hipGetLastError();
  nvfp4::launch_quantize(x, x_dtype == NVFP4_BF16, rows, cols, ld_x, amax, out->codes,
                         out->scales, out->scale_layout == NVFP4_SCALES_TILED,
                         out->global_scale, scratch, as_stream(stream));
  return finish();
}

int nvfp4_quantize_transposed(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                              int64_t ld_x, const float* amax, const nvfp4_tensor_t* out,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (rows < 0 || cols < 0) return NVFP4_EINVAL;
  int st = check_tensor(out);
  if (st) return st;
  if (out->rows != cols || out->cols != rows) return NVFP4_ESHAPE;
  if (cols % 16 || cols > kMaxCols) return NVFP4_ESHAPE;    // grid.y: 128 input columns each
  const int64_t elem = x_dtype == NVFP4_BF16 ? 2 : 4;
  if (!stride_ok(ld_x, cols, elem)) return NVFP4_ESHAPE;
  if (rows > 0 && cols > 0 && !x) return NVFP4_EINVAL;
  if (!aligned(x, 16)) return NVFP4_ESHAPE;
  if (amax && !aligned(amax, 4)) return NVFP4_ESHAPE;
  const size_t need = nvfp4::quantize_workspace_bytes(rows, cols, amax != nullptr);
  if (need && (!workspace || ws_bytes < need || !aligned(workspace, 256))) return NVFP4_EWORKSPACE;
  (void)hipGetLastError();
  nvfp4::launch_quantize_transposed(x, x_dtype == NVFP4_BF16, rows, cols, ld_x, amax, out->codes,
                                    out->scales, out->scale_layout == NVFP4_SCALES_TILED,
                                    out->global_scale, workspace, as_stream(stream));
  return finish();
}

int nvfp4_adaln_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                         int64_t ld_x, const float* shift, const float* scale,
                         int64_t rows_per_group, float eps, float* row_stats,
                         const nvfp4_tensor_t* out, void* workspace, size_t ws_bytes,
                         void* stream) {
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (rows < 0 || cols < 0 || rows_per_group < 1) return NVFP4_EINVAL;
  if (!(eps > 0.0f) || !(eps < INFINITY)) return NVFP4_EINVAL;
  int st = check_tensor(out);
  if (st) return st;
  if (out->rows != rows || out->cols != cols) return NVFP4_ESHAPE;
  const int64_t elem = x_dtype == NVFP4_BF16 ? 2 : 4;
  if (!stride_ok(ld_x, cols, elem)) return NVFP4_ESHAPE;
  if (rows > 0 && cols > 0 && (!x || !shift || !scale || !row_stats)) return NVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(shift, 16) || !aligned(scale, 16) || !aligned(row_stats, 8))
    return NVFP4_ESHAPE;
  const size_t need = nvfp4::adaln_quantize_workspace_bytes(rows, cols);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256)) return NVFP4_EWORKSPACE;
  (void)hipGetLastError();
  nvfp4::launch_adaln_quantize(x, x_dtype == NVFP4_BF16, rows, cols, ld_x, shift, scale,
                               rows_per_group, eps, row_stats, out->codes, out->scales,
                               out->scale_layout == NVFP4_SCALES_TILED, out->global_scale,
                               workspace, as_stream(stream));
  return finish();
}

int nvfp4_dequantize(const nvfp4_tensor_t* in, void* y, int32_t y_dtype, int64_t ld_y,
                     void* stream) {
  int st = check_tensor(in);
  if (st) return st;
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  const int64_t elem = y_dtype == NVFP4_BF16 ? 2 : 4;
  if (!stride_ok(ld_y, in->cols, elem)) return NVFP4_ESHAPE;
  if (in->rows > 0 && in->cols > 0 && !y) return NVFP4_EINVAL;
  if (!aligned(y, 16)) return NVFP4_ESHAPE;
  (void)hipGetLastError();
  nvfp4::launch_dequantize(in->codes, in->scales, in->scale_layout == NVFP4_SCALES_TILED,
                           in->global_scale, in->rows, in->cols, y, y_dtype == NVFP4_BF16, ld_y,
                           as_stream(stream));
  return finish();
}

int nvfp4_gemm_w4a4(const nvfp4_tensor_t* x, const nvfp4_tensor_t* w, void* y, int32_t y_dtype,
                    int64_t ld_y, float* y_amax, void* stream) {
  int st = check_tensor(x);
  if (st) return st;
  st = check_tensor(w);
  if (st) return st;
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (x->cols != w->cols) return NVFP4_ESHAPE;
  const int64_t M = x->rows, N = w->rows, K = x->cols;
  // K % 16 == 0 (check_tensor); K % 64 != 0 implies row-major scales (a tiled
  // operand has cols % 64 == 0), which the GEMM's ragged-K path assumes
  if (ld_y < N || ld_y > kMaxLd) return NVFP4_ESHAPE;
  if (M > 0 && N > 0 && !y) return NVFP4_EINVAL;
  if (!aligned(y, 4) || (y_amax && !aligned(y_amax, 4))) return NVFP4_ESHAPE;
  if (M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31)) return NVFP4_ESHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  (void)hipGetLastError();
  nvfp4::launch_gemm(x->codes, x->scales, x->scale_layout == NVFP4_SCALES_TILED, x->global_scale,
                     w->codes, w->scales, w->scale_layout == NVFP4_SCALES_TILED, w->global_scale,
                     M, N, K, y, y_dtype == NVFP4_BF16, ld_y, y_amax, as_stream(stream));
  return finish();
}

int64_t nvfp4_kv_page_bytes(int32_t n_heads, int32_t head_dim, int32_t page_tokens) {
  if (n_heads <= 0 || head_dim <= 0 || head_dim % 16 || page_tokens <= 0) return 0;
  return (int64_t)2 * n_heads * page_tokens * (head_dim / 2 + head_dim / 16);
}

static int check_cache(const nvfp4_kv_cache_t* c, int32_t layer, nvfp4::KvGeom* g) {
  if (!c || !c->pool || !c->page_table || !c->page_chunk || !c->k_mean || !c->k_gscale ||
      !c->v_gscale)
    return NVFP4_EINVAL;
  if (c->n_layers <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->page_tokens <= 0 ||
      c->max_pages <= 0 || c->max_chunks <= 0 || c->n_phys_pages <= 0)
    return NVFP4_EINVAL;
  if (c->head_dim % 16 || c->head_dim > 256) return NVFP4_ESHAPE;
  if (layer < 0 || layer >= c->n_layers) return NVFP4_ESHAPE;
  if (!aligned(c->pool, 16) || !aligned(c->k_mean, 16)) return NVFP4_ESHAPE;
  if (nvfp4_kv_page_bytes(c->n_heads, c->head_dim, c->page_tokens) % 16) return NVFP4_ESHAPE;
  if (c->n_heads > 65535) return NVFP4_ESHAPE;
  g->pool = c->pool;
  g->n_heads = c->n_heads;
  g->head_dim = c->head_dim;
  g->page_tokens = c->page_tokens;
  g->max_pages = c->max_pages;
  g->max_chunks = c->max_chunks;
  g->page_table = c->page_table + (int64_t)layer * c->max_pages;
  g->page_chunk = c->page_chunk + (int64_t)layer * c->max_pages * 2;
  g->k_mean = c->k_mean + (int64_t)layer * c->max_chunks * c->n_heads * c->head_dim;
  g->k_gscale = c->k_gscale + (int64_t)layer * c->max_chunks;
  g->v_gscale = c->v_gscale + (int64_t)layer * c->max_chunks;
  g->page_bytes = nvfp4_kv_page_bytes(c->n_heads, c->head_dim, c->page_tokens);
  g->n_phys_pages = c->n_phys_pages;
  return NVFP4_OK;
}

int nvfp4_kv_quantize(const nvfp4_kv_cache_t* cache, int32_t layer, int32_t chunk_id,
                      const void* k_bf16, const void* v_bf16, int64_t T, int64_t start_token,
                      void* workspace, size_t ws_bytes, void* stream) {
  nvfp4::KvGeom g;
  int st = check_cache(cache, layer, &g);
  if (st) return st;
  if (T <= 0 || start_token < 0 || !k_bf16 || !v_bf16) return NVFP4_EINVAL;
  if (!aligned(k_bf16, 16) || !aligned(v_bf16, 16)) return NVFP4_ESHAPE;
  if (chunk_id < 0 || chunk_id >= cache->max_chunks) return NVFP4_ESHAPE;
  if (T < cache->page_tokens && chunk_id != 0) return NVFP4_ESHAPE;
  // a chunk that starts inside a page shares it with the chunk before it, so
  // the first chunk of a layer must start on a page boundary
  if (chunk_id == 0 && start_token % cache->page_tokens != 0) return NVFP4_ESHAPE;
  // the token range must end inside the layer's logical pages (no overflow)
  const int64_t layer_tokens = (int64_t)cache->max_pages * cache->page_tokens;
  if (start_token > layer_tokens || T > layer_tokens - start_token) return NVFP4_ESHAPE;
  // the general quantize kernel runs one workgroup per >= 64 tokens on grid.x
  if (T >= (int64_t(1) << 30)) return NVFP4_ESHAPE;
  const size_t need = nvfp4::kv_quantize_workspace_bytes(T, cache->n_heads, cache->head_dim);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256)) return NVFP4_EWORKSPACE;
  (void)hipGetLastError();
  nvfp4::launch_kv_quantize(g, chunk_id, (const uint16_t*)k_bf16, (const uint16_t*)v_bf16, T,
                            start_token, workspace, as_stream(stream));
  return finish();
}

int nvfp4_kv_dequant_blocks(const nvfp4_kv_cache_t* cache, int32_t layer,
                            const int32_t* logical_pages, int32_t n_pages, void* k_out,
                            void* v_out, void* stream) {
  nvfp4::KvGeom g;
  int st = check_cache(cache, layer, &g);
  if (st) return st;
  if (n_pages < 0) return NVFP4_EINVAL;
  if (n_pages == 0) return NVFP4_OK;
  // one workgroup per 8-token tile of every listed page (a 1-D grid)
  if ((int64_t)((g.page_tokens + 7) / 8) * n_pages >= (int64_t(1) << 32)) return NVFP4_ESHAPE;
  if (!logical_pages || !k_out || !v_out) return NVFP4_EINVAL;
  if (!aligned(k_out, 16) || !aligned(v_out, 16) || !aligned(logical_pages, 4))
    return NVFP4_ESHAPE;
  (void)hipGetLastError();
  nvfp4::launch_kv_dequant(g, logical_pages, n_pages, (uint16_t*)k_out, (uint16_t*)v_out,
                           as_stream(stream));
  return finish();
}

int nvfp4_kv_attention(const nvfp4_kv_cache_t* cache, int32_t layer,
                       const int32_t* logical_pages, int32_t n_pages, int32_t last_page_tokens,
                       const void* q_bf16, int64_t n_q, float softmax_scale, void* out_bf16,
                       void* workspace, size_t ws_bytes, void* stream) {
  nvfp4::KvGeom g;
  int st = check_cache(cache, layer, &g);
  if (st) return st;
  if ((cache->head_dim != 64 && cache->head_dim != 128) || cache->page_tokens % 64)
    return NVFP4_ESHAPE;
  // grid.y is the head; page offsets inside the kernel are 32-bit
  if (cache->n_heads > 65535 || g.page_bytes >= (int64_t(1) << 32)) return NVFP4_ESHAPE;
  if (n_pages < 0 || n_q < 0) return NVFP4_EINVAL;
  if (n_pages > 0 && (last_page_tokens < 0 || last_page_tokens > cache->page_tokens))
    return NVFP4_EINVAL;
  if (n_q == 0) return NVFP4_OK;
  if (!q_bf16 || !out_bf16 || (n_pages > 0 && !logical_pages)) return NVFP4_EINVAL;
  if (!aligned(q_bf16, 16) || !aligned(out_bf16, 8) || (n_pages > 0 && !aligned(logical_pages, 4)))
    return NVFP4_ESHAPE;
  if ((n_q + 127) / 128 >= (int64_t(1) << 31)) return NVFP4_ESHAPE;
  const size_t need = nvfp4::kv_attention_workspace_bytes(
      n_q, cache->n_heads, (int64_t)n_pages * cache->page_tokens);
  if (need && (!workspace || ws_bytes < need || !aligned(workspace, 256))) return NVFP4_EWORKSPACE;
  (void)hipGetLastError();
  nvfp4::launch_kv_attention(g, logical_pages, n_pages, last_page_tokens, (const uint16_t*)q_bf16,
                             n_q, softmax_scale, (uint16_t*)out_bf16, workspace,
                             as_stream(stream));
  return finish();
}

int nvfp4_kv_window_pages(int64_t total_tokens, int32_t page_tokens, int64_t global_sink_tokens,
                          int64_t shot_start, int64_t shot_sink_tokens, int64_t window_tokens,
                          int32_t* pages_dev, int32_t max_pages, int32_t* n_pages,
                          int32_t* last_page_tokens, void* stream) {
  if (!n_pages || !last_page_tokens) return NVFP4_EINVAL;
  if (total_tokens < 0 || page_tokens <= 0 || global_sink_tokens < 0 || shot_start < 0 ||
      shot_sink_tokens < 0 || window_tokens < 0 || max_pages < 0)
    return NVFP4_EINVAL;
  const int64_t P = page_tokens;
  if ((total_tokens + P - 1) / P > INT32_MAX) return NVFP4_ESHAPE;
  // the three token ranges, clipped, as page ranges [a, b)
  int64_t ra[3], rb[3];
  int n = 0;
  // (sums clipped to total_tokens before they could overflow)
  const int64_t shot_end = shot_start >= total_tokens ? total_tokens
                         : shot_sink_tokens > total_tokens - shot_start
                             ? total_tokens
                             : shot_start + shot_sink_tokens;
  const int64_t tok[3][2] = {{0, global_sink_tokens},
                             {shot_start, shot_end},
                             {total_tokens - window_tokens, total_tokens}};
  for (int i = 0; i < 3; ++i) {
    const int64_t a = tok[i][0] < 0 ? 0 : tok[i][0];
    const int64_t b = tok[i][1] > total_tokens ? total_tokens : tok[i][1];
    if (a < b) {
      ra[n] = a / P;
      rb[n] = (b + P - 1) / P;
      ++n;
    }
  }
  // sort by start (at most 3 ranges) and merge overlapping or touching ones
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if (ra[j] < ra[i]) {
        const int64_t ta = ra[i], tb = rb[i];
        ra[i] = ra[j];
        rb[i] = rb[j];
        ra[j] = ta;
        rb[j] = tb;
      }
  int m = 0;
  for (int i = 0; i < n; ++i) {
    if (m > 0 && ra[i] <= rb[m - 1]) {
      if (rb[i] > rb[m - 1]) rb[m - 1] = rb[i];
    } else {
      ra[m] = ra[i];
      rb[m] = rb[i];
      ++m;
    }
  }
  int64_t count = 0;
  for (int i = 0; i < m; ++i) count += rb[i] - ra[i];
  if (count > max_pages) return NVFP4_ESHAPE;
  *n_pages = (int32_t)count;
  *last_page_tokens =
      count ? (int32_t)(total_tokens - P * (rb[m - 1] - 1) < P ? total_tokens - P * (rb[m - 1] - 1) : P)
            : 0;
  if (count == 0) return NVFP4_OK;
  if (!pages_dev) return NVFP4_EINVAL;
  if (!aligned(pages_dev, 4)) return NVFP4_ESHAPE;
  int32_t r[6] = {0, 0, 0, 0, 0, 0};
  for (int i = 0; i < m; ++i) {
    r[2 * i] = (int32_t)ra[i];
    r[2 * i + 1] = (int32_t)rb[i];
  }
  (void)hipGetLastError();
  nvfp4::launch_kv_window_pages(r, m, (int32_t)count, pages_dev, as_stream(stream));
  return finish();
}

}  // extern "C"
