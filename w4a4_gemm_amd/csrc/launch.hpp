// Host-side launchers of the NVFP4 kernels.  Arguments are validated by the
// C ABI layer (capi.cpp) before any of these is called; each launcher only
// picks the launch geometry and enqueues on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace nvfp4 {

// Raise `kernel`'s dynamic-LDS limit to `bytes` on the current device, once per
// device: `done` is the calling launcher's own bit set (bit d: device d is
// configured).  A failure is left to the launch, which then reports it.
inline void ensure_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  if (dev < 0 || dev >= 64) {                     // beyond the bit set: set it every time
    (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return;
  }
  const uint64_t bit = uint64_t(1) << dev;
  if (done.load(std::memory_order_acquire) & bit) return;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) ==
      hipSuccess)
    done.fetch_or(bit, std::memory_order_release);
}

// ---- quantize / dequantize (quant.hip)
constexpr int kAmaxPartials = 1024;   // partial maxima written by the amax pass (multiple of 256)

// Workspace floats used by the amax pass (partials), 256-byte rounded.
size_t quantize_workspace_bytes(int64_t rows, int64_t cols, bool has_amax);

void launch_quantize(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld,
                     const float* amax, uint8_t* codes, uint8_t* scales, bool tiled,
                     float* gscale, void* workspace, hipStream_t stream);

// Size of the file-scope device array that nvfp4_quantize_noalloc uses in
// place of a workspace, and its address on the current device (looked up once
// per device; no allocation).
constexpr size_t kQuantizeScratchBytes = 4096;
static_assert(kAmaxPartials * sizeof(float) <= kQuantizeScratchBytes, "scratch holds the partials");
hipError_t quantize_scratch(void** ptr);

void launch_dequantize(const uint8_t* codes, const uint8_t* scales, bool tiled,
                       const float* gscale, int64_t rows, int64_t cols, void* y, bool y_bf16,
                       int64_t ld_y, hipStream_t stream);

// NVFP4 of X^T (blocks along X's rows) into a [cols x rows] tensor (quant.hip);
// same workspace as launch_quantize.
void launch_quantize_transposed(const void* x, bool x_bf16, int64_t rows, int64_t cols,
                                int64_t ld, const float* amax, uint8_t* codes, uint8_t* scales,
                                bool tiled, float* gscale, void* workspace, hipStream_t stream);

// Fused LayerNorm + adaLN modulate + quantize (quant.hip); row_stats is
// [rows][2] fp32 (mean, rstd), shift/scale [groups][cols] fp32.
size_t adaln_quantize_workspace_bytes(int64_t rows, int64_t cols);

void launch_adaln_quantize(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld,
                           const float* shift, const float* scale, int64_t rows_per_group,
                           float eps, float* row_stats, uint8_t* codes, uint8_t* scales,
                           bool tiled, float* gscale, void* workspace, hipStream_t stream);

// ---- W4A4 GEMM (gemm.hip)
void launch_gemm(const uint8_t* xc, const uint8_t* xs, bool x_tiled, const float* xg,
                 const uint8_t* wc, const uint8_t* ws, bool w_tiled, const float* wg,
                 int64_t M, int64_t N, int64_t K, void* y, bool y_bf16, int64_t ld_y,
                 float* y_amax, hipStream_t stream);

// ---- KV cache (kv.hip)
struct KvGeom {
  uint8_t* pool;
  int32_t n_heads, head_dim, page_tokens, max_pages, max_chunks;
  const int32_t* page_table;  // this layer's row
  int32_t* page_chunk;        // this layer's row
  float* k_mean;              // this layer's [max_chunks][H][D]
  float* k_gscale;            // this layer's [max_chunks]
  float* v_gscale;
  int64_t page_bytes;
  int64_t n_phys_pages;
};

size_t kv_quantize_workspace_bytes(int64_t T, int64_t H, int64_t D);

void launch_kv_quantize(const KvGeom& g, int32_t chunk_id, const uint16_t* k, const uint16_t* v,
                        int64_t T, int64_t start_token, void* workspace, hipStream_t stream);

// Fused window attention (kv_attn.hip): head_dim 64 or 128, page_tokens % 64 == 0.
int attention_splits(int64_t n_q, int64_t n_heads, int64_t n_keys);
size_t kv_attention_workspace_bytes(int64_t n_q, int64_t n_heads, int64_t n_keys);
void launch_kv_attention(const KvGeom& g, const int32_t* logical_pages, int32_t n_pages,
                         int32_t last_page_tokens, const uint16_t* q, int64_t n_q,
                         float softmax_scale, uint16_t* out, void* workspace,
                         hipStream_t stream);

// Page list of a window (kv.hip): `ranges` holds m disjoint, increasing page
// ranges [r[2i], r[2i+1]) with `count` pages in total.
void launch_kv_window_pages(const int32_t* ranges, int m, int32_t count, int32_t* pages,
                            hipStream_t stream);

void launch_kv_dequant(const KvGeom& g, const int32_t* logical_pages, int32_t n_pages,
                       uint16_t* k_out, uint16_t* v_out, hipStream_t stream);

}  // namespace nvfp4
