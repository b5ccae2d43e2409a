// NVFP4 quantize and dequantize kernels for gfx950.
//
// Quantize follows the two-level scaling of NVFP4 (techwalker.com LongLive-2.0
// report summary, section 一) in two passes: a tensor-amax pass (skipped when
// a producer already knows max|x|) and one fused pass that, per 16-value
// block, takes the block amax, derives the E4M3 scale and encodes and packs
// the E2M1 codes in registers (the fused scale+quantize kernel the
// ai-manual.ru article credits with a 20% saving).
//
// Layout of work: a workgroup is 4 waves; lane l of wave w handles row
// (64 * blockIdx.x + l) and the 64-column group (4 * blockIdx.y + w), i.e.
// four blocks.  Each lane reads one 128-byte (bf16) or 256-byte (fp32) run with
// 16-byte loads, writes 32 bytes of codes and one dword of scale bytes; in
// the tiled scale layout the 64 lanes' dwords are contiguous.

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

// ------------------------------------------------------------------ amax pass

template <bool kBf16>
__global__ __launch_bounds__(256) void amax_partial_kernel(const void* __restrict__ xv,
                                                           int64_t rows, int64_t cols,
                                                           int64_t ld, float* __restrict__ partial) {
  // 16-byte chunks per row; the host guarantees 16-byte aligned rows
  const int64_t elem = kBf16 ? 2 : 4;
  const int64_t cpr = cols * elem / 16;
  const int64_t total = rows * cpr;
  const int64_t per = (total + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < total ? beg + per : total;
  const char* base = (const char*)xv;
  uint32_t m = 0;                        // max of |x| bit patterns (monotone for |x|)
  int64_t i = beg + threadIdx.x;
  if (i < end) {
    int64_t r = i / cpr, c = i - r * cpr;
    for (; i < end; i += blockDim.x) {
      const u32x4 w = *(const u32x4*)(base + (r * ld * elem) + c * 16);
      if (kBf16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t a = w[j] & 0x7FFF7FFFu;
          m = max(m, max(a & 0xFFFFu, a >> 16));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max(m, w[j] & 0x7FFFFFFFu);
      }
      c += blockDim.x;
      while (c >= cpr) { c -= cpr; ++r; }
    }
  }
  float f = kBf16 ? __uint_as_float(m << 16) : __uint_as_float(m);
  f = wave_max(f);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = f;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ------------------------------------------------------------------ quantize pass

template <bool kBf16>
__device__ __forceinline__ void load_group(const void* xv, int64_t row_off, int64_t col0, int nblk,
                                           float* v) {
  if (kBf16) {
    const uint16_t* p = (const uint16_t*)xv + row_off + col0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < nblk) {
        const u32x4 w0 = *(const u32x4*)(p + 16 * b);
        const u32x4 w1 = *(const u32x4*)(p + 16 * b + 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[16 * b + 2 * j] = bf16_lo(w0[j]);
          v[16 * b + 2 * j + 1] = bf16_hi(w0[j]);
          v[16 * b + 8 + 2 * j] = bf16_lo(w1[j]);
          v[16 * b + 8 + 2 * j + 1] = bf16_hi(w1[j]);
        }
      }
    }
  } else {
    const float* p = (const float*)xv + row_off + col0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < nblk) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 w = *(const f32x4*)(p + 16 * b + 4 * q);
          v[16 * b + 4 * q + 0] = w[0];
          v[16 * b + 4 * q + 1] = w[1];
          v[16 * b + 4 * q + 2] = w[2];
          v[16 * b + 4 * q + 3] = w[3];
        }
      }
    }
  }
}

__device__ __forceinline__ float resolve_amax(const float* amax, const float* partial, int n) {
  if (amax) return *amax;
  float m = 0.0f;
  for (int i = threadIdx.x & 63; i < n; i += 64) m = fmaxf(m, partial[i]);
  return wave_max(m);
}

template <bool kBf16, bool kTiled>
__global__ __launch_bounds__(256) void quantize_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax, const float* __restrict__ partial, int n_partial,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale) {
  const float s_g = global_scale(resolve_amax(amax, partial, n_partial));
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *gscale = s_g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 64 + lane;
  const int64_t g = (int64_t)blockIdx.y * 4 + wave;
  const int64_t col0 = g * 64;
  if (r >= rows || col0 >= cols) return;
  const int64_t left = (cols - col0) / 16;
  const int nblk = left >= 4 ? 4 : (int)left;
  const double six_sg = 6.0 * (double)s_g;

  float v[64];
  load_group<kBf16>(x, r * ld, col0, nblk, v);
  uint32_t cw[8];
  uint32_t sw;
  if (s_g < 0x1p-100f) quantize_group<true>(v, nblk, s_g, six_sg, cw, sw);
  else quantize_group<false>(v, nblk, s_g, six_sg, cw, sw);

  uint8_t* cp = codes + r * (cols / 2) + g * 32;
  if (nblk == 4) {
    *(u32x4*)cp = u32x4{cw[0], cw[1], cw[2], cw[3]};
    *(u32x4*)(cp + 16) = u32x4{cw[4], cw[5], cw[6], cw[7]};
  } else {
    for (int b = 0; b < nblk; ++b) *(u32x2*)(cp + 8 * b) = u32x2{cw[2 * b], cw[2 * b + 1]};
  }
  if (kTiled) {
    const int64_t off = ((r >> 7) * (cols / 64) + g) * 512 + (r & 127) * 4;
    *(uint32_t*)(scales + off) = sw;
  } else {
    uint8_t* sp = scales + r * (cols / 16) + g * 4;
    if (nblk == 4 && (cols % 64) == 0) {
      *(uint32_t*)sp = sw;
    } else {
      for (int b = 0; b < nblk; ++b) sp[b] = (uint8_t)(sw >> (8 * b));
    }
  }
}

// ------------------------------------------------------------------ dequantize

template <bool kTiled, bool kOutBf16>
__global__ __launch_bounds__(256) void dequantize_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ gscale, int64_t rows, int64_t cols, void* __restrict__ y,
    int64_t ld_y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 64 + lane;
  const int64_t g = (int64_t)blockIdx.y * 4 + wave;
  const int64_t col0 = g * 64;
  if (r >= rows || col0 >= cols) return;
  const int64_t left = (cols - col0) / 16;
  const int nblk = left >= 4 ? 4 : (int)left;
  const float s_g = *gscale;

  uint32_t sw;
  if (kTiled) {
    sw = *(const uint32_t*)(scales + ((r >> 7) * (cols / 64) + g) * 512 + (r & 127) * 4);
  } else {
    const uint8_t* sp = scales + r * (cols / 16) + g * 4;
    if (nblk == 4 && (cols % 64) == 0) {
      sw = *(const uint32_t*)sp;
    } else {
      sw = 0;
      for (int b = 0; b < nblk; ++b) sw |= (uint32_t)sp[b] << (8 * b);
    }
  }
  const uint8_t* cp = codes + r * (cols / 2) + g * 32;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b < nblk) {
      const u32x2 cw = *(const u32x2*)(cp + 8 * b);
      const float s_b = e4m3_value((sw >> (8 * b)) & 0xFFu);
      float out[16];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int sel = 0; sel < 4; ++sel) {
          const f32x2 q = e2m1_pair(cw[h], sel);
          const float a0 = q[0] * s_b, a1 = q[1] * s_b;         // exact: <= 6 bits
          if (kOutBf16) {
            out[8 * h + 2 * sel] = mul_for_bf16(a0, s_g);
            out[8 * h + 2 * sel + 1] = mul_for_bf16(a1, s_g);
          } else {
            out[8 * h + 2 * sel] = a0 * s_g;
            out[8 * h + 2 * sel + 1] = a1 * s_g;
          }
        }
      }
      if (kOutBf16) {
        uint16_t* yp = (uint16_t*)y + r * ld_y + col0 + 16 * b;
        u32x4 p0, p1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p0[j] = pack_bf16x2(out[2 * j], out[2 * j + 1]);
          p1[j] = pack_bf16x2(out[8 + 2 * j], out[8 + 2 * j + 1]);
        }
        *(u32x4*)yp = p0;
        *(u32x4*)(yp + 8) = p1;
      } else {
        float* yp = (float*)y + r * ld_y + col0 + 16 * b;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(f32x4*)(yp + 4 * q4) =
              f32x4{out[4 * q4], out[4 * q4 + 1], out[4 * q4 + 2], out[4 * q4 + 3]};
      }
    }
  }
}

// ------------------------------------------------------------------ launchers

static int amax_grid(int64_t rows, int64_t cols, bool bf16) {
  const int64_t chunks = rows * cols * (bf16 ? 2 : 4) / 16;
  int64_t g = (chunks + 255) / 256;
  if (g > kAmaxPartials) g = kAmaxPartials;
  if (g < 1) g = 1;
  return (int)g;
}

size_t quantize_workspace_bytes(int64_t rows, int64_t cols, bool has_amax) {
  (void)rows;
  (void)cols;
  return has_amax ? 0 : (size_t)kAmaxPartials * sizeof(float);
}

void launch_quantize(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld,
                     const float* amax, uint8_t* codes, uint8_t* scales, bool tiled,
                     float* gscale, void* workspace, hipStream_t stream) {
  float* partial = (float*)workspace;
  int n_partial = 0;
  if (!amax) {
    n_partial = amax_grid(rows, cols, x_bf16);
    if (x_bf16)
      hipLaunchKernelGGL(amax_partial_kernel<true>, dim3(n_partial), dim3(256), 0, stream, x,
                         rows, cols, ld, partial);
    else
      hipLaunchKernelGGL(amax_partial_kernel<false>, dim3(n_partial), dim3(256), 0, stream, x,
                         rows, cols, ld, partial);
  }
  const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((cols / 16 + 15) / 16));
  if (rows == 0 || cols == 0) {
    // still publish s_g (1.0 for an empty tensor) with a single idle lane group
    const dim3 one(1, 1);
    if (x_bf16)
      hipLaunchKernelGGL((quantize_kernel<true, false>), one, dim3(256), 0, stream, x, rows,
                         cols, ld, amax, partial, n_partial, codes, scales, gscale);
    else
      hipLaunchKernelGGL((quantize_kernel<false, false>), one, dim3(256), 0, stream, x, rows,
                         cols, ld, amax, partial, n_partial, codes, scales, gscale);
    return;
  }
#define NVFP4_QLAUNCH(B, T)                                                                 \
  hipLaunchKernelGGL((quantize_kernel<B, T>), grid, dim3(256), 0, stream, x, rows, cols, ld, \
                     amax, partial, n_partial, codes, scales, gscale)
  if (x_bf16) {
    if (tiled) NVFP4_QLAUNCH(true, true);
    else NVFP4_QLAUNCH(true, false);
  } else {
    if (tiled) NVFP4_QLAUNCH(false, true);
    else NVFP4_QLAUNCH(false, false);
  }
#undef NVFP4_QLAUNCH
}

void launch_dequantize(const uint8_t* codes, const uint8_t* scales, bool tiled,
                       const float* gscale, int64_t rows, int64_t cols, void* y, bool y_bf16,
                       int64_t ld_y, hipStream_t stream) {
  if (rows == 0 || cols == 0) return;
  const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((cols / 16 + 15) / 16));
#define NVFP4_DLAUNCH(T, B)                                                                  \
  hipLaunchKernelGGL((dequantize_kernel<T, B>), grid, dim3(256), 0, stream, codes, scales,   \
                     gscale, rows, cols, y, ld_y)
  if (tiled) {
    if (y_bf16) NVFP4_DLAUNCH(true, true);
    else NVFP4_DLAUNCH(true, false);
  } else {
    if (y_bf16) NVFP4_DLAUNCH(false, true);
    else NVFP4_DLAUNCH(false, false);
  }
#undef NVFP4_DLAUNCH
}

}  // namespace nvfp4
