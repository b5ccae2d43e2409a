// NVFP4 quantize and dequantize kernels for gfx950.
//
// Quantize follows the two-level scaling of NVFP4 (techwalker.com LongLive-2.0
// report summary, section 一) in two passes: a tensor-amax pass (skipped when
// a producer already knows max|x|) and one fused pass that, per 16-value
// block, takes the block amax, derives the E4M3 scale and encodes and packs
// the E2M1 codes in registers (the fused scale+quantize kernel the
// ai-manual.ru article credits with a 20% saving).
//
// Layout of work (quantize and dequantize): a workgroup covers a tile of 128
// rows x 128 columns.  Lane l of wave w owns 8 consecutive values, column
// chunk j = l % 16 of the tile, in rows 32 w + 4 t + l / 16 for t = 0..7.  A
// wave's load instruction therefore reads 4 rows x 256 contiguous bytes (bf16),
// two neighbouring lanes form one 16-value block (the even one stores its
// scale byte), a lane's 8 codes are one dword (16 lanes store a row's 64
// contiguous bytes), and the workgroup writes both 512-byte tiles of the tiled
// scale layout that its 128 rows touch.

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {
constexpr int kTile = 128;         // tile rows and columns
constexpr int kTasks = 8;          // rows per lane
constexpr int kAmaxUnroll = 8;     // 16-byte loads in flight per lane in the amax pass
}  // namespace

// ------------------------------------------------------------------ amax pass

__device__ __forceinline__ uint32_t fold_abs_bits(uint32_t m, const u32x4 w, bool bf16) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (bf16) {
      const uint32_t a = w[j] & 0x7FFF7FFFu;
      m = max(m, max(a & 0xFFFFu, a >> 16));
    } else {
      m = max(m, w[j] & 0x7FFFFFFFu);
    }
  }
  return m;
}

// Partial max|x| per workgroup, as fp32.  The max of |x| bit patterns is the
// bit pattern of max|x| (finite inputs).  Dense tensors are walked as one flat
// array of 16-byte chunks, consecutive lanes on consecutive chunks; strided
// ones row by row.
template <bool kBf16>
__global__ __launch_bounds__(256) void amax_partial_kernel(const void* __restrict__ xv,
                                                           int64_t rows, int64_t cols,
                                                           int64_t ld, float* __restrict__ partial) {
  const int64_t elem = kBf16 ? 2 : 4;
  const int64_t cpr = cols * elem / 16;             // 16-byte chunks per row (cols % 16 == 0)
  uint32_t m = 0;
  if (ld == cols) {
    const u32x4* p = (const u32x4*)xv;
    const int64_t n = rows * cpr;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += kAmaxUnroll * stride) {
      u32x4 w[kAmaxUnroll];
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u)
        w[u] = i + u * stride < n ? p[i + u * stride] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) m = fold_abs_bits(m, w[u], kBf16);
    }
  } else {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
      const u32x4* p = (const u32x4*)((const char*)xv + r * ld * elem);
      for (int64_t c = threadIdx.x; c < cpr; c += 256) m = fold_abs_bits(m, p[c], kBf16);
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

// 8 values of a lane as fp32 from one 16-byte (bf16) or two 16-byte (fp32) loads.
struct Raw8 {
  u32x4 a, b;
};

// Unconditional loads (the caller clamps the offset into the tensor): keeping
// them out of divergent branches lets the compiler wait for each one
// separately instead of for all of them.
template <bool kBf16>
__device__ __forceinline__ Raw8 load8(const void* x, int64_t off) {
  Raw8 r;
  if (kBf16) {
    r.a = *(const u32x4*)((const uint16_t*)x + off);
    r.b = u32x4{0, 0, 0, 0};
  } else {
    r.a = *(const u32x4*)((const float*)x + off);
    r.b = *(const u32x4*)((const float*)x + off + 4);
  }
  return r;
}

template <bool kBf16>
__device__ __forceinline__ void unpack8(const Raw8& r, float* v) {
  if (kBf16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_lo(r.a[j]);
      v[2 * j + 1] = bf16_hi(r.a[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = __uint_as_float(r.a[j]);
      v[4 + j] = __uint_as_float(r.b[j]);
    }
  }
}

// Tensor amax from the amax pass's kAmaxPartials partials (the pass writes all
// of them): every wave reads them with independent 16-byte loads, so no
// workgroup barrier is needed.
struct Partials {
  f32x4 w[kAmaxPartials / 256];
};

__device__ __forceinline__ Partials load_partials(const float* partial) {
  Partials r;
  const f32x4* p = (const f32x4*)(partial + (kAmaxPartials / 64) * (threadIdx.x & 63));
#pragma unroll
  for (int u = 0; u < kAmaxPartials / 256; ++u) r.w[u] = p[u];
  return r;
}

__device__ __forceinline__ float reduce_partials(const Partials& r) {
  float m = 0.0f;
#pragma unroll
  for (int u = 0; u < kAmaxPartials / 256; ++u)
    m = fmaxf(m, fmaxf(fmaxf(r.w[u][0], r.w[u][1]), fmaxf(r.w[u][2], r.w[u][3])));
  return wave_max(m);
}

// rows == 0 or cols == 0: only s_g is published (1.0 unless amax says otherwise).
__global__ __launch_bounds__(64) void publish_gscale_kernel(const float* __restrict__ amax,
                                                            const float* __restrict__ partial,
                                                            float* __restrict__ gscale) {
  const float m = amax ? *amax : reduce_partials(load_partials(partial));
  if (threadIdx.x == 0) *gscale = global_scale(m);
}

// The 8 row tasks of a lane.  kPre: s_g < 2^-100, x is scaled by 2^64 before
// encoding (a tensor-uniform choice, so the two variants are separate code).
template <bool kBf16, bool kTiled, bool kPre>
__device__ __forceinline__ void quantize_tasks(const Raw8* raw, const TensorEnc& te, int64_t r0,
                                               int64_t rows, bool cok, int j,
                                               uint8_t* __restrict__ cp,
                                               uint8_t* __restrict__ sp, int64_t c_step,
                                               int64_t s_step) {
#pragma unroll
  for (int t = 0; t < kTasks; ++t) {
    float v[8];
    unpack8<kBf16>(raw[t], v);
    float bm = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) bm = fmaxf(bm, __builtin_fabsf(v[e]));
    bm = pair_max(bm);
    const uint32_t sb = block_scale_byte(bm, te);
    const BlockEnc enc = make_block_enc(sb, te);
    if (kPre) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= 0x1p64f;
    }
    const uint32_t cw = encode8(v, enc, te);
    if (cok && r0 + 4 * t < rows) {
      *(uint32_t*)(cp + t * c_step) = cw;
      if ((j & 1) == 0) sp[t * s_step] = (uint8_t)sb;
    }
  }
}

template <bool kBf16, bool kTiled>
__global__ __launch_bounds__(256) void quantize_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax, const float* __restrict__ partial,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int64_t c0 = (int64_t)blockIdx.y * kTile + 8 * j;
  const int64_t r0 = (int64_t)blockIdx.x * kTile + 32 * wave + (lane >> 4);
  const bool cok = c0 < cols;

  // partial maxima first: in-order completion then lets task 0 start as soon
  // as its own load is in
  Partials part;
  if (!amax) part = load_partials(partial);
  // rows >= 1 and cols >= 16 here; out-of-range lanes load a valid element and
  // store nothing (both lanes of a block are in or out together)
  const int64_t cl = cok ? c0 : cols - 8;
  Raw8 raw[kTasks];
#pragma unroll
  for (int t = 0; t < kTasks; ++t) {
    const int64_t r = r0 + 4 * t;
    raw[t] = load8<kBf16>(x, (r < rows ? r : rows - 1) * ld + cl);
  }
  float s_g = global_scale(amax ? *amax : reduce_partials(part));
  s_g = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_g)));   // uniform
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *gscale = s_g;
  const TensorEnc te = make_tensor_enc(s_g);

  // output addresses of task 0; task t is 4 t rows further down
  const int64_t kb = c0 >> 4;                           // block index along the row
  uint8_t* cp = codes + r0 * (cols / 2) + c0 / 2;
  uint8_t* sp = scales + (kTiled ? ((r0 >> 7) * (cols / 64) + (kb >> 2)) * 512 +
                                       (r0 & 127) * 4 + (kb & 3)
                                 : r0 * (cols / 16) + kb);
  const int64_t c_step = 4 * (cols / 2);
  const int64_t s_step = kTiled ? 16 : 4 * (cols / 16);   // tiled: 128-row tiles hold all 8 tasks
  if (te.pre != 1.0f)
    quantize_tasks<kBf16, kTiled, true>(raw, te, r0, rows, cok, j, cp, sp, c_step, s_step);
  else
    quantize_tasks<kBf16, kTiled, false>(raw, te, r0, rows, cok, j, cp, sp, c_step, s_step);
}

// ------------------------------------------------------------------ dequantize

// Same tiling as quantize: per lane and row, one dword of codes and one scale
// byte in, 8 values out (16 or 32 bytes).
template <bool kTiled, bool kOutBf16>
__global__ __launch_bounds__(256) void dequantize_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ gscale, int64_t rows, int64_t cols, void* __restrict__ y,
    int64_t ld_y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int64_t c0 = (int64_t)blockIdx.y * kTile + 8 * j;
  const int64_t r0 = (int64_t)blockIdx.x * kTile + 32 * wave + (lane >> 4);
  if (c0 >= cols) return;

  uint32_t cw[kTasks], sbyte[kTasks];
#pragma unroll
  for (int t = 0; t < kTasks; ++t) {
    const int64_t r = r0 + 4 * t;
    cw[t] = 0;
    sbyte[t] = 0;
    if (r < rows) {
      cw[t] = *(const uint32_t*)(codes + r * (cols / 2) + c0 / 2);
      const int64_t so = kTiled ? ((r >> 7) * (cols / 64) + (c0 >> 6)) * 512 + (r & 127) * 4 +
                                      ((c0 >> 4) & 3)
                                : r * (cols / 16) + (c0 >> 4);
      sbyte[t] = scales[so];
    }
  }
  const float s_g = *gscale;
  // bf16: RN32(q s_b s_g) can be a bf16 midpoint that RN_bf16 would then round
  // the wrong way only for some s_g; decided once (uniform) for this s_g
  const bool check = kOutBf16 && product_needs_check(s_g);

#pragma unroll
  for (int t = 0; t < kTasks; ++t) {
    const int64_t r = r0 + 4 * t;
    if (r >= rows) continue;
    const float s_b = e4m3_value(sbyte[t]);
    float out[8];
#pragma unroll
    for (int sel = 0; sel < 4; ++sel) {
      const f32x2 q = e2m1_pair(cw[t], sel);
      const float a0 = q[0] * s_b, a1 = q[1] * s_b;         // exact: <= 6 bits
      if (check) {
        out[2 * sel] = mul_for_bf16(a0, s_g);
        out[2 * sel + 1] = mul_for_bf16(a1, s_g);
      } else {
        out[2 * sel] = a0 * s_g;
        out[2 * sel + 1] = a1 * s_g;
      }
    }
    if (kOutBf16) {
      u32x4 p;
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = pack_bf16x2(out[2 * e], out[2 * e + 1]);
      *(u32x4*)((uint16_t*)y + r * ld_y + c0) = p;
    } else {
      float* yp = (float*)y + r * ld_y + c0;
      *(f32x4*)yp = f32x4{out[0], out[1], out[2], out[3]};
      *(f32x4*)(yp + 4) = f32x4{out[4], out[5], out[6], out[7]};
    }
  }
}

// ------------------------------------------------------------------ launchers

size_t quantize_workspace_bytes(int64_t rows, int64_t cols, bool has_amax) {
  (void)rows;
  (void)cols;
  return has_amax ? 0 : (size_t)kAmaxPartials * sizeof(float);
}

void launch_quantize(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld,
                     const float* amax, uint8_t* codes, uint8_t* scales, bool tiled,
                     float* gscale, void* workspace, hipStream_t stream) {
  float* partial = (float*)workspace;
  if (!amax) {
    // always kAmaxPartials workgroups: every partial is written (idle ones write 0)
    if (x_bf16)
      hipLaunchKernelGGL(amax_partial_kernel<true>, dim3(kAmaxPartials), dim3(256), 0, stream,
                         x, rows, cols, ld, partial);
    else
      hipLaunchKernelGGL(amax_partial_kernel<false>, dim3(kAmaxPartials), dim3(256), 0, stream,
                         x, rows, cols, ld, partial);
  }
  const dim3 grid((unsigned)((rows + kTile - 1) / kTile), (unsigned)((cols + kTile - 1) / kTile));
  if (rows == 0 || cols == 0) {
    hipLaunchKernelGGL(publish_gscale_kernel, dim3(1), dim3(64), 0, stream, amax, partial, gscale);
    return;
  }
#define NVFP4_QLAUNCH(B, T)                                                                 \
  hipLaunchKernelGGL((quantize_kernel<B, T>), grid, dim3(256), 0, stream, x, rows, cols, ld, \
                     amax, partial, codes, scales, gscale)
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
  const dim3 grid((unsigned)((rows + kTile - 1) / kTile), (unsigned)((cols + kTile - 1) / kTile));
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
