// NVFP4 quantize and dequantize kernels for gfx950.
//
// Quantize follows the two-level scaling of NVFP4 (techwalker.com LongLive-2.0
// report summary, section 一) in two passes: a tensor-amax pass (skipped when
// a producer already knows max|x|) and one fused pass that, per 16-value
// block, takes the block amax, derives the E4M3 scale and encodes and packs
// the E2M1 codes in registers (the fused scale+quantize kernel the
// ai-manual.ru article credits with a 20% saving).
//
// Layout of work (quantize and dequantize): with L = kLpr lanes per row and
// R = 64 / L rows per wave instruction, a workgroup covers a tile of
// 4 R kTasks rows x 8 L columns.  Lane l of wave w owns 8 consecutive values,
// column chunk j = l % L of the tile, in rows R kTasks w + R t + l / L for
// t < kTasks.  A wave's load instruction therefore reads R rows x 16 L
// contiguous bytes (bf16), two neighbouring lanes form one 16-value block (the
// even one stores its scale byte), a lane's 8 codes are one dword (L lanes
// store 4 L contiguous bytes of a row), and the workgroup's rows lie inside one
// 128-row band of the tiled scale layout.

#include <mutex>
#include <unordered_map>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {
#ifndef NVFP4_QUANT_TASKS
#define NVFP4_QUANT_TASKS 4
#endif
#ifndef NVFP4_QUANT_LPR
#define NVFP4_QUANT_LPR 32
#endif
constexpr int kTile = 128;                   // tile of the transposed quantize
constexpr int kTasks = NVFP4_QUANT_TASKS;    // rows per lane
constexpr int kLpr = NVFP4_QUANT_LPR;        // lanes per row (8 values each)
constexpr int kRpi = 64 / kLpr;              // rows per wave instruction
constexpr int kTileCols = 8 * kLpr;          // columns per workgroup
constexpr int kTileRows = 4 * kRpi * kTasks; // rows per workgroup: 4 waves x kRpi rows x kTasks
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
// `pro(t, v)` maps task t's 8 loaded values to the values that are quantized
// (the identity for a plain quantize).
template <int kN, int kStep, bool kBf16, bool kTiled, bool kPre, typename Prologue>
__device__ __forceinline__ void quantize_tasks(const Raw8* raw, const TensorEnc& te, int64_t r0,
                                               int64_t rows, bool cok, int j,
                                               uint8_t* __restrict__ cp,
                                               uint8_t* __restrict__ sp, int64_t c_step,
                                               int64_t s_step, const Prologue& pro) {
#pragma unroll
  for (int t = 0; t < kN; ++t) {
    float v[8];
    unpack8<kBf16>(raw[t], v);
    pro(t, v);
    float bm = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) bm = fmaxf(bm, __builtin_fabsf(v[e]));
    bm = pair_max(bm);
    const uint32_t sb = block_scale_byte<kPre>(bm, te);
    const BlockEnc enc = make_block_enc(sb, te);
    if (kPre) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= 0x1p64f;
    }
    const uint32_t cw = encode8(v, enc, te);
    if (cok && r0 + kStep * t < rows) {
      *(uint32_t*)(cp + t * c_step) = cw;
      if ((j & 1) == 0) sp[t * s_step] = (uint8_t)sb;
    }
  }
}

// Column tiles are taken from the last to the first (grid.y counts down): a
// producer GEMM writes its output's tile columns from the first to the last,
// so the columns written most recently, still in the Infinity Cache, are read
// first.  For the FFN requantize right after GEMM1 (8192 x 14336) this took
// the in-step time from 78 to 68 us.
template <bool kBf16, bool kTiled>
__global__ __launch_bounds__(256) void quantize_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax, const float* __restrict__ partial,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & (kLpr - 1);
  const int64_t c0 = (int64_t)(gridDim.y - 1 - blockIdx.y) * kTileCols + 8 * j;
  const int64_t r0 = (int64_t)blockIdx.x * kTileRows + kRpi * kTasks * wave + lane / kLpr;
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
    const int64_t r = r0 + kRpi * t;
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
  const int64_t c_step = kRpi * (cols / 2);
  const int64_t s_step = kTiled ? 4 * kRpi : kRpi * (cols / 16);   // tiled: a 128-row band holds every task
  const auto identity = [](int, float*) {};
  if (te.pre != 1.0f)
    quantize_tasks<kTasks, kRpi, kBf16, kTiled, true>(raw, te, r0, rows, cok, j, cp, sp, c_step, s_step,
                                        identity);
  else
    quantize_tasks<kTasks, kRpi, kBf16, kTiled, false>(raw, te, r0, rows, cok, j, cp, sp, c_step, s_step,
                                         identity);
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
  const int j = lane & (kLpr - 1);
  const int64_t c0 = (int64_t)blockIdx.y * kTileCols + 8 * j;
  const int64_t r0 = (int64_t)blockIdx.x * kTileRows + kRpi * kTasks * wave + lane / kLpr;
  if (c0 >= cols) return;

  uint32_t cw[kTasks], sbyte[kTasks];
#pragma unroll
  for (int t = 0; t < kTasks; ++t) {
    const int64_t r = r0 + kRpi * t;
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
    const int64_t r = r0 + kRpi * t;
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

// ------------------------------------------------------------------ transposed quantize
//
// NVFP4 of X^T, blocks of 16 along X's rows: the operand layout of the
// backward GEMMs of NVFP4 training (techwalker.com LongLive-2.0 report
// summary, sections 一 and 五), where dgrad contracts over a weight's rows and
// wgrad over the tokens.  A workgroup stages a 128 x 128 tile of X in LDS,
// row-major with each row's 16-byte chunks XOR-permuted by bits 3..6 of the
// row, then reads it column-wise: lane l of wave w takes output row
// k = 32 w + 4 t + l / 16 (a column of X) and the 8 X rows m = 8 (l % 16) + e,
// the per-lane shape of the plain quantize, so the encoder is shared.  With
// the permutation, a wave's column reads hit distinct LDS banks (two lanes
// per dword for bf16).

template <bool kBf16, bool kTiled>
__global__ __launch_bounds__(256) void quantize_t_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax, const float* __restrict__ partial,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale) {
  constexpr int kTT = kTile / 16;                      // rows per lane (128-row tile)
  constexpr int kElem = kBf16 ? 2 : 4;
  constexpr int kChunks = kTile * kElem / 16;          // 16-byte chunks per tile row
  constexpr int kPerChunk = 16 / kElem;                // elements per chunk
  __shared__ u32x4 tile[kTile * kChunks];              // 32 KB (bf16) or 64 KB (fp32)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int64_t m0 = (int64_t)blockIdx.x * kTile;      // X rows of the tile
  const int64_t k0 = (int64_t)blockIdx.y * kTile;      // X columns of the tile
  const auto swz = [](int mr, int c) { return c ^ ((mr >> 3) & 15); };

  Partials part;
  if (!amax) part = load_partials(partial);
  // stage: rows 32 w + l / 16 + 4 t of the tile, columns 8 j .. 8 j + 7;
  // out-of-range rows / columns load a valid element and are never stored
  {
    const int64_t kc = k0 + 8 * j < cols ? k0 + 8 * j : cols - 8;
    Raw8 in[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) {
      const int64_t m = m0 + 32 * wave + (lane >> 4) + 4 * t;
      in[t] = load8<kBf16>(x, (m < rows ? m : rows - 1) * ld + kc);
    }
#pragma unroll
    for (int t = 0; t < kTT; ++t) {
      const int mr = 32 * wave + (lane >> 4) + 4 * t;
      if (kBf16) {
        tile[mr * kChunks + swz(mr, j)] = in[t].a;
      } else {
        tile[mr * kChunks + swz(mr, 2 * j)] = in[t].a;
        tile[mr * kChunks + swz(mr, 2 * j + 1)] = in[t].b;
      }
    }
  }
  __syncthreads();

  // column reads: task t is output row kr = 32 w + l / 16 + 4 t, X rows 8 j + e
  Raw8 raw[kTT];
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    const int kr = 32 * wave + (lane >> 4) + 4 * t;
    const int c = kr / kPerChunk, off = kr % kPerChunk;
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int mr = 8 * j + e;
      const int idx = mr * kChunks + swz(mr, c);
      if (kBf16)
        w[e] = ((const uint16_t*)tile)[idx * 8 + off];
      else
        w[e] = ((const uint32_t*)tile)[idx * 4 + off];
    }
    if (kBf16) {
      raw[t].a = u32x4{w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16),
                       w[6] | (w[7] << 16)};
      raw[t].b = u32x4{0, 0, 0, 0};
    } else {
      raw[t].a = u32x4{w[0], w[1], w[2], w[3]};
      raw[t].b = u32x4{w[4], w[5], w[6], w[7]};
    }
  }

  float s_g = global_scale(amax ? *amax : reduce_partials(part));
  s_g = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_g)));   // uniform
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *gscale = s_g;
  const TensorEnc te = make_tensor_enc(s_g);

  // the output is [cols x rows]: row k0 + kr, columns m0 + 8 j ..
  const int64_t orows = cols, ocols = rows;
  const int64_t r0 = k0 + 32 * wave + (lane >> 4);
  const int64_t c0 = m0 + 8 * j;
  const bool cok = c0 < ocols;
  const int64_t kb = c0 >> 4;
  uint8_t* cp = codes + r0 * (ocols / 2) + c0 / 2;
  uint8_t* sp = scales + (kTiled ? ((r0 >> 7) * (ocols / 64) + (kb >> 2)) * 512 +
                                       (r0 & 127) * 4 + (kb & 3)
                                 : r0 * (ocols / 16) + kb);
  const int64_t c_step = 4 * (ocols / 2);
  const int64_t s_step = kTiled ? 16 : 4 * (ocols / 16);
  const auto identity = [](int, float*) {};
  if (te.pre != 1.0f)
    quantize_tasks<kTT, 4, kBf16, kTiled, true>(raw, te, r0, orows, cok, j, cp, sp, c_step, s_step,
                                        identity);
  else
    quantize_tasks<kTT, 4, kBf16, kTiled, false>(raw, te, r0, orows, cok, j, cp, sp, c_step, s_step,
                                         identity);
}

// ------------------------------------------------------------------ fused LayerNorm + adaLN + quantize
//
// The producer of a W4A4 linear's activations in a DiT block: LayerNorm of
// each residual row (no affine parameters), the adaLN modulation
// x' = n (1 + scale) + shift with one (shift, scale) pair per group of rows,
// then NVFP4 -- adaLN fused into one kernel (zuobiaodaohang LongLive blog,
// section "NVFP4：数据体积砍到 1/4") and scaling fused with quantization
// (ai-manual.ru LongLive-2.0 article, section "Как это работает под
// капотом").  Two passes over x, as for a plain quantize: the stats pass
// writes each row's (mean, rstd) and per-workgroup maxima of |x'|; the encode
// pass recomputes x' from x and the stored statistics and encodes it.  x'
// itself never goes to memory.

// x' of one element: fp32, one rounding per operation in the formula's order
// (no contraction into fused multiply-adds), so both passes get the same bits.
__device__ __forceinline__ float adaln_value(float x, float mu, float rstd, float gain,
                                             float shift) {
#pragma clang fp contract(off)
  const float n = (x - mu) * rstd;
  return n * gain + shift;
}

template <bool kBf16>
__device__ __forceinline__ void chunk_values(const u32x4 w, float* v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (kBf16) {
      v[2 * j] = bf16_lo(w[j]);
      v[2 * j + 1] = bf16_hi(w[j]);
    } else {
      v[j] = __uint_as_float(w[j]);
    }
  }
}

__device__ __forceinline__ void load_f32(const float* __restrict__ p, float* v, int n) {
#pragma unroll
  for (int k = 0; k < n / 4; ++k) {
    const f32x4 w = *(const f32x4*)(p + 4 * k);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * k + e] = w[e];
  }
}

constexpr int kStatRegChunks = 8;   // 16-byte chunks of a row a lane keeps in registers
constexpr int64_t kModLdsBytes = 64 * 1024;   // LDS for one group's gain and shift vectors

__device__ __forceinline__ void wave_sum2(double& a, double& b) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
  }
}

// One wave, one row: statistics, stored by lane 0; returns this lane's max |x'|.
// The sums run in fp64 about a pivot p (the row's first element):
// s1 = sum (x - p), s2 = sum (x - p)^2, mean = p + s1 / n, var = s2 / n - (s1 / n)^2.
// (p - mean)^2 <= n var, so the subtraction loses at most log2(n) of fp64's
// 53 bits.  mean and rstd are rounded once to fp32.  kRegs: the row (at most
// 64 kStatRegChunks chunks) stays in registers for the modulate sweep;
// otherwise that sweep reads it again (from cache).  kLds: gain (= 1 + scale)
// and shift come from LDS, else from global memory.
template <bool kBf16, bool kRegs, bool kLds>
__device__ __forceinline__ float adaln_row(const u32x4* __restrict__ xr, int64_t cpr,
                                           int64_t cols, const float* gain_or_scale,
                                           const float* shift, float eps, int lane,
                                           float2* __restrict__ st) {
  constexpr int kPer = kBf16 ? 8 : 4;
  constexpr int kU = kRegs ? kStatRegChunks : 1;
  u32x4 w[kU];
  if (kRegs) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = lane + 64 * u;
      w[u] = i < cpr ? xr[i] : u32x4{0, 0, 0, 0};
    }
  }
  auto for_chunks = [&](auto&& f) {
    if (kRegs) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = lane + 64 * u;
        if (i < cpr) {
          float v[kPer];
          chunk_values<kBf16>(w[u], v);
          f(i, v);
        }
      }
    } else {
      for (int64_t i = lane; i < cpr; i += 64) {
        float v[kPer];
        chunk_values<kBf16>(xr[i], v);
        f(i, v);
      }
    }
  };
  const uint32_t first = kRegs ? w[0][0] : xr[0][0];
  const double p = kBf16 ? (double)bf16_lo(__builtin_amdgcn_readfirstlane(first))
                         : (double)__uint_as_float(__builtin_amdgcn_readfirstlane(first));
  double s1 = 0.0, s2 = 0.0;
  for_chunks([&](int64_t, const float* v) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const double d = (double)v[e] - p;
      s1 += d;
      s2 = __builtin_fma(d, d, s2);
    }
  });
  wave_sum2(s1, s2);
  const double a1 = s1 / (double)cols;
  const double var = fmax(s2 / (double)cols - a1 * a1, 0.0);
  const float mu = (float)(p + a1);
  const float rstd = (float)(1.0 / sqrt(var + (double)eps));
  float m = 0.0f;
  for_chunks([&](int64_t i, const float* v) {
    float gv[kPer], shv[kPer];
    if (kLds) {
#pragma unroll
      for (int k = 0; k < kPer / 4; ++k) {
        const f32x4 a = *(const f32x4*)(gain_or_scale + i * kPer + 4 * k);
        const f32x4 b = *(const f32x4*)(shift + i * kPer + 4 * k);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gv[4 * k + e] = a[e];
          shv[4 * k + e] = b[e];
        }
      }
    } else {
      load_f32(gain_or_scale + i * kPer, gv, kPer);
      load_f32(shift + i * kPer, shv, kPer);
#pragma unroll
      for (int e = 0; e < kPer; ++e) gv[e] = 1.0f + gv[e];
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      m = fmaxf(m, __builtin_fabsf(adaln_value(v[e], mu, rstd, gv[e], shv[e])));
  });
  if (lane == 0) *st = make_float2(mu, rstd);
  return m;
}

// Stats pass: workgroup b takes the band of rows [b B, b B + B) and walks it
// one modulation group at a time (kLds: the group's gain and shift vectors are
// staged in LDS once, 8 cols bytes); its 4 waves take the group's rows in
// turn.  Every workgroup writes its partial max |x'| (0 if idle).
template <bool kBf16, bool kLds>
__global__ __launch_bounds__(256) void adaln_stats_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ shift, const float* __restrict__ scale, int64_t rpg, float eps,
    int64_t band, float2* __restrict__ stats, float* __restrict__ partial) {
  extern __shared__ f32x4 mod4[];                 // kLds: gain [cols] then shift [cols]
  float* mod = (float*)mod4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t cpr = cols / (kBf16 ? 8 : 4);
  const int64_t b0 = (int64_t)blockIdx.x * band;
  const int64_t b1 = b0 + band < rows ? b0 + band : rows;
  float m = 0.0f;
  for (int64_t g0 = b0; g0 < b1;) {               // uniform over the workgroup
    const int64_t g = g0 / rpg;
    const int64_t g1 = (g + 1) * rpg < b1 ? (g + 1) * rpg : b1;
    const float* sc = scale + g * cols;
    const float* sh = shift + g * cols;
    if (kLds) {
      __syncthreads();                            // readers of the previous group are done
      for (int64_t i = threadIdx.x; i < cols / 4; i += 256) {
        const f32x4 a = ((const f32x4*)sc)[i];
        mod4[i] = f32x4{1.0f + a[0], 1.0f + a[1], 1.0f + a[2], 1.0f + a[3]};
        mod4[cols / 4 + i] = ((const f32x4*)sh)[i];
      }
      __syncthreads();
    }
    for (int64_t r = g0 + wave; r < g1; r += 4) {
      const u32x4* xr = (const u32x4*)((const char*)x + r * ld * (kBf16 ? 2 : 4));
      const float* gs = kLds ? mod : sc;
      const float* shp = kLds ? mod + cols : sh;
      if (cpr <= 64 * kStatRegChunks)
        m = fmaxf(m, adaln_row<kBf16, true, kLds>(xr, cpr, cols, gs, shp, eps, lane, stats + r));
      else
        m = fmaxf(m, adaln_row<kBf16, false, kLds>(xr, cpr, cols, gs, shp, eps, lane, stats + r));
    }
    g0 = g1;
  }
  m = wave_max(m);
  __shared__ float red[4];
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Encode pass: the plain quantize tiling, with x' computed from the loaded x in
// the prologue.  kTwoGroups: rows_per_group > kRpi (kTasks - 1), so a lane's rows
// r0 .. r0 + kRpi (kTasks - 1) meet at most two modulation groups, whose vectors
// are loaded once; otherwise each task loads its own.
template <bool kBf16, bool kTiled, bool kTwoGroups>
__global__ __launch_bounds__(256) void adaln_quantize_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ shift, const float* __restrict__ scale, int64_t rpg,
    const float2* __restrict__ stats, const float* __restrict__ partial,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & (kLpr - 1);
  const int64_t c0 = (int64_t)blockIdx.y * kTileCols + 8 * j;
  const int64_t r0 = (int64_t)blockIdx.x * kTileRows + kRpi * kTasks * wave + lane / kLpr;
  const bool cok = c0 < cols;

  const Partials part = load_partials(partial);
  const int64_t cl = cok ? c0 : cols - 8;
  Raw8 raw[kTasks];
  float2 st[kTasks];
#pragma unroll
  for (int t = 0; t < kTasks; ++t) {
    const int64_t r = r0 + kRpi * t;
    const int64_t rc = r < rows ? r : rows - 1;
    raw[t] = load8<kBf16>(x, rc * ld + cl);
    st[t] = stats[rc];
  }
  const int64_t ra = r0 < rows ? r0 : rows - 1;   // the lane's rows: r0 .. r0 + kRpi (kTasks - 1)
  const int64_t ga = ra / rpg;
  const int64_t next = (ga + 1) * rpg;      // first row of the following group
  float sha[8], gna[8], shb[8], gnb[8];
  if (kTwoGroups) {
    const int64_t gb = ga + 1 < (rows + rpg - 1) / rpg ? ga + 1 : ga;
    load_f32(shift + ga * cols + cl, sha, 8);
    load_f32(scale + ga * cols + cl, gna, 8);
    load_f32(shift + gb * cols + cl, shb, 8);
    load_f32(scale + gb * cols + cl, gnb, 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gna[e] = 1.0f + gna[e];
      gnb[e] = 1.0f + gnb[e];
    }
  }
  const auto modulate = [&](int t, float* v) {
    const int64_t r = r0 + kRpi * t;
    const int64_t rc = r < rows ? r : rows - 1;
    if (kTwoGroups) {
      const bool b = rc >= next;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = adaln_value(v[e], st[t].x, st[t].y, b ? gnb[e] : gna[e], b ? shb[e] : sha[e]);
    } else {
      const int64_t g = rc / rpg;
      float sh[8], gn[8];
      load_f32(shift + g * cols + cl, sh, 8);
      load_f32(scale + g * cols + cl, gn, 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = adaln_value(v[e], st[t].x, st[t].y, 1.0f + gn[e], sh[e]);
    }
  };

  float s_g = global_scale(reduce_partials(part));
  s_g = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_g)));   // uniform
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *gscale = s_g;
  const TensorEnc te = make_tensor_enc(s_g);

  const int64_t kb = c0 >> 4;
  uint8_t* cp = codes + r0 * (cols / 2) + c0 / 2;
  uint8_t* sp = scales + (kTiled ? ((r0 >> 7) * (cols / 64) + (kb >> 2)) * 512 +
                                       (r0 & 127) * 4 + (kb & 3)
                                 : r0 * (cols / 16) + kb);
  const int64_t c_step = kRpi * (cols / 2);
  const int64_t s_step = kTiled ? 4 * kRpi : kRpi * (cols / 16);
  if (te.pre != 1.0f)
    quantize_tasks<kTasks, kRpi, kBf16, kTiled, true>(raw, te, r0, rows, cok, j, cp, sp, c_step, s_step,
                                        modulate);
  else
    quantize_tasks<kTasks, kRpi, kBf16, kTiled, false>(raw, te, r0, rows, cok, j, cp, sp, c_step, s_step,
                                         modulate);
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
  const dim3 grid((unsigned)((rows + kTileRows - 1) / kTileRows),
                  (unsigned)((cols + kTileCols - 1) / kTileCols));
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

// ------------------------------------------------------------------ allocation-free scratch
//
// Device memory of nvfp4_quantize_noalloc: the amax partials live in this
// file-scope array instead of a caller workspace.  Each device holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, so its device address is looked up once per device (with that
// device current) and only that address is handed to kernels.  Every call on
// one device shares the array; the amax pass rewrites every partial before the
// encode pass reads them, so nothing in it needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[kQuantizeScratchBytes];

hipError_t quantize_scratch(void** ptr) {
  static std::mutex mu;
  static std::unordered_map<int, void*> addr;     // device -> address of `scratch`
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = addr.find(dev);
  if (it != addr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
  addr.emplace(dev, p);
  *ptr = p;
  return hipSuccess;
}

void launch_dequantize(const uint8_t* codes, const uint8_t* scales, bool tiled,
                       const float* gscale, int64_t rows, int64_t cols, void* y, bool y_bf16,
                       int64_t ld_y, hipStream_t stream) {
  if (rows == 0 || cols == 0) return;
  const dim3 grid((unsigned)((rows + kTileRows - 1) / kTileRows),
                  (unsigned)((cols + kTileCols - 1) / kTileCols));
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

size_t adaln_quantize_workspace_bytes(int64_t rows, int64_t cols) {
  (void)rows;
  (void)cols;
  return (size_t)kAmaxPartials * sizeof(float);
}

void launch_adaln_quantize(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ld,
                           const float* shift, const float* scale, int64_t rows_per_group,
                           float eps, float* row_stats, uint8_t* codes, uint8_t* scales,
                           bool tiled, float* gscale, void* workspace, hipStream_t stream) {
  float* partial = (float*)workspace;
  float2* stats = (float2*)row_stats;
  // cols == 0: no row has statistics; only s_g (1) is published.  Rows are
  // dealt in contiguous bands, one per workgroup (all kAmaxPartials write).
  const int64_t srows = cols > 0 ? rows : 0;
  const int64_t band = srows > 0 ? (srows + kAmaxPartials - 1) / kAmaxPartials : 1;
  const size_t lds = (size_t)cols * 8;
  const auto stats_go = [&](auto kernel, size_t bytes) {
    hipLaunchKernelGGL(kernel, dim3(kAmaxPartials), dim3(256), bytes, stream, x, srows, cols, ld,
                       shift, scale, rows_per_group, eps, band, stats, partial);
  };
  if (lds <= (size_t)kModLdsBytes) {
    if (x_bf16) stats_go(adaln_stats_kernel<true, true>, lds);
    else stats_go(adaln_stats_kernel<false, true>, lds);
  } else {
    if (x_bf16) stats_go(adaln_stats_kernel<true, false>, 0);
    else stats_go(adaln_stats_kernel<false, false>, 0);
  }
  if (rows == 0 || cols == 0) {
    hipLaunchKernelGGL(publish_gscale_kernel, dim3(1), dim3(64), 0, stream, nullptr, partial,
                       gscale);
    return;
  }
  const dim3 grid((unsigned)((rows + kTileRows - 1) / kTileRows),
                  (unsigned)((cols + kTileCols - 1) / kTileCols));
  const bool two = rows_per_group > kRpi * (kTasks - 1);
  const auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, x, rows, cols, ld, shift, scale,
                       rows_per_group, stats, partial, codes, scales, gscale);
  };
  if (x_bf16) {
    if (tiled) two ? go(adaln_quantize_kernel<true, true, true>)
                   : go(adaln_quantize_kernel<true, true, false>);
    else two ? go(adaln_quantize_kernel<true, false, true>)
             : go(adaln_quantize_kernel<true, false, false>);
  } else {
    if (tiled) two ? go(adaln_quantize_kernel<false, true, true>)
                   : go(adaln_quantize_kernel<false, true, false>);
    else two ? go(adaln_quantize_kernel<false, false, true>)
             : go(adaln_quantize_kernel<false, false, false>);
  }
}

void launch_quantize_transposed(const void* x, bool x_bf16, int64_t rows, int64_t cols,
                                int64_t ld, const float* amax, uint8_t* codes, uint8_t* scales,
                                bool tiled, float* gscale, void* workspace, hipStream_t stream) {
  float* partial = (float*)workspace;
  if (!amax) {
    if (x_bf16)
      hipLaunchKernelGGL(amax_partial_kernel<true>, dim3(kAmaxPartials), dim3(256), 0, stream,
                         x, rows, cols, ld, partial);
    else
      hipLaunchKernelGGL(amax_partial_kernel<false>, dim3(kAmaxPartials), dim3(256), 0, stream,
                         x, rows, cols, ld, partial);
  }
  if (rows == 0 || cols == 0) {
    hipLaunchKernelGGL(publish_gscale_kernel, dim3(1), dim3(64), 0, stream, amax, partial, gscale);
    return;
  }
  const dim3 grid((unsigned)((rows + kTile - 1) / kTile), (unsigned)((cols + kTile - 1) / kTile));
  const auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, x, rows, cols, ld, amax, partial,
                       codes, scales, gscale);
  };
  if (x_bf16) {
    if (tiled) go(quantize_t_kernel<true, true>);
    else go(quantize_t_kernel<true, false>);
  } else {
    if (tiled) go(quantize_t_kernel<false, true>);
    else go(quantize_t_kernel<false, false>);
  }
}

}  // namespace nvfp4
