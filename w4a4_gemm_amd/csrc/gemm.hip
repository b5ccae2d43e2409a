// W4A4 GEMM on gfx950: Y[M x N] = X[M x K] * W[N x K]^T, both operands NVFP4.
//
// "All matrix multiplications run in 4 bits" (techwalker.com LongLive-2.0
// report summary, section 四, first key).  gfx950's scaled FP4 MFMA takes
// power-of-two (E8M0) scales per 32 values, which cannot carry NVFP4's E4M3
// scale per 16 values exactly.  Instead every product q s_b is formed exactly
// in bf16 (q has <= 2 significant bits, s_b <= 4, so q s_b fits bf16's 8) and
// fed to the bf16 MFMA, whose products are exact in fp32; only the fp32
// accumulation and the final multiply by s_gx s_gw round.
//
// Work decomposition
//   * workgroup tile 256 x BN (BN = 256 or 192), K step 64; four waves in a
//     2 x 2 grid, each owning a 128 x BN/2 block of 32 x 32 accumulators
//     (v_mfma_f32_32x32x16_bf16).
//   * Each K step a thread fetches one 64-value slice of one X row and one W
//     row (32 bytes of codes + one scale dword, read straight from either
//     scale layout), decodes it in registers to 64 bf16 and writes it to LDS.
//     Decoding happens once per workgroup per element; the MFMA operands are
//     then read from LDS with 16-byte loads.  Rows are padded to 144 bytes so
//     that both the stores and the fragment loads are free of bank conflicts.
//   * LDS is double-buffered: step s computes on one buffer while the slice
//     of step s+1, fetched from global memory before the MFMAs, is decoded
//     into the other; one barrier per step.
//   * Workgroups are remapped so that each of the 8 XCDs owns a contiguous run
//     of tiles (better L2 reuse of shared X rows / W rows), grouped 8 tile
//     rows at a time.

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;
constexpr int kBK = 64;
constexpr int kLdsRow = kBK + 8;          // bf16 per padded LDS row (144 bytes)
constexpr int kThreads = 256;

struct Operand {
  const uint8_t* codes;
  const uint8_t* scales;
  bool tiled;
};

// Byte offset of the scale dword (4 blocks of 16) of row r, K step ks.
__device__ __forceinline__ int64_t scale_dword_offset(int64_t r, int ks, int64_t K, bool tiled) {
  return tiled ? ((r >> 7) * (K / 64) + ks) * 512 + (r & 127) * 4 : r * (K / 16) + ks * 4;
}

struct Slice {
  u32x4 c0, c1;      // 64 codes
  uint32_t s;        // 4 scale bytes
};

__device__ __forceinline__ Slice fetch(const Operand& o, int64_t r, int ks, int64_t K) {
  Slice sl;
  const uint8_t* cp = o.codes + r * (K / 2) + ks * 32;
  sl.c0 = *(const u32x4*)cp;
  sl.c1 = *(const u32x4*)(cp + 16);
  sl.s = *(const uint32_t*)(o.scales + scale_dword_offset(r, ks, K, o.tiled));
  return sl;
}

// 8 codes (one dword) times s_b -> 4 dwords of bf16 pairs.  The products are
// exact fp32 numbers with <= 6 significant bits, so their top halves are the
// exact bf16 values.
__device__ __forceinline__ void decode8(uint32_t w, float s_b, uint32_t* out) {
#define NVFP4_DEC(SEL)                                                                 \
  {                                                                                    \
    const f32x2 q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);            \
    const uint32_t lo = __float_as_uint(q[0] * s_b), hi = __float_as_uint(q[1] * s_b); \
    out[SEL] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);                             \
  }
  NVFP4_DEC(0)
  NVFP4_DEC(1)
  NVFP4_DEC(2)
  NVFP4_DEC(3)
#undef NVFP4_DEC
}

__device__ __forceinline__ void decode_to_lds(const Slice& sl, uint16_t* row) {
  const uint32_t cw[8] = {sl.c0[0], sl.c0[1], sl.c0[2], sl.c0[3],
                          sl.c1[0], sl.c1[1], sl.c1[2], sl.c1[3]};
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float s_b = e4m3_value((sl.s >> (8 * b)) & 0xFFu);
    uint32_t o[8];
    decode8(cw[2 * b], s_b, o);
    decode8(cw[2 * b + 1], s_b, o + 4);
    *(u32x4*)(row + 16 * b) = u32x4{o[0], o[1], o[2], o[3]};
    *(u32x4*)(row + 16 * b + 8) = u32x4{o[4], o[5], o[6], o[7]};
  }
}

// Linear workgroup id -> (tile row, tile col): XCD-contiguous, then grouped.
__device__ __forceinline__ void tile_of(int bid, int nbm, int nbn, int& tm, int& tn) {
  const int total = nbm * nbn;
  int t = bid;
  if ((total & 7) == 0) t = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int G = 8;
  const int per_group = G * nbn;
  const int group = t / per_group;
  const int first = group * G;
  const int rows = nbm - first < G ? nbm - first : G;
  const int in = t - group * per_group;
  tm = first + in % rows;
  tn = in / rows;
}

}  // namespace

template <int BN, bool kOutBf16>
__global__ __launch_bounds__(kThreads, 1) void gemm_w4a4_kernel(
    Operand xa, Operand wb, const float* __restrict__ xg, const float* __restrict__ wg, int M,
    int N, int64_t K, void* __restrict__ y, int64_t ld_y, float* __restrict__ y_amax, int nbm,
    int nbn) {
  constexpr int WN = BN / 2;                // wave tile 128 x WN
  constexpr int TM = 4, TN = WN / 32;
  constexpr int kStage = (kBM + BN) * kLdsRow;   // bf16 per LDS stage
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  int tm, tn;
  tile_of(blockIdx.x, nbm, nbn, tm, tn);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = (int)(K / kBK);

  // loader rows (clamped into range; results of clamped rows are never stored)
  const int64_t ar = min((int64_t)tm * kBM + tid, (int64_t)M - 1);
  const bool has_b = tid < BN;
  const int64_t br = min((int64_t)tn * BN + (has_b ? tid : 0), (int64_t)N - 1);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  {
    const Slice a = fetch(xa, ar, 0, K);
    decode_to_lds(a, lds + tid * kLdsRow);
    if (has_b) {
      const Slice b = fetch(wb, br, 0, K);
      decode_to_lds(b, lds + (kBM + tid) * kLdsRow);
    }
  }
  __syncthreads();

  for (int s = 0; s < nk; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nk;
    Slice na, nb;
    if (more) {
      na = fetch(xa, ar, s + 1, K);
      if (has_b) nb = fetch(wb, br, s + 1, K);
    }
    const uint16_t* As = lds + cur * kStage;
    const uint16_t* Bs = As + kBM * kLdsRow;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int kc = kk * 16 + (lane >> 5) * 8;
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const bf16x8*)(As + (wm * 128 + i * 32 + (lane & 31)) * kLdsRow + kc);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *(const bf16x8*)(Bs + (wn * WN + j * 32 + (lane & 31)) * kLdsRow + kc);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      uint16_t* An = lds + (cur ^ 1) * kStage;
      decode_to_lds(na, An + tid * kLdsRow);
      if (has_b) decode_to_lds(nb, An + (kBM + tid) * kLdsRow);
    }
    __syncthreads();
  }

  // epilogue: Y = acc * (s_gx s_gw), rounded once to the output type
  const float scale = (*xg) * (*wg);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = tn * BN + wn * WN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tm * kBM + wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const float v = acc[i][j][r] * scale;
        if (row < M && col < N) {
          if (kOutBf16) {
            const uint32_t b = f32_to_bf16_bits(v);
            ((uint16_t*)y)[(int64_t)row * ld_y + col] = (uint16_t)b;
            amax = fmaxf(amax, __builtin_fabsf(__uint_as_float(b << 16)));
          } else {
            ((float*)y)[(int64_t)row * ld_y + col] = v;
            amax = fmaxf(amax, __builtin_fabsf(v));
          }
        }
      }
    }
  }
  if (y_amax) {
    amax = wave_max(amax);
    if (lane == 0) atomicMax((unsigned int*)y_amax, __float_as_uint(amax));
  }
}

template <int BN, bool kOutBf16>
static void launch_bn(const Operand& xa, const Operand& wb, const float* xg, const float* wg,
                      int64_t M, int64_t N, int64_t K, void* y, int64_t ld_y, float* y_amax,
                      hipStream_t stream) {
  const int nbm = (int)((M + kBM - 1) / kBM), nbn = (int)((N + BN - 1) / BN);
  const size_t lds = 2 * (size_t)(kBM + BN) * kLdsRow * sizeof(uint16_t);
  auto kern = gemm_w4a4_kernel<BN, kOutBf16>;
  // raise the dynamic-LDS limit once per instantiation (thread-safe static init)
  static const bool configured =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)lds) == hipSuccess;
  (void)configured;
  hipLaunchKernelGGL(kern, dim3((unsigned)(nbm * nbn)), dim3(kThreads), lds, stream, xa, wb, xg,
                     wg, (int)M, (int)N, K, y, ld_y, y_amax, nbm, nbn);
}

void launch_gemm(const uint8_t* xc, const uint8_t* xs, bool x_tiled, const float* xg,
                 const uint8_t* wc, const uint8_t* ws, bool w_tiled, const float* wg, int64_t M,
                 int64_t N, int64_t K, void* y, bool y_bf16, int64_t ld_y, float* y_amax,
                 hipStream_t stream) {
  const Operand xa{xc, xs, x_tiled}, wb{wc, ws, w_tiled};
  // Pick the tile width with the shorter estimated run time: the number of
  // waves of workgroups over the 256 CUs times the work of one tile.
  const int64_t nbm = (M + kBM - 1) / kBM;
  const int64_t t256 = nbm * ((N + 255) / 256), t192 = nbm * ((N + 191) / 192);
  auto waves = [](int64_t t) { return (t + 255) / 256; };
  const bool use192 = waves(t192) * 192 < waves(t256) * 256;
  if (use192) {
    if (y_bf16) launch_bn<192, true>(xa, wb, xg, wg, M, N, K, y, ld_y, y_amax, stream);
    else launch_bn<192, false>(xa, wb, xg, wg, M, N, K, y, ld_y, y_amax, stream);
  } else {
    if (y_bf16) launch_bn<256, true>(xa, wb, xg, wg, M, N, K, y, ld_y, y_amax, stream);
    else launch_bn<256, false>(xa, wb, xg, wg, M, N, K, y, ld_y, y_amax, stream);
  }
}

}  // namespace nvfp4
