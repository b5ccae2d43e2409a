// W4A4 GEMM on gfx950: Y[M x N] = X[M x K] * W[N x K]^T, both operands NVFP4.
//
// Every matmul of the model runs in 4-bit NVFP4 (techwalker.com LongLive-2.0
// report summary, section 四, first key).  gfx950's scaled FP4 MFMA takes
// power-of-two (E8M0) scales per 32 values, which cannot carry NVFP4's E4M3
// scale per 16 values exactly.  Instead every product q s_b is formed exactly
// in fp16 and fed to the fp16 MFMA: q has <= 2 significant bits and s_b <= 4,
// so q s_b has <= 6 (fp16 keeps 11), and |q s_b| lies in [2^-10, 2688], inside
// fp16's normal range.  The MFMA products are exact in fp32; only the fp32
// accumulation and the final multiply by s_gx s_gw round.  Decoding is two
// instructions per two values: gfx950's fp4 -> fp16 pair conversion and one
// packed fp16 multiply by s_b (both exact, as above, and checked on the device
// over every code and scale byte).
//
// Work decomposition
//   * workgroup tile 256 x BN (BN = 256 or 192), K step 64 (a K that is not a
//     multiple of 64 ends with a partial step, zero-filled); four waves in a
//     2 x 2 grid, each owning a 128 x BN/2 block of 32 x 32 accumulators
//     (v_mfma_f32_32x32x16_f16).
//   * Each K step a thread fetches one 64-value slice of one X row and one W
//     row (32 bytes of codes + one scale dword, read straight from either
//     scale layout), decodes it in registers to 64 fp16 and writes it to LDS.
//     Decoding happens once per workgroup per element; the MFMA operands are
//     then read from LDS with 16-byte loads.  Rows are padded to 144 bytes so
//     that both the stores and the fragment loads are free of bank conflicts.
//   * LDS is double-buffered: step s computes on one buffer while the slice
//     of step s+1, fetched from global memory before the MFMAs, is decoded
//     into the other; one barrier per step.
//   * Workgroups are remapped so that each of the 8 XCDs owns a contiguous run
//     of tiles (better L2 reuse of shared X rows / W rows), grouped 8 tile
//     rows at a time.
//   * Epilogue: a wave tile inside Y is stored with row addresses formed on
//     the scalar unit and a 32-bit offset per lane (three VALU instructions
//     per two bf16 values); tiles on Y's edges check every element.

#include <type_traits>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;
constexpr int kBK = 64;
constexpr int kLdsRow = kBK + 8;          // fp16 per padded LDS row (144 bytes)
constexpr int kThreads = 256;

struct Operand {
  const uint8_t* codes;
  const uint8_t* scales;
  bool tiled;
};

struct Slice {
  u32x4 c0, c1;      // 64 codes
  uint32_t s;        // 4 scale bytes
};

// Per-thread source of one operand row: K step ks reads 32 bytes of codes at
// codes + 32 ks and the scale dword (blocks 4 ks .. 4 ks + 3) at
// scales + ks * sstride.  In the row-major layout the dword follows the
// previous one (stride 4); in the 128-row tiled layout the next 64 columns
// of the same row are one 512-byte tile further on (stride 512).
struct RowSrc {
  const uint8_t* codes;
  const uint8_t* scales;
  int sstride;
};

__device__ __forceinline__ RowSrc row_src(const Operand& o, int64_t r, int64_t K) {
  RowSrc rs;
  rs.codes = o.codes + r * (K / 2);
  rs.scales = o.scales + (o.tiled ? (r >> 7) * (K / 64) * 512 + (r & 127) * 4 : r * (K / 16));
  rs.sstride = o.tiled ? 512 : 4;
  return rs;
}

// Slice of K step ks.  kRag (K % 64 != 0, so row-major scales): rows start on
// 8-byte code and 1-byte scale boundaries, so the slice is read in 8-byte code
// pieces and single scale bytes, and of the last step only its vb valid blocks
// are read (the rest are zero: zero codes with a zero scale contribute 0).
template <bool kRag>
__device__ __forceinline__ Slice fetch(const RowSrc& rs, int ks, int vb) {
  Slice sl;
  const uint8_t* cp = rs.codes + ks * 32;
  if (!kRag) {
    sl.c0 = *(const u32x4*)cp;
    sl.c1 = *(const u32x4*)(cp + 16);
    sl.s = *(const uint32_t*)(rs.scales + (int64_t)ks * rs.sstride);
    return sl;
  }
  const uint8_t* sp = rs.scales + (int64_t)ks * 4;
  uint32_t c[8], s = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int bb = b < vb ? b : vb - 1;             // in-bounds address; value masked below
    const u32x2 v = *(const u32x2*)(cp + 8 * bb);
    const uint32_t sb = sp[bb];
    c[2 * b] = b < vb ? v[0] : 0u;
    c[2 * b + 1] = b < vb ? v[1] : 0u;
    s |= (b < vb ? sb : 0u) << (8 * b);
  }
  sl.c0 = u32x4{c[0], c[1], c[2], c[3]};
  sl.c1 = u32x4{c[4], c[5], c[6], c[7]};
  sl.s = s;
  return sl;
}

// Codes byte SEL of w (two values) times s_b (half HI of the fp16 pair sp):
// one fp4 -> fp16 pair conversion and one packed multiply, both exact
// (products of <= 6 significant bits).
template <int SEL>
__device__ __forceinline__ uint32_t dec2(uint32_t w, uint32_t sp, int hi) {
  const _Float16 s_b = __builtin_bit_cast(f16x2, sp)[hi];
  const f16x2 q = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, q * (f16x2){s_b, s_b});
}

// 8 codes (one dword) times s_b -> 4 dwords of fp16 pairs.
__device__ __forceinline__ void decode8(uint32_t w, uint32_t sp, int hi, uint32_t* out) {
  out[0] = dec2<0>(w, sp, hi);
  out[1] = dec2<1>(w, sp, hi);
  out[2] = dec2<2>(w, sp, hi);
  out[3] = dec2<3>(w, sp, hi);
}

// The four E4M3 scale bytes of a dword as two fp16 pairs (exact: E4M3 fits
// fp16): p[0] = blocks 0, 1; p[1] = blocks 2, 3.
__device__ __forceinline__ void scales4(uint32_t s, uint32_t* p) {
  p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false));
  p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true));
}

__device__ __forceinline__ void decode_to_lds(const Slice& sl, uint16_t* row) {
  const uint32_t cw[8] = {sl.c0[0], sl.c0[1], sl.c0[2], sl.c0[3],
                          sl.c1[0], sl.c1[1], sl.c1[2], sl.c1[3]};
  uint32_t sp[2];
  scales4(sl.s, sp);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t o[8];
    decode8(cw[2 * b], sp[b >> 1], b & 1, o);
    decode8(cw[2 * b + 1], sp[b >> 1], b & 1, o + 4);
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

template <int TM, int TN, int WN>
struct Frags {
  f16x8 a[TM], b[TN];
};

template <int TM, int TN, int WN>
__device__ __forceinline__ void load_frags(Frags<TM, TN, WN>& f, const uint16_t* __restrict__ As,
                                           const uint16_t* __restrict__ Bs, int kk, int lane,
                                           int wm, int wn) {
  const int kc = kk * 16 + (lane >> 5) * 8;
#pragma unroll
  for (int i = 0; i < TM; ++i)
    f.a[i] = *(const f16x8*)(As + (wm * 128 + i * 32 + (lane & 31)) * kLdsRow + kc);
#pragma unroll
  for (int j = 0; j < TN; ++j)
    f.b[j] = *(const f16x8*)(Bs + (wn * WN + j * 32 + (lane & 31)) * kLdsRow + kc);
}

// One K step, software-pipelined, with an explicit instruction order.
//
// On entry `f0` holds the fragments of k16 sub-step 0 of stage As/Bs.  The
// step issues TM*TN*4 MFMAs.  Between consecutive MFMAs it places a slice of
// the decode of the next step (16 units: the 8 code dwords of the X slice and
// the 8 of the W slice, each 4 x {fp4->fp16 pair, one packed multiply} plus
// one 16-byte LDS store into stage An), and during the first MFMAs
// of sub-step kk the fragment loads of kk+1.  Scheduling fences keep that
// order: an MFMA occupies the matrix pipe for 32 cycles, and the VALU work that
// follows it in program order issues underneath instead of queueing behind the
// next MFMA.  The stage pointers are restrict-qualified (the stages never
// overlap), so stores to An may pass loads from As/Bs.
template <int TM, int TN, int WN>
__device__ __forceinline__ void gemm_step(f32x16 (&acc)[TM][TN], Frags<TM, TN, WN>& f0,
                                          Frags<TM, TN, WN>& f1,
                                          const uint16_t* __restrict__ As,
                                          const uint16_t* __restrict__ Bs,
                                          uint16_t* __restrict__ An, const Slice& ca,
                                          const Slice& cb, int tid, int lane, int wm, int wn) {
  constexpr int kSub = kBK / 16;
  constexpr int kPer = TM * TN;                    // MFMAs per sub-step
  constexpr int kTotal = kPer * kSub;              // MFMAs per step
  constexpr int kUnits = 16;                       // decode units per step
  static_assert(kTotal % kUnits == 0, "MFMA count must split evenly over the decode units");
  constexpr int kMpu = kTotal / kUnits;            // MFMAs per decode unit (4 or 3)

  const uint32_t cw[16] = {ca.c0[0], ca.c0[1], ca.c0[2], ca.c0[3], ca.c1[0], ca.c1[1],
                           ca.c1[2], ca.c1[3], cb.c0[0], cb.c0[1], cb.c0[2], cb.c0[3],
                           cb.c1[0], cb.c1[1], cb.c1[2], cb.c1[3]};
  uint32_t sc[4];                                  // fp16 scale pairs: X blocks 0-1, 2-3, W 0-1, 2-3
  scales4(ca.s, sc);
  scales4(cb.s, sc + 2);
  uint16_t* rowA = An + tid * kLdsRow;
  uint16_t* rowB = An + (kBM + tid) * kLdsRow;
  uint32_t out[4];
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int kk = 0; kk < kSub; ++kk) {
    Frags<TM, TN, WN>& cur = (kk & 1) ? f1 : f0;
    Frags<TM, TN, WN>& nxt = (kk & 1) ? f0 : f1;
    const int kc = (kk + 1) * 16 + (lane >> 5) * 8;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int i = kk * kPer + m;                 // MFMA index within the step
      // fragment load for sub-step kk+1 (one per MFMA until all are issued)
      if (kk + 1 < kSub && m < TM + TN) {
        if (m < TM)
          nxt.a[m] = *(const f16x8*)(As + (wm * 128 + m * 32 + (lane & 31)) * kLdsRow + kc);
        else
          nxt.b[m - TM] =
              *(const f16x8*)(Bs + (wn * WN + (m - TM) * 32 + (lane & 31)) * kLdsRow + kc);
      }
      acc[m / TN][m % TN] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
          cur.a[m / TN], cur.b[m % TN], acc[m / TN][m % TN], 0, 0, 0);
      // decode slice: unit u, part p of kMpu; the 4 selectors of the unit's code
      // dword are split over the parts
      const int u = i / kMpu, p = i % kMpu;
      const int sel0 = p * 4 / kMpu, sel1 = (p + 1) * 4 / kMpu;
#pragma unroll
      for (int sel = 0; sel < 4; ++sel) {
        if (sel >= sel0 && sel < sel1) {
          const int blk = (u & 7) >> 1;            // block of code dword u within its slice
          const uint32_t sp = sc[(u >> 3) * 2 + (blk >> 1)];
          out[sel] = sel == 0 ? dec2<0>(cw[u], sp, blk & 1)
                   : sel == 1 ? dec2<1>(cw[u], sp, blk & 1)
                   : sel == 2 ? dec2<2>(cw[u], sp, blk & 1)
                              : dec2<3>(cw[u], sp, blk & 1);
        }
      }
      if (p == kMpu - 1) {
        uint16_t* row = (u < 8) ? rowA : rowB;
        *(u32x4*)(row + 8 * (u & 7)) = u32x4{out[0], out[1], out[2], out[3]};
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One 32 x 32 accumulator tile to Y (lane: column lane % 32; register r:
// row (r / 4) * 8 + (lane / 32) * 4 + r % 4), also folding max |Y| as stored.
// Every element is bounds-checked: the path for wave tiles that straddle an
// edge of Y.
template <bool kOutBf16>
__device__ __forceinline__ void store_tile(const f32x16& a, float scale, void* y, int64_t ld_y,
                                           int row0, int col0, int M, int N, int lane,
                                           float& amax) {
  const int col = col0 + (lane & 31);
  const int rbase = row0 + (lane >> 5) * 4;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = rbase + (r >> 2) * 8 + (r & 3);
    const float v = a[r] * scale;
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

// The same store for a 32 x 32 tile that lies inside Y.  base is the tile's
// first element (wave-uniform, so the row addresses are formed on the scalar
// unit) and off[r] the lane's byte offset of register r's element, which fits
// 32 bits.  Per element that leaves the scale multiply, half a packed bf16
// conversion, half a max3 and the store.  m folds max |acc * scale| before the
// bf16 rounding: rounding is monotone and odd, so the largest stored magnitude
// is m rounded (done once per wave).
template <bool kOutBf16>
__device__ __forceinline__ void store_tile_whole(const f32x16& a, float scale, char* base,
                                                 const uint32_t (&off)[16], float& m) {
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float v0 = a[r] * scale, v1 = a[r + 1] * scale;
    m = fmaxf(m, fmaxf(__builtin_fabsf(v0), __builtin_fabsf(v1)));
    if (kOutBf16) {
      const uint32_t pk = pack_bf16x2(v0, v1);
      *(uint16_t*)(base + (uint64_t)off[r]) = (uint16_t)pk;
      *(uint16_t*)(base + (uint64_t)off[r + 1]) = (uint16_t)(pk >> 16);
    } else {
      *(float*)(base + (uint64_t)off[r]) = v0;
      *(float*)(base + (uint64_t)off[r + 1]) = v1;
    }
  }
}

}  // namespace

template <int BN, bool kOutBf16, bool kRag>
__global__ __launch_bounds__(kThreads, 1) void gemm_w4a4_kernel(
    Operand xa, Operand wb, const float* __restrict__ xg, const float* __restrict__ wg, int M,
    int N, int64_t K, void* __restrict__ y, int64_t ld_y, float* __restrict__ y_amax, int nbm,
    int nbn) {
  constexpr int WN = BN / 2;                // wave tile 128 x WN
  constexpr int TM = 4, TN = WN / 32;
  constexpr int kStage = 2 * kBM * kLdsRow;  // fp16 per LDS stage: 256 A rows + 256 B rows
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  int tm, tn;
  tile_of(blockIdx.x, nbm, nbn, tm, tn);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = (int)((K + kBK - 1) / kBK);      // K steps; the last is partial when kRag
  const int kbt = (int)(K / 16);                  // 16-value blocks along K
  auto vb = [&](int ks) { return kbt - 4 * ks < 4 ? kbt - 4 * ks : 4; };

  // Loader rows, clamped into range (results of clamped rows are never
  // stored).  With BN < 256 the spare threads load a valid W row and write it
  // to LDS rows the MFMAs never read, which keeps the main loop branch-free.
  const RowSrc ra = row_src(xa, min((int64_t)tm * kBM + tid, (int64_t)M - 1), K);
  const RowSrc rb = row_src(wb, min((int64_t)tn * BN + (tid < BN ? tid : BN - 1), (int64_t)N - 1), K);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Pipeline: step s computes on LDS stage s&1, decodes the slices of step
  // s+1 (fetched during step s-1) into the other stage, and issues the global
  // loads of step s+2.  The decode (VALU + LDS stores) and the MFMAs of a step
  // are independent, so they form one basic block that the scheduler
  // interleaves; one barrier per step.
  if (nk > 0) {             // K == 0: no step, Y = 0
    {
      const Slice a0 = fetch<kRag>(ra, 0, vb(0)), b0 = fetch<kRag>(rb, 0, vb(0));
      decode_to_lds(a0, lds + tid * kLdsRow);
      decode_to_lds(b0, lds + (kBM + tid) * kLdsRow);
    }
    const int s1 = nk > 1 ? 1 : 0;
    Slice ca = fetch<kRag>(ra, s1, vb(s1)), cb = fetch<kRag>(rb, s1, vb(s1));
    __syncthreads();
    Frags<TM, TN, WN> f0, f1;
    load_frags(f0, lds, lds + kBM * kLdsRow, 0, lane, wm, wn);

    for (int s = 0; s < nk; ++s) {
      const int cur = s & 1;
      const int s2 = s + 2 < nk ? s + 2 : nk - 1;
      const Slice na = fetch<kRag>(ra, s2, vb(s2)), nb = fetch<kRag>(rb, s2, vb(s2));
      const uint16_t* As = lds + cur * kStage;
      uint16_t* An = lds + (cur ^ 1) * kStage;
      gemm_step<TM, TN, WN>(acc, f0, f1, As, As + kBM * kLdsRow, An, ca, cb, tid, lane, wm, wn);
      __syncthreads();
      load_frags(f0, An, An + kBM * kLdsRow, 0, lane, wm, wn);   // sub-step 0 of the next step
      ca = na;
      cb = nb;
    }
  }

  // epilogue: Y = acc * (s_gx s_gw), rounded once to the output type
  const float scale = (*xg) * (*wg);
  constexpr int kEs = kOutBf16 ? 2 : 4;            // bytes per Y element
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int row_w = tm * kBM + (wave_u >> 1) * 128, col_w = tn * BN + (wave_u & 1) * WN;
  // whole wave tile inside Y, and every lane offset below 2^32 bytes
  const bool whole = row_w + 128 <= M && col_w + WN <= N && ld_y * kEs <= (int64_t(1) << 27);
  float amax = 0.0f;
  if (whole) {
    const int64_t ldb = ld_y * kEs;
    uint32_t off[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      off[r] = (uint32_t)(((lane >> 5) * 4 + (r >> 2) * 8 + (r & 3)) * ldb + (lane & 31) * kEs);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      char* base = (char*)y + ((int64_t)(row_w + i * 32) * ld_y + col_w) * kEs;
#pragma unroll
      for (int j = 0; j < TN; ++j)
        store_tile_whole<kOutBf16>(acc[i][j], scale, base + j * 32 * kEs, off, amax);
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row0 = tm * kBM + wm * 128 + i * 32, col0 = tn * BN + wn * WN + j * 32;
        store_tile<kOutBf16>(acc[i][j], scale, y, ld_y, row0, col0, M, N, lane, amax);
      }
    }
  }
  if (y_amax) {
    amax = wave_max(amax);
    if (kOutBf16 && whole) amax = __uint_as_float(f32_to_bf16_bits(amax) << 16);
    if (lane == 0) atomicMax((unsigned int*)y_amax, __float_as_uint(amax));
  }
}

template <int BN, bool kOutBf16, bool kRag>
static void launch_bn(const Operand& xa, const Operand& wb, const float* xg, const float* wg,
                      int64_t M, int64_t N, int64_t K, void* y, int64_t ld_y, float* y_amax,
                      hipStream_t stream) {
  const int nbm = (int)((M + kBM - 1) / kBM), nbn = (int)((N + BN - 1) / BN);
  const size_t lds = 2 * (size_t)(2 * kBM) * kLdsRow * sizeof(uint16_t);
  auto kern = gemm_w4a4_kernel<BN, kOutBf16, kRag>;
  static std::atomic<uint64_t> lds_done{0};         // per instantiation, per device
  ensure_dynamic_lds((const void*)kern, (int)lds, lds_done);
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
  const bool rag = K % kBK != 0;
  auto go = [&](auto bn, auto out_bf16, auto ragged) {
    launch_bn<decltype(bn)::value, decltype(out_bf16)::value, decltype(ragged)::value>(
        xa, wb, xg, wg, M, N, K, y, ld_y, y_amax, stream);
  };
  using T = std::true_type;
  using F = std::false_type;
  auto go_rag = [&](auto bn, auto out_bf16) { rag ? go(bn, out_bf16, T{}) : go(bn, out_bf16, F{}); };
  auto go_out = [&](auto bn) { y_bf16 ? go_rag(bn, T{}) : go_rag(bn, F{}); };
  if (use192) go_out(std::integral_constant<int, 192>{});
  else go_out(std::integral_constant<int, 256>{});
}

}  // namespace nvfp4
