// Device-side NVFP4 helpers for gfx950 (CDNA4).
//
// NVFP4 (techwalker.com LongLive-2.0 report summary, section 一): E2M1 4-bit
// values, one E4M3 scale per 16 values, one fp32 scale per tensor.  Every
// rounding below reproduces a single round-to-nearest-even of the exact real
// value; the argument for each shortcut is stated where it is used.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;                  // values per E4M3 block scale

// ------------------------------------------------------------------ bit views

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// f32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  uint16_t s;
  __builtin_memcpy(&s, &b, 2);
  return s;
}

// Two fp32 -> one dword of bf16 (lo in bits 15:0), both round to nearest even:
// a vector conversion, which gfx950 does in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ------------------------------------------------------------------ scales

// Value of an E4M3FN byte in 0x00..0x7E (bias 7; exponent field 0 is m/8 * 2^-6).
// gfx950's fp8 -> fp32 conversion uses the OCP E4M3FN encoding; it was checked
// on the device against the bit definition for all 127 finite non-negative
// bytes, and the dequantize parity tests cover every scale byte.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// s_g = RN32(amax / 2688), or 1 when amax == 0.  __fdiv_rn is the correctly
// rounded fp32 quotient.  A nonzero amax below 2688 * 2^-150 would give s_g =
// 0, for which no block scale is defined; s_g is then the smallest positive
// fp32, 2^-149.
__device__ __forceinline__ float global_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  const float q = __fdiv_rn(amax, 2688.0f);
  return q == 0.0f ? 0x1p-149f : q;
}

// E4M3 byte nearest to the exact quotient t = b / six (ties to even,
// saturating at 448), with six = 6 s_g (times the tensor's pre-scaling, which
// also multiplies b).
//
// t64 = RN64(b / six) is on the same side of every E4M3 midpoint as the
// exact t, and equals a midpoint only when t does: b has 24 significant bits
// and six M (M a midpoint, 5 bits) has at most 31, so a nonzero b - six M
// is at least 2^-33 relative, far above fp64's 2^-53 division error.  Rounding
// t64 to 3 mantissa bits with RNE therefore gives the exact answer.
__device__ __forceinline__ uint32_t e4m3_block_scale(float b, double six) {
  double t = (double)b / six;
  if (t >= 464.0) return 0x7Eu;             // [448, 464] rounds to 448; beyond saturates
  if (t < 0x1p-6) {                         // subnormal range: m = RNE(t * 2^9) in 0..8
    return (uint32_t)__builtin_rint(t * 512.0);   // 8 is byte 0x08 = 2^-6
  }
  uint64_t bits = (uint64_t)__double_as_longlong(t);
  bits += (1ull << 48) - 1ull + ((bits >> 49) & 1ull);  // RNE to 3 fraction bits
  return (uint32_t)(bits >> 49) - ((1023u - 7u) << 3);  // rebias exponent 1023 -> 7
}

// ------------------------------------------------------------------ encoding

// Per-tensor encoder constants.
//   pre    1, or 2^64 when s_g < 2^-100: x (and a block's amax) is scaled up
//          exactly so that every reciprocal below stays inside the fp32 range
//          (s_g can be as small as 2^-149); it cancels in the codes and bytes.
//   sg_pre s_g pre, exact, at least 2^-85.
//   i6_lo, i6_hi  bracket R = 1 / (6 sg_pre) from below and above:
//          r = rcp(RN32(6 sg_pre)) is within 2^-22.4 of R (one rounding of the
//          product, one ulp of the reciprocal), and RN32(r (1 -/+ 2^-19))
//          keeps each end more than 2^-19.2 away from R on its side.
struct TensorEnc {
  float s_g, pre, sg_pre, i6_lo, i6_hi;
};

__device__ __forceinline__ TensorEnc make_tensor_enc(float s_g) {
  TensorEnc t;
  t.s_g = s_g;
  t.pre = s_g < 0x1p-100f ? 0x1p64f : 1.0f;
  t.sg_pre = s_g * t.pre;
  const float r = __builtin_amdgcn_rcpf(6.0f * t.sg_pre);
  t.i6_lo = r * (1.0f - 0x1p-19f);
  t.i6_hi = r * (1.0f + 0x1p-19f);
  return t;
}

// Block scale byte = E4M3 value nearest to t = b / (6 s_g) = b pre R.  b pre
// i6_lo < t < b pre i6_hi (each product within 2^-24 of its exact value).
// gfx950's fp32 -> E4M3 conversion is RNE (checked on the device against the
// exact rule for every fp32 in [0, 448]) and monotone, so equal bytes for both
// ends are the byte of t.  Otherwise t lies within about 2^-19 of an E4M3
// midpoint, or on one, and the two bytes are neighbours (consecutive midpoints
// are more than 6 % apart): the exact side of that midpoint Mid decides.
// 6 Mid = 3 (E(lo) + E(hi)) has at most 7 significant bits, so one fp32 FMA
// gives b - 6 Mid s_g with a single rounding; while s_g >= 2^-100 (no
// pre-scaling) that difference is a multiple of 2^-149 and so rounds to zero
// only when it is zero, and its sign is exact.  With pre-scaling the fp64
// quotient decides.  Clamping at 448 is exact: with saturation every t >= 448
// gives 448.  Products below the fp32 normal range are far below 2^-10 and
// give byte 0 either way.
template <bool kPre>
__device__ __forceinline__ uint32_t block_scale_byte(float b, const TensorEnc& t) {
  const float bp = kPre ? b * t.pre : b;                       // exact
  const float tl = fminf(bp * t.i6_lo, 448.0f), th = fminf(bp * t.i6_hi, 448.0f);
  const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(tl, th, 0, false);
  const uint32_t lo = pk & 0xFFu, hi = (pk >> 8) & 0xFFu;
  if (__builtin_expect(lo == hi, 1)) return lo;
  if (kPre) return e4m3_block_scale(bp, 6.0 * (double)t.sg_pre);
  const f32x2 e = __builtin_amdgcn_cvt_pk_f32_fp8((int)pk, false);   // E(lo), E(hi)
  const float d = __builtin_fmaf(-3.0f * (e[0] + e[1]), t.s_g, b);
  return (d > 0.0f || (d == 0.0f && (lo & 1u))) ? hi : lo;     // a tie goes to the even byte
}

// Per-block encoder.  Codes come from gfx950's fp32 -> E2M1 conversion (RNE,
// saturating at 6, sign kept; checked on the device against the exact rule
// for every fp32 with |x| <= 8) applied to y = x c for two multipliers that
// bracket R = 1 / (s_b s_g pre):  p = RN32(s_b s_g pre) (relative error <=
// 2^-24), r = rcp(p) (<= 1 ulp), c = RN32(r (1 -/+ 2^-19)); hence
//   |x| c_lo (1 + 2^-24) < |x| R < |x| c_hi (1 - 2^-24).
// The conversion is monotone, so equal codes for both are the code of |x| R.
// Where they differ (|x| R within about 2^-19 of an E2M1 midpoint M, or on it)
// the exact comparison |x| - M s_b s_g decides: M s_b has at most 7 bits, so
// one fp32 FMA gives that difference with a single rounding and an exact sign.
struct BlockEnc {
  float c_lo, c_hi;   // 0 when s_b == 0: every code is then sign | 0
  float s_b;
};

__device__ __forceinline__ BlockEnc make_block_enc(uint32_t sb_byte, const TensorEnc& t) {
  BlockEnc e;
  e.s_b = e4m3_value(sb_byte);
  const float r = __builtin_amdgcn_rcpf(e.s_b * t.sg_pre);
  e.c_lo = sb_byte ? r * (1.0f - 0x1p-19f) : 0.0f;
  e.c_hi = sb_byte ? r * (1.0f + 0x1p-19f) : 0.0f;
  return e;
}

// x[k] for k in 0..7: a select tree on the bits of k over register copies of
// the values.  The empty asm makes each copy an opaque register value, so the
// selects are not folded into a variable index into x (which would move x out
// of registers).
__device__ __forceinline__ float select8(const float* x, uint32_t k) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = x[i];
    __asm__("" : "+v"(v[i]));
  }
  const bool b0 = (k & 1u) != 0, b1 = (k & 2u) != 0, b2 = (k & 4u) != 0;
  const float a0 = b0 ? v[1] : v[0], a1 = b0 ? v[3] : v[2];
  const float a2 = b0 ? v[5] : v[4], a3 = b0 ? v[7] : v[6];
  const float c0 = b1 ? a1 : a0, c1 = b1 ? a3 : a2;
  return b2 ? c1 : c0;
}

// Codes of 8 values (x already multiplied by `pre`) -> 8 nibbles, value j in
// bits 4j+3..4j (so byte i holds values 2i, 2i+1 with the even one low).
//
// Where the two conversions disagree, hi's magnitude is lo's plus one: the
// conversion is monotone, the products differ by less than 2^-18 relative, and
// neighbouring E2M1 midpoints are at least a factor 1.4 apart.  The exact side
// of the midpoint M between the two magnitudes then decides: M s_b has at most
// 7 significant bits, so one FMA gives |x| - M s_b s_g with a single rounding
// and an exact sign (zero only on a tie, which goes to the even magnitude).
// Each pass of the loop settles one such nibble of the lane; lanes rarely have
// more than one.
__device__ __forceinline__ uint32_t encode8(const float* x, const BlockEnc& e,
                                            const TensorEnc& t) {
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[0] * e.c_lo, x[1] * e.c_lo, 1.0f, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[0] * e.c_hi, x[1] * e.c_hi, 1.0f, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[2] * e.c_lo, x[3] * e.c_lo, 1.0f, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[2] * e.c_hi, x[3] * e.c_hi, 1.0f, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[4] * e.c_lo, x[5] * e.c_lo, 1.0f, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[4] * e.c_hi, x[5] * e.c_hi, 1.0f, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[6] * e.c_lo, x[7] * e.c_lo, 1.0f, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[6] * e.c_hi, x[7] * e.c_hi, 1.0f, 3);
  uint32_t diff = lo ^ hi;
  if (__builtin_expect(diff != 0u, 0)) {
    const float hs = 0.5f * e.s_b;                    // exact
    const float sg_pre = t.sg_pre;
    do {
      const uint32_t sh = (uint32_t)__builtin_ctz(diff) & ~3u;     // bit offset of the nibble
      const uint32_t ml = (lo >> sh) & 7u;                          // magnitude code of lo
      const f32x2 q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ml | ((ml + 1u) << 4), 1.0f, 0);
      const float ms = (q[0] + q[1]) * hs;                          // M s_b, exact
      const float d = __builtin_fmaf(-ms, sg_pre, __builtin_fabsf(select8(x, sh >> 2)));
      lo += (d > 0.0f || (d == 0.0f && (ml & 1u))) ? (1u << sh) : 0u;
      diff &= ~(0xFu << sh);
    } while (diff != 0u);
  }
  return lo;
}

// ------------------------------------------------------------------ 64-value groups

// Quantize `nblk` (1..4) blocks held in v[0 .. 16*nblk) into codes and scale bytes.
template <bool kPre>
__device__ __forceinline__ void quantize_group(float* v, int nblk, const TensorEnc& t,
                                               uint32_t* code_words, uint32_t& scale_word) {
  scale_word = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b < nblk) {
      float bm = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) bm = fmaxf(bm, __builtin_fabsf(v[16 * b + j]));
      const uint32_t sb = block_scale_byte<kPre>(bm, t);
      const BlockEnc enc = make_block_enc(sb, t);
      if (kPre) {
#pragma unroll
        for (int j = 0; j < 16; ++j) v[16 * b + j] *= 0x1p64f;
      }
      code_words[2 * b] = encode8(v + 16 * b, enc, t);
      code_words[2 * b + 1] = encode8(v + 16 * b + 8, enc, t);
      scale_word |= sb << (8 * b);
    }
  }
}

// Dispatch on the (tensor-uniform) pre-scaling.
__device__ __forceinline__ void quantize_group(float* v, int nblk, const TensorEnc& t,
                                               uint32_t* code_words, uint32_t& scale_word) {
  if (t.pre != 1.0f) quantize_group<true>(v, nblk, t, code_words, scale_word);
  else quantize_group<false>(v, nblk, t, code_words, scale_word);
}

// ------------------------------------------------------------------ decoding

// q (E2M1 value) for the two nibbles of byte `sel` of w, as fp32 (exact).
__device__ __forceinline__ f32x2 e2m1_pair(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

// RN_bf16(a * g) with one rounding of the exact product (a has <= 6
// significant bits, g is fp32): p = RN32(a g) gives the right bf16 rounding
// unless p is exactly a bf16 midpoint; then the exact residual a g - p (one
// FMA, exact) says on which side the true product lies, and p is moved one
// fp32 ulp toward it before the RNE conversion.
__device__ __forceinline__ float mul_for_bf16(float a, float g) {
  float p = a * g;
  uint32_t pb = __float_as_uint(p);
  if (__builtin_expect((pb & 0xFFFFu) == 0x8000u, 0)) {
    float r = __builtin_fmaf(a, g, -p);
    if (r != 0.0f) {
      bool away = (r > 0.0f) == (p > 0.0f);          // exact value further from zero
      p = __uint_as_float(away ? pb + 1u : pb - 1u);
    }
  }
  return p;
}

// Whether mul_for_bf16(a, g) can ever take its slow branch for this g, over
// every decoded a = q s_b (q an E2M1 magnitude, s_b an E4M3 scale).  While
// a g is a normal fp32 number, the low bits of RN32(a g) depend only on the
// significands of a and g, and a's significand is one of the 16 products
// {1, 1.5} x (1 + m/8); so testing those 16 values of a decides it for all.
// g below 2^-116 (products that may be subnormal) always answers yes.
__device__ __forceinline__ bool product_needs_check(float g) {
  if (!(g >= 0x1p-116f)) return true;
  bool need = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = ((i & 8) ? 1.5f : 1.0f) * (1.0f + (float)(i & 7) * 0.125f);
    const float p = a * g;
    need |= (__float_as_uint(p) & 0xFFFFu) == 0x8000u && __builtin_fmaf(a, g, -p) != 0.0f;
  }
  return need;
}

// Nonzero unless the fp32 number f is exactly a bf16 midpoint (low 16 bits 0x8000).
__device__ __forceinline__ uint32_t off_midpoint(float f) {
  return (__float_as_uint(f) & 0xFFFFu) ^ 0x8000u;
}

// RN_bf16(a * g + mu) with one rounding of the exact value.  f = RN32(a g + mu)
// (one FMA) decides correctly unless it is exactly a bf16 midpoint; then the
// exact value is compared with f in fp64: A = a g is exact in fp64 (30 bits),
// s + e = A + mu exactly (TwoSum), and (s - f) is exact (Sterbenz), so the sign
// of (s - f) + e is the sign of the true offset from the midpoint.
__device__ __forceinline__ float fma_for_bf16(float a, float g, float mu) {
  float f = __builtin_fmaf(a, g, mu);
  uint32_t fb = __float_as_uint(f);
  if (__builtin_expect((fb & 0xFFFFu) == 0x8000u, 0)) {
    double A = (double)a * (double)g;
    double m = (double)mu;
    double s = A + m;
    double bb = s - A;
    double e = (A - (s - bb)) + (m - bb);
    double off = (s - (double)f) + e;
    if (off != 0.0) {
      bool away = (off > 0.0) == (f > 0.0f);
      f = __uint_as_float(away ? fb + 1u : fb - 1u);
    }
  }
  return f;
}

// ------------------------------------------------------------------ KV decode

// One (token, head) unit of the paged KV cache: 8 codes of K and of V (one
// dword each) and their scale bytes -> K^ = RN_bf16(q s_b s_gK + mu) and
// V^ = RN_bf16(q s_b s_gV) with one rounding each, as 4 dwords of bf16 pairs.
// V: RN32(a s_gV) can land on a bf16 midpoint only for the s_gV that
// product_needs_check() flags (kVCheck, decided per scale); K: the eight fp32
// FMA results are tested together and the exact slow path runs only when one
// of them is a bf16 midpoint.
template <bool kVCheck>
__device__ __forceinline__ void kv_unit_bf16(uint32_t kcw, uint32_t ksb, uint32_t vcw, uint32_t vsb,
                                             float sgk, float sgv, const float* mu, u32x4& ko,
                                             u32x4& vo) {
  const float sbk = e4m3_value(ksb), sbv = e4m3_value(vsb);
  float ka[8], kf[8], vf[8];
  uint32_t off = 0xFFFFFFFFu;
#pragma unroll
  for (int sel = 0; sel < 4; ++sel) {
    const f32x2 qk = e2m1_pair(kcw, sel);
    const f32x2 qv = e2m1_pair(vcw, sel);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int n = 2 * sel + e;
      ka[n] = qk[e] * sbk;                                  // exact
      kf[n] = __builtin_fmaf(ka[n], sgk, mu[n]);
      off = min(off, off_midpoint(kf[n]));
      vf[n] = kVCheck ? mul_for_bf16(qv[e] * sbv, sgv) : (qv[e] * sbv) * sgv;
    }
  }
  if (__builtin_expect(off == 0u, 0)) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      // (the barrier keeps this rare path's fp64 conversion of mu inside it)
      float mun = mu[n];
      __asm__ volatile("" : "+v"(mun));
      kf[n] = fma_for_bf16(ka[n], sgk, mun);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ko[q] = pack_bf16x2(kf[2 * q], kf[2 * q + 1]);
    vo[q] = pack_bf16x2(vf[2 * q], vf[2 * q + 1]);
  }
}

// ------------------------------------------------------------------ reductions

// max(v, v of lane ^ 1): the two lanes of a 16-value block (DPP quad_perm 1,0,3,2).
__device__ __forceinline__ float pair_max(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(o));
}

// Max over the wave (every lane active; values >= 0): DPP within each row of 16
// lanes, then the four row maxima.  The result is wave-uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

}  // namespace nvfp4
