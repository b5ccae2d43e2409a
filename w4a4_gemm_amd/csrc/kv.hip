// Paged NVFP4 KV cache kernels for gfx950.
//
// Write path (techwalker.com LongLive-2.0 report summary, section 四, second
// key: K is mean-subtracted, then K and V are stored in NVFP4; zuobiaodaohang
// LongLive blog: the quantized cache is updated in place):
//   1. kv_stats:     one read of K and V: per (head, channel) fp64 sum, min,
//                    max and smallest nonzero |K| over a token slice; per
//                    workgroup max|V|.
//   2. kv_finalize:  per channel mu = RN32(S / T) (S exact: the fp64 sum when
//                    the channel's range allows, else an integer sum of the
//                    channel); max|K - mu| from min/max
//                    (RN32 is monotone, so max |RN32(K - mu)| is
//                    max(RN32(Kmax - mu), RN32(mu - Kmin))); mu is stored.
//   3. kv_quantize:  second read (usually from the 256 MB Infinity Cache):
//                    K' = RN32(K - mu), K' and V quantized along head_dim into
//                    the pages named by the page table, in place.
// Read path (same section: one parallel kernel decompresses many cache
// blocks of a window): kv_dequant, one grid over (listed page, head, slot
// tile), K^ = RN_bf16(q s_b s_gK + mu), V^ = RN_bf16(q s_b s_gV).

#include <type_traits>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kStatsSlices = 32;          // token slices of the stats pass
constexpr int kStatsCols = 64;            // channels per stats workgroup (8 lanes x 8)
constexpr int kFinalizeThreads = 256;
static_assert(kStatsSlices % 8 == 0, "the finalize folds the slices eight at a time");

struct KvWorkspace {
  double* sum;      // [slices][C]
  float* kmin;      // [slices][C]
  float* kmax;      // [slices][C]
  uint32_t* knz;    // [slices][C]: smallest nonzero |K| as fp32 bits, minus one (all ones: none)
  float* vamax;     // [stats workgroups]
  float* kamax;     // [finalize workgroups]
  float* vamax_f;   // [finalize workgroups]: the stats partials of V folded per finalize workgroup
};

inline size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

KvWorkspace carve(void* ws, int64_t C, int n_stats_wg, int n_fin_wg) {
  char* p = (char*)ws;
  KvWorkspace w;
  w.sum = (double*)p;
  p += round256(sizeof(double) * kStatsSlices * C);
  w.kmin = (float*)p;
  p += round256(sizeof(float) * kStatsSlices * C);
  w.kmax = (float*)p;
  p += round256(sizeof(float) * kStatsSlices * C);
  w.knz = (uint32_t*)p;
  p += round256(sizeof(uint32_t) * kStatsSlices * C);
  w.vamax = (float*)p;
  p += round256(sizeof(float) * n_stats_wg);
  w.kamax = (float*)p;
  p += round256(sizeof(float) * n_fin_wg);
  w.vamax_f = (float*)p;
  return w;
}

int stats_wgs(int64_t C) { return (int)((C + kStatsCols - 1) / kStatsCols) * kStatsSlices; }
int finalize_wgs(int64_t C) { return (int)((C + kFinalizeThreads - 1) / kFinalizeThreads); }

}  // namespace

size_t kv_quantize_workspace_bytes(int64_t T, int64_t H, int64_t D) {
  (void)T;
  const int64_t C = H * D;
  return round256(sizeof(double) * kStatsSlices * C) + 3 * round256(sizeof(float) * kStatsSlices * C) +
         round256(sizeof(float) * stats_wgs(C)) + 2 * round256(sizeof(float) * finalize_wgs(C));
}

// ------------------------------------------------------------------ 1. stats

// Workgroup (colgroup, slice): 8 lanes cover 64 channels (8 each, one 16-byte
// load), 32 token lanes stride over the slice's tokens, kStatsUnroll tokens at
// a time.
constexpr int kStatsUnroll = 8;
__global__ __launch_bounds__(256) void kv_stats_kernel(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       int64_t T, int64_t C, KvWorkspace ws) {
  const int cg = blockIdx.x / kStatsSlices, slice = blockIdx.x % kStatsSlices;
  const int cl = threadIdx.x & 7, tl = threadIdx.x >> 3;     // 8 channel lanes x 32 token lanes
  const int64_t c0 = (int64_t)cg * kStatsCols + cl * 8;
  const int64_t per = (T + kStatsSlices - 1) / kStatsSlices;
  const int64_t t0 = slice * per, t1 = t0 + per < T ? t0 + per : T;
  double s[8];
  float mn[8], mx[8];
  uint32_t nz[8];        // smallest nonzero |K| bits minus one (zero wraps to all ones)
  uint32_t va = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s[j] = 0.0;
    mn[j] = __builtin_inff();
    mx[j] = -__builtin_inff();
    nz[j] = 0xFFFFFFFFu;
  }
  const bool active = c0 < C;
  if (active && t0 < t1) {
    // kStatsUnroll tokens' loads in flight per lane; a token past the slice
    // loads the slice's last row again (min, max and amax unchanged) and is
    // left out of the sum
    for (int64_t tb = t0 + tl; tb < t1; tb += 32 * kStatsUnroll) {
      u32x4 kw[kStatsUnroll], vw[kStatsUnroll];
#pragma unroll
      for (int u = 0; u < kStatsUnroll; ++u) {
        const int64_t t = tb + 32 * u < t1 ? tb + 32 * u : t1 - 1;
        kw[u] = *(const u32x4*)(k + t * C + c0);
        vw[u] = *(const u32x4*)(v + t * C + c0);
      }
#pragma unroll
      for (int u = 0; u < kStatsUnroll; ++u) {
        const bool in = tb + 32 * u < t1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = bf16_lo(kw[u][j]), b = bf16_hi(kw[u][j]);
          s[2 * j] += in ? (double)a : 0.0;
          s[2 * j + 1] += in ? (double)b : 0.0;
          mn[2 * j] = fminf(mn[2 * j], a);
          mn[2 * j + 1] = fminf(mn[2 * j + 1], b);
          mx[2 * j] = fmaxf(mx[2 * j], a);
          mx[2 * j + 1] = fmaxf(mx[2 * j + 1], b);
          nz[2 * j] = min(nz[2 * j], (__float_as_uint(a) & 0x7FFFFFFFu) - 1u);
          nz[2 * j + 1] = min(nz[2 * j + 1], (__float_as_uint(b) & 0x7FFFFFFFu) - 1u);
          const uint32_t av = vw[u][j] & 0x7FFF7FFFu;
          va = max(va, max(av & 0xFFFFu, av >> 16));
        }
      }
    }
  }
  // reduce the 32 token lanes of each channel through LDS (fixed order)
  __shared__ double ssum[32][kStatsCols + 1];
  __shared__ float smin[32][kStatsCols + 1];
  __shared__ float smax[32][kStatsCols + 1];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ssum[tl][cl * 8 + j] = s[j];
    smin[tl][cl * 8 + j] = mn[j];
    smax[tl][cl * 8 + j] = mx[j];
  }
  float vf = wave_max(__uint_as_float(va << 16));
  __shared__ float svmax[4];
  if ((threadIdx.x & 63) == 0) svmax[threadIdx.x >> 6] = vf;
  __syncthreads();
  if (threadIdx.x < kStatsCols) {
    const int ch = threadIdx.x;
    double a = 0.0;
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int i = 0; i < 32; ++i) {
      a += ssum[i][ch];
      lo = fminf(lo, smin[i][ch]);
      hi = fmaxf(hi, smax[i][ch]);
    }
    const int64_t c = (int64_t)cg * kStatsCols + ch;
    if (c < C) {
      ws.sum[slice * C + c] = a;
      ws.kmin[slice * C + c] = lo;
      ws.kmax[slice * C + c] = hi;
    }
  }
  // the smallest nonzero |K| through smin's space once it has been read (an
  // array of its own would cost a resident workgroup per CU)
  __syncthreads();
  uint32_t(*snz)[kStatsCols + 1] = (uint32_t(*)[kStatsCols + 1])smin;
#pragma unroll
  for (int j = 0; j < 8; ++j) snz[tl][cl * 8 + j] = nz[j];
  __syncthreads();
  if (threadIdx.x < kStatsCols) {
    const int ch = threadIdx.x;
    uint32_t z = 0xFFFFFFFFu;
    for (int i = 0; i < 32; ++i) z = min(z, snz[i][ch]);
    const int64_t c = (int64_t)cg * kStatsCols + ch;
    if (c < C) ws.knz[slice * C + c] = z;
  }
  if (threadIdx.x == 0)
    ws.vamax[blockIdx.x] = fmaxf(fmaxf(svmax[0], svmax[1]), fmaxf(svmax[2], svmax[3]));
}

// ------------------------------------------------------------------ 2. finalize

// mu = RN32(S / T) from the exact fp64 sum S.  q = RN64(S / T) is correctly
// rounded; converting it to fp32 can only differ from RN32(S / T) when q is
// exactly an fp32 midpoint, in which case the sign of S - q T (one fp64 FMA,
// exact sign) tells on which side the true quotient lies.
__device__ __forceinline__ float mean_rn32(double S, int64_t T) {
  const double Td = (double)T;
  const double q = S / Td;
  float f = (float)q;
  const double df = (double)f;
  if (df != q) {
    // the fp32 neighbour of q on the other side; q is a midpoint if equidistant
    const float f2 = nextafterf(f, q > df ? __builtin_inff() : -__builtin_inff());
    if ((double)f2 - q == q - df) {
      const double r = __builtin_fma(-q, Td, S);               // sign of S/T - q
      if (r != 0.0) f = r > 0.0 ? fmaxf(f, f2) : fminf(f, f2);
    }
  }
  return f;
}

// The exact sum for a channel whose values span too many binades for fp64:
// every bf16 value is m 2^(max(E, 1) - 134) with m < 2^8 (E the exponent
// field), so S is an integer in units of 2^-133 below 2^(8 + 254 + log2 T);
// positive and negative parts are summed in five 64-bit limbs each.
__device__ __forceinline__ void add_shifted(uint64_t (&a)[5], uint32_t m, int sh) {
  const int limb = sh >> 6, off = sh & 63;
  const uint64_t lo = (uint64_t)m << off;
  const uint64_t hi = off > 56 ? (uint64_t)m >> (64 - off) : 0;
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint64_t add = i == limb ? lo : (i == limb + 1 ? hi : 0);
    const uint64_t s1 = a[i] + add;
    const uint64_t s2 = s1 + carry;
    carry = (uint64_t)(s1 < add) | (uint64_t)(s2 < carry);
    a[i] = s2;
  }
}

// limb j of a (a select over the five, so the limbs stay in registers)
__device__ __forceinline__ uint64_t pick(const uint64_t (&a)[5], int j) {
  uint64_t v = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) v = i == j ? a[i] : v;
  return v;
}

// a += the a of lane ^ off (exact: five-limb addition with carries)
__device__ __forceinline__ void add_lane_xor(uint64_t (&a)[5], int off) {
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)a[i], off, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(a[i] >> 32), off, 64);
    const uint64_t b = ((uint64_t)hi << 32) | lo;
    const uint64_t s1 = a[i] + b;
    const uint64_t s2 = s1 + carry;
    carry = (uint64_t)(s1 < b) | (uint64_t)(s2 < carry);
    a[i] = s2;
  }
}

// mu = RN32(S / T) for channel c of K ([T][C] bf16) from the exact integer sum,
// computed by the whole wave (every lane calls it with the same c; the result
// is uniform): lane l sums tokens l, l + 64, ..., and the 64 partial sums are
// added exactly across lanes.  The top 64 bits N of |S| (the rest folded into
// a sticky bit) are divided by T, which leaves at least 25 quotient bits for
// T < 2^39, and the quotient is rounded to fp32 (ties to even, subnormal
// results included).  It runs only for channels that fail the fp64 exactness
// test below.
__device__ __forceinline__ float exact_mean_wave(const uint16_t* __restrict__ k, int64_t T,
                                                 int64_t C, int64_t c, int lane) {
  uint64_t P[5] = {0, 0, 0, 0, 0}, N[5] = {0, 0, 0, 0, 0};
  constexpr int kU = 4;                                   // loads in flight per lane
  for (int64_t t0 = lane; t0 < T; t0 += 64 * kU) {
    uint32_t uv[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int64_t t = t0 + 64 * j;
      uv[j] = t < T ? (uint32_t)k[t * C + c] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const uint32_t u = uv[j];
      const uint32_t mag = u & 0x7FFFu, E = mag >> 7;
      if (mag == 0) continue;
      const uint32_t m = (mag & 0x7Fu) | (E ? 0x80u : 0u);
      const int sh = (int)(E ? E : 1u) - 1;
      if (u & 0x8000u) add_shifted(N, m, sh);
      else add_shifted(P, m, sh);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    add_lane_xor(P, off);
    add_lane_xor(N, off);
  }
  bool neg = false;
  for (int i = 4; i >= 0; --i) {
    if (P[i] != N[i]) {
      neg = N[i] > P[i];
      break;
    }
  }
  uint64_t D[5];
  uint64_t borrow = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint64_t x = neg ? N[i] : P[i], y = neg ? P[i] : N[i];
    const uint64_t d1 = x - y, d2 = d1 - borrow;
    borrow = (uint64_t)(x < y) | (uint64_t)(d1 < borrow);
    D[i] = d2;
  }
  int top = -1;
#pragma unroll
  for (int i = 0; i < 5; ++i) top = D[i] != 0 ? i : top;
  if (top < 0) return 0.0f;
  const int n = 64 * top + (64 - __builtin_clzll(pick(D, top)));   // bit length of |S|
  uint64_t Nt;
  bool sticky = false;
  if (n <= 64) {
    Nt = D[0] << (64 - n);
  } else {
    const int sft = n - 64, li = sft >> 6, lo = sft & 63;
    const uint64_t dl = pick(D, li), dh = pick(D, li + 1);
    Nt = lo ? (dl >> lo) | (dh << (64 - lo)) : dl;
    sticky = lo ? (dl & ((1ull << lo) - 1)) != 0 : false;
#pragma unroll
    for (int i = 0; i < 5; ++i) sticky = sticky || (i < li && D[i] != 0);
  }
  const uint64_t Tu = (uint64_t)T, Q = Nt / Tu, R = Nt % Tu;
  const bool st = sticky || R != 0;
  const int qb = 64 - __builtin_clzll(Q);
  const int lsb = n - 197;                                          // exponent of Q's last bit
  const int target = max(qb - 1 + lsb - 23, -149);                  // exponent of the fp32 ulp
  const int shift = target - lsb;                                   // >= 1
  uint32_t mant;
  if (shift >= 65) {
    mant = 0;
  } else if (shift == 64) {
    mant = (Q > (1ull << 63) || (Q == (1ull << 63) && st)) ? 1u : 0u;
  } else {
    mant = (uint32_t)(Q >> shift);
    const uint64_t rem = Q & ((1ull << shift) - 1), half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (st || (mant & 1u)))) ++mant;
  }
  const float f = ldexpf((float)mant, target);
  return neg ? -f : f;
}

// The fp64 sums are exact when every partial sum fits 53 bits above the last
// bit of the channel's smallest nonzero value: every value is a multiple of
// u = 2^(max(Emin, 1) - 134) and every partial sum is below T 2^(Emax - 126),
// so Emax - max(Emin, 1) + ceil(log2 T) <= 45 suffices.  Other channels take
// exact_mean_wave.  Each workgroup also folds its share of the stats pass's V
// maxima, so the quantize pass reads 2 x (finalize workgroups) partials for
// both tensor scales.
__global__ __launch_bounds__(kFinalizeThreads) void kv_finalize_kernel(KvWorkspace ws,
                                                                      const uint16_t* __restrict__ k,
                                                                      int64_t T, int64_t C,
                                                                      int n_stats_wg,
                                                                      float* __restrict__ mu_out) {
  const int64_t c = (int64_t)blockIdx.x * kFinalizeThreads + threadIdx.x;
  const bool in = c < C;
  float amax = 0.0f;
  double S = 0.0;
  float lo = __builtin_inff(), hi = -__builtin_inff();
  uint32_t z = 0xFFFFFFFFu;
  if (in) {
    // eight slices' partials loaded before any is folded (all loads in flight)
    for (int i0 = 0; i0 < kStatsSlices; i0 += 8) {
      double sv[8];
      float lv[8], hv[8];
      uint32_t zv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t o = (int64_t)(i0 + u) * C + c;
        sv[u] = ws.sum[o];
        lv[u] = ws.kmin[o];
        hv[u] = ws.kmax[o];
        zv[u] = ws.knz[o];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        S += sv[u];
        lo = fminf(lo, lv[u]);
        hi = fmaxf(hi, hv[u]);
        z = min(z, zv[u]);
      }
    }
  }
  bool exact = true;
  if (in && z != 0xFFFFFFFFu) {
    const int emax = (int)(__float_as_uint(fmaxf(fabsf(lo), fabsf(hi))) >> 23);
    const int emin = (int)((z + 1u) >> 23);
    const int lg_t = T > 1 ? 64 - __builtin_clzll((uint64_t)(T - 1)) : 0;
    exact = emax - (emin > 1 ? emin : 1) + lg_t <= 45;
  }
  float mu = in && exact ? mean_rn32(S, T) : 0.0f;
  // channels whose fp64 sum may round: the wave sums each one exactly in turn
  const int lane = threadIdx.x & 63;
  uint64_t todo = __ballot(in && !exact);
  while (todo) {
    const int src = __builtin_ctzll(todo);
    todo &= todo - 1;
    const int64_t cc = (int64_t)blockIdx.x * kFinalizeThreads + (threadIdx.x & ~63) + src;
    const float m = exact_mean_wave(k, T, C, cc, lane);
    if (lane == src) mu = m;
  }
  if (in) {
    mu_out[c] = mu;
    amax = fmaxf(hi - mu, mu - lo);              // each an RN32 of an exact difference
  }
  float va = 0.0f;
  for (int i = blockIdx.x * kFinalizeThreads + threadIdx.x; i < n_stats_wg;
       i += gridDim.x * kFinalizeThreads)
    va = fmaxf(va, ws.vamax[i]);
  amax = wave_max(amax);
  va = wave_max(va);
  __shared__ float red[kFinalizeThreads / 64], redv[kFinalizeThreads / 64];
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = amax;
    redv[threadIdx.x >> 6] = va;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0], mv = redv[0];
    for (int i = 1; i < kFinalizeThreads / 64; ++i) {
      m = fmaxf(m, red[i]);
      mv = fmaxf(mv, redv[i]);
    }
    ws.kamax[blockIdx.x] = m;
    ws.vamax_f[blockIdx.x] = mv;
  }
}

// ------------------------------------------------------------------ 3. quantize into pages

__device__ __forceinline__ float max_of(const float* p, int n) {
  float m = 0.0f;
  for (int i = threadIdx.x & 63; i < n; i += 64) m = fmaxf(m, p[i]);
  return wave_max(m);
}

// Thread -> (token, 64-channel group of head_dim) for one head (blockIdx.y).
__global__ __launch_bounds__(256) void kv_quantize_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t T,
    int64_t start_token, int32_t chunk_id, KvWorkspace ws, int n_fin_wg,
    KvGeom g, int64_t n_phys, const float* __restrict__ mu_chunk) {
  const float s_gk = global_scale(max_of(ws.kamax, n_fin_wg));
  const float s_gv = global_scale(max_of(ws.vamax_f, n_fin_wg));
  const TensorEnc tk = make_tensor_enc(s_gk), tv = make_tensor_enc(s_gv);
  const int H = g.n_heads, D = g.head_dim, P = g.page_tokens;
  const int gpr = (D + 63) / 64;                     // 64-value groups per (token, head)
  const int tpw = 256 / gpr;                         // tokens per workgroup
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    g.k_gscale[chunk_id] = s_gk;
    g.v_gscale[chunk_id] = s_gv;
  }
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid >= tpw * gpr) return;
  const int64_t t = (int64_t)blockIdx.x * tpw + tid / gpr;
  const int grp = tid % gpr;
  if (t >= T) return;
  const int64_t pos = start_token + t;
  const int64_t lp = pos / P;
  const int slot = (int)(pos - lp * P);
  // page -> chunk bookkeeping (one thread per touched page)
  if (h == 0 && grp == 0) {
    if (t == 0) {
      // a chunk starting inside a page: the slots before it are chunk_id - 1's
      g.page_chunk[2 * lp] = slot ? chunk_id - 1 : chunk_id;
      g.page_chunk[2 * lp + 1] = slot ? (int32_t)slot : P;
    } else if (slot == 0) {
      g.page_chunk[2 * lp] = chunk_id;
      g.page_chunk[2 * lp + 1] = P;
    }
  }
  const int64_t phys = g.page_table[lp];
  if (phys < 0 || phys >= n_phys) return;
  const int64_t col0 = (int64_t)grp * 64;
  const int left = (D - (int)col0) / 16;
  const int nblk = left >= 4 ? 4 : left;
  const int64_t C = (int64_t)H * D;

  uint8_t* page = g.pool + phys * g.page_bytes;
  const int64_t row = (int64_t)h * P + slot;          // (head, slot) row inside a region
  const int64_t codes_region = (int64_t)H * P * (D / 2);
  const int64_t scales_region = (int64_t)H * P * (D / 16);
  uint8_t* kc = page + row * (D / 2) + grp * 32;
  uint8_t* ks = page + codes_region + row * (D / 16) + grp * 4;
  uint8_t* vc = page + codes_region + scales_region + row * (D / 2) + grp * 32;
  uint8_t* vs = page + 2 * codes_region + scales_region + row * (D / 16) + grp * 4;

  for (int which = 0; which < 2; ++which) {
    const uint16_t* src = (which == 0 ? k : v) + t * C + (int64_t)h * D + col0;
    float x[64];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < nblk) {
        const u32x4 w0 = *(const u32x4*)(src + 16 * b);
        const u32x4 w1 = *(const u32x4*)(src + 16 * b + 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[16 * b + 2 * j] = bf16_lo(w0[j]);
          x[16 * b + 2 * j + 1] = bf16_hi(w0[j]);
          x[16 * b + 8 + 2 * j] = bf16_lo(w1[j]);
          x[16 * b + 8 + 2 * j + 1] = bf16_hi(w1[j]);
        }
      }
    }
    if (which == 0) {
      const float* mu = mu_chunk + (int64_t)h * D + col0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b < nblk) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 m4 = *(const f32x4*)(mu + 16 * b + 4 * q);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[16 * b + 4 * q + j] = x[16 * b + 4 * q + j] - m4[j];
          }
        }
      }
    }
    uint32_t cw[8];
    uint32_t sw;
    quantize_group(x, nblk, which == 0 ? tk : tv, cw, sw);
    uint8_t* cp = which == 0 ? kc : vc;
    uint8_t* sp = which == 0 ? ks : vs;
    // rows of codes are head_dim/2 bytes: 8-byte aligned for any head_dim % 16 == 0
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (b < nblk) *(u32x2*)(cp + 8 * b) = u32x2{cw[2 * b], cw[2 * b + 1]};
    if (nblk == 4 && (D % 64) == 0) {
      *(uint32_t*)sp = sw;
    } else {
      for (int b = 0; b < nblk; ++b) sp[b] = (uint8_t)(sw >> (8 * b));
    }
  }
}

// ------------------------------------------------------------------ read: dequantize pages

// Work unit = 8 consecutive values of one (token, head) row: one dword of codes
// and half a scale byte in, 16 bytes of bf16 out, for K and for V.
//
// A workgroup covers `tt` tokens of one listed page and all heads.  Thread
// `pos` owns the unit position (head h, value group sub) of a token row and
// walks the tile's tokens, so its K mean stays in registers and the loop
// carries no index arithmetic beyond strides.  The output of a token is one
// contiguous run of H * D bf16 values, unit pos at bytes [16 pos, 16 pos + 16):
// consecutive lanes store consecutive 16 bytes.
//
// Exact rounding at low cost: V^ = RN_bf16(a s_gV) needs the midpoint fix-up
// only for the rare s_gV that product_needs_check() flags (decided once per
// tile, and the two cases are separate code); for K^ = RN_bf16(a s_gK + mu)
// the eight fp32 FMA results of a unit are tested together and the exact slow
// path runs only when one of them is a bf16 midpoint.

struct UnitPtrs {
  const uint8_t *kc, *ks, *vc, *vs;   // codes dword / scale byte of token 0 of the tile
  int64_t c_stride, s_stride;          // bytes per token (row) in the codes / scale regions
};

// One token of one unit: 8 K and 8 V values, stored as 16 bytes each.
template <bool kVCheck>
__device__ __forceinline__ void dequant_unit(uint32_t kcw, uint32_t ksb, uint32_t vcw,
                                             uint32_t vsb, float sgk, float sgv, const float* mu,
                                             uint16_t* ko_p, uint16_t* vo_p) {
  u32x4 ko, vo;
  kv_unit_bf16<kVCheck>(kcw, ksb, vcw, vsb, sgk, sgv, mu, ko, vo);
  *(u32x4*)ko_p = ko;
  *(u32x4*)vo_p = vo;
}

// Fast path: all kTT tokens of the tile exist and belong to one chunk.
template <int kTT, bool kVCheck>
__device__ __forceinline__ void dequant_tile_uniform(const UnitPtrs& u, float sgk, float sgv,
                                                     const float* mu, uint16_t* ko,
                                                     uint16_t* vo, int64_t row_elems) {
  uint32_t kcw[kTT], vcw[kTT], ksb[kTT], vsb[kTT];
#pragma unroll
  for (int j = 0; j < kTT; ++j) {
    kcw[j] = *(const uint32_t*)(u.kc + j * u.c_stride);
    vcw[j] = *(const uint32_t*)(u.vc + j * u.c_stride);
    ksb[j] = u.ks[j * u.s_stride];
    vsb[j] = u.vs[j * u.s_stride];
  }
#pragma unroll
  for (int j = 0; j < kTT; ++j)
    dequant_unit<kVCheck>(kcw[j], ksb[j], vcw[j], vsb[j], sgk, sgv, mu, ko + j * row_elems,
                          vo + j * row_elems);
}

// ---- quad path (head_dim % 32 == 0): the four lanes of a quad own value groups
// 4m..4m+3 of one head.  Lane k loads token k's 16 bytes of codes for those
// four groups (one load instead of four), and a 4 x 4 dword transpose across
// the quad (DPP lane swaps) gives each lane its own group for the 4 tokens.

__device__ __forceinline__ uint32_t quad_swap1(uint32_t v) {      // value of lane ^ 1
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {      // value of lane ^ 2
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}
template <int kLane>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {      // value of quad lane kLane
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kLane * 0x55, 0xF, 0xF, false);
}

// In: lane k (k = lane % 4) holds row k of a 4 x 4 matrix.  Out: column k.
// Two butterfly stages; in stage b, element e is taken from lane k ^ 2^b
// (its element e ^ 2^b) exactly when bit b of e and of k differ.
__device__ __forceinline__ u32x4 quad_transpose(u32x4 a, int k) {
  const bool o0 = k & 1, o1 = k & 2;
  const uint32_t x0 = quad_swap1(a[1]), x1 = quad_swap1(a[0]);
  const uint32_t x2 = quad_swap1(a[3]), x3 = quad_swap1(a[2]);
  a = u32x4{o0 ? x0 : a[0], o0 ? a[1] : x1, o0 ? x2 : a[2], o0 ? a[3] : x3};
  const uint32_t y0 = quad_swap2(a[2]), y1 = quad_swap2(a[3]);
  const uint32_t y2 = quad_swap2(a[0]), y3 = quad_swap2(a[1]);
  return u32x4{o1 ? y0 : a[0], o1 ? y1 : a[1], o1 ? a[2] : y2, o1 ? a[3] : y3};
}

// Scale byte of this lane's group for token j of the quad: lane j loaded the
// two scale bytes (groups 4m..4m+3 span two blocks) of token j.
template <int kJ>
__device__ __forceinline__ uint32_t quad_scale(uint32_t two_bytes, int k) {
  return (quad_bcast<kJ>(two_bytes) >> (8 * (k >> 1))) & 0xFFu;
}

// Fast path with the quad loads: kTT tokens (a multiple of 4), one chunk.
// `u` points at this lane's own group of token 0; `q` at the quad's 16-byte
// code block / 2-byte scale pair of token k (lane k of the quad).
template <int kTT, bool kVCheck>
__device__ __forceinline__ void dequant_tile_quad(const UnitPtrs& q, int k, float sgk, float sgv,
                                                  const float* mu, uint16_t* ko, uint16_t* vo,
                                                  int64_t row_elems) {
  constexpr int kG = kTT / 4;
  u32x4 kc[kG], vc[kG];
  uint32_t ks[kG], vs[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    kc[g] = *(const u32x4*)(q.kc + 4 * g * q.c_stride);
    vc[g] = *(const u32x4*)(q.vc + 4 * g * q.c_stride);
    ks[g] = *(const uint16_t*)(q.ks + 4 * g * q.s_stride);
    vs[g] = *(const uint16_t*)(q.vs + 4 * g * q.s_stride);
  }
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const u32x4 kt = quad_transpose(kc[g], k), vt = quad_transpose(vc[g], k);
    uint16_t* kg = ko + 4 * g * row_elems;
    uint16_t* vg = vo + 4 * g * row_elems;
    dequant_unit<kVCheck>(kt[0], quad_scale<0>(ks[g], k), vt[0], quad_scale<0>(vs[g], k), sgk,
                          sgv, mu, kg, vg);
    dequant_unit<kVCheck>(kt[1], quad_scale<1>(ks[g], k), vt[1], quad_scale<1>(vs[g], k), sgk,
                          sgv, mu, kg + row_elems, vg + row_elems);
    dequant_unit<kVCheck>(kt[2], quad_scale<2>(ks[g], k), vt[2], quad_scale<2>(vs[g], k), sgk,
                          sgv, mu, kg + 2 * row_elems, vg + 2 * row_elems);
    dequant_unit<kVCheck>(kt[3], quad_scale<3>(ks[g], k), vt[3], quad_scale<3>(vs[g], k), sgk,
                          sgv, mu, kg + 3 * row_elems, vg + 3 * row_elems);
  }
}

__device__ __forceinline__ void load_mu8(const float* p, float* mu) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mu[j] = a[j];
    mu[4 + j] = b[j];
  }
}

// Wave-uniform product_needs_check(g): lane l tests significand l % 16 and the
// wave votes.  Every lane of the wave must be active.
__device__ __forceinline__ bool needs_check_wave(float g) {
  if (!(g >= 0x1p-116f)) return true;
  const int i = threadIdx.x & 15;
  const float a = ((i & 8) ? 1.5f : 1.0f) * (1.0f + (float)(i & 7) * 0.125f);
  const float p = a * g;
  const bool need = (__float_as_uint(p) & 0xFFFFu) == 0x8000u && __builtin_fmaf(a, g, -p) != 0.0f;
  return __builtin_amdgcn_ballot_w64(need) != 0;
}

template <int kTT, bool kQuad>
__global__ __launch_bounds__(512) void kv_dequant_kernel(KvGeom g, int64_t n_phys,
                                                         const int32_t* __restrict__ pages,
                                                         uint16_t* __restrict__ k_out,
                                                         uint16_t* __restrict__ v_out) {
  const int H = g.n_heads, D = g.head_dim, P = g.page_tokens;
  const int upr = D / 8;                                  // units per (token, head) row
  const int npos = H * upr;                               // units per token
  const int tiles = (P + kTT - 1) / kTT;
  // Workgroup b runs on XCD b % 8.  Tiles 2j and 2j + 1 share the 128-byte
  // lines of their heads' scale bytes (16 tokens x 8 bytes), so they are given
  // to workgroups b and b + 8 -- the same XCD, dispatched back to back -- and
  // the line is fetched into that XCD's L2 once instead of into two.
  int bid = blockIdx.x;
  if ((gridDim.x & 15u) == 0) {
    const int x = bid & 7, s = bid >> 3;
    bid = (s >> 1) * 16 + x * 2 + (s & 1);
  }
  const int64_t i = bid / tiles;
  const int t0 = (bid % tiles) * kTT;
  const int ntok = min(kTT, P - t0);
  const int32_t lp = pages[i];
  bool valid = lp >= 0 && lp < g.max_pages;
  const int64_t phys = valid ? (int64_t)g.page_table[lp] : -1;
  valid = valid && phys >= 0 && phys < n_phys;
  const int64_t row_elems = (int64_t)H * D;               // bf16 values per output token
  uint16_t* k_tile = k_out + (i * P + t0) * row_elems;
  uint16_t* v_tile = v_out + (i * P + t0) * row_elems;
  if (!valid) {
    for (int64_t u = threadIdx.x; u < (int64_t)ntok * npos; u += blockDim.x) {
      *(u32x4*)(k_tile + 8 * u) = u32x4{0, 0, 0, 0};
      *(u32x4*)(v_tile + 8 * u) = u32x4{0, 0, 0, 0};
    }
    return;
  }
  int c0 = g.page_chunk[2 * lp];
  const int split = g.page_chunk[2 * lp + 1];
  c0 = c0 < 0 ? 0 : (c0 >= g.max_chunks ? g.max_chunks - 1 : c0);
  const int c1 = c0 + 1 < g.max_chunks ? c0 + 1 : g.max_chunks - 1;
  // tile entirely in one chunk (the common case) and complete
  const bool uniform = ntok == kTT && (t0 + kTT <= split || t0 >= split);
  const int cu = t0 >= split ? c1 : c0;
  const float sgk0 = g.k_gscale[c0], sgk1 = g.k_gscale[c1];
  const float sgv0 = g.v_gscale[c0], sgv1 = g.v_gscale[c1];
  const bool vcheck = uniform ? needs_check_wave(cu == c0 ? sgv0 : sgv1)
                              : needs_check_wave(sgv0) || needs_check_wave(sgv1);

  const uint8_t* page = g.pool + phys * g.page_bytes;
  const int64_t codes_region = (int64_t)H * P * (D / 2);
  const int64_t scales_region = (int64_t)H * P * (D / 16);

  for (int pos = threadIdx.x; pos < npos; pos += blockDim.x) {
    const int h = pos / upr, sub = pos - (pos / upr) * upr;
    const int64_t r0 = (int64_t)h * P + t0;                // (head, slot) row of token t0
    UnitPtrs u;
    u.kc = page + r0 * (D / 2) + 4 * sub;
    u.ks = page + codes_region + r0 * (D / 16) + (sub >> 1);
    u.vc = page + codes_region + scales_region + r0 * (D / 2) + 4 * sub;
    u.vs = page + 2 * codes_region + scales_region + r0 * (D / 16) + (sub >> 1);
    u.c_stride = D / 2;
    u.s_stride = D / 16;
    const int64_t mu_off = (int64_t)h * D + 8 * sub;
    if (kQuad && uniform) {
      // head_dim % 32 == 0 and the block size a multiple of 64: quads are whole
      const int k = pos & 3;
      const int64_t rq = r0 + k;                            // token k of the quad
      UnitPtrs q;
      q.kc = page + rq * (D / 2) + 16 * (sub >> 2);
      q.ks = page + codes_region + rq * (D / 16) + 2 * (sub >> 2);
      q.vc = page + codes_region + scales_region + rq * (D / 2) + 16 * (sub >> 2);
      q.vs = page + 2 * codes_region + scales_region + rq * (D / 16) + 2 * (sub >> 2);
      q.c_stride = D / 2;
      q.s_stride = D / 16;
      float mu[8];
      load_mu8(g.k_mean + (int64_t)cu * H * D + mu_off, mu);
      const float sgk = cu == c0 ? sgk0 : sgk1, sgv = cu == c0 ? sgv0 : sgv1;
      if (vcheck)
        dequant_tile_quad<kTT, true>(q, k, sgk, sgv, mu, k_tile + 8 * pos, v_tile + 8 * pos,
                                     row_elems);
      else
        dequant_tile_quad<kTT, false>(q, k, sgk, sgv, mu, k_tile + 8 * pos, v_tile + 8 * pos,
                                      row_elems);
    } else if (uniform) {
      float mu[8];
      load_mu8(g.k_mean + (int64_t)cu * H * D + mu_off, mu);
      const float sgk = cu == c0 ? sgk0 : sgk1, sgv = cu == c0 ? sgv0 : sgv1;
      if (vcheck)
        dequant_tile_uniform<kTT, true>(u, sgk, sgv, mu, k_tile + 8 * pos, v_tile + 8 * pos,
                                        row_elems);
      else
        dequant_tile_uniform<kTT, false>(u, sgk, sgv, mu, k_tile + 8 * pos, v_tile + 8 * pos,
                                         row_elems);
    } else {
      // ragged tile or a tile across the chunk boundary: token by token
      float mu0[8], mu1[8];
      load_mu8(g.k_mean + (int64_t)c0 * H * D + mu_off, mu0);
      load_mu8(g.k_mean + (int64_t)c1 * H * D + mu_off, mu1);
      for (int t = 0; t < ntok; ++t) {
        const bool second = t0 + t >= split;
        const uint32_t kcw = *(const uint32_t*)(u.kc + t * u.c_stride);
        const uint32_t vcw = *(const uint32_t*)(u.vc + t * u.c_stride);
        const uint32_t ksb = u.ks[t * u.s_stride], vsb = u.vs[t * u.s_stride];
        dequant_unit<true>(kcw, ksb, vcw, vsb, second ? sgk1 : sgk0, second ? sgv1 : sgv0,
                           second ? mu1 : mu0, k_tile + t * row_elems + 8 * pos,
                           v_tile + t * row_elems + 8 * pos);
      }
    }
  }
}

// ------------------------------------------------------------------ launchers

// Flat variant for head_dim dividing 512 (64, 128, 256).  A row is one
// (head, token) pair, taken head-major (row r = h T + t); lane u of the grid
// owns channels 8 j .. 8 j + 7 (j = u % (D / 8)) of row u / (D / 8): one
// 16-byte load per tensor.  A workgroup thus covers consecutive tokens of one
// head, whose page rows are consecutive too: it writes whole runs of codes and
// of scale bytes (16 tokens x 8 bytes = 128 bytes of scales for head_dim 128)
// instead of leaving neighbouring tokens' scale bytes to workgroups on other
// XCDs, whose L2s would each write back a partial span.  The two lanes of a
// 16-value block exchange their maxima with one DPP swap (the scheme of the
// activation quantize).  Whole waves stay in the loop (lanes past the end take
// the last unit and store nothing) so the swap always has both lanes; the
// loop strides over the grid.
template <int kD, bool kPre>
__device__ __forceinline__ void kv_flat_unit(const uint16_t* __restrict__ src,
                                             const float* __restrict__ mu, uint32_t e0,
                                             const TensorEnc& te, bool store, uint8_t* cp,
                                             uint8_t* sp, int j) {
  const u32x4 w = *(const u32x4*)(src + e0);
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(w[e]);
    x[2 * e + 1] = bf16_hi(w[e]);
  }
  if (mu) {                                            // K' = RN32(K - mu)
    const f32x4 m0 = *(const f32x4*)mu, m1 = *(const f32x4*)(mu + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = x[e] - m0[e];
      x[4 + e] = x[4 + e] - m1[e];
    }
  }
  float bm = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) bm = fmaxf(bm, __builtin_fabsf(x[e]));
  bm = pair_max(bm);
  const uint32_t sb = block_scale_byte<kPre>(bm, te);
  const BlockEnc enc = make_block_enc(sb, te);
  if (kPre) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= 0x1p64f;
  }
  const uint32_t cw = encode8(x, enc, te);
  if (store) {
    *(uint32_t*)cp = cw;
    if ((j & 1) == 0) *sp = (uint8_t)sb;
  }
}

// p_shift: log2(page_tokens) when that is a power of two, else -1 (divide).
template <int kD>
__global__ __launch_bounds__(256) void kv_quantize_flat_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t T,
    int64_t start_token, int32_t chunk_id, KvWorkspace ws, int n_fin_wg,
    KvGeom g, int64_t n_phys, const float* __restrict__ mu_chunk, int p_shift) {
  const float s_gk = global_scale(max_of(ws.kamax, n_fin_wg));
  const float s_gv = global_scale(max_of(ws.vamax_f, n_fin_wg));
  const TensorEnc tk = make_tensor_enc(s_gk), tv = make_tensor_enc(s_gv);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    g.k_gscale[chunk_id] = s_gk;
    g.v_gscale[chunk_id] = s_gv;
  }
  // 32-bit indices (the launcher checks T H D and start_token + T < 2^31, and
  // page_bytes < 2^32; T >= 1).  The grid stride is a whole number of rows, so a
  // lane's (head, token) moves by a fixed step each iteration and its channel
  // chunk j never changes.
  constexpr uint32_t kLpr = kD / 8;                     // lanes per row
  const uint32_t H = g.n_heads, P = g.page_tokens, Tu = (uint32_t)T;
  const uint32_t n = Tu * H * kLpr;
  const uint32_t codes_region = H * P * (kD / 2);
  const uint32_t scales_region = H * P * (kD / 16);
  const uint32_t stride = gridDim.x * 256u;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t u0 = blockIdx.x * 256u + threadIdx.x;
  const uint32_t j = u0 % kLpr;
  const uint32_t dr = stride / kLpr, dh = dr / Tu, dt = dr % Tu;
  uint32_t r0 = u0 / kLpr;
  uint32_t h = r0 / Tu, t = r0 % Tu;
  const uint32_t rs = H * kD;                           // elements per token of K and V
  const float* mu = mu_chunk + 8 * j;
  // the encoders' pre-scaling is uniform per tensor: pick it outside the loop so
  // the loop body has no branch between the K and V loads
  const auto run = [&](auto pre_k, auto pre_v) {
    constexpr bool kPk = decltype(pre_k)::value, kPv = decltype(pre_v)::value;
    for (uint32_t base = blockIdx.x * 256u + (threadIdx.x - lane); base < n; base += stride) {
      const uint32_t u = base + lane;
      const bool in = u < n;
      const uint32_t tc = in ? t : Tu - 1;              // lanes past the end: valid addresses
      const uint32_t hc = in ? h : H - 1;
      const uint32_t pos = (uint32_t)start_token + tc;
      const uint32_t lp = p_shift >= 0 ? pos >> p_shift : pos / P;
      const uint32_t slot = pos - lp * P;
      // page -> chunk bookkeeping (one lane per touched page)
      if (in && h == 0 && j == 0) {
        if (t == 0) {
          // a chunk starting inside a page: the slots before it are chunk_id - 1's
          g.page_chunk[2 * lp] = slot ? chunk_id - 1 : chunk_id;
          g.page_chunk[2 * lp + 1] = slot ? (int32_t)slot : (int32_t)P;
        } else if (slot == 0) {
          g.page_chunk[2 * lp] = chunk_id;
          g.page_chunk[2 * lp + 1] = P;
        }
      }
      const int64_t phys = g.page_table[lp];
      const bool store = in && phys >= 0 && phys < n_phys;
      uint8_t* page = g.pool + (store ? phys : 0) * g.page_bytes;
      const uint32_t row = hc * P + slot;
      uint8_t* kc = page + (row * (kD / 2) + 4 * j);
      uint8_t* ks = page + (codes_region + row * (kD / 16) + (j >> 1));
      uint8_t* vc = page + (codes_region + scales_region + row * (kD / 2) + 4 * j);
      uint8_t* vs = page + (2 * codes_region + scales_region + row * (kD / 16) + (j >> 1));
      const uint32_t e0 = tc * rs + hc * kD + 8 * j;    // first element of the lane's 8
      kv_flat_unit<kD, kPk>(k, mu + hc * kD, e0, tk, store, kc, ks, j);
      kv_flat_unit<kD, kPv>(v, nullptr, e0, tv, store, vc, vs, j);
      // next iteration's (head, token)
      t += dt;
      h += dh;
      if (t >= Tu) {
        t -= Tu;
        h += 1;
      }
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  const bool pk = tk.pre != 1.0f, pv = tv.pre != 1.0f;
  if (pk) {
    if (pv) run(yes{}, yes{});
    else run(yes{}, no{});
  } else {
    if (pv) run(no{}, yes{});
    else run(no{}, no{});
  }
}

void launch_kv_quantize(const KvGeom& g, int32_t chunk_id, const uint16_t* k, const uint16_t* v,
                        int64_t T, int64_t start_token, void* workspace, hipStream_t stream) {
  const int64_t C = (int64_t)g.n_heads * g.head_dim;
  const int nsw = stats_wgs(C), nfw = finalize_wgs(C);
  KvWorkspace ws = carve(workspace, C, nsw, nfw);
  float* mu = g.k_mean + (int64_t)chunk_id * C;
  hipLaunchKernelGGL(kv_stats_kernel, dim3(nsw), dim3(256), 0, stream, k, v, T, C, ws);
  hipLaunchKernelGGL(kv_finalize_kernel, dim3(nfw), dim3(kFinalizeThreads), 0, stream, ws, k, T,
                     C, nsw, mu);
  const int D = g.head_dim;
  const bool small = T * g.n_heads * D < (int64_t(1) << 31) &&
                     start_token + T < (int64_t(1) << 31) &&
                     g.page_bytes < (int64_t(1) << 32);
  if ((D == 64 || D == 128 || D == 256) && small) {
    const int64_t lanes = T * g.n_heads * (D / 8);
    // at most one resident round of workgroups (256 CUs x 8 of 256 threads),
    // each lane striding over several units: measured 11 % faster for a
    // 7040-token chunk than 8192 short workgroups (too few waves stay resident)
    int64_t wgs = (lanes + 255) / 256;
    wgs = wgs < 2048 ? wgs : 2048;
    const int P = g.page_tokens;
    const int p_shift = (P & (P - 1)) == 0 ? __builtin_ctz((unsigned)P) : -1;
    const auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(256), 0, stream, k, v, T, start_token,
                         chunk_id, ws, nfw, g, g.n_phys_pages, (const float*)mu, p_shift);
    };
    if (D == 64) go(kv_quantize_flat_kernel<64>);
    else if (D == 128) go(kv_quantize_flat_kernel<128>);
    else go(kv_quantize_flat_kernel<256>);
    return;
  }
  const int gpr = (D + 63) / 64;
  const int tpw = 256 / gpr;
  const dim3 grid((unsigned)((T + tpw - 1) / tpw), (unsigned)g.n_heads);
  hipLaunchKernelGGL(kv_quantize_kernel, grid, dim3(256), 0, stream, k, v, T, start_token,
                     chunk_id, ws, nfw, g, g.n_phys_pages, (const float*)mu);
}

// Entry i of the list: the i-th page of the concatenated ranges.
__global__ __launch_bounds__(256) void kv_window_pages_kernel(int32_t a0, int32_t b0, int32_t a1,
                                                              int32_t b1, int32_t a2,
                                                              int32_t count,
                                                              int32_t* __restrict__ pages) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const int64_t l0 = b0 - a0, l1 = b1 - a1;
  pages[i] = (int32_t)(i < l0 ? a0 + i : (i < l0 + l1 ? a1 + (i - l0) : a2 + (i - l0 - l1)));
}

void launch_kv_window_pages(const int32_t* r, int m, int32_t count, int32_t* pages,
                            hipStream_t stream) {
  (void)m;                                  // unused ranges are empty ([0, 0))
  hipLaunchKernelGGL(kv_window_pages_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                     stream, r[0], r[1], r[2], r[3], r[4], count, pages);
}

#ifndef NVFP4_KV_READ_TOKENS
#define NVFP4_KV_READ_TOKENS 8
#endif

void launch_kv_dequant(const KvGeom& g, const int32_t* logical_pages, int32_t n_pages,
                       uint16_t* k_out, uint16_t* v_out, hipStream_t stream) {
  // One thread per unit position of a token row (up to 512) and a few tokens
  // per workgroup: each workgroup then writes short contiguous runs (H * D * 2
  // bytes per token for K and for V), and the chip's concurrent writes stay
  // close together, which sustains a higher HBM write rate than long
  // per-workgroup runs.
  constexpr int kTT = NVFP4_KV_READ_TOKENS;
  const int npos = g.n_heads * (g.head_dim / 8);
  int threads = ((npos + 63) / 64) * 64;
  threads = threads > 512 ? 512 : threads;
  const int64_t tiles = (g.page_tokens + kTT - 1) / kTT;
  // quad loads need whole quads of value groups per head (head_dim % 32) and
  // lanes that line up with them (block size a multiple of 4, which 64 is)
  if (g.head_dim % 32 == 0 && kTT % 4 == 0)
    hipLaunchKernelGGL((kv_dequant_kernel<kTT, true>), dim3((unsigned)(tiles * n_pages)),
                       dim3(threads), 0, stream, g, g.n_phys_pages, logical_pages, k_out, v_out);
  else
    hipLaunchKernelGGL((kv_dequant_kernel<kTT, false>), dim3((unsigned)(tiles * n_pages)),
                       dim3(threads), 0, stream, g, g.n_phys_pages, logical_pages, k_out, v_out);
}

}  // namespace nvfp4
