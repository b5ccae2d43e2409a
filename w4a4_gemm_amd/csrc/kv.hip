// Paged NVFP4 KV cache kernels for gfx950.
//
// Write path (techwalker.com LongLive-2.0 report summary, section 四, second
// key: K is mean-subtracted, then K and V are stored in NVFP4; zuobiaodaohang
// LongLive blog: the quantized cache is updated in place):
//   1. kv_stats:     one read of K and V: per (head, channel) fp64 sum, min and
//                    max of K over a token slice; per workgroup max|V|.
//   2. kv_finalize:  per channel mu = RN32(S / T); max|K - mu| from min/max
//                    (RN32 is monotone, so max |RN32(K - mu)| is
//                    max(RN32(Kmax - mu), RN32(mu - Kmin))); mu is stored.
//   3. kv_quantize:  second read (usually from the 256 MB Infinity Cache):
//                    K' = RN32(K - mu), K' and V quantized along head_dim into
//                    the pages named by the page table, in place.
// Read path (same section: one parallel kernel decompresses many cache
// blocks of a window): kv_dequant, one grid over (listed page, head, slot
// tile), K^ = RN_bf16(q s_b s_gK + mu), V^ = RN_bf16(q s_b s_gV).

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kStatsSlices = 8;           // token slices of the stats pass
constexpr int kStatsCols = 64;            // channels per stats workgroup (8 lanes x 8)
constexpr int kFinalizeThreads = 256;

struct KvWorkspace {
  double* sum;      // [slices][C]
  float* kmin;      // [slices][C]
  float* kmax;      // [slices][C]
  float* vamax;     // [stats workgroups]
  float* kamax;     // [finalize workgroups]
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
  w.vamax = (float*)p;
  p += round256(sizeof(float) * n_stats_wg);
  w.kamax = (float*)p;
  (void)n_fin_wg;
  return w;
}

int stats_wgs(int64_t C) { return (int)((C + kStatsCols - 1) / kStatsCols) * kStatsSlices; }
int finalize_wgs(int64_t C) { return (int)((C + kFinalizeThreads - 1) / kFinalizeThreads); }

}  // namespace

size_t kv_quantize_workspace_bytes(int64_t T, int64_t H, int64_t D) {
  (void)T;
  const int64_t C = H * D;
  return round256(sizeof(double) * kStatsSlices * C) + 2 * round256(sizeof(float) * kStatsSlices * C) +
         round256(sizeof(float) * stats_wgs(C)) + round256(sizeof(float) * finalize_wgs(C));
}

// ------------------------------------------------------------------ 1. stats

// Workgroup (colgroup, slice): 8 lanes cover 64 channels (8 each, one 16-byte
// load), 32 token lanes stride over the slice's tokens.
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
  uint32_t va = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) { s[j] = 0.0; mn[j] = __builtin_inff(); mx[j] = -__builtin_inff(); }
  const bool active = c0 < C;
  if (active) {
    for (int64_t t = t0 + tl; t < t1; t += 32) {
      const u32x4 kw = *(const u32x4*)(k + t * C + c0);
      const u32x4 vw = *(const u32x4*)(v + t * C + c0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = bf16_lo(kw[j]), b = bf16_hi(kw[j]);
        s[2 * j] += (double)a;
        s[2 * j + 1] += (double)b;
        mn[2 * j] = fminf(mn[2 * j], a);
        mn[2 * j + 1] = fminf(mn[2 * j + 1], b);
        mx[2 * j] = fmaxf(mx[2 * j], a);
        mx[2 * j + 1] = fmaxf(mx[2 * j + 1], b);
        const uint32_t av = vw[j] & 0x7FFF7FFFu;
        va = max(va, max(av & 0xFFFFu, av >> 16));
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

__global__ __launch_bounds__(kFinalizeThreads) void kv_finalize_kernel(KvWorkspace ws, int64_t T,
                                                                      int64_t C,
                                                                      float* __restrict__ mu_out) {
  const int64_t c = (int64_t)blockIdx.x * kFinalizeThreads + threadIdx.x;
  float amax = 0.0f;
  if (c < C) {
    double S = 0.0;
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int i = 0; i < kStatsSlices; ++i) {
      S += ws.sum[i * C + c];
      lo = fminf(lo, ws.kmin[i * C + c]);
      hi = fmaxf(hi, ws.kmax[i * C + c]);
    }
    const float mu = mean_rn32(S, T);
    mu_out[c] = mu;
    amax = fmaxf(hi - mu, mu - lo);              // each an RN32 of an exact difference
  }
  amax = wave_max(amax);
  __shared__ float red[kFinalizeThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
    for (int i = 1; i < kFinalizeThreads / 64; ++i) m = fmaxf(m, red[i]);
    ws.kamax[blockIdx.x] = m;
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
    int64_t start_token, int32_t chunk_id, KvWorkspace ws, int n_stats_wg, int n_fin_wg,
    KvGeom g, int64_t n_phys, const float* __restrict__ mu_chunk) {
  const float s_gk = global_scale(max_of(ws.kamax, n_fin_wg));
  const float s_gv = global_scale(max_of(ws.vamax, n_stats_wg));
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
      if (slot) g.page_chunk[2 * lp + 1] = slot;
      else { g.page_chunk[2 * lp] = chunk_id; g.page_chunk[2 * lp + 1] = P; }
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
// walks the tile's tokens, so its K mean (both chunks a page can hold) stays
// in registers and the loop carries no index arithmetic beyond strides.  The
// output of a token is one contiguous run of H * D bf16 values, unit pos at
// bytes [16 pos, 16 pos + 16): consecutive lanes store consecutive 16 bytes.
//
// Exact rounding at low cost: V^ = RN_bf16(a s_gV) needs the midpoint fix-up
// only for the rare s_gV that product_needs_check() flags (decided once per
// chunk); for K^ = RN_bf16(a s_gK + mu) the eight fp32 FMA results of a unit
// are tested together and the exact slow path runs only when one of them is
// a bf16 midpoint.
template <int kTok>
__global__ __launch_bounds__(512) void kv_dequant_kernel(KvGeom g, int64_t n_phys,
                                                         const int32_t* __restrict__ pages, int tt,
                                                         uint16_t* __restrict__ k_out,
                                                         uint16_t* __restrict__ v_out) {
  const int H = g.n_heads, D = g.head_dim, P = g.page_tokens;
  const int upr = D / 8;                                  // units per (token, head) row
  const int npos = H * upr;                               // units per token
  const int tiles = (P + tt - 1) / tt;
  const int64_t i = blockIdx.x / tiles;
  const int t0 = (blockIdx.x % tiles) * tt;
  const int ntok = min(tt, P - t0);
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
  const float sgk0 = g.k_gscale[c0], sgk1 = g.k_gscale[c1];
  const float sgv0 = g.v_gscale[c0], sgv1 = g.v_gscale[c1];
  const bool vcheck = product_needs_check(sgv0) || product_needs_check(sgv1);

  const uint8_t* page = g.pool + phys * g.page_bytes;
  const int64_t codes_region = (int64_t)H * P * (D / 2);
  const int64_t scales_region = (int64_t)H * P * (D / 16);

  for (int pos = threadIdx.x; pos < npos; pos += blockDim.x) {
    const int h = pos / upr, sub = pos - (pos / upr) * upr;
    float mu0[8], mu1[8];
    {
      const float* m0 = g.k_mean + ((int64_t)c0 * H + h) * D + 8 * sub;
      const float* m1 = g.k_mean + ((int64_t)c1 * H + h) * D + 8 * sub;
      const f32x4 a0 = *(const f32x4*)m0, a1 = *(const f32x4*)(m0 + 4);
      const f32x4 b0 = *(const f32x4*)m1, b1 = *(const f32x4*)(m1 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mu0[j] = a0[j]; mu0[4 + j] = a1[j];
        mu1[j] = b0[j]; mu1[4 + j] = b1[j];
      }
    }
    const int64_t r0 = (int64_t)h * P + t0;                // (head, slot) row of token t0
    const uint8_t* kc = page + r0 * (D / 2) + 4 * sub;
    const uint8_t* ks = page + codes_region + r0 * (D / 16) + (sub >> 1);
    const uint8_t* vc = page + codes_region + scales_region + r0 * (D / 2) + 4 * sub;
    const uint8_t* vs = page + 2 * codes_region + scales_region + r0 * (D / 16) + (sub >> 1);
    for (int t = 0; t < ntok; t += kTok) {
      uint32_t kcw[kTok], vcw[kTok], ksb[kTok], vsb[kTok];
#pragma unroll
      for (int j = 0; j < kTok; ++j) {
        if (t + j < ntok) {
          kcw[j] = *(const uint32_t*)(kc + (int64_t)(t + j) * (D / 2));
          vcw[j] = *(const uint32_t*)(vc + (int64_t)(t + j) * (D / 2));
          ksb[j] = ks[(int64_t)(t + j) * (D / 16)];
          vsb[j] = vs[(int64_t)(t + j) * (D / 16)];
        }
      }
#pragma unroll
      for (int j = 0; j < kTok; ++j) {
        if (t + j < ntok) {
          const bool second = t0 + t + j >= split;
          const float sgk = second ? sgk1 : sgk0, sgv = second ? sgv1 : sgv0;
          const float sbk = e4m3_value(ksb[j]), sbv = e4m3_value(vsb[j]);
          float ka[8], kf[8], vf[8];
          uint32_t off = 0xFFFFFFFFu;
#pragma unroll
          for (int sel = 0; sel < 4; ++sel) {
            const f32x2 qk = e2m1_pair(kcw[j], sel);
            const f32x2 qv = e2m1_pair(vcw[j], sel);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int n = 2 * sel + e;
              ka[n] = qk[e] * sbk;                          // exact
              kf[n] = __builtin_fmaf(ka[n], sgk, second ? mu1[n] : mu0[n]);
              off = min(off, off_midpoint(kf[n]));
              vf[n] = vcheck ? mul_for_bf16(qv[e] * sbv, sgv) : (qv[e] * sbv) * sgv;
            }
          }
          if (__builtin_expect(off == 0u, 0)) {
#pragma unroll
            for (int n = 0; n < 8; ++n)
              kf[n] = fma_for_bf16(ka[n], sgk, second ? mu1[n] : mu0[n]);
          }
          u32x4 ko, vo;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            ko[q] = pack_bf16x2(kf[2 * q], kf[2 * q + 1]);
            vo[q] = pack_bf16x2(vf[2 * q], vf[2 * q + 1]);
          }
          const int64_t o = (int64_t)(t + j) * row_elems + 8 * pos;
          *(u32x4*)(k_tile + o) = ko;
          *(u32x4*)(v_tile + o) = vo;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launchers

void launch_kv_quantize(const KvGeom& g, int32_t chunk_id, const uint16_t* k, const uint16_t* v,
                        int64_t T, int64_t start_token, void* workspace, hipStream_t stream) {
  const int64_t C = (int64_t)g.n_heads * g.head_dim;
  const int nsw = stats_wgs(C), nfw = finalize_wgs(C);
  KvWorkspace ws = carve(workspace, C, nsw, nfw);
  float* mu = g.k_mean + (int64_t)chunk_id * C;
  hipLaunchKernelGGL(kv_stats_kernel, dim3(nsw), dim3(256), 0, stream, k, v, T, C, ws);
  hipLaunchKernelGGL(kv_finalize_kernel, dim3(nfw), dim3(kFinalizeThreads), 0, stream, ws, T, C,
                     mu);
  const int gpr = (g.head_dim + 63) / 64;
  const int tpw = 256 / gpr;
  const dim3 grid((unsigned)((T + tpw - 1) / tpw), (unsigned)g.n_heads);
  hipLaunchKernelGGL(kv_quantize_kernel, grid, dim3(256), 0, stream, k, v, T, start_token,
                     chunk_id, ws, nsw, nfw, g, g.n_phys_pages, (const float*)mu);
}

void launch_kv_dequant(const KvGeom& g, const int32_t* logical_pages, int32_t n_pages,
                       uint16_t* k_out, uint16_t* v_out, hipStream_t stream) {
  // one thread per unit position of a token row (up to 512), 16 tokens per workgroup
  const int npos = g.n_heads * (g.head_dim / 8);
  int threads = ((npos + 63) / 64) * 64;
  threads = threads > 512 ? 512 : threads;
  const int tt = g.page_tokens < 16 ? g.page_tokens : 16;
  const int64_t tiles = (g.page_tokens + tt - 1) / tt;
  hipLaunchKernelGGL(kv_dequant_kernel<4>, dim3((unsigned)(tiles * n_pages)), dim3(threads), 0,
                     stream, g, g.n_phys_pages, logical_pages, tt, k_out, v_out);
}

}  // namespace nvfp4
