// Fused attention over the paged NVFP4 KV cache for gfx950.
//
// The cache is read block by block (techwalker.com LongLive-2.0 report
// summary, section 四, second key: many cache blocks of the time window are
// decompressed in parallel); here each 64-key block is decompressed into LDS
// with exactly the rounding of the window-read kernel (K^ = RN_bf16(q s_b
// s_gK + mu), V^ = RN_bf16(q s_b s_gV)) and consumed at once by a
// flash-attention step, so no bf16 K or V reaches HBM.
//
// Layout of work: a workgroup is one head and 128 queries (4 waves x 32).
// Each wave computes the transposed products on the bf16 MFMA
//   S^T = K^ Q^T    (32 keys x 32 queries per v_mfma_f32_32x32x16_bf16 tile)
//   O^T += V^T P^T  (32 channels x 32 queries per tile)
// so that in both accumulators a lane owns one query (column lane % 32) and
// its registers run over keys or channels.  The online softmax (running max
// m, running sum l, rescaling of O) is then per lane plus one exchange with
// lane ^ 32, and P goes from the S^T registers straight into the second
// MFMA: the MFMA sums over its 16 k values in any order, so the k order of
// a step is taken to be the key order of the S^T registers, and V^T is read
// from LDS in that same order.  Logits are scaled by scale * log2(e) and
// exponentiated with exp2.

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;               // head_dim
constexpr int kQB = 128;              // queries per workgroup
constexpr int kKB = 64;               // keys per block
constexpr int kKsRow = kD + 8;        // bf16 per K^ row in LDS (272 bytes: conflict-free reads)
constexpr int kVtRow = kKB + 8;       // bf16 per V^T row in LDS (144 bytes)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Per-page facts, uniform over the workgroup.
struct PageInfo {
  const uint8_t* page;    // null when the page is not mapped
  int valid;              // valid slots of the page (keys beyond are masked)
  int split;              // slots [0, split) belong to chunk c0, the rest to c1
  int c0, c1;
  float sgk0, sgk1, sgv0, sgv1;
  bool vcheck;            // some V product of this page may need the midpoint fix-up
};

__device__ __forceinline__ PageInfo page_info(const KvGeom& g, int64_t n_phys,
                                              const int32_t* pages, int pi, int n_pages,
                                              int last_tokens) {
  PageInfo p;
  const int32_t lp = pages[pi];
  bool mapped = lp >= 0 && lp < g.max_pages;
  const int64_t phys = mapped ? (int64_t)g.page_table[lp] : -1;
  mapped = mapped && phys >= 0 && phys < n_phys;
  p.page = mapped ? g.pool + phys * g.page_bytes : nullptr;
  p.valid = !mapped ? 0 : (pi == n_pages - 1 ? last_tokens : g.page_tokens);
  int c0 = mapped ? g.page_chunk[2 * lp] : 0;
  p.split = mapped ? g.page_chunk[2 * lp + 1] : g.page_tokens;
  c0 = c0 < 0 ? 0 : (c0 >= g.max_chunks ? g.max_chunks - 1 : c0);
  p.c0 = c0;
  p.c1 = c0 + 1 < g.max_chunks ? c0 + 1 : g.max_chunks - 1;
  p.sgk0 = g.k_gscale[p.c0];
  p.sgk1 = g.k_gscale[p.c1];
  p.sgv0 = g.v_gscale[p.c0];
  p.sgv1 = g.v_gscale[p.c1];
  p.vcheck = product_needs_check(p.sgv0) || product_needs_check(p.sgv1);
  return p;
}

// Decode keys [s0, s0 + 64) of head h of one page into K^ rows and V^T
// columns of LDS.  Thread t handles units t + 256 i (i = 0..3): key u / 16,
// channel group u % 16 (8 channels).
__device__ __forceinline__ void decode_block(const KvGeom& g, const PageInfo& p, int h, int s0,
                                             uint16_t* __restrict__ Ks,
                                             uint16_t* __restrict__ Vt) {
  const int H = g.n_heads, P = g.page_tokens;
  const int64_t codes_region = (int64_t)H * P * (kD / 2);
  const int64_t scales_region = (int64_t)H * P * (kD / 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = threadIdx.x + 256 * i;
    const int key = u >> 4, sub = u & 15;
    const int slot = s0 + key;
    u32x4 ko = u32x4{0, 0, 0, 0}, vo = u32x4{0, 0, 0, 0};
    if (p.page) {
      const int64_t row = (int64_t)h * P + slot;
      const uint32_t kcw = *(const uint32_t*)(p.page + row * (kD / 2) + 4 * sub);
      const uint32_t ksb = p.page[codes_region + row * (kD / 16) + (sub >> 1)];
      const uint32_t vcw =
          *(const uint32_t*)(p.page + codes_region + scales_region + row * (kD / 2) + 4 * sub);
      const uint32_t vsb =
          p.page[2 * codes_region + scales_region + row * (kD / 16) + (sub >> 1)];
      const bool second = slot >= p.split;
      const int c = second ? p.c1 : p.c0;
      const float* mp = g.k_mean + ((int64_t)c * H + h) * kD + 8 * sub;
      const f32x4 m0 = *(const f32x4*)mp, m1 = *(const f32x4*)(mp + 4);
      const float mu[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
      const float sgk = second ? p.sgk1 : p.sgk0, sgv = second ? p.sgv1 : p.sgv0;
      if (p.vcheck) kv_unit_bf16<true>(kcw, ksb, vcw, vsb, sgk, sgv, mu, ko, vo);
      else kv_unit_bf16<false>(kcw, ksb, vcw, vsb, sgk, sgv, mu, ko, vo);
    }
    *(u32x4*)(Ks + key * kKsRow + 8 * sub) = ko;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Vt[(8 * sub + 2 * e) * kVtRow + key] = (uint16_t)(vo[e] & 0xFFFFu);
      Vt[(8 * sub + 2 * e + 1) * kVtRow + key] = (uint16_t)(vo[e] >> 16);
    }
  }
}

}  // namespace

__global__ __launch_bounds__(256) void kv_attention_kernel(KvGeom g, int64_t n_phys,
                                                           const int32_t* __restrict__ pages,
                                                           int n_pages, int last_tokens,
                                                           const uint16_t* __restrict__ q,
                                                           int64_t n_q, float scale_log2e,
                                                           uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kKB * kKsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kD * kVtRow];
  const int H = g.n_heads, P = g.page_tokens;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5;
  const int64_t qrow = (int64_t)blockIdx.x * kQB + wave * 32 + (lane & 31);
  const int64_t qn = qrow < n_q ? qrow : n_q - 1;          // clamped rows are never stored

  // Q as the B operand of S^T = K^ Q^T: step s covers channels 16 s .. 16 s + 15,
  // lane half `half` the 8 channels 16 s + 8 half ..
  u32x4 qf[kD / 16];
  {
    const uint16_t* qp = q + (qn * H + h) * kD + 8 * half;
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) qf[s] = *(const u32x4*)(qp + 16 * s);
  }
  f32x16 o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m = -__builtin_inff(), l = 0.0f;

  const int bpp = P / kKB;                                  // blocks per page
  PageInfo pinfo;
  int cur_page = -1;
  for (int b = 0; b < n_pages * bpp; ++b) {
    const int pi = b / bpp, s0 = (b - pi * bpp) * kKB;
    if (pi != cur_page) {
      pinfo = page_info(g, n_phys, pages, pi, n_pages, last_tokens);
      cur_page = pi;
    }
    if (pinfo.valid <= s0) continue;                        // whole block masked (uniform)
    __syncthreads();                                        // previous block's LDS reads done
    decode_block(g, pinfo, h, s0, Ks, Vt);
    __syncthreads();

    // S^T tiles: keys 32 kt + (r / 4) * 8 + 4 half + r % 4 of this block, query lane % 32
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kt][r] = 0.0f;
      const uint16_t* kp = Ks + (32 * kt + (lane & 31)) * kKsRow + 8 * half;
#pragma unroll
      for (int s = 0; s < kD / 16; ++s)
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*(const u32x4*)(kp + 16 * s)),
                                                         as_bf16x8(qf[s]), st[kt], 0, 0, 0);
    }
    // online softmax for this lane's query (keys split between lane and lane ^ 32)
    float mb = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + (r >> 2) * 8 + 4 * half + (r & 3);
        const float t = s0 + key < pinfo.valid ? st[kt][r] * scale_log2e : -__builtin_inff();
        st[kt][r] = t;
        mb = fmaxf(mb, t);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float m_new = fmaxf(m, mb);                       // finite: the block has a valid key
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first block
    float ps = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(st[kt][r] - m_new);
        st[kt][r] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 32, 64);
    l = l * alpha + ps;
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

    // O^T += V^T P^T.  Step kk of key tile kt: k index j of lane half `half` is
    // key 32 kt + 16 kk + (j / 4) * 8 + 4 half + j % 4 = S^T register 8 kk + j.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 pb;
#pragma unroll
        for (int j = 0; j < 4; ++j) pb[j] = pack_bf16x2(st[kt][8 * kk + 2 * j], st[kt][8 * kk + 2 * j + 1]);
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) {
          const uint16_t* vp = Vt + (32 * dt + (lane & 31)) * kVtRow + 32 * kt + 16 * kk + 4 * half;
          const u32x2 v0 = *(const u32x2*)vp, v1 = *(const u32x2*)(vp + 8);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(u32x4{v0[0], v0[1], v1[0], v1[1]}), as_bf16x8(pb), o[dt], 0, 0, 0);
        }
      }
    }
  }

  // O = O^T / l, rounded once to bf16; register r of tile dt is channel
  // 32 dt + (r / 4) * 8 + 4 half + r % 4.
  if (qrow < n_q) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* op = out + (qrow * H + h) * kD + 4 * half;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(u32x2*)(op + 32 * dt + 8 * g4) =
            u32x2{pack_bf16x2(o[dt][4 * g4] * inv, o[dt][4 * g4 + 1] * inv),
                  pack_bf16x2(o[dt][4 * g4 + 2] * inv, o[dt][4 * g4 + 3] * inv)};
  }
}

void launch_kv_attention(const KvGeom& g, const int32_t* logical_pages, int32_t n_pages,
                         int32_t last_page_tokens, const uint16_t* q, int64_t n_q,
                         float softmax_scale, uint16_t* out, hipStream_t stream) {
  const float scale_log2e = (float)((double)softmax_scale * 1.4426950408889634);
  const dim3 grid((unsigned)((n_q + kQB - 1) / kQB), (unsigned)g.n_heads);
  hipLaunchKernelGGL(kv_attention_kernel, grid, dim3(256), 0, stream, g, g.n_phys_pages,
                     logical_pages, n_pages, last_page_tokens, q, n_q, scale_log2e, out);
}

}  // namespace nvfp4
