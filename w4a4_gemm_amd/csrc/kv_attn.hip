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

#include <type_traits>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef NVFP4_ATTN_WAVES
#define NVFP4_ATTN_WAVES 4
#endif
constexpr int kWaves = NVFP4_ATTN_WAVES;  // waves per workgroup, 32 queries each
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 32 * kWaves;          // queries per workgroup
constexpr int kKB = 64;               // keys per block
constexpr int kVtRow = kKB + 8;       // bf16 per V^T row in LDS (144 bytes)
constexpr int kMaxD = 128;            // largest head_dim (sizes the split workspace)

// Head-dim dependent shapes (head_dim kD = 64 or 128).
template <int kD>
struct Shape {
  static constexpr int kGroups = kD / 8;                 // 8-channel units per key
  static constexpr int kKPT = kKB * kGroups / kThreads;  // keys per thread in a block's decode
  static constexpr int kKsRow = kD + 8;                  // bf16 per Q / K^ row in LDS (conflict-free)
  static constexpr size_t kLds =                         // Q rows + K^ rows + V^T rows + K means
      2 * ((size_t)kQB * kKsRow + (size_t)kKB * kKsRow + (size_t)kD * kVtRow) + 2 * kD * 4;
  static_assert(kKPT == 2 || kKPT == 4, "a thread decodes 2 or 4 keys of a block");
  static_assert(kThreads >= 2 * kD && kThreads == 2 * kQB, "thread roles of the Q and mean loads");
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Per-page facts, uniform over the workgroup.
struct PageInfo {
  const uint8_t* page;    // a valid page address (page 0 when unmapped: loads stay in bounds)
  bool mapped;
  int valid;              // valid slots of the page (keys beyond are masked)
  int split;              // slots [0, split) belong to chunk c0, the rest to c1
  int c0, c1;
  float sgk0, sgk1, sgv0, sgv1;
  bool vcheck;            // a V^ product of this page may need the bf16 midpoint fix-up
};

__device__ __forceinline__ PageInfo page_info(const KvGeom& g, int64_t n_phys,
                                              const int32_t* pages, int pi, int n_pages,
                                              int last_tokens) {
  PageInfo p;
  const int32_t lp = pages[pi];
  bool mapped = lp >= 0 && lp < g.max_pages;
  const int64_t phys = mapped ? (int64_t)g.page_table[lp] : -1;
  mapped = mapped && phys >= 0 && phys < n_phys;
  p.mapped = mapped;
  p.page = g.pool + (mapped ? phys : 0) * g.page_bytes;
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

// The raw inputs of one block for this thread: with G = kD / 8 channel groups
// per key, its units are the kKPT adjacent keys kKPT (tid / G) + i in channel
// group tid % G (the same 8 channels for every unit), written to V^T as
// kKPT-key runs.  The K means of the page's two chunks (2 x kD floats) travel
// one per thread and are shared through LDS.
template <int kKPT>
struct BlockRaw {
  uint32_t kc[kKPT], ks[kKPT], vc[kKPT], vs[kKPT];
  float mu;               // K mean of chunk (tid < kD ? c0 : c1), channel tid % kD (tid < 2 kD)
};

template <int kD>
__device__ __forceinline__ void fetch_block(const KvGeom& g, const PageInfo& p, int h, int s0,
                                            BlockRaw<Shape<kD>::kKPT>& r) {
  constexpr int kKPT = Shape<kD>::kKPT, kGroups = Shape<kD>::kGroups;
  // 32-bit offsets from the (uniform) page address: a page is far below 4 GiB
  const uint32_t H = g.n_heads, P = g.page_tokens;
  const uint32_t codes_region = H * P * (kD / 2);
  const uint32_t scales_region = H * P * (kD / 16);
  const uint32_t sub = threadIdx.x % kGroups;
  const uint32_t row0 = (uint32_t)h * P + s0 + kKPT * (threadIdx.x / kGroups);
#pragma unroll
  for (int i = 0; i < kKPT; ++i) {
    const uint32_t row = row0 + i;
    r.kc[i] = *(const uint32_t*)(p.page + (row * (kD / 2) + 4 * sub));
    r.ks[i] = p.page[codes_region + row * (kD / 16) + (sub >> 1)];
    r.vc[i] = *(const uint32_t*)(p.page + (codes_region + scales_region + row * (kD / 2) + 4 * sub));
    r.vs[i] = p.page[2 * codes_region + scales_region + row * (kD / 16) + (sub >> 1)];
  }
  if (threadIdx.x < 2 * kD)
    r.mu = g.k_mean[((int64_t)(threadIdx.x < kD ? p.c0 : p.c1) * H + h) * kD + (threadIdx.x & (kD - 1))];
}

// Decode a fetched block into K^ rows and V^T columns of LDS.  Slots that hold
// no key (unmapped page, past the last valid slot) give zeros: their weights are
// 0, and zero values keep 0 * V^ finite whatever bytes the slot holds.
// kSimple: the block is mapped, every slot holds a key and all belong to chunk
// `cs` (uniform), so no per-key choice of chunk or mask is needed.
template <int kD, bool kVCheck, bool kSimple>
__device__ __forceinline__ void decode_block(const PageInfo& p, int s0, int cs,
                                             const BlockRaw<Shape<kD>::kKPT>& r,
                                             const float* __restrict__ Mu,
                                             uint16_t* __restrict__ Ks,
                                             uint16_t* __restrict__ Vt) {
  constexpr int kKPT = Shape<kD>::kKPT, kGroups = Shape<kD>::kGroups;
  constexpr int kKsRow = Shape<kD>::kKsRow;
  const int sub = threadIdx.x % kGroups;
  const float* m0p = Mu + (kSimple ? cs * kD : 0) + 8 * sub;
  const f32x4 a0 = *(const f32x4*)m0p, b0 = *(const f32x4*)(m0p + 4);
  const float mu0[8] = {a0[0], a0[1], a0[2], a0[3], b0[0], b0[1], b0[2], b0[3]};
  float mu1[8];
  if (!kSimple) {
    const f32x4 a1 = *(const f32x4*)(Mu + kD + 8 * sub), b1 = *(const f32x4*)(Mu + kD + 8 * sub + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mu1[e] = a1[e];
      mu1[4 + e] = b1[e];
    }
  }
  const float sgk_s = cs ? p.sgk1 : p.sgk0, sgv_s = cs ? p.sgv1 : p.sgv0;
  uint32_t vw[kKPT][4];                                     // V^ words of the thread's keys
#pragma unroll
  for (int i = 0; i < kKPT; ++i) {
    const int key = kKPT * (threadIdx.x / kGroups) + i;
    u32x4 ko, vo;
    if (kSimple) {
      kv_unit_bf16<kVCheck>(r.kc[i], r.ks[i], r.vc[i], r.vs[i], sgk_s, sgv_s, mu0, ko, vo);
    } else {
      const bool second = s0 + key >= p.split;
      kv_unit_bf16<kVCheck>(r.kc[i], r.ks[i], r.vc[i], r.vs[i], second ? p.sgk1 : p.sgk0,
                            second ? p.sgv1 : p.sgv0, second ? mu1 : mu0, ko, vo);
      if (!p.mapped || s0 + key >= p.valid) {               // no key: zeros, never NaN
        ko = u32x4{0, 0, 0, 0};
        vo = u32x4{0, 0, 0, 0};
      }
    }
    *(u32x4*)(Ks + key * kKsRow + 8 * sub) = ko;
#pragma unroll
    for (int e = 0; e < 4; ++e) vw[i][e] = vo[e];
  }
  // V^T row 8 sub + c holds channel c of the 4 keys: bf16 of key i is the
  // low (c even) or high (c odd) half of vw[i][c / 2]
  const int k0 = kKPT * (threadIdx.x / kGroups);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t lo = __builtin_amdgcn_perm(vw[1][c >> 1], vw[0][c >> 1], sel);
    if (kKPT == 4) {
      const uint32_t hi = __builtin_amdgcn_perm(vw[kKPT - 1][c >> 1], vw[kKPT - 2][c >> 1], sel);
      *(u32x2*)(Vt + (8 * sub + c) * kVtRow + k0) = u32x2{lo, hi};
    } else {
      *(uint32_t*)(Vt + (8 * sub + c) * kVtRow + k0) = lo;
    }
  }
}

}  // namespace

// Key splits: when the grid of (query block, head) is small, the window is
// split over several workgroups whose partial results are merged by
// kv_attention_combine.  A pure function of the sizes, shared by the
// workspace query and the launcher.
int attention_splits(int64_t n_q, int64_t n_heads, int64_t n_keys) {
  const int64_t base = ((n_q + kQB - 1) / kQB) * n_heads;
  const int64_t blocks = (n_keys + kKB - 1) / kKB;
  if (base >= 512 || blocks < 16) return 1;
  // Workgroups run two per CU (512 at once on 256 CUs).  Time ~ rounds of
  // workgroups x blocks per workgroup, plus the merge, which reads every split's
  // partial O (about 0.6 block-times per split here); each split keeps >= 8 blocks.
  constexpr int64_t kSlots = 512;
  const int64_t s_max = blocks / 8 < 64 ? blocks / 8 : 64;
  int64_t best_s = 1;
  double best = (double)blocks * ((base + kSlots - 1) / kSlots);
  for (int64_t s = 2; s <= s_max; ++s) {
    const double cost = (double)((base * s + kSlots - 1) / kSlots) * ((blocks + s - 1) / s) +
                        0.6 * (double)s;
    if (cost < best) {
      best = cost;
      best_s = s;
    }
  }
  return (int)best_s;
}

size_t kv_attention_workspace_bytes(int64_t n_q, int64_t n_heads, int64_t n_keys) {
  const int s = attention_splits(n_q, n_heads, n_keys);
  if (s == 1) return 0;
  return (size_t)s * n_q * n_heads * (kMaxD + 2) * sizeof(float);
}

// Split `split` of `n_split` handles key blocks [b0, b1) of the window.  With
// one split the result is normalized and written as bf16; otherwise the
// unnormalized fp32 O^T, the running max m (log2 units) and the sum l go to
// the workspace: O at part + ((split * n_q + n) * H + h) * D, (m, l) after all
// O values.
// Two workgroups per CU (registers capped at 256 per lane), so one
// workgroup's decode overlaps the other's MFMAs.
template <int kD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void kv_attention_kernel(KvGeom g, int64_t n_phys,
                                                           const int32_t* __restrict__ pages,
                                                           int n_pages, int last_tokens,
                                                           const uint16_t* __restrict__ q,
                                                           int64_t n_q, float scale_log2e,
                                                           uint32_t q_sign,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ part, int n_split) {
  // LDS (Shape<kD>::kLds bytes, dynamic): Q rows, K^ rows, V^T rows, K means of chunk c0 then c1
  constexpr int kKsRow = Shape<kD>::kKsRow;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* Qs = smem;
  uint16_t* Ks = Qs + kQB * kKsRow;
  uint16_t* Vt = Ks + kKB * kKsRow;
  float* Mu = (float*)(Vt + kD * kVtRow);
  const int H = g.n_heads, P = g.page_tokens;
  const int h = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5;
  const int64_t qrow = (int64_t)blockIdx.x * kQB + wave * 32 + (lane & 31);

  // The workgroup's 128 query rows go to LDS once (two threads per row, kD / 2
  // channels each); the first barrier of the block loop publishes them.  They
  // are the B operand of S^T = K^ Q^T: step s covers channels 16 s .. 16 s + 15,
  // lane half `half` the 8 channels 16 s + 8 half ..
  {
    const int row = tid >> 1;
    const int64_t qr = (int64_t)blockIdx.x * kQB + row;
    const uint16_t* qp = q + ((qr < n_q ? qr : n_q - 1) * H + h) * kD + (kD / 2) * (tid & 1);
    uint16_t* qs = Qs + row * kKsRow + (kD / 2) * (tid & 1);
#pragma unroll
    for (int i = 0; i < kD / 16; ++i) {
      u32x4 v = *(const u32x4*)(qp + 8 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] ^= q_sign;           // -q when the scale is negative
      *(u32x4*)(qs + 8 * i) = v;
    }
  }
  f32x16 o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m = -__builtin_inff(), l = 0.0f;

  const int bpp = P / kKB;                                  // blocks per page
  const int nb = n_pages * bpp;
  const int b0 = (int)((int64_t)nb * split / n_split), b1 = (int)((int64_t)nb * (split + 1) / n_split);

  // software pipeline: the raw inputs of block b + 1 are in flight while
  // block b is decoded and consumed
  PageInfo pn;
  BlockRaw<Shape<kD>::kKPT> rn;
  if (b0 < b1) {
    pn = page_info(g, n_phys, pages, b0 / bpp, n_pages, last_tokens);
    fetch_block<kD>(g, pn, h, (b0 % bpp) * kKB, rn);
  }
  for (int b = b0; b < b1; ++b) {
    const int s0 = (b % bpp) * kKB;
    const PageInfo pc = pn;
    const BlockRaw<Shape<kD>::kKPT> rc = rn;
    if (b + 1 < b1) {
      if ((b + 1) % bpp == 0) pn = page_info(g, n_phys, pages, (b + 1) / bpp, n_pages, last_tokens);
      fetch_block<kD>(g, pn, h, ((b + 1) % bpp) * kKB, rn);
    }
    if (pc.valid <= s0) continue;                           // whole block masked (uniform)
    if (tid < 2 * kD) Mu[tid] = rc.mu;     // safe: the previous decode's reads of Mu
    __syncthreads();                       // finished before the previous block's MFMAs
    {
      const bool one_chunk = s0 + kKB <= pc.split || s0 >= pc.split;
      const bool simple = pc.mapped && s0 + kKB <= pc.valid && one_chunk;
      const int cs = s0 >= pc.split ? 1 : 0;
      if (simple) {
        if (pc.vcheck) decode_block<kD, true, true>(pc, s0, cs, rc, Mu, Ks, Vt);
        else decode_block<kD, false, true>(pc, s0, cs, rc, Mu, Ks, Vt);
      } else {
        if (pc.vcheck) decode_block<kD, true, false>(pc, s0, 0, rc, Mu, Ks, Vt);
        else decode_block<kD, false, false>(pc, s0, 0, rc, Mu, Ks, Vt);
      }
    }
    __syncthreads();

    // S^T tiles: keys 32 kt + (r / 4) * 8 + 4 half + r % 4 of this block, query lane % 32
    // (the two key tiles' MFMA chains alternate, sharing each Q fragment)
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kt][r] = 0.0f;
    {
      const uint16_t* kp = Ks + (lane & 31) * kKsRow + 8 * half;
      const uint16_t* qs = Qs + (wave * 32 + (lane & 31)) * kKsRow + 8 * half;
#pragma unroll
      for (int s = 0; s < kD / 16; ++s) {
        const bf16x8 qv = as_bf16x8(*(const u32x4*)(qs + 16 * s));
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(*(const u32x4*)(kp + 32 * kt * kKsRow + 16 * s)), qv, st[kt], 0, 0, 0);
      }
    }
    // online softmax for this lane's query (keys split between lane and lane ^ 32),
    // in log2 units: t = S c with c = |scale| log2(e) >= 0, so the block max of t is
    // RN(c max S) and each weight is exp2(fma(S, c, -m)).  Keys past the last
    // valid slot only occur in a block that is not full (uniform test).
    const bool full = s0 + kKB <= pc.valid;
    float mb = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + (r >> 2) * 8 + 4 * half + (r & 3);
        if (full || s0 + key < pc.valid) mb = fmaxf(mb, st[kt][r]);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float m_new = fmaxf(m, mb * scale_log2e);         // finite: the block has a valid key
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first block
    float ps = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + (r >> 2) * 8 + 4 * half + (r & 3);
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kt][r], scale_log2e, -m_new));
        if (!full && s0 + key >= pc.valid) p = 0.0f;
        st[kt][r] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 32, 64);
    l = l * alpha + ps;
    m = m_new;
    if (__any(alpha != 1.0f)) {                             // the running max moved
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }

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

  // register r of tile dt is channel 32 dt + (r / 4) * 8 + 4 half + r % 4
  if (qrow < n_q) {
    if (n_split == 1) {
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      uint16_t* op = out + (qrow * H + h) * kD + 4 * half;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(u32x2*)(op + 32 * dt + 8 * g4) =
              u32x2{pack_bf16x2(o[dt][4 * g4] * inv, o[dt][4 * g4 + 1] * inv),
                    pack_bf16x2(o[dt][4 * g4 + 2] * inv, o[dt][4 * g4 + 3] * inv)};
    } else {
      float* op = part + (((int64_t)split * n_q + qrow) * H + h) * kD + 4 * half;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(f32x4*)(op + 32 * dt + 8 * g4) =
              f32x4{o[dt][4 * g4], o[dt][4 * g4 + 1], o[dt][4 * g4 + 2], o[dt][4 * g4 + 3]};
      if (half == 0) {
        float* ml = part + (int64_t)n_split * n_q * H * kD + (((int64_t)split * n_q + qrow) * H + h) * 2;
        *(f32x2*)ml = f32x2{m, l};
      }
    }
  }
}

// Merge the splits of one (query, head) row: M = max m_s, L = sum l_s 2^(m_s - M),
// O = sum O_s 2^(m_s - M) / L, rounded once to bf16.  One wave per row, kD / 64
// channels per lane.
template <int kD>
__global__ __launch_bounds__(256) void kv_attention_combine(const float* __restrict__ part,
                                                            int n_split, int64_t rows,
                                                            uint16_t* __restrict__ out) {
  constexpr int kCpl = kD / 64;                             // channels per lane: 1 or 2
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* ml = part + (int64_t)n_split * rows * kD;
  float M = -__builtin_inff();
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, ml[((int64_t)s * rows + row) * 2]);
  float L = 0.0f, a[kCpl] = {};
  if (M != -__builtin_inff()) {
    for (int s = 0; s < n_split; ++s) {
      const f32x2 v = *(const f32x2*)(ml + ((int64_t)s * rows + row) * 2);
      const float w = __builtin_amdgcn_exp2f(v[0] - M);    // 0 for an empty split (m = -inf)
      const float* os = part + ((int64_t)s * rows + row) * kD + kCpl * lane;
      L += v[1] * w;
#pragma unroll
      for (int c = 0; c < kCpl; ++c) a[c] += os[c] * w;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  if (kCpl == 2)
    *(uint32_t*)(out + row * kD + 2 * lane) = pack_bf16x2(a[0] * inv, a[kCpl - 1] * inv);
  else
    out[row * kD + lane] = (uint16_t)f32_to_bf16_bits(a[0] * inv);
}

void launch_kv_attention(const KvGeom& g, const int32_t* logical_pages, int32_t n_pages,
                         int32_t last_page_tokens, const uint16_t* q, int64_t n_q,
                         float softmax_scale, uint16_t* out, void* workspace,
                         hipStream_t stream) {
  // logits in log2 units with a non-negative factor; a negative scale negates q
  // instead (exact in bf16), so the block max maps to the max weight
  const float scale_log2e = (float)(fabs((double)softmax_scale) * 1.4426950408889634);
  const uint32_t q_sign = softmax_scale < 0.0f ? 0x80008000u : 0u;
  const int n_split = attention_splits(n_q, g.n_heads, (int64_t)n_pages * g.page_tokens);
  const dim3 grid((unsigned)((n_q + kQB - 1) / kQB), (unsigned)g.n_heads, (unsigned)n_split);
  const auto go = [&](auto d) {
    constexpr int kD = decltype(d)::value;
    constexpr size_t kLds = Shape<kD>::kLds;
    // dynamic LDS above the default 64 KB limit (head_dim 128), raised once per device
    static std::atomic<uint64_t> lds_done{0};
    if (kLds > 65536) ensure_dynamic_lds((const void*)kv_attention_kernel<kD>, (int)kLds, lds_done);
    hipLaunchKernelGGL(kv_attention_kernel<kD>, grid, dim3(kThreads), kLds, stream, g,
                       g.n_phys_pages, logical_pages, n_pages, last_page_tokens, q, n_q,
                       scale_log2e, q_sign, out, (float*)workspace, n_split);
    if (n_split > 1) {
      const int64_t rows = n_q * g.n_heads;
      hipLaunchKernelGGL(kv_attention_combine<kD>, dim3((unsigned)((rows + 3) / 4)), dim3(256),
                         0, stream, (const float*)workspace, n_split, rows, out);
    }
  };
  if (g.head_dim == 64) go(std::integral_constant<int, 64>{});
  else go(std::integral_constant<int, 128>{});
}

}  // namespace nvfp4
