// Fused attention over the paged NVFP4 KV cache for gfx950.
//
// The cache is read block by block (techwalker.com LongLive-2.0 report
// summary, section 四, second key: many cache blocks of the time window are
// decompressed in parallel); here each 64-key block is decompressed into LDS
// with exactly the rounding of the window-read kernel (K^ = RN_bf16(q s_b
// s_gK + mu), V^ = RN_bf16(q s_b s_gV)) and consumed at once by a
// flash-attention step, so no bf16 K or V reaches HBM.
//
// Layout of work: a workgroup is one head and 256 queries (8 waves x 32, two
// waves per SIMD), so each decoded block serves 256 queries; a wave keeps its
// 32 query rows in registers.  K^ and V^T are double-buffered in LDS: while
// the waves multiply block b from one buffer, the workgroup decodes block
// b + 1 into the other (the decode's VALU work issues under the MFMAs), so a
// block costs one barrier.  Each wave computes the transposed products on the
// bf16 MFMA
//   S^T = K^ Q^T    (32 keys x 32 queries per v_mfma_f32_32x32x16_bf16 tile)
//   O^T += V^T P^T  (32 channels x 32 queries per tile)
// so that in both accumulators a lane owns one query (column lane % 32) and
// its registers run over keys or channels.  The online softmax (reference
// max m, running sum l, rescaling of O) is then per lane plus one exchange with
// lane ^ 32 (a permlane swap), and P goes from the S^T registers straight into the second
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
#define NVFP4_ATTN_WAVES 8
#endif
constexpr int kWaves = NVFP4_ATTN_WAVES;  // waves per workgroup, 32 queries each
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 32 * kWaves;          // queries per workgroup
constexpr int kKB = 64;               // keys per block
constexpr int kVtRow = kKB + 8;       // bf16 per V^T row in LDS (144 bytes)
constexpr int kMaxD = 128;            // largest head_dim (sizes the split workspace)
constexpr float kLazy = 8.0f;         // slack of the softmax reference max (log2 units)

// Head-dim dependent shapes (head_dim kD = 64 or 128).
template <int kD>
struct Shape {
  static constexpr int kGroups = kD / 8;                 // 8-channel units per key
  static constexpr int kKPT = kKB * kGroups / kThreads;  // keys per thread in a block's decode
  static constexpr int kKsRow = kD + 8;                  // bf16 per K^ row in LDS (conflict-free)
  static constexpr size_t kKsElems = (size_t)kKB * kKsRow;   // bf16 per K^ buffer
  static constexpr size_t kVtElems = (size_t)kD * kVtRow;    // bf16 per V^T buffer
  static constexpr size_t kLds = 2 * 2 * (kKsElems + kVtElems);   // bytes: 2 x (K^ rows + V^T rows)
  static_assert(kKPT == 1 || kKPT == 2 || kKPT == 4, "a thread decodes 1, 2 or 4 keys of a block");
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// x combined with the x of lane ^ 32, without LDS: gfx950's permlane32 swap
// exchanges the upper half of one copy with the lower half of another, so
// lane i of the two results holds x of lanes i % 32 and i % 32 + 32 (in some
// order); max and + of the two are symmetric in that order.
__device__ __forceinline__ float max_lane32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_lane32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of key k (0..63) in a V^T row: bits 2 and 3 of k swapped.  The
// O^T MFMA's lane half `half` takes, in step kk of key tile kt, the keys
// 32 kt + 16 kk + 4 half + {0..3} and the same plus 8; with this order they
// are the 8 contiguous positions 32 kt + 16 kk + 8 half .. (one 16-byte read).
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Offset (bf16) of channel ch's V^T row at key position pos in a V^T buffer.
// The row of channel ch is ch with bit 0 flipped when bit 4 is set, and the
// row's 16-byte chunks are permuted, chunk pos / 8 stored at chunk
// (pos / 8) ^ (2 ((ch / 32) % 4)).  A decode write instruction covers the
// rows of channel c of the 16 channel groups (8 apart, so without a
// permutation they share a few LDS banks) and, with unit_key0's key order,
// four dwords of one chunk; these two permutations spread them over all
// banks, while the O^T fragment reads (32 rows of one 32-channel block, one
// chunk) keep their conflict-free pattern.  Measured on the device: a
// transposed write instruction takes 2 LDS cycles (64 with plain rows) and a
// fragment read 4, neither with bank conflicts.
__device__ __forceinline__ int vt_index(int ch, int pos) {
  return (ch ^ ((ch >> 4) & 1)) * kVtRow + 8 * ((pos >> 3) ^ (2 * ((ch >> 5) & 3))) + (pos & 7);
}

// First key of this thread's decode units (kKPT adjacent keys; kGroups =
// kD / 8 threads share a key run).  With two keys per thread the wave's four
// key pairs are keys {0, 2, 8, 10} + 4 (bit 0 of the wave) + 16 m, i.e. the
// four dwords of one V^T chunk (the pair index has bits 1 and 2 swapped), and
// a thread of odd channel group takes the pair of the other half of the wave
// (slot XOR 2), so that each 32-lane half of a write covers all four dwords.
template <int kKPT, int kGroups>
__device__ __forceinline__ int unit_key0() {
  int j = (int)threadIdx.x / kGroups;
  if (kKPT == 2) {
    j = (j & ~3) | ((j & 3) ^ (2 * ((int)(threadIdx.x % kGroups) & 1)));
    j = (j & ~6) | ((j & 2) << 1) | ((j & 4) >> 1);
  }
  return kKPT * j;
}

// A workgroup-uniform value read through the scalar unit (the page table,
// page->chunk table and chunk scales are not written while the kernel runs),
// so that waiting for it does not also wait for the vector loads in flight.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Per-page facts, uniform over the workgroup.
// (32-bit fields only: a struct with padding bytes is copied through scratch
// memory when the pipeline rotates it.)
struct PageInfo {
  const uint8_t* page;    // a valid page address (page 0 when unmapped: loads stay in bounds)
  int mapped;
  int valid;              // valid slots of the page (keys beyond are masked)
  int split;              // slots [0, split) belong to chunk c0, the rest to c1
  int c0, c1;
  float sgk0, sgk1, sgv0, sgv1;
  int vcheck;             // a V^ product of this page may need the bf16 midpoint fix-up
};

// `prev`: the facts of the page before, when `has_prev` (consecutive pages
// usually hold the same chunks, whose V scale test is then reused instead of
// recomputed).
__device__ __forceinline__ PageInfo page_info(const KvGeom& g, int64_t n_phys,
                                              const int32_t* pages, int pi, int n_pages,
                                              int last_tokens, const PageInfo& prev,
                                              bool has_prev) {
  PageInfo p;
  const int32_t lp = load_uniform(pages + pi);
  bool mapped = lp >= 0 && lp < g.max_pages;
  const int64_t phys = mapped ? (int64_t)load_uniform(g.page_table + lp) : -1;
  mapped = mapped && phys >= 0 && phys < n_phys;
  p.mapped = mapped;
  p.page = g.pool + (mapped ? phys : 0) * g.page_bytes;
  p.valid = !mapped ? 0 : (pi == n_pages - 1 ? last_tokens : g.page_tokens);
  int c0 = mapped ? load_uniform(g.page_chunk + 2 * lp) : 0;
  p.split = mapped ? load_uniform(g.page_chunk + 2 * lp + 1) : g.page_tokens;
  c0 = c0 < 0 ? 0 : (c0 >= g.max_chunks ? g.max_chunks - 1 : c0);
  p.c0 = c0;
  p.c1 = c0 + 1 < g.max_chunks ? c0 + 1 : g.max_chunks - 1;
  p.sgk0 = load_uniform(g.k_gscale + p.c0);
  p.sgk1 = load_uniform(g.k_gscale + p.c1);
  p.sgv0 = load_uniform(g.v_gscale + p.c0);
  p.sgv1 = load_uniform(g.v_gscale + p.c1);
  if (has_prev && prev.sgv0 == p.sgv0 && prev.sgv1 == p.sgv1)
    p.vcheck = prev.vcheck;
  else
    p.vcheck = product_needs_check(p.sgv0) || product_needs_check(p.sgv1);
  return p;
}

// The raw inputs of one block for this thread: with G = kD / 8 channel groups
// per key, its units are the kKPT adjacent keys unit_key0() + i in channel
// group tid % G (the same 8 channels for every unit), written to V^T as
// kKPT-key runs.  The K means of those 8 channels, for the chunk of the
// block's first slot, travel with them (the only chunk of a block that needs
// no per-key choice; the other blocks read theirs when they are decoded), so
// a block's decode waits only for loads issued one block earlier.
template <int kKPT>
struct BlockRaw {
  uint32_t kc[kKPT], ks[kKPT], vc[kKPT], vs[kKPT];
  f32x4 mu_lo, mu_hi;     // K means of channels 8 (tid % G) + 0..3 and + 4..7
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
  const uint32_t row0 = (uint32_t)h * P + s0 + unit_key0<kKPT, kGroups>();
#pragma unroll
  for (int i = 0; i < kKPT; ++i) {
    const uint32_t row = row0 + i;
    r.kc[i] = *(const uint32_t*)(p.page + (row * (kD / 2) + 4 * sub));
    r.ks[i] = p.page[codes_region + row * (kD / 16) + (sub >> 1)];
    r.vc[i] = *(const uint32_t*)(p.page + (codes_region + scales_region + row * (kD / 2) + 4 * sub));
    r.vs[i] = p.page[2 * codes_region + scales_region + row * (kD / 16) + (sub >> 1)];
  }
  const float* mp = g.k_mean + ((int64_t)(s0 >= p.split ? p.c1 : p.c0) * H + h) * kD + 8 * sub;
  r.mu_lo = *(const f32x4*)mp;
  r.mu_hi = *(const f32x4*)(mp + 4);
}

// Decode a fetched block into K^ rows and V^T columns of LDS.  Slots that hold
// no key (unmapped page, past the last valid slot) give zeros: their weights are
// 0, and zero values keep 0 * V^ finite whatever bytes the slot holds.
// kSimple: the block is mapped, every slot holds a key and all belong to chunk
// `cs` (uniform), so no per-key choice of chunk or mask is needed.
template <int kD, bool kVCheck, bool kSimple>
__device__ __forceinline__ void decode_block(const KvGeom& g, int h, const PageInfo& p, int s0,
                                             int cs, const BlockRaw<Shape<kD>::kKPT>& r,
                                             uint16_t* __restrict__ Ks,
                                             uint16_t* __restrict__ Vt) {
  constexpr int kKPT = Shape<kD>::kKPT, kGroups = Shape<kD>::kGroups;
  constexpr int kKsRow = Shape<kD>::kKsRow;
  const int sub = threadIdx.x % kGroups;
  // K means: the fetched ones (chunk cs) for a simple block; both chunks'
  // from memory otherwise (chunk boundaries, unmapped or partial pages)
  f32x4 a0 = r.mu_lo, b0 = r.mu_hi, a1, b1;
  if (!kSimple) {
    const float* m0p = g.k_mean + ((int64_t)p.c0 * g.n_heads + h) * kD + 8 * sub;
    const float* m1p = g.k_mean + ((int64_t)p.c1 * g.n_heads + h) * kD + 8 * sub;
    a0 = *(const f32x4*)m0p;
    b0 = *(const f32x4*)(m0p + 4);
    a1 = *(const f32x4*)m1p;
    b1 = *(const f32x4*)(m1p + 4);
  }
  const float mu0[8] = {a0[0], a0[1], a0[2], a0[3], b0[0], b0[1], b0[2], b0[3]};
  float mu1[8];
  if (!kSimple) {
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
    const int key = unit_key0<kKPT, kGroups>() + i;
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
  // Channel 8 sub + c: bf16 of key i is the low (c even) or high (c odd)
  // half of vw[i][c / 2].  Keys sit at position vt_pos(key) of the row (runs
  // of 4 keys stay contiguous), stored at vt_index: for this thread's
  // channels the chunk permutation is one constant and the row is 8 sub + c
  // moved by +b (c even) or -b (c odd), b = bit 1 of sub.
  const int k0 = vt_pos(unit_key0<kKPT, kGroups>());
  const int vb = (sub >> 1) & 1;
  uint16_t* const vt0 = Vt + (8 * sub) * kVtRow + 8 * ((k0 >> 3) ^ (2 * ((sub >> 2) & 3))) + (k0 & 7);
  uint16_t* const vt_even = vt0 + vb * kVtRow;
  uint16_t* const vt_odd = vt0 - vb * kVtRow;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint16_t* vt = ((c & 1) ? vt_odd : vt_even) + c * kVtRow;
    if (kKPT == 1) {
      *vt = (uint16_t)((c & 1) ? vw[0][c >> 1] >> 16 : vw[0][c >> 1]);
      continue;
    }
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t lo = __builtin_amdgcn_perm(vw[kKPT > 1 ? 1 : 0][c >> 1], vw[0][c >> 1], sel);
    if (kKPT == 4) {
      const uint32_t hi = __builtin_amdgcn_perm(vw[kKPT - 1][c >> 1], vw[kKPT - 2][c >> 1], sel);
      *(u32x2*)vt = u32x2{lo, hi};
    } else {
      *(uint32_t*)vt = lo;
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
  // Two waves per SIMD: 8 / kWaves workgroups per CU run at once.  Time ~ rounds of
  // workgroups x blocks per workgroup, plus the merge, which reads every split's
  // partial O (about 0.6 block-times per split here); each split keeps >= 8 blocks.
  constexpr int64_t kSlots = 256 * (8 / kWaves);
  if (base >= kSlots || blocks < 16) return 1;
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

// One block of keys for a wave's 32 queries: S^T = K^ Q^T from buffer (Kc, Vc),
// the online-softmax update of (m, l, O), and O^T += V^T P^T.  `decode_next`
// runs between the S^T MFMAs and the softmax: it decodes the next block into
// the other buffer (restrict-qualified, so its LDS stores may pass these
// reads and its VALU work can issue under the MFMAs).
template <int kD, typename Decode>
__device__ __forceinline__ void attend_block(const uint16_t* __restrict__ Kc,
                                             const uint16_t* __restrict__ Vc,
                                             const bf16x8 (&qr)[kD / 16], int lane, int s0,
                                             int valid, float scale_log2e, float& m, float& l,
                                             f32x16 (&o)[kD / 32], const Decode& decode_next) {
  constexpr int kKsRow = Shape<kD>::kKsRow;
  const int half = lane >> 5;
  // S^T tiles: keys 32 kt + (r / 4) * 8 + 4 half + r % 4 of this block, query lane % 32
  // (the two key tiles' MFMA chains alternate, sharing each Q fragment)
  f32x16 st[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st[kt][r] = 0.0f;
  {
    const uint16_t* kp = Kc + (lane & 31) * kKsRow + 8 * half;
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(*(const u32x4*)(kp + 32 * kt * kKsRow + 16 * s)), qr[s], st[kt], 0, 0, 0);
    }
  }
  decode_next();
  // online softmax for this lane's query (keys split between lane and lane ^ 32),
  // in log2 units: t = S c with c = |scale| log2(e) >= 0, so the block max of t is
  // RN(c max S) and each weight is exp2(fma(S, c, -m)) for the reference m.  Keys past the last
  // valid slot only occur in a block that is not full: a full block (the
  // usual case, a uniform test) takes a loop without per-key masks.  (This
  // file is compiled without NaN support, so fmaxf is one instruction.)
  const bool full = s0 + kKB <= valid;
  float mb = -__builtin_inff();
  if (full) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mb = fmaxf(mb, st[kt][r]);
  } else {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + (r >> 2) * 8 + 4 * half + (r & 3);
        if (s0 + key < valid) mb = fmaxf(mb, st[kt][r]);
      }
  }
  mb = max_lane32(mb);
  // m is a reference, not always the running max: it moves only when a block's
  // max exceeds it by more than kLazy (log2 units), so weights stay below
  // 2^kLazy (exact in scale for bf16 and fp32) and O is rescaled rarely.
  const float bmax = mb * scale_log2e;                    // finite: the block has a valid key
  const float m_new = bmax > m + kLazy ? bmax : m;         // the first block always moves m
  const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first block
  float ps = 0.0f;
  if (full) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kt][r], scale_log2e, -m_new));
        st[kt][r] = p;
        ps += p;
      }
  } else {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + (r >> 2) * 8 + 4 * half + (r & 3);
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kt][r], scale_log2e, -m_new));
        if (s0 + key >= valid) p = 0.0f;
        st[kt][r] = p;
        ps += p;
      }
  }
  ps = sum_lane32(ps);
  l = l * alpha + ps;
  m = m_new;
  if (__any(alpha != 1.0f)) {                             // a reference moved
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
  }

  // O^T += V^T P^T.  Step kk of key tile kt: k index j of lane half `half` is
  // key 32 kt + 16 kk + (j / 4) * 8 + 4 half + j % 4 = S^T register 8 kk + j.
  // Lane reads channel 32 dt + x (x = lane % 32) at position 32 kt + 16 kk +
  // 8 half, i.e. vt_index: row 32 dt + (x with bit 0 flipped when bit 4 is
  // set), chunk ((4 kt + 2 kk) ^ 2 dt) + half.
  const int vx = lane & 31;
  const uint16_t* vrow = Vc + (vx ^ ((vx >> 4) & 1)) * kVtRow + 8 * half;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 pb;
#pragma unroll
      for (int j = 0; j < 4; ++j) pb[j] = pack_bf16x2(st[kt][8 * kk + 2 * j], st[kt][8 * kk + 2 * j + 1]);
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) {
        // the 8 keys of this lane half are contiguous in the V^T row (vt_pos)
        const uint16_t* vp = vrow + 32 * dt * kVtRow + 8 * ((4 * kt + 2 * kk) ^ (2 * dt));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*(const u32x4*)vp),
                                                        as_bf16x8(pb), o[dt], 0, 0, 0);
      }
    }
  }
}

// Decode block (page facts p, first slot s0, raw inputs r) of head h into (Kn, Vn).
template <int kD>
__device__ __forceinline__ void decode_any(const KvGeom& g, int h, const PageInfo& p, int s0,
                                           const BlockRaw<Shape<kD>::kKPT>& r,
                                           uint16_t* __restrict__ Kn, uint16_t* __restrict__ Vn) {
  const bool one_chunk = s0 + kKB <= p.split || s0 >= p.split;
  const bool simple = p.mapped && s0 + kKB <= p.valid && one_chunk;
  const int cs = s0 >= p.split ? 1 : 0;
  if (simple) {
    if (p.vcheck) decode_block<kD, true, true>(g, h, p, s0, cs, r, Kn, Vn);
    else decode_block<kD, false, true>(g, h, p, s0, cs, r, Kn, Vn);
  } else {
    if (p.vcheck) decode_block<kD, true, false>(g, h, p, s0, 0, r, Kn, Vn);
    else decode_block<kD, false, false>(g, h, p, s0, 0, r, Kn, Vn);
  }
}

// Split `split` of `n_split` handles key blocks [b0, b1) of the window.  With
// one split the result is normalized and written as bf16; otherwise the
// unnormalized fp32 O^T, the reference max m (log2 units) and the sum l go to
// the workspace: O at part + ((split * n_q + n) * H + h) * D, (m, l) after all
// O values.
// Two waves per SIMD (registers capped at 256 per lane): one wave's softmax
// and decode overlap the other's MFMAs.
template <int kD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void kv_attention_kernel(KvGeom g, int64_t n_phys,
                                                           const int32_t* __restrict__ pages,
                                                           int n_pages, int last_tokens,
                                                           const uint16_t* __restrict__ q,
                                                           int64_t n_q, float scale_log2e,
                                                           uint32_t q_sign,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ part, int n_split) {
  // LDS (Shape<kD>::kLds bytes, dynamic): K^ rows, V^T rows
  constexpr int kKsRow = Shape<kD>::kKsRow;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  constexpr size_t kKsElems = Shape<kD>::kKsElems, kVtElems = Shape<kD>::kVtElems;
  uint16_t* Kb = smem;                                    // buffer i at Kb + i kKsElems
  uint16_t* Vb = Kb + 2 * kKsElems;                       // buffer i at Vb + i kVtElems
  const int H = g.n_heads, P = g.page_tokens;
  // Work order: the (head, split) pairs of query block 0, then of block 1, ...
  // so the last query block, the one that may be partial and then runs faster,
  // is dispatched last and fills the tail; the query blocks of one (head,
  // split), which read the same pages, are heads x splits workgroups apart,
  // on one XCD when that count is a multiple of 8.
  const int n_hs = (int)(gridDim.y * gridDim.z);
  const int wg = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
  const int qblk = wg / n_hs, hs = wg % n_hs;
  const int h = hs % (int)gridDim.y, split = hs / (int)gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5;
  const int64_t wave_q0 = (int64_t)qblk * kQB + wave * 32;   // the wave's first query
  const int64_t qrow = wave_q0 + (lane & 31);

  // The lane's query row in registers, as the B operand of S^T = K^ Q^T:
  // step s covers channels 16 s .. 16 s + 15, lane half `half` the 8 channels
  // 16 s + 8 half ..
  bf16x8 qr[kD / 16];
  {
    const uint16_t* qp = q + ((qrow < n_q ? qrow : n_q - 1) * H + h) * kD + 8 * half;
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) {
      u32x4 v = *(const u32x4*)(qp + 16 * s);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] ^= q_sign;           // -q when the scale is negative
      qr[s] = as_bf16x8(v);
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

  // Pipeline: on entry to iteration b, buffer b & 1 holds decoded block b and
  // the raw inputs of block b + 1 (with their K means) are in flight (rn).
  // Iteration b multiplies block b and, between its S^T MFMAs and its softmax,
  // decodes block b + 1 and then reuses rn to fetch block b + 2; one barrier
  // ends it, and nothing before that barrier waits for the fetch.
  if (b0 < b1) {
    PageInfo pc;
    pc = page_info(g, n_phys, pages, b0 / bpp, n_pages, last_tokens, pc, false);
    BlockRaw<Shape<kD>::kKPT> rn;
    fetch_block<kD>(g, pc, h, (b0 % bpp) * kKB, rn);
    decode_any<kD>(g, h, pc, (b0 % bpp) * kKB, rn, Kb + (b0 & 1) * kKsElems,
                   Vb + (b0 & 1) * kVtElems);
    PageInfo pn = pc;
    if (b0 + 1 < b1) {
      if ((b0 + 1) % bpp == 0)
        pn = page_info(g, n_phys, pages, (b0 + 1) / bpp, n_pages, last_tokens, pc, true);
      fetch_block<kD>(g, pn, h, ((b0 + 1) % bpp) * kKB, rn);
    }
    __syncthreads();

    for (int b = b0; b < b1; ++b) {
      const int cur = b & 1, nxt = cur ^ 1;
      const int s0 = (b % bpp) * kKB;
      const bool has1 = b + 1 < b1, has2 = b + 2 < b1;
      PageInfo pn2 = pn;
      if (has2 && (b + 2) % bpp == 0)
        pn2 = page_info(g, n_phys, pages, (b + 2) / bpp, n_pages, last_tokens, pn, true);
      const auto decode_next = [&]() {
        if (has1) {
          decode_any<kD>(g, h, pn, ((b + 1) % bpp) * kKB, rn, Kb + nxt * kKsElems,
                         Vb + nxt * kVtElems);
          if (has2) fetch_block<kD>(g, pn2, h, ((b + 2) % bpp) * kKB, rn);
        }
      };
      // a block with a key, for a wave with a query (both uniform per wave: the
      // waves past the last query only help decode)
      if (pc.valid > s0 && wave_q0 < n_q)
        attend_block<kD>(Kb + cur * kKsElems, Vb + cur * kVtElems, qr, lane, s0, pc.valid,
                         scale_log2e, m, l, o, decode_next);
      else
        decode_next();
      __syncthreads();
      pc = pn;
      pn = pn2;
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
// channels per lane.  Up to kChunk splits are read in one round of loads (m, l
// and O together); more splits take a first pass for M and then kChunk at a
// time with all their loads in flight.  The sums run over s in increasing
// order either way.
template <int kD>
__global__ __launch_bounds__(256) void kv_attention_combine(const float* __restrict__ part,
                                                            int n_split, int64_t rows,
                                                            uint16_t* __restrict__ out) {
  constexpr int kCpl = kD / 64;                             // channels per lane: 1 or 2
  constexpr int kChunk = 8;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* ml = part + (int64_t)n_split * rows * kD;
  float M = -__builtin_inff();
  if (n_split <= kChunk) {
    f32x2 v[kChunk];
    float ov[kChunk][kCpl];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      v[i] = f32x2{-__builtin_inff(), 0.0f};
      if (i < n_split) {
        v[i] = *(const f32x2*)(ml + ((int64_t)i * rows + row) * 2);
        const float* os = part + ((int64_t)i * rows + row) * kD + kCpl * lane;
#pragma unroll
        for (int c = 0; c < kCpl; ++c) ov[i][c] = os[c];
      }
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) M = fmaxf(M, v[i][0]);
    float L = 0.0f, a[kCpl] = {};
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        if (i < n_split) {
          const float w = __builtin_amdgcn_exp2f(v[i][0] - M);   // 0 for an empty split (m = -inf)
          L += v[i][1] * w;
#pragma unroll
          for (int c = 0; c < kCpl; ++c) a[c] += ov[i][c] * w;
        }
      }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (kCpl == 2)
      *(uint32_t*)(out + row * kD + 2 * lane) = pack_bf16x2(a[0] * inv, a[kCpl - 1] * inv);
    else
      out[row * kD + lane] = (uint16_t)f32_to_bf16_bits(a[0] * inv);
    return;
  }
  for (int s0 = 0; s0 < n_split; s0 += kChunk) {
    float mv[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      mv[i] = s0 + i < n_split ? ml[((int64_t)(s0 + i) * rows + row) * 2] : -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kChunk; ++i) M = fmaxf(M, mv[i]);
  }
  float L = 0.0f, a[kCpl] = {};
  if (M != -__builtin_inff()) {
    for (int s0 = 0; s0 < n_split; s0 += kChunk) {
      f32x2 v[kChunk];
      float ov[kChunk][kCpl];
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        const int64_t s = s0 + i;
        if (s < n_split) {
          v[i] = *(const f32x2*)(ml + (s * rows + row) * 2);
          const float* os = part + (s * rows + row) * kD + kCpl * lane;
#pragma unroll
          for (int c = 0; c < kCpl; ++c) ov[i][c] = os[c];
        }
      }
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        if (s0 + i < n_split) {
          const float w = __builtin_amdgcn_exp2f(v[i][0] - M);   // 0 for an empty split (m = -inf)
          L += v[i][1] * w;
#pragma unroll
          for (int c = 0; c < kCpl; ++c) a[c] += ov[i][c] * w;
        }
      }
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
