// Sparse paged decode attention: split-K flash-decode over a page list, then
// an LSE merge of the splits.
//
// [Locks] §2 "Decode-time attention": o = sum_t alpha_t v_t with
// alpha = softmax(scale * q . k_t), here over the tokens of the selected pages
// only (the most recent page contributes its filled slots); App. E, Stage B.
// All G query heads of a KV head read each K/V page once.
//
// Split kernel: a workgroup of 4 waves per (sequence, KV head, split); each
// wave takes a run of consecutive units of the page list, 32 tokens each: half
// a page of 64 tokens, or two consecutive list entries of 16-token pages.  Lane
// (sg = lane / 8, e = lane % 8) owns dims 16e..16e+15 of tokens sg, sg+8, ...,
// so K and V are read with coalesced 16-byte loads (eight tokens x 256 bytes
// per instruction), all issued before any arithmetic; the first half page's
// loads go out together with the sequence length and the selection count.
// q . k is summed over the 8 lanes of a token group with DPP; every lane then
// runs its own online softmax over its tokens (running max m, sum l, output o).
// At the end every lane is rescaled to its wave's maximum, token groups are
// added in pairs (or fours) on the VALU, and the workgroup's partials are
// combined in LDS into one partial per workgroup; the partials of a
// (sequence, KV head) are then combined for all G heads (by the merge kernel
// below, or in the decode step's build launch):
// o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s and
// lse = M + log sum_s e^{m_s - M} l_s.

#include "common.cuh"
#include "kernels.h"
#include "select_impl.cuh"

namespace lk {

// q . k over 16 dims: bf16 uses the packed bf16 dot product (exact products,
// fp32 accumulate); fp32 uses FMAs.
struct QSliceBF16 {
  uint32_t w[8];
  __device__ __forceinline__ void load(const bf16_t* p) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0];
    const uint4 b = reinterpret_cast<const uint4*>(p)[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  __device__ __forceinline__ float dot(const uint4& a, const uint4& b) const {
    float acc = 0.f;
    const uint32_t k[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]),
                                            __builtin_bit_cast(bf16x2_t, k[i]), acc, false);
    return acc;
  }
};

template <typename T> struct KV16;  // 16 consecutive elements of one K or V row
template <> struct KV16<bf16_t> {
  uint4 a, b;
  __device__ __forceinline__ void load(const bf16_t* p) {
    a = reinterpret_cast<const uint4*>(p)[0];
    b = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ __forceinline__ void zero() { a = make_uint4(0, 0, 0, 0); b = a; }
  __device__ __forceinline__ void to_f32(float (&x)[16]) const {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
  }
};
template <> struct KV16<float> {
  float4 v[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const float4*>(p)[i];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __device__ __forceinline__ void to_f32(float (&x)[16]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[4 * i] = v[i].x; x[4 * i + 1] = v[i].y; x[4 * i + 2] = v[i].z; x[4 * i + 3] = v[i].w; }
  }
};

constexpr int kAttnWaves = 4;
constexpr int kAttnTG = 8;                     // token groups per wave
constexpr int kAttnHalf = 32;                  // tokens per unit (half a page)
constexpr int kAttnTPG = kAttnHalf / kAttnTG;  // tokens per group per unit

// Partials per workgroup combined through LDS: the 8 token groups of a wave
// are first paired (G <= 4) or grouped by four (G = 8) on the VALU.
template <int G, int NWV> struct AttnCombine {
  static constexpr int kGroupsPerPartial = G <= 4 ? 2 : 4;
  static constexpr int kPartialsPerWave = kAttnTG / kGroupsPerPartial;
  static constexpr int kPartials = NWV * kPartialsPerWave;
};

// The lane's query slices (dims 16e..16e+15) of the G heads of a KV head.
template <typename T, int G> struct QLane {
  QSliceBF16 qb[G];
  float qf[G][16];
  __device__ __forceinline__ void load(const AttnArgs& a, int seq, int kvh, int e) {
    constexpr int D = kHeadDim;
    const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)seq * a.hq + (size_t)kvh * G) * D + e * 16;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int g = 0; g < G; ++g) qb[g].load(reinterpret_cast<const bf16_t*>(qp) + (size_t)g * D);
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) qf[g][i] = reinterpret_cast<const float*>(qp)[(size_t)g * D + i];
    }
  }
};

// K and V loads of half `half` of physical page ph for this lane: tokens
// sg, sg + 8, ... of the half, dims 16e..16e+15 (coalesced 16-byte loads).
template <typename T>
__device__ __forceinline__ void issue_unit(const AttnArgs& a, int kvh, int ph, int half, int sg, int e,
                                           KV16<T> (&kr)[kAttnTPG], KV16<T> (&vr)[kAttnTPG]) {
  constexpr int B = 64;
  constexpr int D = kHeadDim;
  const size_t base = (((size_t)ph * a.hkv + kvh) * B + half * kAttnHalf) * D + e * 16;
  const T* Kp = reinterpret_cast<const T*>(a.k_pool) + base;
  const T* Vp = reinterpret_cast<const T*>(a.v_pool) + base;
#pragma unroll
  for (int x = 0; x < kAttnTPG; ++x) {
    kr[x].load(Kp + (size_t)(sg + kAttnTG * x) * D);
    vr[x].load(Vp + (size_t)(sg + kAttnTG * x) * D);
  }
}

// The same for a unit of two 16-token pages ph0, ph1 (list entries 2u, 2u + 1):
// unit token 8 x + sg is token sg + 8 (x & 1) of page x >> 1, so the unit's 32
// tokens are page ph0's 16 then page ph1's 16, in the order attend_unit masks.
template <typename T>
__device__ __forceinline__ void issue_unit16(const AttnArgs& a, int kvh, int ph0, int ph1, int sg, int e,
                                             KV16<T> (&kr)[kAttnTPG], KV16<T> (&vr)[kAttnTPG]) {
  constexpr int B = 16;
  constexpr int D = kHeadDim;
  const T* Kp = reinterpret_cast<const T*>(a.k_pool);
  const T* Vp = reinterpret_cast<const T*>(a.v_pool);
#pragma unroll
  for (int x = 0; x < kAttnTPG; ++x) {
    const int ph = x < 2 ? ph0 : ph1;
    const size_t off = (((size_t)ph * a.hkv + kvh) * B + sg + kAttnTG * (x & 1)) * D + e * 16;
    kr[x].load(Kp + off);
    vr[x].load(Vp + off);
  }
}

// Online-softmax update of the lane's (m, l, o) with the first n_tok tokens
// (0 < n_tok) of a loaded unit: q . k summed over the 8 lanes of a token
// group with DPP, then running max, rescale and probabilities per head (a
// head with no token yet keeps m = -inf and gets p = 0), then P V one token
// at a time.
template <typename T, int G>
__device__ __forceinline__ void attend_unit(const QLane<T, G>& q, KV16<T> (&kr)[kAttnTPG], KV16<T> (&vr)[kAttnTPG],
                                            int n_tok, int sg, float zscale, float (&m)[G], float (&l)[G],
                                            float (&o)[G][16]) {
  constexpr int TPG = kAttnTPG;
  if (n_tok < kAttnHalf) {  // the filled part of the most recent page only
#pragma unroll
    for (int x = 0; x < TPG; ++x)
      if (sg + kAttnTG * x >= n_tok) { kr[x].zero(); vr[x].zero(); }
  }
  float z[TPG][G];
#pragma unroll
  for (int x = 0; x < TPG; ++x) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc;
      if constexpr (sizeof(T) == 2) {
        acc = q.qb[g].dot(kr[x].a, kr[x].b);
      } else {
        float kx[16];
        kr[x].to_f32(kx);
        acc = 0.f;
#pragma unroll
        for (int y = 0; y < 16; ++y) acc = fmaf(q.qf[g][y], kx[y], acc);
      }
      z[x][g] = acc;
    }
  }
#pragma unroll
  for (int x = 0; x < TPG; ++x)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float full = group_sum<8>(z[x][g]);
      z[x][g] = (sg + kAttnTG * x < n_tok) ? full * zscale : -INFINITY;
    }
  float p[TPG][G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float pm = -INFINITY;
#pragma unroll
    for (int x = 0; x < TPG; ++x) pm = fmaxf(pm, z[x][g]);
    const float m_new = fmaxf(m[g], pm);
    const float mref = (m_new == -INFINITY) ? 0.f : m_new;
    const float corr = fast_exp2(m[g] - mref);
    m[g] = m_new;
    l[g] *= corr;
#pragma unroll
    for (int y = 0; y < 16; ++y) o[g][y] *= corr;
#pragma unroll
    for (int x = 0; x < TPG; ++x) {
      p[x][g] = fast_exp2(z[x][g] - mref);
      l[g] += p[x][g];
    }
  }
#pragma unroll
  for (int x = 0; x < TPG; ++x) {
    float vx[16];
    vr[x].to_f32(vx);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int y = 0; y < 16; ++y) o[g][y] = fmaf(p[x][g], vx[y], o[g][y]);
  }
}

// Combine the (m, l, o) of every lane of NWV waves into the workgroup's
// partial, written at index pidx of part_o / part_ml: every lane is rescaled
// to its wave's running max, token groups are added in pairs (or fours) on
// the VALU, and the workgroup's partials are combined in LDS with the waves'
// weights e^{M_w - M}.  Every thread of the workgroup must call it.
template <int G, int NWV>
__device__ __forceinline__ void combine_write(const AttnArgs& a, size_t pidx, int wave, int lane, float (&m)[G],
                                              float (&l)[G], float (&o)[G][16]) {
  constexpr int D = kHeadDim;
  constexpr int NT = NWV * kWave;
  constexpr int NP = AttnCombine<G, NWV>::kPartials;
  constexpr int PPW = AttnCombine<G, NWV>::kPartialsPerWave;
  constexpr int GPP = AttnCombine<G, NWV>::kGroupsPerPartial;
  __shared__ float4 s_o[NP][G][D / 4];
  __shared__ float s_l[NP][G];
  __shared__ float s_m[NWV][G];
  const int sg = lane >> 3;
  const int e = lane & 7;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = vmax(m[g], dpp<kDppRor8>(m[g]));
    M = xor32_max(xor16_max(M));
    const float f = (M == -INFINITY) ? 0.f : fast_exp2(m[g] - M);
    float lg = l[g] * f;
    lg += dpp<kDppRor8>(lg);
    if constexpr (GPP == 4) lg = xor16_sum(lg);
    l[g] = lg;
#pragma unroll
    for (int y = 0; y < 16; ++y) {
      float v = o[g][y] * f;
      v += dpp<kDppRor8>(v);
      if constexpr (GPP == 4) v = xor16_sum(v);
      o[g][y] = v;
    }
    m[g] = M;
  }
  if (sg % GPP == 0) {
    const int p = wave * PPW + sg / GPP;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int y = 0; y < 4; ++y)
        s_o[p][g][e * 4 + y] = make_float4(o[g][4 * y], o[g][4 * y + 1], o[g][4 * y + 2], o[g][4 * y + 3]);
      if (e == 0) s_l[p][g] = l[g];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) s_m[wave][g] = m[g];
  }
  __syncthreads();
  if constexpr (NWV == kAttnWaves) {  // one float4 of the output per thread
    for (int x = threadIdx.x; x < G * (D / 4); x += NT) {
      const int g = x / (D / 4), d4 = x % (D / 4);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWV; ++w) M = vmax(M, s_m[w][g]);
      float4 ov = make_float4(0.f, 0.f, 0.f, 0.f);
      float lv = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
          const float f = s_m[w][g] == -INFINITY ? 0.f : fast_exp2(s_m[w][g] - M);
#pragma unroll
          for (int q = 0; q < PPW; ++q) {
            const float4 v = s_o[w * PPW + q][g][d4];
            ov.x = fmaf(f, v.x, ov.x); ov.y = fmaf(f, v.y, ov.y);
            ov.z = fmaf(f, v.z, ov.z); ov.w = fmaf(f, v.w, ov.w);
            lv = fmaf(f, s_l[w * PPW + q][g], lv);
          }
        }
      }
      reinterpret_cast<float4*>(a.part_o + (pidx * G + g) * D)[d4] = ov;
      if (d4 == 0) {
        a.part_ml[(pidx * G + g) * 2 + 0] = M;
        a.part_ml[(pidx * G + g) * 2 + 1] = lv;
      }
    }
  } else {  // one output element per thread
    const float* so = reinterpret_cast<const float*>(&s_o[0][0][0]);
    for (int x = threadIdx.x; x < G * D; x += NT) {
      const int g = x / D, d = x % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWV; ++w) M = vmax(M, s_m[w][g]);
      float ov = 0.f, lv = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
          const float f = s_m[w][g] == -INFINITY ? 0.f : fast_exp2(s_m[w][g] - M);
#pragma unroll
          for (int q = 0; q < PPW; ++q) {
            ov = fmaf(f, so[((size_t)(w * PPW + q) * G + g) * D + d], ov);
            lv = fmaf(f, s_l[w * PPW + q][g], lv);
          }
        }
      }
      a.part_o[(pidx * G + g) * D + d] = ov;
      if (d == 0) {
        a.part_ml[(pidx * G + g) * 2 + 0] = M;
        a.part_ml[(pidx * G + g) * 2 + 1] = lv;
      }
    }
  }
}

// One workgroup's split of the attention of (seq, kvh) over the page list
// `list` (logical pages; nullptr: every page of the sequence), `plist` their
// physical pages (nullptr: looked up) and `cnt_p` the list length; the lists
// may live in global memory or LDS.  seq_len is a.seq_lens[seq], loaded by
// the caller.
// attn_split_block for pages of 16 tokens: unit u is list entries 2u and
// 2u + 1 (issue_unit16); the first unit's loads go out before the lengths are
// used, as at 64 tokens.
template <typename T, int G>
__device__ __forceinline__ void attn_split_block16(const AttnArgs& a, int split, int kvh, int seq, int seq_len,
                                                   const int32_t* list, const int32_t* plist, const int32_t* cnt_p) {
  constexpr int B = 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int sg = lane >> 3;
  const int e = lane & 7;
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;
  const int ups = a.pages_per_split;
  const int u0 = (split * kAttnWaves + wave) * ups;
  const int n_entries = list ? a.k : a.max_pages;  // list entries that exist in memory
  // logical and physical page of list entry x (-1 past the entries in memory)
  auto entry = [&](int x, int& pg, int& ph) {
    pg = -1;
    ph = -1;
    if (x >= n_entries) return;
    pg = list ? list[x] : x;
    ph = plist ? plist[x] : ((pg >= 0 && pg < a.max_pages) ? bt[pg] : -1);
  };
  auto valid_phys = [&](int ph) { return ph >= 0 && ph < a.num_phys; };
  int pg0, ph0, pg1, ph1;
  entry(2 * u0, pg0, ph0);
  entry(2 * u0 + 1, pg1, ph1);
  const int len = seq_len + a.len_add;
  const int cnt = list ? *cnt_p : 0;

  QLane<T, G> q;
  q.load(a, seq, kvh, e);
  float m[G], l[G], o[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[g][i] = 0.f;
  }
  const float zscale = a.scale * kLog2e;
  KV16<T> kr[kAttnTPG], vr[kAttnTPG];
  bool loaded = false;
  if (len > 0 && valid_phys(ph0)) {
    issue_unit16<T>(a, kvh, ph0, valid_phys(ph1) ? ph1 : ph0, sg, e, kr, vr);
    loaded = true;
  }
  int n_mr = len > 0 ? (len - 1) / B : -1;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  const int n_list = len <= 0 ? 0 : (list ? min(cnt, a.k) : n_mr + 1);
  const int u1 = min(u0 + ups, (n_list + 1) / 2);
  for (int u = u0; u < u1; ++u) {
    if (u != u0) {
      entry(2 * u, pg0, ph0);
      entry(2 * u + 1, pg1, ph1);
      loaded = valid_phys(ph0);
      if (loaded) issue_unit16<T>(a, kvh, ph0, valid_phys(ph1) ? ph1 : ph0, sg, e, kr, vr);
    }
    if (!loaded || pg0 < 0 || pg0 > n_mr) continue;
    // tokens from the unit's start on: page 0 whole (or its filled part when
    // it is the most recent page, the last entry), then page 1 when present
    int n_tok = pg0 == n_mr ? len - n_mr * B : B;
    if (pg0 != n_mr && 2 * u + 1 < n_list && pg1 >= 0 && pg1 <= n_mr && valid_phys(ph1))
      n_tok += pg1 == n_mr ? len - n_mr * B : B;
    attend_unit<T, G>(q, kr, vr, n_tok, sg, zscale, m, l, o);
  }
  combine_write<G, kAttnWaves>(a, ((size_t)seq * a.hkv + kvh) * a.n_splits + split, wave, lane, m, l, o);
}

template <typename T, int G, int B>
__device__ __forceinline__ void attn_split_block(const AttnArgs& a, int split, int kvh, int seq, int seq_len,
                                                 const int32_t* list, const int32_t* plist, const int32_t* cnt_p) {
  if constexpr (B == 16) {
    attn_split_block16<T, G>(a, split, kvh, seq, seq_len, list, plist, cnt_p);
    return;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar page-list loads
  const int sg = lane >> 3;
  const int e = lane & 7;
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;

  // units are half pages: unit u is half (u & 1) of list entry u >> 1; wave w
  // of split s takes units [(4 s + w) * ups, +ups)
  const int ups = a.pages_per_split;
  const int u0 = (split * kAttnWaves + wave) * ups;
  const int n_entries = list ? a.k : a.max_pages;  // list entries that exist in memory

  // The first unit's page and physical page are fetched together with the
  // lengths; its K/V loads are issued before the lengths are used (every
  // address is inside the physical page, tokens past the end are masked).
  int pg_first = -1, phys_first = -1;
  if (u0 < 2 * n_entries) {
    const int x = u0 >> 1;
    pg_first = list ? list[x] : x;
    phys_first = plist ? plist[x] : -2;  // -2: look up through the block table
  }
  const int len = seq_len + a.len_add;
  const int cnt = list ? *cnt_p : 0;

  QLane<T, G> q;
  q.load(a, seq, kvh, e);
  float m[G], l[G], o[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[g][i] = 0.f;
  }
  const float zscale = a.scale * kLog2e;

  int u = u0;
  int pg = pg_first, phys = phys_first;
  if (phys == -2) phys = (pg >= 0 && pg < a.max_pages) ? bt[pg] : -1;
  // Every load site below issues a whole unit (an invalid page reads page 0
  // and is not attended), so the unit's registers are always redefined there
  // and never held across a reload.
  KV16<T> kr[kAttnTPG], vr[kAttnTPG];
  bool loaded = phys >= 0 && phys < a.num_phys;
  if (u0 < 2 * n_entries) issue_unit<T>(a, kvh, loaded ? phys : 0, u & 1, sg, e, kr, vr);
  loaded = loaded && len > 0;

  int n_mr = len > 0 ? (len - 1) / B : -1;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  const int n_list = len <= 0 ? 0 : (list ? min(cnt, a.k) : n_mr + 1);
  const int u1 = min(u0 + ups, 2 * n_list);

  for (; u < u1; ++u) {
    if (u != u0) {
      pg = list ? list[u >> 1] : (u >> 1);
      phys = plist ? plist[u >> 1] : ((pg >= 0 && pg < a.max_pages) ? bt[pg] : -1);
      loaded = phys >= 0 && phys < a.num_phys;
      issue_unit<T>(a, kvh, loaded ? phys : 0, u & 1, sg, e, kr, vr);
    }
    if (!loaded || pg < 0 || pg > n_mr) continue;
    const int n_tok = ((pg == n_mr) ? len - n_mr * B : B) - (u & 1) * kAttnHalf;  // tokens from the unit's start on
    if (n_tok <= 0) continue;
    attend_unit<T, G>(q, kr, vr, n_tok, sg, zscale, m, l, o);
  }
  combine_write<G, kAttnWaves>(a, ((size_t)seq * a.hkv + kvh) * a.n_splits + split, wave, lane, m, l, o);
}

// attn_split_block when every wave attends exactly one unit (the sparse
// split count): straight-line code, the unit's K/V registers live only
// around the one attend, so a wave holds fewer registers than the looping
// form (which keeps the running (m, l, o) and the queries across reloads).
template <typename T, int G, int B>
__device__ __forceinline__ void attn_one_unit_block(const AttnArgs& a, int split, int kvh, int seq, int seq_len,
                                                    const int32_t* list, const int32_t* plist, const int32_t* cnt_p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int sg = lane >> 3;
  const int e = lane & 7;
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;
  const int u = split * kAttnWaves + wave;
  const int n_entries = list ? a.k : a.max_pages;  // list entries that exist in memory
  // list entry x -> logical page and physical page (-1 past the entries in memory)
  auto entry = [&](int x, int& pg, int& ph) {
    pg = -1;
    ph = -1;
    if (x >= n_entries) return;
    pg = list ? list[x] : x;
    ph = plist ? plist[x] : ((pg >= 0 && pg < a.max_pages) ? bt[pg] : -1);
  };
  auto valid_phys = [&](int ph) { return ph >= 0 && ph < a.num_phys; };
  // unit u: half (u & 1) of entry u >> 1 (64-token pages), entries 2u, 2u + 1 (16)
  int pg0, ph0, pg1 = -1, ph1 = -1;
  entry(B == 64 ? u >> 1 : 2 * u, pg0, ph0);
  if constexpr (B == 16) entry(2 * u + 1, pg1, ph1);
  const int len = seq_len + a.len_add;
  const int cnt = list ? *cnt_p : 0;

  QLane<T, G> q;
  q.load(a, seq, kvh, e);
  float m[G], l[G], o[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[g][i] = 0.f;
  }
  int n_mr = len > 0 ? (len - 1) / B : -1;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  const int n_list = len <= 0 ? 0 : (list ? min(cnt, a.k) : n_mr + 1);
  const int first = B == 64 ? u >> 1 : 2 * u;  // the unit's first list entry
  if (first < n_list && pg0 >= 0 && pg0 <= n_mr && valid_phys(ph0)) {
    KV16<T> kr[kAttnTPG], vr[kAttnTPG];
    int n_tok;
    if constexpr (B == 64) {
      issue_unit<T>(a, kvh, ph0, u & 1, sg, e, kr, vr);
      n_tok = ((pg0 == n_mr) ? len - n_mr * B : B) - (u & 1) * kAttnHalf;  // tokens from the unit's start on
    } else {
      const bool two = pg0 != n_mr && 2 * u + 1 < n_list && pg1 >= 0 && pg1 <= n_mr && valid_phys(ph1);
      issue_unit16<T>(a, kvh, ph0, two ? ph1 : ph0, sg, e, kr, vr);
      n_tok = pg0 == n_mr ? len - n_mr * B : B;
      if (two) n_tok += pg1 == n_mr ? len - n_mr * B : B;
    }
    if (n_tok > 0) attend_unit<T, G>(q, kr, vr, n_tok, sg, a.scale * kLog2e, m, l, o);
  }
  combine_write<G, kAttnWaves>(a, ((size_t)seq * a.hkv + kvh) * a.n_splits + split, wave, lane, m, l, o);
}

// ONE: every wave attends one unit (pages_per_split == 1).
template <typename T, int G, int B, bool ONE>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_split_kernel(AttnArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const size_t pair = (size_t)seq * a.hkv + kvh;
  const int32_t* list = a.sel_pages ? a.sel_pages + pair * a.k : nullptr;
  const int32_t* plist = (list && a.sel_phys) ? a.sel_phys + pair * a.k : nullptr;
  if constexpr (ONE)
    attn_one_unit_block<T, G, B>(a, split, kvh, seq, a.seq_lens[seq], list, plist,
                                 list ? a.sel_count + pair : nullptr);
  else
    attn_split_block<T, G, B>(a, split, kvh, seq, a.seq_lens[seq], list, plist, list ? a.sel_count + pair : nullptr);
}

// ---------------------------------------------------------------------------
// Decode step: selection and attention in one launch.
//
// Workgroup = 8 waves per (split, KV head, sequence); wave w of split s
// attends unit u = 8 s + w of the selection list: half u & 1 of list entry
// u >> 1 (64-token pages), or list entries 2u and 2u + 1 (16-token pages).
// Every workgroup of a (sequence, KV head) computes that pair's selection
// itself (the same selection as select_block: the sink, the most recent page
// and the top k - 2 candidates by m_bar, ties to the lower page index, in
// page order), with three barriers:
//  1. per-head normalizers (thread t holds pages (8 NPT (t / 64) + 64 i)
//     + t % 64, i < NPT: each wave owns a contiguous page range);
//  2. ranking keys; each thread's largest key goes to LDS;
//  3. every wave finds the same pivot (the (k-2)-th largest of the maxima of
//     groups of 8 threads when there are enough groups, else of the
//     threads' maxima, with the key bits below 16 left clear; at least k-2
//     keys reach it) and appends its keys >= pivot to its own LDS list, in
//     page order.
// Then every wave reads the concatenated lists (page order), finds the exact
// cut by bisection on ballot counts (CR keys per lane) and takes its unit's
// pages from the lanes that hold them: no further barrier before the K/V
// loads.  More than CR * 64 keys at the pivot (massive ties) fall back to
// select_block over LDS.
constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * kWave;

template <typename T, int NPT, int G, int B, int CR>
__global__ __launch_bounds__(kFusedThreads) void select_attn_kernel(SelectArgs se, AttnArgs a) {
  constexpr int BS = kFusedThreads;
  constexpr int NW = kFusedWaves;
  constexpr int TR = BS / kWave;  // threads per pivot group
  constexpr int CAP = CR * kWave;  // list entries the exact cut holds in registers
  static_assert(B == 64 || B == 16, "page size");
  __shared__ float s_pm[G][NW], s_ps[G][NW];
  __shared__ uint32_t s_tmax[BS];
  __shared__ uint32_t s_ck[NW][CAP];
  __shared__ int32_t s_cp[NW][CAP];
  __shared__ int32_t s_cph[NW][CAP];
  __shared__ int32_t s_wc[NW];
  __shared__ int32_t s_fix[2];
  __shared__ int32_t s_sel[kMaxSelect], s_selp[kMaxSelect];  // fallback selection
  __shared__ int32_t s_cnt;
  __shared__ uint32_t s_piv;

  // 1-D grid, XCD-aware: the splits of a (sequence, KV head), which all read
  // its page scores and block table, are logically adjacent and share an L2
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int split = lin % a.n_splits;
  const int kvh = (lin / a.n_splits) % se.hkv;
  const int seq = lin / (a.n_splits * se.hkv);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const size_t pair = (size_t)seq * se.hkv + kvh;
  const int k = se.k;
  const int32_t* bt = se.block_table + (size_t)seq * se.max_pages;
  const float* lse = se.page_lse + ((size_t)seq * se.hkv * G + (size_t)kvh * G) * se.max_pages;
  auto page = [&](int i) { return (wave * NPT + i) * kWave + lane; };
  auto valid_phys = [&](int ph) { return (ph >= 0 && ph < se.num_phys) ? ph : -1; };

  // Loads that need no length go out first: the scores and block-table
  // entries of this thread's pages (clamped in bounds, masked below) and the
  // lane's query slices.
  float v[G][NPT];
  int ph[NPT];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NPT; ++i) v[g][i] = lse[(size_t)g * se.max_pages + min(page(i), se.max_pages - 1)];
#pragma unroll
  for (int i = 0; i < NPT; ++i) ph[i] = bt[min(page(i), se.max_pages - 1)];
  const int sg = lane >> 3;
  const int e = lane & 7;
  QLane<T, G> q;
  q.load(a, seq, kvh, e);
  const int seq_len = se.seq_lens[seq];

  const int len = seq_len + se.len_add;
  int n_mr = len > 0 ? (len - 1) / B : -1;
  if (n_mr > se.max_pages - 1) n_mr = se.max_pages - 1;
  const int n_cand = n_mr > 0 ? n_mr - 1 : 0;
  const int n_top = min(k - 2, n_cand);
  const int unit = split * NW + wave;  // this wave's unit of the selection list
  // its list entries: x (and x1 at 16-token pages)
  const int x = B == 64 ? unit >> 1 : 2 * unit;
  const int x1 = 2 * unit + 1;
  int cnt = 0, pg = -1, phys = -1, pg1 = -1, phys1 = -1;
  int mode = 0;  // 0: no page or every page, 1: the selection in LDS (s_sel / s_selp), 2: k = 2

  if (len > 0 && n_top == n_cand) {  // every page 0 .. n_mr is selected
    cnt = n_mr + 1;
    if (x <= n_mr) { pg = x; phys = bt[x]; }
    if (B == 16 && x1 <= n_mr) { pg1 = x1; phys1 = bt[x1]; }
  } else if (len > 0) {
    // 1) per-head normalizers M_g, S_g (scores in log2 units); v then holds
    //    2^(s2 - m_g) (m_g: this thread's maximum of head g)
    float mg[G], sl[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mg[g] = -INFINITY;
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        v[g][i] = page(i) < n_mr ? v[g][i] * kLog2e : -INFINITY;
        mg[g] = vmax(mg[g], v[g][i]);
      }
      sl[g] = 0.f;
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        v[g][i] = mg[g] == -INFINITY ? 0.f : fast_exp2(v[g][i] - mg[g]);
        sl[g] += v[g][i];
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float wm = wave_max(mg[g]);
      const float ws = wave_sum(wm == -INFINITY || mg[g] == -INFINITY ? 0.f : sl[g] * fast_exp2(mg[g] - wm));
      if (lane == 0) { s_pm[g][wave] = wm; s_ps[g][wave] = ws; }
    }
    __syncthreads();
    // lane g * 8 + w combines wave w's partial of head g; groups of 8 lanes
    // reduce with DPP and every lane reads the G results
    float Mg[G], scale[G], log2S[G];
    {
      static_assert(G * NW <= kWave && NW == 8, "one lane per (head, wave)");
      const int gl = min(lane / NW, G - 1), wl = lane % NW;
      const float pm = s_pm[gl][wl], ps = s_ps[gl][wl];
      const float M = group_max<NW>(pm);
      const float S = group_sum<NW>(pm == -INFINITY ? 0.f : ps * fast_exp2(pm - M));
#pragma unroll
      for (int g = 0; g < G; ++g) {
        Mg[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M), g * NW));
        const float Sg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(S), g * NW));
        log2S[g] = fast_log2(Sg);
        scale[g] = (mg[g] == -INFINITY || !(Sg > 0.f)) ? 0.f : fast_exp2(mg[g] - Mg[g]) / Sg;
      }
    }
    // 2) ranking keys of the candidates 1 .. n_mr - 1; the fixed pages'
    //    physical pages for every wave
    const float invG = 1.f / (float)G;
    const float log2G = fast_log2((float)G);
    uint32_t key[NPT];
    uint32_t tmax = 0u;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int j = page(i);
      key[i] = 0u;
      if (j == 0) s_fix[0] = ph[i];
      if (j == n_mr) s_fix[1] = ph[i];
      if (j < 1 || j >= n_mr) continue;
      // m_bar_j; a share below 2^-120 is taken in the log domain from the
      // page's scores, read again (rare)
      float mb = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) mb = fmaf(v[g][i], scale[g], mb);
      mb *= invG;
      float lm;
      if (mb >= 0x1p-120f) {
        lm = fast_log2(mb);
      } else {
        float xg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) xg[g] = lse[(size_t)g * se.max_pages + j] * kLog2e;
        lm = share_log2_small<G>(xg, Mg, log2S, log2G, mb);
      }
      key[i] = order_key(lm);
      tmax = max(tmax, key[i]);
    }
    s_tmax[tid] = tmax;
    __syncthreads();
    cnt = n_top + 2;
    if (n_top > 0) {
      // 3) pivot, by wave 0 (the bisections below run on one wave: their
      //    ballot counts use the CU's one scalar unit)
      if (wave == 0) {
        uint32_t piv;
        uint32_t gm[1] = {0u};
#pragma unroll
        for (int r = 0; r < TR; ++r) gm[0] = max(gm[0], s_tmax[lane * TR + r]);
        if (__popcll(__ballot(gm[0] != 0u)) >= n_top) {
          piv = wave_nth_largest<1>(gm, n_top);
        } else {
          uint32_t tv[TR];
          int nz = 0;
#pragma unroll
          for (int r = 0; r < TR; ++r) {
            tv[r] = s_tmax[lane + kWave * r];
            nz += __popcll(__ballot(tv[r] != 0u));
          }
          piv = nz >= n_top ? wave_nth_largest<TR>(tv, n_top) : 1u;
        }
        if (lane == 0) s_piv = piv;
      }
      __syncthreads();
      const uint32_t piv = s_piv;
      //    every wave's keys >= pivot, in page order, to its own list
      int wc = 0;
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const bool c = key[i] >= piv && key[i] != 0u;
        const uint64_t bm = __ballot(c);
        const int pos = wc + lanes_below(bm);
        if (c && pos < CAP) {
          s_ck[wave][pos] = key[i];
          s_cp[wave][pos] = page(i);
          s_cph[wave][pos] = ph[i];
        }
        wc += __popcll(bm);
      }
      if (lane == 0) s_wc[wave] = wc;
      __syncthreads();
      int C = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) C += s_wc[w];
      mode = 1;
      if (C <= CAP) {
        // 4) exact cut over the concatenated lists (entry lane + 64 r) by
        //    wave 0, which writes the selection to LDS in page order
        if (wave == 0) {
          int off[NW + 1];
          off[0] = 0;
#pragma unroll
          for (int w = 0; w < NW; ++w) off[w + 1] = off[w] + s_wc[w];
          uint32_t ck[CR];
          int cpg[CR], cph[CR];
#pragma unroll
          for (int r = 0; r < CR; ++r) {
            const int en = lane + kWave * r;
            ck[r] = 0u;
            cpg[r] = -1;
            cph[r] = -1;
            if (en < C) {
              int w = 0, base = 0;
#pragma unroll
              for (int ww = 1; ww < NW; ++ww)
                if (en >= off[ww]) { w = ww; base = off[ww]; }
              ck[r] = s_ck[w][en - base];
              cpg[r] = s_cp[w][en - base];
              cph[r] = s_cph[w][en - base];
            }
          }
          wave_take_in_order<CR>(ck, n_top, [&](int sl, int r) {
            s_sel[1 + sl] = cpg[r];
            s_selp[1 + sl] = cph[r];
          });
          if (lane == 0) {
            s_sel[0] = 0;
            s_selp[0] = s_fix[0];
            s_sel[n_top + 1] = n_mr;
            s_selp[n_top + 1] = s_fix[1];
          }
        }
      } else {
        // massive ties at the pivot: the general selection over LDS
        select_block<BS, NPT, G>(se, seq, kvh, seq_len, s_sel, &s_cnt, s_selp);
        __syncthreads();
        cnt = s_cnt;
      }
      __syncthreads();
      if (x < cnt) { pg = s_sel[x]; phys = s_selp[x]; }
      if (B == 16 && x1 < cnt) { pg1 = s_sel[x1]; phys1 = s_selp[x1]; }
    } else {  // k = 2: the sink and the most recent page
      mode = 2;
      if (x == 0) { pg = 0; phys = s_fix[0]; }
      else if (x == 1) { pg = n_mr; phys = s_fix[1]; }
      if (B == 16 && x1 == 1) { pg1 = n_mr; phys1 = s_fix[1]; }
    }
  }

  // the selection, when asked for, from split 0
  if (split == 0 && se.sel_pages) {
    int32_t* so = se.sel_pages + pair * k;
    int32_t* sp = se.sel_phys ? se.sel_phys + pair * k : nullptr;
    for (int sl0 = tid; sl0 < k; sl0 += BS) {
      const bool in = sl0 < cnt;
      int pv = -1, fv = -1;
      if (in && mode == 0) { pv = sl0; fv = valid_phys(bt[sl0]); }
      if (in && mode == 1) { pv = s_sel[sl0]; fv = valid_phys(s_selp[sl0]); }
      if (in && mode == 2) { pv = sl0 == 0 ? 0 : n_mr; fv = valid_phys(s_fix[sl0 == 0 ? 0 : 1]); }
      so[sl0] = pv;
      if (sp) sp[sl0] = fv;
    }
    if (tid == 0) se.sel_count[pair] = cnt;
  }

  // attention over this wave's unit
  float m[G], l[G], o[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[g][i] = 0.f;
  }
  if (x < cnt && pg >= 0 && pg <= n_mr && phys >= 0 && phys < a.num_phys) {
    KV16<T> kr[kAttnTPG], vr[kAttnTPG];
    if constexpr (B == 64) {
      const int half = unit & 1;
      issue_unit<T>(a, kvh, phys, half, sg, e, kr, vr);
      const int n_tok = ((pg == n_mr) ? len - n_mr * B : B) - half * kAttnHalf;
      if (n_tok > 0) attend_unit<T, G>(q, kr, vr, n_tok, sg, a.scale * kLog2e, m, l, o);
    } else {
      // the unit's first page whole (or its filled part when it is the most
      // recent page, the last entry), then the second when present
      const bool has1 = pg != n_mr && x1 < cnt && pg1 >= 0 && pg1 <= n_mr && phys1 >= 0 && phys1 < a.num_phys;
      issue_unit16<T>(a, kvh, phys, has1 ? phys1 : phys, sg, e, kr, vr);
      int n_tok = pg == n_mr ? len - n_mr * B : B;
      if (has1) n_tok += pg1 == n_mr ? len - n_mr * B : B;
      attend_unit<T, G>(q, kr, vr, n_tok, sg, a.scale * kLog2e, m, l, o);
    }
  }
  combine_write<G, NW>(a, pair * a.n_splits + split, wave, lane, m, l, o);
}

// Merge: one workgroup per (sequence, KV head) combines the split partials of
// all G heads: o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s and
// lse = M + log sum_s e^{m_s - M} l_s.
// Merge for the standalone attention entry points: one workgroup of 4 waves
// per (sequence, query head); wave w takes splits w, w+4, ...; lane owns dims
// 2 lane, 2 lane + 1.  (The decode step merges inside its build launch.)
template <typename T, int G>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_merge_kernel(AttnArgs a) {
  constexpr int D = kHeadDim;
  __shared__ float s_m[kAttnWaves], s_o[kAttnWaves][D], s_l[kAttnWaves];
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int kvh = h / G;
  const int g = h % G;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const size_t pbase = ((size_t)seq * a.hkv + kvh) * a.n_splits;
  const float* ml = a.part_ml;
  float M = -INFINITY;
  for (int s0 = threadIdx.x; s0 < a.n_splits; s0 += kAttnWaves * kWave)
    M = vmax(M, ml[((pbase + s0) * G + g) * 2]);
  M = group_max<kWave>(M);
  if (lane == 0) s_m[wave] = M;
  __syncthreads();
  M = vmax(vmax(s_m[0], s_m[1]), vmax(s_m[2], s_m[3]));
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s0 = wave; s0 < a.n_splits; s0 += kAttnWaves) {
      const float ms = ml[((pbase + s0) * G + g) * 2];
      const float ls = ml[((pbase + s0) * G + g) * 2 + 1];
      const float2 ov = reinterpret_cast<const float2*>(a.part_o + ((pbase + s0) * G + g) * D)[lane];
      const float w = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
      L = fmaf(w, ls, L);
      o0 = fmaf(w, ov.x, o0);
      o1 = fmaf(w, ov.y, o1);
    }
  }
  s_o[wave][2 * lane] = o0;
  s_o[wave][2 * lane + 1] = o1;
  if (lane == 0) s_l[wave] = L;
  __syncthreads();
  if (wave == 0) {
    float Lt = 0.f, x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      Lt += s_l[w];
      x0 += s_o[w][2 * lane];
      x1 += s_o[w][2 * lane + 1];
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    T* out = reinterpret_cast<T*>(a.out) + ((size_t)seq * a.hq + h) * D + 2 * lane;
    Elem<T>::store(out, x0 * inv);
    Elem<T>::store(out + 1, x1 * inv);
    if (a.lse_out && lane == 0)
      a.lse_out[(size_t)seq * a.hq + h] = Lt > 0.f ? (M + fast_log2(Lt)) * kLn2 : -INFINITY;
  }
}

template <typename T, int B>
static hipError_t launch_attn_tb(int group, const AttnArgs& a, bool merge, hipStream_t s) {
  dim3 grid(a.n_splits, a.hkv, a.batch);
  dim3 block(kAttnWaves * kWave);
  dim3 mgrid(a.hq, a.batch);
  const bool one = a.pages_per_split == 1;
#define LK_SPLIT(GG)                                                                                  \
  if (one) hipLaunchKernelGGL((attn_split_kernel<T, GG, B, true>), grid, block, 0, s, a);             \
  else hipLaunchKernelGGL((attn_split_kernel<T, GG, B, false>), grid, block, 0, s, a);                \
  if (merge) hipLaunchKernelGGL((attn_merge_kernel<T, GG>), mgrid, block, 0, s, a);
  switch (group) {
    case 1: LK_SPLIT(1) break;
    case 2: LK_SPLIT(2) break;
    case 4: LK_SPLIT(4) break;
    case 8: LK_SPLIT(8) break;
    default: return hipErrorInvalidValue;
  }
#undef LK_SPLIT
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_attn_t(int group, const AttnArgs& a, bool merge, hipStream_t s) {
  if (a.page_size == 64) return launch_attn_tb<T, 64>(group, a, merge, s);
  if (a.page_size == 16) return launch_attn_tb<T, 16>(group, a, merge, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn(DType dt, int group, const AttnArgs& a, bool merge, hipStream_t s) {
  return dt == kBF16 ? launch_attn_t<bf16_t>(group, a, merge, s) : launch_attn_t<float>(group, a, merge, s);
}

template <typename T, int NPT, int B, int CR>
static hipError_t launch_select_attn_n(const SelectArgs& se, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.n_splits * a.hkv * a.batch);
  dim3 block(kFusedThreads);
  switch (se.group) {
    case 1: hipLaunchKernelGGL((select_attn_kernel<T, NPT, 1, B, CR>), grid, block, 0, s, se, a); break;
    case 2: hipLaunchKernelGGL((select_attn_kernel<T, NPT, 2, B, CR>), grid, block, 0, s, se, a); break;
    case 4: hipLaunchKernelGGL((select_attn_kernel<T, NPT, 4, B, CR>), grid, block, 0, s, se, a); break;
    default: return hipErrorInvalidValue;  // G = 8 keeps the two launches (registers)
  }
  return hipGetLastError();
}

// Tiers of pages per thread: 64-token pages up to 3,072 pages per sequence,
// 16-token pages up to 8,704.
constexpr int kFusedMaxPages64 = kFusedThreads * 6;
constexpr int kFusedMaxPages16 = kFusedThreads * 17;

template <typename T, int B, int CR>
static hipError_t launch_select_attn_b(const SelectArgs& se, const AttnArgs& a, hipStream_t s) {
  const int n = se.max_pages;
  if constexpr (B == 64) {
    if (n <= kFusedThreads * 2) return launch_select_attn_n<T, 2, B, CR>(se, a, s);
    if (n <= kFusedThreads * 4) return launch_select_attn_n<T, 4, B, CR>(se, a, s);
    if (n <= kFusedThreads * 5) return launch_select_attn_n<T, 5, B, CR>(se, a, s);
    if (n <= kFusedThreads * 6) return launch_select_attn_n<T, 6, B, CR>(se, a, s);
  } else {
    if (n <= kFusedThreads * 6) return launch_select_attn_n<T, 6, B, CR>(se, a, s);
    if (n <= kFusedThreads * 12) return launch_select_attn_n<T, 12, B, CR>(se, a, s);
    if (n <= kFusedThreads * 17) return launch_select_attn_n<T, 17, B, CR>(se, a, s);
  }
  return hipErrorNotSupported;
}

// List entries per lane of the exact cut: twice the candidates kept, rounded
// up to lanes (the keys at or above the pivot are typically a few more than
// k - 2); 64-token pages keep two (more keys at the pivot take the fallback).
static int fused_list_regs(const SelectArgs& se) {
  if (se.page_size == 64) return 2;
  return 2 * (se.k - 2) <= 2 * kWave ? 2 : (2 * (se.k - 2) <= 4 * kWave ? 4 : 0);
}

bool select_attn_fusable(const SelectArgs& se) {
  if (se.group > 4 || se.share_out != nullptr || se.k > kMaxSelect) return false;
  if (se.page_size == 64) return se.max_pages <= kFusedMaxPages64;
  return se.page_size == 16 && se.max_pages <= kFusedMaxPages16 && fused_list_regs(se) > 0;
}

int select_attn_splits(int k, int page_size) {
  const int units = page_size == 64 ? 2 * k : (k + 1) / 2;
  return (units + kFusedWaves - 1) / kFusedWaves;
}

hipError_t launch_select_attn(DType dt, const SelectArgs& se, const AttnArgs& a, hipStream_t s) {
  if (!select_attn_fusable(se)) return hipErrorNotSupported;
  if (se.seq_lens != a.seq_lens || a.page_size != se.page_size ||
      a.n_splits != select_attn_splits(se.k, se.page_size))
    return hipErrorInvalidValue;
  const bool bf = dt == kBF16;
  if (se.page_size == 64)
    return bf ? launch_select_attn_b<bf16_t, 64, 2>(se, a, s) : launch_select_attn_b<float, 64, 2>(se, a, s);
  if (fused_list_regs(se) == 2)
    return bf ? launch_select_attn_b<bf16_t, 16, 2>(se, a, s) : launch_select_attn_b<float, 16, 2>(se, a, s);
  return bf ? launch_select_attn_b<bf16_t, 16, 4>(se, a, s) : launch_select_attn_b<float, 16, 4>(se, a, s);
}


// ---------------------------------------------------------------------------
// Decode step, chunked selection (long tables, few (sequence, KV head) pairs):
// attention whose waves merge the pair's chunk lists themselves.  Workgroup =
// 4 waves per (split, KV head, sequence); wave w of split s attends unit
// 4 s + w (half (4 s + w) & 1 of selection entry (4 s + w) >> 1).  Every wave
// reads the list slots and counts of its pair (one round trip, with its
// queries), takes the top-(k-2) entries as the selection merge does (ties to
// the earlier entry = the lower page) and picks its own entry from the lane
// that holds it: no barrier before the K/V loads.  Wave 0 of split 0 writes
// the selection when it is asked for.
template <typename T, int G, int CR, int B>
__global__ __launch_bounds__(kAttnWaves * kWave) void list_attn_kernel(SelectArgs se, AttnArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const size_t pair = (size_t)seq * se.hkv + kvh;
  const int k = se.k, ktop = k - 2, C = se.n_chunks;
  const int32_t* bt = se.block_table + (size_t)seq * se.max_pages;
  uint32_t ck[CR];
  int cp[CR], cq[CR];
#pragma unroll
  for (int r = 0; r < CR; ++r) {
    const int x = lane + kWave * r;
    const int c = x / ktop, i = x - c * ktop;
    const bool in = c < C;
    const size_t at = pair * C * ktop + (in ? x : 0);
    const int n = se.cand_cnt[pair * C + (in ? c : 0)];
    const uint32_t kv = se.cand_key[at];
    ck[r] = (in && i < n) ? kv : 0u;
    cp[r] = se.cand_page[at];
    cq[r] = se.cand_phys[at];
  }
  const int sg = lane >> 3;
  const int e = lane & 7;
  QLane<T, G> q;
  q.load(a, seq, kvh, e);
  const int len = se.seq_lens[seq] + se.len_add;
  int n_mr = len > 0 ? (len - 1) / B : 0;
  if (n_mr > se.max_pages - 1) n_mr = se.max_pages - 1;
  const int ph0 = bt[0], phr = bt[n_mr];
  const int n_cand = n_mr > 0 ? n_mr - 1 : 0;
  const int u = split * kAttnWaves + wave;
  // this wave's selection entries: entry u >> 1 (half u & 1 of a 64-token
  // page), or entries 2u and 2u + 1 (16-token pages)
  const int x = B == 64 ? u >> 1 : 2 * u;
  const int x1 = 2 * u + 1;
  int32_t* so = (split == 0 && wave == 0 && se.sel_pages) ? se.sel_pages + pair * k : nullptr;
  int pg = -1, phys = -1, cnt = 0;
  int pg1 = -1, phys1 = -1;
  if (len <= 0) {
    if (so) {
      for (int s = lane; s < k; s += kWave) so[s] = -1;
      if (lane == 0) se.sel_count[pair] = 0;
    }
  } else if (min(ktop, n_cand) == n_cand) {  // every page 0 .. n_mr
    cnt = n_mr + 1;
    if (x <= n_mr) { pg = x; phys = bt[x]; }
    if (B == 16 && x1 <= n_mr) { pg1 = x1; phys1 = bt[x1]; }
    if (so) {
      for (int s = lane; s < k; s += kWave) so[s] = s <= n_mr ? s : -1;
      if (lane == 0) se.sel_count[pair] = cnt;
    }
  } else {
    int nz = 0;  // k - 2, fewer only if non-finite scores left keys at zero
#pragma unroll
    for (int r = 0; r < CR; ++r) nz += __popcll(__ballot(ck[r] != 0u));
    const int n_top = min(ktop, nz);
    cnt = n_top + 2;
    if (x == 0) { pg = 0; phys = ph0; }
    else if (x == n_top + 1) { pg = n_mr; phys = phr; }
    if (B == 16 && x1 == n_top + 1) { pg1 = n_mr; phys1 = phr; }
    if (n_top > 0) {
      int mp = -1, mq = -1, mp1 = -1, mq1 = -1;
      bool have = false, have1 = false;
      wave_take_in_order<CR>(ck, n_top, [&](int slot, int r) {
        if (slot == x - 1) { mp = cp[r]; mq = cq[r]; have = true; }
        if (B == 16 && slot == x1 - 1) { mp1 = cp[r]; mq1 = cq[r]; have1 = true; }
        if (so) so[1 + slot] = cp[r];
      });
      const uint64_t hb = __ballot(have);
      if (hb) {
        const int src = __ffsll((unsigned long long)hb) - 1;
        pg = __builtin_amdgcn_readlane(mp, src);
        phys = __builtin_amdgcn_readlane(mq, src);
      }
      if constexpr (B == 16) {
        const uint64_t hb1 = __ballot(have1);
        if (hb1) {
          const int src = __ffsll((unsigned long long)hb1) - 1;
          pg1 = __builtin_amdgcn_readlane(mp1, src);
          phys1 = __builtin_amdgcn_readlane(mq1, src);
        }
      }
    }
    if (so) {
      if (lane == 0) { so[0] = 0; so[n_top + 1] = n_mr; se.sel_count[pair] = cnt; }
      for (int s = n_top + 2 + lane; s < k; s += kWave) so[s] = -1;
    }
  }

  float m[G], l[G], o[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[g][i] = 0.f;
  }
  if (x < cnt && pg >= 0 && pg <= n_mr && phys >= 0 && phys < a.num_phys) {
    KV16<T> kr[kAttnTPG], vr[kAttnTPG];
    if constexpr (B == 64) {
      const int half = u & 1;
      issue_unit<T>(a, kvh, phys, half, sg, e, kr, vr);
      const int n_tok = ((pg == n_mr) ? len - n_mr * B : B) - half * kAttnHalf;
      if (n_tok > 0) attend_unit<T, G>(q, kr, vr, n_tok, sg, a.scale * kLog2e, m, l, o);
    } else {
      const bool has1 = pg != n_mr && x1 < cnt && pg1 >= 0 && pg1 <= n_mr && phys1 >= 0 && phys1 < a.num_phys;
      issue_unit16<T>(a, kvh, phys, has1 ? phys1 : phys, sg, e, kr, vr);
      int n_tok = pg == n_mr ? len - n_mr * B : B;
      if (has1) n_tok += pg1 == n_mr ? len - n_mr * B : B;
      attend_unit<T, G>(q, kr, vr, n_tok, sg, a.scale * kLog2e, m, l, o);
    }
  }
  combine_write<G, kAttnWaves>(a, pair * a.n_splits + split, wave, lane, m, l, o);
}

int list_attn_splits(int k, int page_size) {
  const int units = page_size == 64 ? 2 * k : (k + 1) / 2;
  return (units + kAttnWaves - 1) / kAttnWaves;
}

template <typename T, int G, int B>
static hipError_t launch_list_attn_gb(const SelectArgs& se, const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.n_splits, a.hkv, a.batch), block(kAttnWaves * kWave);
  const int entries = se.n_chunks * (se.k - 2);
  if (entries <= 4 * kWave) hipLaunchKernelGGL((list_attn_kernel<T, G, 4, B>), grid, block, 0, s, se, a);
  else if (entries <= 8 * kWave) hipLaunchKernelGGL((list_attn_kernel<T, G, 8, B>), grid, block, 0, s, se, a);
  else if (entries <= 12 * kWave) hipLaunchKernelGGL((list_attn_kernel<T, G, 12, B>), grid, block, 0, s, se, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, int G>
static hipError_t launch_list_attn_g(const SelectArgs& se, const AttnArgs& a, hipStream_t s) {
  return se.page_size == 64 ? launch_list_attn_gb<T, G, 64>(se, a, s) : launch_list_attn_gb<T, G, 16>(se, a, s);
}

template <typename T>
static hipError_t launch_list_attn_t(const SelectArgs& se, const AttnArgs& a, hipStream_t s) {
  switch (se.group) {
    case 1: return launch_list_attn_g<T, 1>(se, a, s);
    case 2: return launch_list_attn_g<T, 2>(se, a, s);
    case 4: return launch_list_attn_g<T, 4>(se, a, s);
    case 8: return launch_list_attn_g<T, 8>(se, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_list_attn(DType dt, const SelectArgs& se, const AttnArgs& a, hipStream_t s) {
  if (se.n_chunks <= 0 || !se.cand_key || !se.cand_page || !se.cand_phys || !se.cand_cnt || se.k < 3 ||
      (se.page_size != 64 && se.page_size != 16) || a.page_size != se.page_size || se.seq_lens != a.seq_lens ||
      a.n_splits != list_attn_splits(se.k, se.page_size) ||
      se.hkv != a.hkv || se.batch != a.batch)
    return hipErrorInvalidValue;
  return dt == kBF16 ? launch_list_attn_t<bf16_t>(se, a, s) : launch_list_attn_t<float>(se, a, s);
}

}  // namespace lk
