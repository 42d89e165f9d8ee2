// Sparse paged decode attention: split-K flash-decode over a page list, then
// an LSE merge of the splits.
//
// [Locks] §2 "Decode-time attention": o = sum_t alpha_t v_t with
// alpha = softmax(scale * q . k_t), here over the tokens of the selected pages
// only (the most recent page contributes its filled slots); App. E, Stage B.
// All G query heads of a KV head read each K/V page once.
//
// Split kernel: a workgroup of 4 waves per (sequence, KV head, split); each
// wave takes a run of consecutive half pages of the page list (32 tokens each).  Lane
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

// Partials per workgroup combined through LDS: the 8 token groups of a wave
// are first paired (G <= 4) or grouped by four (G = 8) on the VALU.
template <int G> struct AttnCombine {
  static constexpr int kGroupsPerPartial = G <= 4 ? 2 : 4;
  static constexpr int kPartialsPerWave = 8 / kGroupsPerPartial;
  static constexpr int kPartials = kAttnWaves * kPartialsPerWave;
};

// One workgroup's split of the attention of (seq, kvh) over the page list
// `list` (logical pages; nullptr: every page of the sequence), `plist` their
// physical pages (nullptr: looked up) and `cnt_p` the list length; the lists
// may live in global memory or LDS.
template <typename T, int G>
__device__ __forceinline__ void attn_split_block(const AttnArgs& a, int split, int kvh, int seq, const int32_t* list,
                                                 const int32_t* plist, const int32_t* cnt_p) {
  constexpr int B = 64;
  constexpr int D = kHeadDim;
  constexpr int TG = 8;               // token groups per wave
  constexpr int HALF = B / 2;         // tokens per unit (half a page)
  constexpr int TPG = HALF / TG;      // tokens per group per unit
  constexpr int NP = AttnCombine<G>::kPartials;
  constexpr int PPW = AttnCombine<G>::kPartialsPerWave;
  constexpr int GPP = AttnCombine<G>::kGroupsPerPartial;
  __shared__ float4 s_o[NP][G][D / 4];
  __shared__ float s_l[NP][G];
  __shared__ float s_m[kAttnWaves][G];

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
  const int len = a.seq_lens[seq] + a.len_add;
  const int cnt = list ? *cnt_p : 0;

  const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)seq * a.hq + (size_t)kvh * G) * D + e * 16;
  QSliceBF16 qb[G];
  float qf[G][16];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int g = 0; g < G; ++g) qb[g].load(reinterpret_cast<const bf16_t*>(qp) + (size_t)g * D);
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) qf[g][i] = reinterpret_cast<const float*>(qp)[(size_t)g * D + i];
  }

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
  KV16<T> kr[TPG], vr[TPG];
  auto issue = [&](int ph, int unit) {
    const size_t base = (((size_t)ph * a.hkv + kvh) * B + (unit & 1) * HALF) * D + e * 16;
    const T* Kp = reinterpret_cast<const T*>(a.k_pool) + base;
    const T* Vp = reinterpret_cast<const T*>(a.v_pool) + base;
#pragma unroll
    for (int x = 0; x < TPG; ++x) {
      kr[x].load(Kp + (size_t)(sg + TG * x) * D);
      vr[x].load(Vp + (size_t)(sg + TG * x) * D);
    }
  };
  bool loaded = false;
  if (len > 0 && phys >= 0 && phys < a.num_phys) { issue(phys, u); loaded = true; }

  int n_mr = len > 0 ? (len - 1) / B : -1;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  const int n_list = len <= 0 ? 0 : (list ? min(cnt, a.k) : n_mr + 1);
  const int u1 = min(u0 + ups, 2 * n_list);

  for (; u < u1; ++u) {
    if (u != u0) {
      pg = list ? list[u >> 1] : (u >> 1);
      phys = plist ? plist[u >> 1] : ((pg >= 0 && pg < a.max_pages) ? bt[pg] : -1);
      loaded = phys >= 0 && phys < a.num_phys;
      if (loaded) issue(phys, u);
    }
    if (!loaded || pg < 0 || pg > n_mr) continue;
    const int t_base = (u & 1) * HALF;
    const int n_tok = ((pg == n_mr) ? len - n_mr * B : B) - t_base;  // tokens from t_base on
    if (n_tok <= 0) continue;
    if (n_tok < HALF) {  // the filled part of the most recent page only
#pragma unroll
      for (int x = 0; x < TPG; ++x)
        if (sg + TG * x >= n_tok) { kr[x].zero(); vr[x].zero(); }
    }

    float z[TPG][G];
#pragma unroll
    for (int x = 0; x < TPG; ++x) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc;
        if constexpr (sizeof(T) == 2) {
          acc = qb[g].dot(kr[x].a, kr[x].b);
        } else {
          float kx[16];
          kr[x].to_f32(kx);
          acc = 0.f;
#pragma unroll
          for (int y = 0; y < 16; ++y) acc = fmaf(qf[g][y], kx[y], acc);
        }
        z[x][g] = acc;
      }
    }
#pragma unroll
    for (int x = 0; x < TPG; ++x)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float full = group_sum<8>(z[x][g]);
        z[x][g] = (sg + TG * x < n_tok) ? full * zscale : -INFINITY;
      }
    // running max, rescale and probabilities per head (a head with no token
    // yet keeps m = -inf and gets p = 0), then P V one token at a time
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

  // Combine: rescale every lane to its wave's running max, add token groups
  // pairwise (G <= 4) or by four (G = 8) on the VALU, then the workgroup's
  // NP partials in LDS with the waves' weights e^{M_w - M}.
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = fmaxf(m[g], dpp<kDppRor8>(m[g]));
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
  const size_t pidx = ((size_t)seq * a.hkv + kvh) * a.n_splits + split;
  for (int x = threadIdx.x; x < G * (D / 4); x += kAttnWaves * kWave) {
    const int g = x / (D / 4), d4 = x % (D / 4);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float4 ov = make_float4(0.f, 0.f, 0.f, 0.f);
    float lv = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
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
}

template <typename T, int G>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_split_kernel(AttnArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const size_t pair = (size_t)seq * a.hkv + kvh;
  const int32_t* list = a.sel_pages ? a.sel_pages + pair * a.k : nullptr;
  const int32_t* plist = (list && a.sel_phys) ? a.sel_phys + pair * a.k : nullptr;
  attn_split_block<T, G>(a, split, kvh, seq, list, plist, list ? a.sel_count + pair : nullptr);
}

// Decode step: selection and attention in one launch.  Every workgroup of a
// (sequence, KV head) runs the (deterministic) selection of that pair itself
// into LDS, then attends its split of the selected pages; workgroup 0 also
// writes the selection out when asked.  This trades redundant selection work
// for one kernel boundary and one dependent global round trip.
template <typename T, int NPT, int G>
__global__ __launch_bounds__(kAttnWaves * kWave) void select_attn_kernel(SelectArgs se, AttnArgs a) {
  __shared__ int32_t s_sel[kMaxSelect], s_selp[kMaxSelect];
  __shared__ int32_t s_cnt;
  const int split = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  select_block<kAttnWaves * kWave, NPT, G>(se, seq, kvh, s_sel, &s_cnt, s_selp);
  __syncthreads();
  if (split == 0 && se.sel_pages) {
    const size_t pair = (size_t)seq * se.hkv + kvh;
    for (int i = threadIdx.x; i < se.k; i += kAttnWaves * kWave) se.sel_pages[pair * se.k + i] = s_sel[i];
    if (threadIdx.x == 0) se.sel_count[pair] = s_cnt;
  }
  attn_split_block<T, G>(a, split, kvh, seq, s_sel, s_selp, &s_cnt);
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
    M = fmaxf(M, ml[((pbase + s0) * G + g) * 2]);
  M = group_max<kWave>(M);
  if (lane == 0) s_m[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
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

template <typename T>
static hipError_t launch_attn_t(int group, const AttnArgs& a, bool merge, hipStream_t s) {
  dim3 grid(a.n_splits, a.hkv, a.batch);
  dim3 block(kAttnWaves * kWave);
  dim3 mgrid(a.hq, a.batch);
  switch (group) {
    case 1: hipLaunchKernelGGL((attn_split_kernel<T, 1>), grid, block, 0, s, a);
            if (merge) hipLaunchKernelGGL((attn_merge_kernel<T, 1>), mgrid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_split_kernel<T, 2>), grid, block, 0, s, a);
            if (merge) hipLaunchKernelGGL((attn_merge_kernel<T, 2>), mgrid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_split_kernel<T, 4>), grid, block, 0, s, a);
            if (merge) hipLaunchKernelGGL((attn_merge_kernel<T, 4>), mgrid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((attn_split_kernel<T, 8>), grid, block, 0, s, a);
            if (merge) hipLaunchKernelGGL((attn_merge_kernel<T, 8>), mgrid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn(DType dt, int group, const AttnArgs& a, bool merge, hipStream_t s) {
  return dt == kBF16 ? launch_attn_t<bf16_t>(group, a, merge, s) : launch_attn_t<float>(group, a, merge, s);
}

template <typename T, int NPT>
static hipError_t launch_select_attn_n(const SelectArgs& se, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.n_splits, a.hkv, a.batch);
  dim3 block(kAttnWaves * kWave);
  switch (se.group) {
    case 1: hipLaunchKernelGGL((select_attn_kernel<T, NPT, 1>), grid, block, 0, s, se, a); break;
    case 2: hipLaunchKernelGGL((select_attn_kernel<T, NPT, 2>), grid, block, 0, s, se, a); break;
    case 4: hipLaunchKernelGGL((select_attn_kernel<T, NPT, 4>), grid, block, 0, s, se, a); break;
    case 8: hipLaunchKernelGGL((select_attn_kernel<T, NPT, 8>), grid, block, 0, s, se, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_select_attn_t(const SelectArgs& se, const AttnArgs& a, hipStream_t s) {
  const int n = se.max_pages;
  if (n <= kAttnWaves * kWave * 4) return launch_select_attn_n<T, 4>(se, a, s);
  if (n <= kAttnWaves * kWave * 8) return launch_select_attn_n<T, 8>(se, a, s);
  if (n <= kAttnWaves * kWave * 12) return launch_select_attn_n<T, 12>(se, a, s);
  return hipErrorNotSupported;
}

bool select_attn_fusable(const SelectArgs& se) {
  return se.max_pages <= kAttnWaves * kWave * 12 && se.k <= kMaxSelect && se.group <= kMaxGroup;
}

hipError_t launch_select_attn(DType dt, const SelectArgs& se, const AttnArgs& a, hipStream_t s) {
  if (!select_attn_fusable(se)) return hipErrorNotSupported;
  return dt == kBF16 ? launch_select_attn_t<bf16_t>(se, a, s) : launch_select_attn_t<float>(se, a, s);
}

}  // namespace lk
