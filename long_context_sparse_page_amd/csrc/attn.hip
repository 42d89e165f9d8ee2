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
// per instruction), both issued before any arithmetic.  q . k is
// summed over the 8 lanes of a token group with DPP; every lane then runs its
// own online softmax over its tokens (running max m, sum l, output o), and
// the 8 token groups are combined at the end of the split.
// The 4 waves' results are combined in LDS into one partial per workgroup;
// the partials of a (sequence, KV head) are then combined for all G heads
// (by the merge kernel below, or in the decode step's build launch): o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s and
// lse = M + log sum_s e^{m_s - M} l_s.

#include "common.cuh"
#include "kernels.h"

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

template <typename T, int G>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_split_kernel(AttnArgs a) {
  constexpr int B = 64;
  constexpr int D = kHeadDim;
  constexpr int TG = 8;               // token groups per wave
  constexpr int HALF = B / 2;         // tokens per unit (half a page)
  constexpr int TPG = HALF / TG;      // tokens per group per unit
  __shared__ float s_m[kAttnWaves][G], s_l[kAttnWaves][G];
  __shared__ float s_o[kAttnWaves][G][D];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sg = lane >> 3;
  const int e = lane & 7;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;

  const int len = a.seq_lens[seq] + a.len_add;
  int n_mr = len > 0 ? (len - 1) / B : -1;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  int n_list;
  const int32_t* list = nullptr;
  const int32_t* plist = nullptr;  // physical pages of list (else looked up)
  if (len <= 0) {
    n_list = 0;
  } else if (a.sel_pages) {
    list = a.sel_pages + ((size_t)seq * a.hkv + kvh) * a.k;
    if (a.sel_phys) plist = a.sel_phys + ((size_t)seq * a.hkv + kvh) * a.k;
    n_list = min(a.sel_count[(size_t)seq * a.hkv + kvh], a.k);
  } else {
    n_list = n_mr + 1;
  }
  // units are half pages: unit u is half (u & 1) of list entry u >> 1; wave w
  // of split s takes units [(4 s + w) * ups, +ups)
  const int ups = a.pages_per_split;
  const int u0 = (split * kAttnWaves + wave) * ups;
  const int u1 = min(u0 + ups, 2 * n_list);

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
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;

  for (int u = u0; u < u1; ++u) {
    const int pg = list ? list[u >> 1] : (u >> 1);
    if (pg < 0 || pg > n_mr) continue;
    const int phys = plist ? plist[u >> 1] : bt[pg];
    if (phys < 0 || phys >= a.num_phys) continue;
    const int t_base = (u & 1) * HALF;
    const int n_tok = ((pg == n_mr) ? len - n_mr * B : B) - t_base;  // tokens from t_base on
    if (n_tok <= 0) continue;
    const size_t base = (((size_t)phys * a.hkv + kvh) * B + t_base) * D + e * 16;
    const T* Kp = reinterpret_cast<const T*>(a.k_pool) + base;
    const T* Vp = reinterpret_cast<const T*>(a.v_pool) + base;

    KV16<T> kr[TPG], vr[TPG];
#pragma unroll
    for (int x = 0; x < TPG; ++x) {
      const int t = sg + TG * x;
      if (t < n_tok) { kr[x].load(Kp + (size_t)t * D); vr[x].load(Vp + (size_t)t * D); }
      else { kr[x].zero(); vr[x].zero(); }
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
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float pm = -INFINITY;
#pragma unroll
      for (int x = 0; x < TPG; ++x) pm = fmaxf(pm, z[x][g]);
      const float m_new = fmaxf(m[g], pm);
      if (m_new == -INFINITY) continue;  // no token of this lane yet
      const float corr = fast_exp2(m[g] - m_new);
      m[g] = m_new;
      l[g] *= corr;
#pragma unroll
      for (int y = 0; y < 16; ++y) o[g][y] *= corr;
#pragma unroll
      for (int x = 0; x < TPG; ++x) {
        const float p = fast_exp2(z[x][g] - m_new);
        l[g] += p;
        float vx[16];
        vr[x].to_f32(vx);
#pragma unroll
        for (int y = 0; y < 16; ++y) o[g][y] = fmaf(p, vx[y], o[g][y]);
      }
    }
  }

  // combine the 8 token groups of this wave (lanes e, e+8, ..., e+56)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = fmaxf(m[g], dpp<kDppRor8>(m[g]));
    M = xor32_max(xor16_max(M));
    const float f = (M == -INFINITY) ? 0.f : fast_exp2(m[g] - M);
    float lg = l[g] * f;
    lg += dpp<kDppRor8>(lg);
    lg = xor32_sum(xor16_sum(lg));
#pragma unroll
    for (int y = 0; y < 16; ++y) {
      float v = o[g][y] * f;
      v += dpp<kDppRor8>(v);
      o[g][y] = xor32_sum(xor16_sum(v));
    }
    m[g] = M;
    l[g] = lg;
  }
  // combine the workgroup's waves through LDS into one partial per workgroup
  if (sg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int y = 0; y < 16; ++y) s_o[wave][g][e * 16 + y] = o[g][y];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) { s_m[wave][g] = m[g]; s_l[wave][g] = l[g]; }
  }
  __syncthreads();
  const size_t pidx = ((size_t)seq * a.hkv + kvh) * a.n_splits + split;
  for (int x = threadIdx.x; x < G * D; x += kAttnWaves * kWave) {
    const int g = x / D, dim = x % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float ov = 0.f, lv = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float f = s_m[w][g] == -INFINITY ? 0.f : fast_exp2(s_m[w][g] - M);
        ov = fmaf(f, s_o[w][g][dim], ov);
        lv = fmaf(f, s_l[w][g], lv);
      }
    }
    a.part_o[(pidx * G + g) * D + dim] = ov;
    if (dim == 0) {
      a.part_ml[(pidx * G + g) * 2 + 0] = M;
      a.part_ml[(pidx * G + g) * 2 + 1] = lv;
    }
  }

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

}  // namespace lk
