// Sparse paged decode attention: split-K flash-decode over a page list, then
// an LSE merge of the splits.
//
// [Locks] §2 "Decode-time attention": o = sum_t alpha_t v_t with
// alpha = softmax(scale * q . k_t), here over the tokens of the selected pages
// only (the most recent page contributes its filled slots); App. E, Stage B.
// All G query heads of a KV head read each K/V page once.
//
// Split kernel: one wave per (sequence, KV head, split); a split is a run of
// consecutive entries of the page list.  Lane (sg = lane / 8, e = lane % 8)
// owns dims 16e..16e+15 of tokens sg, sg+8, ..., so K and V are read with
// coalesced 16-byte loads (eight tokens x 256 bytes per instruction).  q . k is
// summed over the 8 lanes of a token group with DPP; every lane then runs its
// own online softmax over its tokens (running max m, sum l, output o), and
// the 8 token groups are combined at the end of the split.
// Merge kernel: per (sequence, query head), o = sum_s e^{m_s - M} o_s /
// sum_s e^{m_s - M} l_s and lse = M + log sum_s e^{m_s - M} l_s.

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

template <typename T, int G>
__global__ __launch_bounds__(kWave) void attn_split_kernel(AttnArgs a) {
  constexpr int B = 64;
  constexpr int D = kHeadDim;
  constexpr int TG = 8;               // token groups per wave
  constexpr int TPG = B / TG;         // tokens per group per page
  const int lane = threadIdx.x;
  const int sg = lane >> 3;
  const int e = lane & 7;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;

  const int len = a.seq_lens[seq];
  int n_mr = len > 0 ? (len - 1) / B : -1;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  int n_list;
  const int32_t* list = nullptr;
  if (len <= 0) {
    n_list = 0;
  } else if (a.sel_pages) {
    list = a.sel_pages + ((size_t)seq * a.hkv + kvh) * a.k;
    n_list = min(a.sel_count[(size_t)seq * a.hkv + kvh], a.k);
  } else {
    n_list = n_mr + 1;
  }
  const int i0 = split * a.pages_per_split;
  const int i1 = min(i0 + a.pages_per_split, n_list);

  // query slices (dims 16e..16e+15) of the group's G heads
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

  for (int i = i0; i < i1; ++i) {
    const int pg = list ? list[i] : i;
    if (pg < 0 || pg > n_mr) continue;
    const int phys = bt[pg];
    if (phys < 0 || phys >= a.num_phys) continue;
    const int n_tok = (pg == n_mr) ? len - n_mr * B : B;
    const size_t base = (((size_t)phys * a.hkv + kvh) * B) * D + e * 16;
    const T* Kp = reinterpret_cast<const T*>(a.k_pool) + base;
    const T* Vp = reinterpret_cast<const T*>(a.v_pool) + base;

    KV16<T> kr[TPG];
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
      const int t = sg + TG * u;
      if (t < n_tok) kr[u].load(Kp + (size_t)t * D); else kr[u].zero();
    }
    float z[TPG][G];
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc;
        if constexpr (sizeof(T) == 2) {
          acc = qb[g].dot(kr[u].a, kr[u].b);
        } else {
          float kx[16];
          kr[u].to_f32(kx);
          acc = 0.f;
#pragma unroll
          for (int x = 0; x < 16; ++x) acc = fmaf(qf[g][x], kx[x], acc);
        }
        z[u][g] = acc;
      }
    }
#pragma unroll
    for (int u = 0; u < TPG; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float full = group_sum<8>(z[u][g]);
        z[u][g] = (sg + TG * u < n_tok) ? full * zscale : -INFINITY;
      }

    KV16<T> vr[TPG];
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
      const int t = sg + TG * u;
      if (t < n_tok) vr[u].load(Vp + (size_t)t * D); else vr[u].zero();
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float pm = -INFINITY;
#pragma unroll
      for (int u = 0; u < TPG; ++u) pm = fmaxf(pm, z[u][g]);
      const float m_new = fmaxf(m[g], pm);
      if (m_new == -INFINITY) continue;  // no token of this lane yet
      const float corr = fast_exp2(m[g] - m_new);
      m[g] = m_new;
      l[g] *= corr;
#pragma unroll
      for (int x = 0; x < 16; ++x) o[g][x] *= corr;
#pragma unroll
      for (int u = 0; u < TPG; ++u) {
        const float p = fast_exp2(z[u][g] - m_new);
        l[g] += p;
        float vx[16];
        vr[u].to_f32(vx);
#pragma unroll
        for (int x = 0; x < 16; ++x) o[g][x] = fmaf(p, vx[x], o[g][x]);
      }
    }
  }

  // combine the 8 token groups (lanes e, e+8, ..., e+56)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = fmaxf(m[g], dpp<kDppRor8>(m[g]));
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = (M == -INFINITY) ? 0.f : fast_exp2(m[g] - M);
    float lg = l[g] * f;
    lg += dpp<kDppRor8>(lg);
    lg += __shfl_xor(lg, 16);
    lg += __shfl_xor(lg, 32);
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      float v = o[g][x] * f;
      v += dpp<kDppRor8>(v);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      o[g][x] = v;
    }
    m[g] = M;
    l[g] = lg;
  }
  const size_t pidx = ((size_t)seq * a.hkv + kvh) * a.n_splits + split;
  if (sg == 0) {
    float* po = a.part_o + pidx * G * D + e * 16;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float4* dst = reinterpret_cast<float4*>(po + (size_t)g * D);
#pragma unroll
      for (int x = 0; x < 4; ++x) dst[x] = make_float4(o[g][4 * x], o[g][4 * x + 1], o[g][4 * x + 2], o[g][4 * x + 3]);
    }
    if (e == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        a.part_ml[(pidx * G + g) * 2 + 0] = m[g];
        a.part_ml[(pidx * G + g) * 2 + 1] = l[g];
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kWave) void attn_merge_kernel(AttnArgs a, int group) {
  constexpr int D = kHeadDim;
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int kvh = h / group;
  const int g = h % group;
  const int lane = threadIdx.x;
  const size_t pbase = ((size_t)seq * a.hkv + kvh) * a.n_splits;
  float M = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, a.part_ml[((pbase + s) * group + g) * 2]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.n_splits; ++s) {
      const float ms = a.part_ml[((pbase + s) * group + g) * 2];
      if (ms == -INFINITY) continue;
      const float w = fast_exp2(ms - M);
      L = fmaf(w, a.part_ml[((pbase + s) * group + g) * 2 + 1], L);
      const float2 ov = reinterpret_cast<const float2*>(a.part_o + ((pbase + s) * group + g) * D)[lane];
      o0 = fmaf(w, ov.x, o0);
      o1 = fmaf(w, ov.y, o1);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* out = reinterpret_cast<T*>(a.out) + ((size_t)seq * a.hq + h) * D + 2 * lane;
  Elem<T>::store(out, o0 * inv);
  Elem<T>::store(out + 1, o1 * inv);
  if (a.lse_out && lane == 0)
    a.lse_out[(size_t)seq * a.hq + h] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
}

template <typename T>
static hipError_t launch_attn_t(int group, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.n_splits, a.hkv, a.batch);
  switch (group) {
    case 1: hipLaunchKernelGGL((attn_split_kernel<T, 1>), grid, dim3(kWave), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_split_kernel<T, 2>), grid, dim3(kWave), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_split_kernel<T, 4>), grid, dim3(kWave), 0, s, a); break;
    case 8: hipLaunchKernelGGL((attn_split_kernel<T, 8>), grid, dim3(kWave), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(attn_merge_kernel<T>, dim3(a.hq, a.batch), dim3(kWave), 0, s, a, group);
  return hipGetLastError();
}

hipError_t launch_attn(DType dt, int group, const AttnArgs& a, hipStream_t s) {
  return dt == kBF16 ? launch_attn_t<bf16_t>(group, a, s) : launch_attn_t<float>(group, a, s);
}

}  // namespace lk
