// Share-average and top-k page selection, one workgroup per (sequence, KV head).
//
// [Locks] §4 (after Eq. (1)) and Cor. 3: query head g's page-mass share is
//   m_hat_g(j) = exp(s_hat_j(q_g)) / sum_{j'} exp(s_hat_j'(q_g))
// over the scored pages j' < n_mr (sink included); the group average
//   m_bar_j = (1/G) sum_g m_hat_g(j)
// ranks the candidates 1 .. n_mr-1, and the selection is the sink page 0, the
// most recent page n_mr and the top-(k-2) candidates (ties to the lower page
// index), written in ascending page order.
//
// The ranking key is log m_bar_j (same order as m_bar_j, but never underflows),
// mapped to an order-preserving uint32 and kept in registers (NPT per thread).
// The (k-2)-th largest key is found by bisection on its bits, one block-wide
// count per bit (DPP row sums, lane reads and one barrier), then the selected
// indices are collected in LDS and ordered by rank counting.

#include "common.cuh"
#include "kernels.h"

namespace lk {

constexpr int kMaxGroup = 8;
constexpr int kMaxSelect = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide sum / max, returned uniform (DPP within rows, then the four row
// results are read from lanes 0, 16, 32, 48).
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
}
__device__ __forceinline__ float wave_max(float x) {
  x = group_max<16>(x);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ uint32_t dpp_u32(uint32_t x, int ctrl_id) {
  switch (ctrl_id) {
    case 0: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppXor1, 0xf, 0xf, false);
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppXor2, 0xf, 0xf, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppHalfMirror, 0xf, 0xf, false);
    default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppMirror, 0xf, 0xf, false);
  }
}
// Wave-wide max and min of uint32 values, returned uniform.
__device__ __forceinline__ void wave_minmax_u32(uint32_t& mx, uint32_t& mn) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    mx = max(mx, dpp_u32(mx, c));
    mn = min(mn, dpp_u32(mn, c));
  }
  uint32_t a0 = (uint32_t)__builtin_amdgcn_readlane((int)mx, 0), a1 = (uint32_t)__builtin_amdgcn_readlane((int)mx, 16);
  uint32_t a2 = (uint32_t)__builtin_amdgcn_readlane((int)mx, 32), a3 = (uint32_t)__builtin_amdgcn_readlane((int)mx, 48);
  mx = max(max(a0, a1), max(a2, a3));
  a0 = (uint32_t)__builtin_amdgcn_readlane((int)mn, 0); a1 = (uint32_t)__builtin_amdgcn_readlane((int)mn, 16);
  a2 = (uint32_t)__builtin_amdgcn_readlane((int)mn, 32); a3 = (uint32_t)__builtin_amdgcn_readlane((int)mn, 48);
  mn = min(min(a0, a1), min(a2, a3));
}

template <int BS>
struct BlockReduce {
  static constexpr int NW = BS / kWave;
  float* buf;      // [2][NW] in LDS
  int parity = 0;
  // Block-wide sum of one value per thread (one barrier; buffers alternate so
  // the next call does not overwrite values still being read).
  __device__ __forceinline__ float sum(float x) {
    x = wave_sum(x);
    if ((threadIdx.x & (kWave - 1)) == 0) buf[parity * NW + threadIdx.x / kWave] = x;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += buf[parity * NW + w];
    parity ^= 1;
    return t;
  }
  // Element-wise block max / sum of G (<= 8) values per thread, one barrier;
  // uses the [2][8][NW] buffer gbuf.
  float* gbuf;
  int gparity = 0;
  __device__ __forceinline__ void maxG(float (&x)[8], int G) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g < G) {
        const float w = wave_max(x[g]);
        if ((threadIdx.x & (kWave - 1)) == 0) gbuf[(gparity * 8 + g) * NW + threadIdx.x / kWave] = w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g < G) {
        float t = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) t = fmaxf(t, gbuf[(gparity * 8 + g) * NW + w]);
        x[g] = t;
      }
    }
    gparity ^= 1;
  }
  __device__ __forceinline__ void sumG(float (&x)[8], int G) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g < G) {
        const float w = wave_sum(x[g]);
        if ((threadIdx.x & (kWave - 1)) == 0) gbuf[(gparity * 8 + g) * NW + threadIdx.x / kWave] = w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g < G) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) t += gbuf[(gparity * 8 + g) * NW + w];
        x[g] = t;
      }
    }
    gparity ^= 1;
  }
  __device__ __forceinline__ float max(float x) {
    x = wave_max(x);
    if ((threadIdx.x & (kWave - 1)) == 0) buf[parity * NW + threadIdx.x / kWave] = x;
    __syncthreads();
    float t = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) t = fmaxf(t, buf[parity * NW + w]);
    parity ^= 1;
    return t;
  }
};

template <int BS, int NPT, int G>
__global__ __launch_bounds__(BS) void select_kernel(SelectArgs a) {
  constexpr int NW = BS / kWave;
  __shared__ float s_red[2 * NW];
  __shared__ float s_gred[2 * 8 * NW];
  __shared__ int s_list[kMaxSelect];
  __shared__ int s_cnt;

  const int tid = threadIdx.x;
  const int kvh = blockIdx.x;
  const int seq = blockIdx.y;
  const int k = a.k;
  int32_t* sel = a.sel_pages + ((size_t)seq * a.hkv + kvh) * k;
  int32_t* cnt_out = a.sel_count + (size_t)seq * a.hkv + kvh;
  BlockReduce<BS> red{s_red, 0, s_gred};

  int32_t* selp = a.sel_phys ? a.sel_phys + ((size_t)seq * a.hkv + kvh) * k : nullptr;
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;
  // write selection slot i (and its physical page when asked for)
  auto emit = [&](int i, int page) {
    sel[i] = page;
    if (selp) {
      int ph = page >= 0 ? bt[page] : -1;
      selp[i] = (ph >= 0 && ph < a.num_phys) ? ph : -1;
    }
  };
  const int len = a.seq_lens[seq] + a.len_add;
  if (len <= 0) {
    for (int i = tid; i < k; i += BS) emit(i, -1);
    if (tid == 0) *cnt_out = 0;
    return;
  }
  int n_mr = (len - 1) / a.page_size;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  const int n_scored = n_mr;
  const int n_cand = n_mr > 0 ? n_mr - 1 : 0;
  const int n_top = min(k - 2, n_cand);
  const size_t hq = (size_t)a.hkv * G;
  const float* lse = a.page_lse + ((size_t)seq * hq + (size_t)kvh * G) * a.max_pages;

  // trivial selections: one page, or every candidate fits the budget
  if (n_mr == 0) {
    for (int i = tid; i < k; i += BS) emit(i, i == 0 ? 0 : -1);
    if (tid == 0) *cnt_out = 1;
    return;
  }
  if (n_top == n_cand && a.share_out == nullptr) {  // every candidate is selected
    for (int i = tid; i < k; i += BS) emit(i, i <= n_mr ? i : -1);
    if (tid == 0) *cnt_out = n_mr + 1;
    return;
  }

  // 1) this thread's scores s_hat_j(g) for pages j = tid + BS*i (one batch of
  //    independent loads), and the per-head normalizers
  //    L_g = log sum_{j < n_scored} exp(s_hat_j(g))
  float v[G][NPT];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int j = tid + BS * i;
      v[g][i] = (j < n_scored) ? lse[(size_t)g * a.max_pages + j] : -INFINITY;
    }
  float M[kMaxGroup], S[kMaxGroup], L[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    M[g] = -INFINITY;
    if (g >= G) continue;
#pragma unroll
    for (int i = 0; i < NPT; ++i) M[g] = fmaxf(M[g], v[g][i]);
  }
  red.maxG(M, G);
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    S[g] = 0.f;
    if (g < G && M[g] != -INFINITY) {
#pragma unroll
      for (int i = 0; i < NPT; ++i) S[g] += __expf(v[g][i] - M[g]);
    }
  }
  red.sumG(S, G);
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) L[g] = M[g] + __logf(S[g]);

  const float logG = __logf((float)G);
  // log m_bar_j of this thread's i-th page
  auto log_mbar = [&](int i) -> float {
    float mx = -INFINITY;
    float d[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      d[g] = v[g][i] - L[g];
      mx = fmaxf(mx, d[g]);
    }
    if (mx == -INFINITY) return -INFINITY;
    float sm = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) sm += __expf(d[g] - mx);
    return mx + __logf(sm) - logG;
  };

  if (a.share_out) {
    float* so = a.share_out + ((size_t)seq * a.hkv + kvh) * a.max_pages;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int j = tid + BS * i;
      if (j < n_scored) so[j] = __expf(log_mbar(i));
    }
  }

  if (n_top == n_cand) {  // every candidate is selected
    for (int i = tid; i < k; i += BS) emit(i, i <= n_mr ? i : -1);
    if (tid == 0) *cnt_out = n_mr + 1;
    return;
  }

  // 2) ranking keys of the candidates (pages 1 .. n_mr-1; the sink is not one)
  uint32_t key[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = tid + BS * i;
    key[i] = (j >= 1 && j < n_mr) ? order_key(log_mbar(i)) : 0u;
  }
  if (tid == 0) s_cnt = 0;

  if (n_top > 0) {
    // 3) t = the n_top-th largest key, by bisection on its bits.  Bits above
    //    the highest bit in which the largest and smallest candidate keys
    //    differ are common to all keys; the rest are decided two per barrier.
    uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      if (key[i]) { kmax = max(kmax, key[i]); kmin = min(kmin, key[i]); }
    }
    wave_minmax_u32(kmax, kmin);
    {
      uint32_t* ib = reinterpret_cast<uint32_t*>(s_gred);
      if ((tid & (kWave - 1)) == 0) { ib[tid / kWave] = kmax; ib[NW + tid / kWave] = kmin; }
      __syncthreads();
#pragma unroll
      for (int w = 0; w < NW; ++w) { kmax = max(kmax, ib[w]); kmin = min(kmin, ib[NW + w]); }
      __syncthreads();
    }
    uint32_t t = kmax;
    const uint32_t diff = kmax ^ kmin;
    if (diff) {
      const int hb = 31 - __clz(diff);
      t = kmax & ~((hb == 31) ? 0xffffffffu : ((2u << hb) - 1u));
      for (int bit = hb; bit >= 0; bit -= 2) {
        const uint32_t b1 = 1u << bit;
        const uint32_t b0 = bit > 0 ? (1u << (bit - 1)) : 0u;
        // wave counts from ballots (scalar popcounts), then one barrier
        int c1 = 0, c0 = 0, c3 = 0;
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
          c1 += __popcll(__ballot(key[i] >= (t | b1)));
          c0 += __popcll(__ballot(key[i] >= (t | b0)));
          c3 += __popcll(__ballot(key[i] >= (t | b1 | b0)));
        }
        int* cb = reinterpret_cast<int*>(s_gred) + red.gparity * 3 * NW;
        if ((tid & (kWave - 1)) == 0) {
          cb[tid / kWave] = c1;
          cb[NW + tid / kWave] = c0;
          cb[2 * NW + tid / kWave] = c3;
        }
        __syncthreads();
        c1 = c0 = c3 = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) { c1 += cb[w]; c0 += cb[NW + w]; c3 += cb[2 * NW + w]; }
        red.gparity ^= 1;
        if (b0 && c3 >= n_top) t |= b1 | b0;
        else if (c1 >= n_top) t |= b1;
        else if (b0 && c0 >= n_top) t |= b0;
      }
    }
    int ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) { ngt += key[i] > t ? 1 : 0; neq += key[i] == t ? 1 : 0; }
    const int n_gt = (int)red.sum((float)ngt);
    const int n_eq = (int)red.sum((float)neq);
    const int take_eq = n_top - n_gt;
    // 4) collect every key > t, and the take_eq lowest-index keys == t
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      if (key[i] > t || (key[i] == t && take_eq == n_eq)) s_list[atomicAdd(&s_cnt, 1)] = tid + BS * i;
    }
    if (take_eq < n_eq) {
      // rare: ties straddle the cut.  Walk index chunks of BS candidates in order.
      int before = 0;
      const int lane = tid & (kWave - 1);
      const int wave = tid / kWave;
      for (int i = 0; i < NPT; ++i) {
        const int eq = key[i] == t ? 1 : 0;
        int incl = eq;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int v = __shfl_up(incl, off);
          if (lane >= off) incl += v;
        }
        if (lane == kWave - 1) s_red[red.parity * NW + wave] = (float)incl;
        __syncthreads();
        int wave_off = 0, chunk_total = 0;
        for (int w = 0; w < NW; ++w) {
          const int v = (int)s_red[red.parity * NW + w];
          if (w < wave) wave_off += v;
          chunk_total += v;
        }
        red.parity ^= 1;
        const int rank_eq = before + wave_off + incl - eq;
        if (eq && rank_eq < take_eq) s_list[atomicAdd(&s_cnt, 1)] = tid + BS * i;
        before += chunk_total;
      }
    }
  }
  __syncthreads();

  // 5) ordered output: 0, selected candidates ascending, n_mr
  for (int i = tid; i < k; i += BS) {
    if (i < n_top) {
      const int v = s_list[i];
      int rank = 0;
      for (int x = 0; x < n_top; ++x) rank += s_list[x] < v ? 1 : 0;
      emit(1 + rank, v);
    } else if (i == n_top) {
      emit(0, 0);
      emit(n_top + 1, n_mr);
    } else if (i >= n_top + 2) {
      emit(i, -1);
    }
  }
  if (tid == 0) *cnt_out = n_top + 2;
}

template <int BS, int NPT>
static hipError_t launch_sel_g(int G, dim3 grid, const SelectArgs& a, hipStream_t s) {
  switch (G) {
    case 1: hipLaunchKernelGGL((select_kernel<BS, NPT, 1>), grid, dim3(BS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((select_kernel<BS, NPT, 2>), grid, dim3(BS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((select_kernel<BS, NPT, 4>), grid, dim3(BS), 0, s, a); break;
    case 8:
      if constexpr (NPT * 8 <= 96) {
        hipLaunchKernelGGL((select_kernel<BS, NPT, 8>), grid, dim3(BS), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.k > kMaxSelect || a.group > kMaxGroup) return hipErrorInvalidValue;
  const int n = a.max_pages;  // bound on scored pages per sequence
  const int G = a.group;
  dim3 grid(a.hkv, a.batch);
  // smallest (block, keys per thread) covering n pages with G * NPT <= 96
  if (n <= 256 * 4) return launch_sel_g<256, 4>(G, grid, a, s);
  if (n <= 256 * 12) return launch_sel_g<256, 12>(G, grid, a, s);
  if (n <= 1024 * 8) return launch_sel_g<1024, 8>(G, grid, a, s);
  if (n <= 1024 * 12) return launch_sel_g<1024, 12>(G, grid, a, s);
  if (n <= 1024 * 17 && G <= 4) return launch_sel_g<1024, 17>(G, grid, a, s);
  if (n <= 1024 * 24 && G <= 4) return launch_sel_g<1024, 24>(G, grid, a, s);
  return hipErrorInvalidValue;
}

}  // namespace lk
