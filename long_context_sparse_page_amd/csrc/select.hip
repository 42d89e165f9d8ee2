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
// mapped to an order-preserving uint32.  The (k-2)-th largest key is found by
// bisection on its 32 bits (one block-wide count per bit), then the selected
// indices are collected and ordered by rank counting.

#include "common.cuh"
#include "kernels.h"

namespace lk {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxGroup = 8;
constexpr int kMaxSelect = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Block-wide integer sum; `buf` is a [2][kSelWaves] LDS array, `parity`
// alternates between calls so that one barrier per call suffices.
__device__ __forceinline__ int block_sum_int(int x, int (*buf)[kSelWaves], int& parity) {
  x = wave_sum_int(x);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) buf[parity][wave] = x;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) total += buf[parity][w];
  parity ^= 1;
  return total;
}

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

template <int NPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ float s_m[kSelWaves][kMaxGroup];
  __shared__ float s_s[kSelWaves][kMaxGroup];
  __shared__ float s_L[kMaxGroup];
  __shared__ int s_red[2][kSelWaves];
  __shared__ int s_list[kMaxSelect];
  __shared__ int s_cnt;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int kvh = blockIdx.x;
  const int seq = blockIdx.y;
  const int G = a.group;
  const int k = a.k;
  int32_t* sel = a.sel_pages + ((size_t)seq * a.hkv + kvh) * k;
  int32_t* cnt_out = a.sel_count + (size_t)seq * a.hkv + kvh;

  const int T = a.seq_lens[seq];
  if (T <= 0) {
    for (int i = tid; i < k; i += kSelThreads) sel[i] = -1;
    if (tid == 0) *cnt_out = 0;
    return;
  }
  int n_mr = (T - 1) / a.page_size;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  const int n_scored = n_mr;
  const int n_cand = n_mr > 0 ? n_mr - 1 : 0;
  const int n_top = min(k - 2, n_cand);
  const size_t hq = (size_t)a.hkv * G;
  const float* lse = a.page_lse + ((size_t)seq * hq + (size_t)kvh * G) * a.max_pages;

  // 1) per-head normalizers L_g = log sum_{j < n_scored} exp(s_hat_j(g))
  if (n_scored > 0) {
    float m[kMaxGroup], s[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) { m[g] = -INFINITY; s[g] = 0.f; }
    for (int j = tid; j < n_scored; j += kSelThreads) {
#pragma unroll
      for (int g = 0; g < kMaxGroup; ++g) {
        if (g < G) lse_merge(m[g], s[g], lse[(size_t)g * a.max_pages + j], 1.f);
      }
    }
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
      if (g < G) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const float m2 = __shfl_xor(m[g], off);
          const float s2 = __shfl_xor(s[g], off);
          lse_merge(m[g], s[g], m2, s2);
        }
        if (lane == 0) { s_m[wave][g] = m[g]; s_s[wave][g] = s[g]; }
      }
    }
    __syncthreads();
    if (tid < G) {
      float M = -INFINITY, S = 0.f;
      for (int w = 0; w < kSelWaves; ++w) lse_merge(M, S, s_m[w][tid], s_s[w][tid]);
      s_L[tid] = M + __logf(S);
    }
    __syncthreads();
  }
  float L[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) L[g] = (g < G && n_scored > 0) ? s_L[g] : 0.f;
  const float logG = __logf((float)G);

  auto log_mbar = [&](int j) -> float {
    float mx = -INFINITY, sm = 0.f;
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
      if (g < G) lse_merge(mx, sm, lse[(size_t)g * a.max_pages + j] - L[g], 1.f);
    }
    return mx + __logf(sm) - logG;
  };

  // optional share output m_bar_j for every scored page
  if (a.share_out) {
    float* so = a.share_out + ((size_t)seq * a.hkv + kvh) * a.max_pages;
    for (int j = tid; j < n_scored; j += kSelThreads) so[j] = __expf(log_mbar(j));
  }

  // 2) ranking keys of the candidates
  uint32_t key[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = 1 + tid + kSelThreads * i;
    key[i] = (j < n_mr) ? order_key(log_mbar(j)) : 0u;
  }

  if (tid == 0) s_cnt = 0;
  int parity = 0;
  if (n_top > 0 && n_top < n_cand) {
    // 3) threshold t = the n_top-th largest key
    uint32_t t = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = t | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < NPT; ++i) cnt += key[i] >= c ? 1 : 0;
      if (block_sum_int(cnt, s_red, parity) >= n_top) t = c;
    }
    int ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) { ngt += key[i] > t ? 1 : 0; neq += key[i] == t ? 1 : 0; }
    const int n_gt = block_sum_int(ngt, s_red, parity);
    const int n_eq = block_sum_int(neq, s_red, parity);
    const int take_eq = n_top - n_gt;
    // 4) collect: every key > t, and the take_eq lowest-index keys == t
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      if (key[i] > t || (key[i] == t && take_eq == n_eq)) {
        s_list[atomicAdd(&s_cnt, 1)] = 1 + tid + kSelThreads * i;
      }
    }
    if (take_eq < n_eq) {
      int before = 0;  // equal keys at lower indices (chunks are index ranges)
      for (int i = 0; i < NPT; ++i) {
        const int eq = key[i] == t ? 1 : 0;
        // exclusive prefix of eq over the threads of this chunk
        int incl = eq;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int v = __shfl_up(incl, off);
          if (lane >= off) incl += v;
        }
        if (lane == kWave - 1) s_red[parity][wave] = incl;
        __syncthreads();
        int wave_off = 0, chunk_total = 0;
        for (int w = 0; w < kSelWaves; ++w) {
          const int v = s_red[parity][w];
          if (w < wave) wave_off += v;
          chunk_total += v;
        }
        parity ^= 1;
        const int rank_eq = before + wave_off + incl - eq;
        if (eq && rank_eq < take_eq) s_list[atomicAdd(&s_cnt, 1)] = 1 + tid + kSelThreads * i;
        before += chunk_total;
      }
    }
    __syncthreads();
  }

  // 5) ordered output: 0, selected candidates ascending, n_mr
  if (n_mr == 0) {
    for (int i = tid; i < k; i += kSelThreads) sel[i] = i == 0 ? 0 : -1;
    if (tid == 0) *cnt_out = 1;
    return;
  }
  if (n_top == n_cand) {
    for (int i = tid; i < k; i += kSelThreads) sel[i] = i <= n_mr ? i : -1;
    if (tid == 0) *cnt_out = n_mr + 1;
    return;
  }
  for (int i = tid; i < k; i += kSelThreads) {
    if (i < n_top) {
      const int v = s_list[i];
      int rank = 0;
      for (int x = 0; x < n_top; ++x) rank += s_list[x] < v ? 1 : 0;
      sel[1 + rank] = v;
    } else if (i == n_top) {
      sel[0] = 0;
      sel[n_top + 1] = n_mr;
    } else if (i >= n_top + 2) {
      sel[i] = -1;
    }
  }
  if (tid == 0) *cnt_out = n_top + 2;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const int max_cand = a.max_pages;  // upper bound on candidates per sequence
  dim3 grid(a.hkv, a.batch);
  dim3 block(kSelThreads);
  if (a.k > kMaxSelect || a.group > kMaxGroup) return hipErrorInvalidValue;
  if (max_cand <= kSelThreads * 16) {
    hipLaunchKernelGGL(select_kernel<16>, grid, block, 0, s, a);
  } else if (max_cand <= kSelThreads * 32) {
    hipLaunchKernelGGL(select_kernel<32>, grid, block, 0, s, a);
  } else if (max_cand <= kSelThreads * 64) {
    hipLaunchKernelGGL(select_kernel<64>, grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lk
