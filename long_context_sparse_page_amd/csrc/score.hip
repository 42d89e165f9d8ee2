// Page scorer: reconstructed log-sum-exp of every complete page.
//
// [Locks] §4 "Score", Eq. (1): for page j with centroid mu_j, basis V_j (d x r)
// and coefficients c_i, and query head g,
//   s_hat_j(q_g) = log sum_i exp(scale * (q_g . mu_j + (V_j^T q_g) . c_i)).
// The record stores centroid | basis rows | coeffs, so rows 0..r of the
// record form W = [mu; v_1; ...; v_r] and the projection is P = W q_g.
//
// Layout of the work (one wave per page at a time, pages of one
// (sequence, KV head) per workgroup):
//   projection: lane (s = lane / 16, e = lane % 16) owns dims 8e..8e+7 of rows
//     s, s+4, s+8, ...; partial dots are summed over the 16 lanes of a row
//     group with DPP, giving P[row][g] for every query head of the group;
//   reconstruction: lane i = token i computes z_i(g) = P[0][g] + sum_m c_i[m] P[m+1][g]
//     (P broadcast from LDS);
//   LSE: z is transposed through LDS so that each query head's B logits sit
//     on a group of 64/G lanes, reduced with DPP (max, then sum of exp2).
// The page's bytes are read once, with 16-byte loads.

#include "common.cuh"
#include "kernels.h"

namespace lk {

constexpr int kScoreWaves = 4;
constexpr int kScorePagesPerWave = 8;
constexpr int kScorePagesPerBlock = kScoreWaves * kScorePagesPerWave;

template <typename T, int R>
__device__ __forceinline__ void load_coeffs(const T* p, float (&c)[R]) {
  if constexpr (R % 8 == 0) {
#pragma unroll
    for (int m = 0; m < R; m += 8) {
      float x[8];
      load8(p + m, x);
#pragma unroll
      for (int t = 0; t < 8; ++t) c[m + t] = x[t];
    }
  } else {
#pragma unroll
    for (int m = 0; m < R; ++m) c[m] = Elem<T>::load(p + m);
  }
}

template <typename T, int R, int G>
__global__ __launch_bounds__(kScoreWaves * kWave) void score_kernel(ScoreArgs a) {
  constexpr int B = 64;
  constexpr int D = kHeadDim;
  constexpr int ROWS = R + 1;                 // centroid + r basis rows
  constexpr int RG = (ROWS + 3) / 4;          // rows per lane group
  constexpr int LPH = kWave / G;              // lanes per query head in the LSE
  constexpr int TPL = B / LPH;                // logits per lane in the LSE
  constexpr size_t REC = (size_t)ROWS * D + (size_t)B * R;

  __shared__ float sP[kScoreWaves][ROWS * G];
  __shared__ float sZ[kScoreWaves][G * B];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int seq = blockIdx.z;
  const int kvh = blockIdx.y;
  const int len = a.seq_lens[seq];
  if (len <= 0) return;
  int n_scored = (len - 1) / B;
  if (n_scored > a.max_pages - 1) n_scored = a.max_pages - 1;
  const int j0 = blockIdx.x * kScorePagesPerBlock + wave * kScorePagesPerWave;
  if (j0 >= n_scored) return;

  const int s = lane >> 4;
  const int e = lane & 15;
  const T* q = reinterpret_cast<const T*>(a.q) + ((size_t)seq * a.hq + (size_t)kvh * G) * D;
  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) load8(q + (size_t)g * D + e * 8, qv[g]);

  const float zscale = a.scale * kLog2e;
  const T* summ = reinterpret_cast<const T*>(a.summary);
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;
  float* out = a.page_lse + ((size_t)seq * a.hq + (size_t)kvh * G) * a.max_pages;
  float* P = sP[wave];
  float* Z = sZ[wave];

  for (int jj = 0; jj < kScorePagesPerWave; ++jj) {
    const int j = j0 + jj;
    if (j >= n_scored) break;
    const int phys = bt[j];
    if (phys < 0 || phys >= a.num_phys) {
      if (lane < G) out[(size_t)lane * a.max_pages + j] = -INFINITY;
      continue;
    }
    const T* rec = summ + ((size_t)phys * a.hkv + kvh) * REC;

    // projection P[row][g] = W[row] . q_g
    float part[RG][G];
#pragma unroll
    for (int u = 0; u < RG; ++u) {
      const int row = s + 4 * u;
#pragma unroll
      for (int g = 0; g < G; ++g) part[u][g] = 0.f;
      if (row < ROWS) {
        float w[8];
        load8(rec + (size_t)row * D + e * 8, w);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = 0.f;
#pragma unroll
          for (int t = 0; t < 8; ++t) acc = fmaf(w[t], qv[g][t], acc);
          part[u][g] = acc;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RG; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g) part[u][g] = group_sum<16>(part[u][g]);
    if (e == 0) {
#pragma unroll
      for (int u = 0; u < RG; ++u) {
        const int row = s + 4 * u;
        if (row < ROWS) {
#pragma unroll
          for (int g = 0; g < G; ++g) P[row * G + g] = part[u][g];
        }
      }
    }
    wave_lds_fence();

    // reconstructed logits, lane = token
    float c[R];
    load_coeffs<T, R>(rec + (size_t)ROWS * D + (size_t)lane * R, c);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float z = P[g];
#pragma unroll
      for (int m = 0; m < R; ++m) z = fmaf(c[m], P[(m + 1) * G + g], z);
      Z[g * B + lane] = z * zscale;
    }
    wave_lds_fence();

    // per-head log-sum-exp over the page's B logits
    const int hg = lane / LPH;
    const int t0 = (lane % LPH) * TPL;
    float v[TPL];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      v[t] = Z[hg * B + t0 + t];
      mx = fmaxf(mx, v[t]);
    }
    mx = group_max<LPH>(mx);
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < TPL; ++t) sum += fast_exp2(v[t] - mx);
    sum = group_sum<LPH>(sum);
    if (lane % LPH == 0) out[(size_t)hg * a.max_pages + j] = (mx + fast_log2(sum)) * kLn2;
    wave_lds_fence();
  }
}

template <typename T, int R>
static hipError_t launch_score_rg(int group, const ScoreArgs& a, hipStream_t s) {
  dim3 grid((a.max_pages + kScorePagesPerBlock - 1) / kScorePagesPerBlock, a.hkv, a.batch);
  dim3 block(kScoreWaves * kWave);
  switch (group) {
    case 1: hipLaunchKernelGGL((score_kernel<T, R, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((score_kernel<T, R, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((score_kernel<T, R, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((score_kernel<T, R, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_score_t(int rank, int group, const ScoreArgs& a, hipStream_t s) {
  switch (rank) {
    case 1: return launch_score_rg<T, 1>(group, a, s);
    case 2: return launch_score_rg<T, 2>(group, a, s);
    case 4: return launch_score_rg<T, 4>(group, a, s);
    case 8: return launch_score_rg<T, 8>(group, a, s);
    case 16: return launch_score_rg<T, 16>(group, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_score(DType dt, int rank, int group, const ScoreArgs& a, hipStream_t s) {
  return dt == kBF16 ? launch_score_t<bf16_t>(rank, group, a, s)
                     : launch_score_t<float>(rank, group, a, s);
}

}  // namespace lk
