// Page summary builder: one workgroup of 1024 threads per (page, KV head).
//
// [Locks] §4 "Build (once, when a page completes)": centre the page,
// k_i = mu + delta_i; stack the deviations as rows of D (B x d); eigendecompose
// the B x B Gram D D^T = U Sigma^2 U^T with eigenvalues descending; keep r
// components, C = U_r Sigma_r (coefficients c_i = rows of C) and the
// orthonormal basis V = D^T U_r Sigma_r^{-1}; zero modes are dropped with
// zero coefficients.
//
// Device plan: the K tile is widened to fp32 and centred in LDS (stored
// transposed, D^T, so the Gram and basis reads are bank-conflict free); the
// Gram is formed in fp32; the eigendecomposition is a cyclic parallel Jacobi
// method held in LDS: each round rotates 32 disjoint index pairs chosen by the
// circle (round-robin) ordering, with the symmetric Schur rotation of Golub &
// Van Loan (Matrix Computations, sym.schur2).  A round is one 2 x 2 block
// update of the upper block triangle per thread (mirrored, so A stays exactly
// symmetric; the rotated pair is set exactly: a_pp - t a_pq, a_qq + t a_pq, 0)
// plus two column-pair updates of the accumulated eigenvector matrix U.
// Sweeps stop when the off-diagonal energy is below 1e-10 of the total.
//
// Zero-mode rule: eigenvalue <= 1e-5 * lambda_1 or <= 1e-10 * sum_i ||k_i||^2.
// Sign rule: each basis vector's largest-magnitude entry is made positive.

#include "common.cuh"
#include "kernels.h"

namespace lk {

constexpr int kBuildThreads = 1024;
constexpr int kBuildWaves = kBuildThreads / kWave;
constexpr int kBuildMaxSweeps = 15;
constexpr float kJacobiTol = 1e-10f;
constexpr float kZeroModeRtol = 1e-5f;
constexpr float kZeroModeFloor = 1e-10f;

// Decode step: combine the attention split partials of (seq, kvh) for its G
// heads, o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s and
// lse = M + log sum_s e^{m_s - M} l_s (max in log2 units); one output per thread.
template <typename T>
__device__ __forceinline__ void merge_partials(const BuildArgs& a, int seq, int kvh) {
  constexpr int D = kHeadDim;
  const int G = a.merge.group;
  const int x = threadIdx.x;
  if (x >= G * D) return;
  const int g = x / D, dim = x % D;
  const int ns = a.merge.n_splits;
  const float* ml = a.merge.part_ml + ((size_t)seq * a.hkv + kvh) * ns * G * 2;
  const float* ob = a.merge.part_o + ((size_t)seq * a.hkv + kvh) * ns * G * D;
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; ++s0) M = fmaxf(M, ml[((size_t)s0 * G + g) * 2]);
  float ov = 0.f, lv = 0.f;
  if (M != -INFINITY) {
#pragma unroll 8
    for (int s0 = 0; s0 < ns; ++s0) {
      const float ms = ml[((size_t)s0 * G + g) * 2];
      const float f = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      ov = fmaf(f, ob[((size_t)s0 * G + g) * D + dim], ov);
      lv = fmaf(f, ml[((size_t)s0 * G + g) * 2 + 1], lv);
    }
  }
  const int h = kvh * G + g;
  Elem<T>::store(reinterpret_cast<T*>(a.merge.out) + ((size_t)seq * a.merge.hq + h) * D + dim,
                 lv > 0.f ? ov / lv : 0.f);
  if (a.merge.lse_out && dim == 0)
    a.merge.lse_out[(size_t)seq * a.merge.hq + h] =
        lv > 0.f ? (M + __builtin_amdgcn_logf(lv)) * kLn2 : -INFINITY;
}

template <typename T, int R>
__global__ __launch_bounds__(kBuildThreads) void build_kernel(BuildArgs a) {
  constexpr int B = 64;
  constexpr int D = kHeadDim;
  constexpr int NP = B / 2;                 // pairs per round
  constexpr int NBLK = NP * (NP + 1) / 2;   // upper 2x2 blocks (528)
  constexpr int KEPT = R < B ? R : B;
  constexpr int LDA = B + 1;

  __shared__ float sDT[D][LDA];             // D^T: sDT[c][i] = delta_i[c]
  __shared__ float sA[B][LDA];              // Gram -> diagonal; later the basis
  __shared__ float sU[B][LDA];
  __shared__ float sMu[D];
  __shared__ float4 sPar[NP];               // c, s, t, (p | q << 8) as bits
  __shared__ float sLam[B];
  __shared__ int sOrder[B];
  __shared__ float sRed[2][kBuildWaves];
  __shared__ float sSigma[KEPT], sSign[KEPT];
  __shared__ int sCol[KEPT], sNz[KEPT];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int idx = blockIdx.x;
  const int kvh = blockIdx.y;
  if (a.commit_seq_lens && kvh == 0 && tid == 0) {
    // decode step: the append of sequence idx was valid -> advance its length
    const int len = a.commit_seq_lens[idx];
    const int page = len / B;
    int ph = -1;
    if (len >= 0 && page < a.max_pages) ph = a.block_table[(size_t)idx * a.max_pages + page];
    if (ph >= 0 && ph < a.num_phys) a.commit_seq_lens[idx] = len + 1;
  }
  if (a.merge.part_o) merge_partials<T>(a, idx, kvh);
  const int phys = a.phys_ids[idx];
  if (phys < 0 || phys >= a.num_phys) return;

  // this thread's upper block (k1 <= k2), if any
  int k1 = -1, k2 = -1;
  if (tid < NBLK) {
    int rem = tid;
    k1 = 0;
    while (rem >= NP - k1) { rem -= NP - k1; ++k1; }
    k2 = k1 + rem;
  }

  // 1) load K (8 elements per thread), energy, transpose into LDS
  const T* K = reinterpret_cast<const T*>(a.k_pool) + (((size_t)phys * a.hkv + kvh) * B) * D;
  float en = 0.f;
  {
    const int row = tid >> 4;
    const int c0 = (tid & 15) * 8;
    float v[8];
    load8(K + (size_t)row * D + c0, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) { sDT[c0 + t][row] = v[t]; en = fmaf(v[t], v[t], en); }
  }
  en = group_sum<kWave>(en);
  if (lane == 0) sRed[0][wave] = en;
  __syncthreads();
  float energy = 0.f;
#pragma unroll
  for (int w = 0; w < kBuildWaves; ++w) energy += sRed[0][w];
  // 2) centroid and centring
  if (tid < D) {
    float s = 0.f;
    for (int i = 0; i < B; ++i) s += sDT[tid][i];
    sMu[tid] = s * (1.0f / B);
  }
  __syncthreads();
  {
    const int row = tid >> 4;
    const int c0 = (tid & 15) * 8;
#pragma unroll
    for (int t = 0; t < 8; ++t) sDT[c0 + t][row] -= sMu[c0 + t];
  }
  __syncthreads();

  // 3) Gram A = D D^T (2 x 2 tile per thread), U = I
  {
    const int bi = tid >> 5, bj = tid & 31;
    float a00 = 0.f, a01 = 0.f, a10 = 0.f, a11 = 0.f;
    for (int c = 0; c < D; ++c) {
      const float x0 = sDT[c][2 * bi], x1 = sDT[c][2 * bi + 1];
      const float y0 = sDT[c][2 * bj], y1 = sDT[c][2 * bj + 1];
      a00 = fmaf(x0, y0, a00); a01 = fmaf(x0, y1, a01);
      a10 = fmaf(x1, y0, a10); a11 = fmaf(x1, y1, a11);
    }
    sA[2 * bi][2 * bj] = a00; sA[2 * bi][2 * bj + 1] = a01;
    sA[2 * bi + 1][2 * bj] = a10; sA[2 * bi + 1][2 * bj + 1] = a11;
    sU[2 * bi][2 * bj] = (bi == bj) ? 1.f : 0.f;
    sU[2 * bi][2 * bj + 1] = 0.f;
    sU[2 * bi + 1][2 * bj] = 0.f;
    sU[2 * bi + 1][2 * bj + 1] = (bi == bj) ? 1.f : 0.f;
  }
  __syncthreads();

  // 4) cyclic parallel Jacobi
  for (int sweep = 0; sweep < kBuildMaxSweeps; ++sweep) {
    for (int r = 0; r < B - 1; ++r) {
      if (tid < NP) {
        const int k = tid;
        const int p = k == 0 ? B - 1 : (r + k) % (B - 1);
        const int q = k == 0 ? r : (r - k + (B - 1)) % (B - 1);
        const float app = sA[p][p], aqq = sA[q][q], apq = sA[p][q];
        float c = 1.f, s = 0.f, t = 0.f;
        if (apq != 0.f) {
          const float tau = (aqq - app) / (2.f * apq);
          t = (tau >= 0.f ? 1.f : -1.f) / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + t * t);
          s = t * c;
        }
        sPar[k] = make_float4(c, s, t, __int_as_float(p | (q << 8)));
      }
      __syncthreads();
      if (k1 >= 0) {
        const float4 P1 = sPar[k1];
        const int p1 = __float_as_int(P1.w) & 0xff, q1 = __float_as_int(P1.w) >> 8;
        if (k1 == k2) {
          const float apq = sA[p1][q1];
          sA[p1][p1] -= P1.z * apq;
          sA[q1][q1] += P1.z * apq;
          sA[p1][q1] = 0.f;
          sA[q1][p1] = 0.f;
        } else {
          const float4 P2 = sPar[k2];
          const int p2 = __float_as_int(P2.w) & 0xff, q2 = __float_as_int(P2.w) >> 8;
          const float c1 = P1.x, s1 = P1.y, c2 = P2.x, s2 = P2.y;
          const float x00 = sA[p1][p2], x01 = sA[p1][q2], x10 = sA[q1][p2], x11 = sA[q1][q2];
          const float y00 = c1 * x00 - s1 * x10, y01 = c1 * x01 - s1 * x11;
          const float y10 = s1 * x00 + c1 * x10, y11 = s1 * x01 + c1 * x11;
          const float z00 = c2 * y00 - s2 * y01, z01 = s2 * y00 + c2 * y01;
          const float z10 = c2 * y10 - s2 * y11, z11 = s2 * y10 + c2 * y11;
          sA[p1][p2] = z00; sA[p2][p1] = z00;
          sA[p1][q2] = z01; sA[q2][p1] = z01;
          sA[q1][p2] = z10; sA[p2][q1] = z10;
          sA[q1][q2] = z11; sA[q2][q1] = z11;
        }
      }
      // U <- U J: columns p, q of rows i (two (row, pair) items per thread)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int w = tid + x * kBuildThreads;
        const int i = w >> 5, k = w & 31;
        const float4 P = sPar[k];
        const int p = __float_as_int(P.w) & 0xff, q = __float_as_int(P.w) >> 8;
        const float up = sU[i][p], uq = sU[i][q];
        sU[i][p] = P.x * up - P.y * uq;
        sU[i][q] = P.y * up + P.x * uq;
      }
      __syncthreads();
    }
    // convergence: off-diagonal energy vs total (4 entries per thread)
    float off = 0.f, tot = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int w = tid + x * kBuildThreads;
      const int i = w >> 6, j = w & 63;
      const float v = sA[i][j];
      tot = fmaf(v, v, tot);
      if (i != j) off = fmaf(v, v, off);
    }
    off = group_sum<kWave>(off);
    tot = group_sum<kWave>(tot);
    if (lane == 0) { sRed[0][wave] = off; sRed[1][wave] = tot; }
    __syncthreads();
    float o = 0.f, tt = 0.f;
#pragma unroll
    for (int w = 0; w < kBuildWaves; ++w) { o += sRed[0][w]; tt += sRed[1][w]; }
    __syncthreads();
    if (o <= kJacobiTol * tt) break;
  }

  // 5) eigenvalues sorted descending (ties to the lower index)
  if (tid < B) sLam[tid] = sA[tid][tid];
  __syncthreads();
  if (tid < B) {
    const float li = sLam[tid];
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const float lj = sLam[j];
      rank += (lj > li || (lj == li && j < tid)) ? 1 : 0;
    }
    sOrder[rank] = tid;
  }
  __syncthreads();
  if (tid < KEPT) {
    const float lam1 = sLam[sOrder[0]];
    const int col = sOrder[tid];
    const float lam = sLam[col];
    const float thresh = fmaxf(kZeroModeRtol * lam1, kZeroModeFloor * energy);
    const int nz = (lam1 > 0.f && lam > thresh) ? 1 : 0;
    sCol[tid] = col;
    sNz[tid] = nz;
    sSigma[tid] = nz ? sqrtf(lam) : 1.f;
  }
  if (a.eigvals_out && tid < B) {
    a.eigvals_out[((size_t)idx * a.hkv + kvh) * B + tid] = fmaxf(sLam[sOrder[tid]], 0.f);
  }
  __syncthreads();

  // 6) basis V[k][c] = sum_i D[i][c] U[i][col_k] / sigma_k  (stored in sA)
  float* sV = &sA[0][0];
  for (int w = tid; w < KEPT * D; w += kBuildThreads) {
    const int k = w / D, c = w % D;
    float v = 0.f;
    if (sNz[k]) {
      const int col = sCol[k];
      for (int i = 0; i < B; ++i) v = fmaf(sDT[c][i], sU[i][col], v);
      v /= sSigma[k];
    }
    sV[k * D + c] = v;
  }
  __syncthreads();
  // sign: largest |entry| positive (ties to the lower dim)
  for (int k = wave; k < KEPT; k += kBuildWaves) {
    float best = -1.f, val = 0.f;
    int bidx = D;
#pragma unroll
    for (int x = 0; x < D / kWave; ++x) {
      const int c = lane + kWave * x;
      const float v = sV[k * D + c];
      if (fabsf(v) > best || (fabsf(v) == best && c < bidx)) { best = fabsf(v); val = v; bidx = c; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float b2 = __shfl_xor(best, off);
      const float v2 = __shfl_xor(val, off);
      const int i2 = __shfl_xor(bidx, off);
      if (b2 > best || (b2 == best && i2 < bidx)) { best = b2; val = v2; bidx = i2; }
    }
    if (lane == 0) sSign[k] = val < 0.f ? -1.f : 1.f;
  }
  __syncthreads();

  // 7) write the record: centroid | basis rows | coefficients
  constexpr int REC = D + R * D + B * R;
  T* rec = reinterpret_cast<T*>(a.summary) + ((size_t)phys * a.hkv + kvh) * REC;
  for (int x = tid; x < REC; x += kBuildThreads) {
    float v;
    if (x < D) {
      v = sMu[x];
    } else if (x < D + R * D) {
      const int k = (x - D) / D, c = (x - D) % D;
      v = (k < KEPT) ? sV[k * D + c] * sSign[k] : 0.f;
    } else {
      const int i = (x - D - R * D) / R, k = (x - D - R * D) % R;
      v = (k < KEPT && sNz[k]) ? sU[i][sCol[k]] * sSigma[k] * sSign[k] : 0.f;
    }
    Elem<T>::store(rec + x, v);
  }
}

template <typename T>
static hipError_t launch_build_t(int rank, const BuildArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  dim3 grid(a.n, a.hkv);
  dim3 block(kBuildThreads);
  switch (rank) {
    case 1: hipLaunchKernelGGL((build_kernel<T, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((build_kernel<T, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((build_kernel<T, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((build_kernel<T, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((build_kernel<T, 16>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_build(DType dt, int rank, const BuildArgs& a, hipStream_t s) {
  return dt == kBF16 ? launch_build_t<bf16_t>(rank, a, s) : launch_build_t<float>(rank, a, s);
}

}  // namespace lk
