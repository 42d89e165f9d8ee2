// Page summary builder: one workgroup per (page, KV head).
//
// [Locks] §4 "Build (once, when a page completes)": centre the page,
// k_i = mu + delta_i; stack the deviations as rows of D (B x d); eigendecompose
// the B x B Gram D D^T = U Sigma^2 U^T with eigenvalues descending; keep r
// components, C = U_r Sigma_r (coefficients c_i = rows of C) and the
// orthonormal basis V = D^T U_r Sigma_r^{-1}; zero modes are dropped with
// zero coefficients.
//
// Device plan: the K tile is widened to fp32 in LDS and centred; the Gram is
// formed in fp32 from LDS; the eigendecomposition is a cyclic parallel Jacobi
// method held in LDS: each round rotates 32 disjoint index pairs chosen by the
// circle (round-robin) ordering, with the symmetric Schur rotation of Golub &
// Van Loan (Matrix Computations, sym.schur2), applied as 2 x 2 block updates
// of the upper block triangle (mirrored, so A stays exactly symmetric) and to
// the accumulated eigenvector matrix U.  Sweeps stop when the off-diagonal
// energy falls below 1e-13 of the total.
//
// Zero-mode rule: eigenvalue <= 1e-5 * lambda_1 or <= 1e-10 * sum_i ||k_i||^2.
// Sign rule: each basis vector's largest-magnitude entry is made positive.

#include "common.cuh"
#include "kernels.h"

namespace lk {

constexpr int kBuildThreads = 256;
constexpr int kBuildMaxSweeps = 12;
constexpr float kZeroModeRtol = 1e-5f;
constexpr float kZeroModeFloor = 1e-10f;

template <typename T, int R>
__global__ __launch_bounds__(kBuildThreads) void build_kernel(BuildArgs a) {
  constexpr int B = 64;
  constexpr int D = kHeadDim;
  constexpr int NP = B / 2;                 // pairs per round
  constexpr int NBLK = NP * (NP + 1) / 2;   // upper 2x2 blocks
  constexpr int KEPT = R < B ? R : B;
  constexpr int LDA = B + 1;

  __shared__ float sD[B][D + 4];
  __shared__ float sA[B][LDA];              // Gram -> eigenvalues; later the basis
  __shared__ float sU[B][LDA];
  __shared__ float sMu[D];
  __shared__ float sRc[NP], sRs[NP], sRt[NP];
  __shared__ int sRp[NP], sRq[NP];
  __shared__ unsigned short sBlk[NBLK];
  __shared__ float sLam[B];
  __shared__ int sOrder[B];
  __shared__ float sRed[2][kBuildThreads / kWave];
  __shared__ float sSigma[KEPT], sSign[KEPT];
  __shared__ int sCol[KEPT], sNz[KEPT];
  __shared__ float sEnergy;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int idx = blockIdx.x;
  const int kvh = blockIdx.y;
  const int phys = a.phys_ids[idx];
  if (phys < 0 || phys >= a.num_phys) return;

  // upper block table (k1 <= k2)
  for (int b = tid; b < NBLK; b += kBuildThreads) {
    int k1 = 0, rem = b;
    while (rem >= NP - k1) { rem -= NP - k1; ++k1; }
    sBlk[b] = (unsigned short)((k1 << 8) | (k1 + rem));
  }

  // 1) load K (fp32 in LDS), page energy
  const T* K = reinterpret_cast<const T*>(a.k_pool) + (((size_t)phys * a.hkv + kvh) * B) * D;
  float en = 0.f;
  {
    const int row = tid >> 2;
    const int c0 = (tid & 3) * 32;
#pragma unroll
    for (int x = 0; x < 32; x += 8) {
      float v[8];
      load8(K + (size_t)row * D + c0 + x, v);
#pragma unroll
      for (int t = 0; t < 8; ++t) { sD[row][c0 + x + t] = v[t]; en = fmaf(v[t], v[t], en); }
    }
  }
  en = group_sum<kWave>(en);
  if (lane == 0) sRed[0][wave] = en;
  __syncthreads();
  if (tid == 0) {
    float e = 0.f;
    for (int w = 0; w < kBuildThreads / kWave; ++w) e += sRed[0][w];
    sEnergy = e;
  }
  // 2) centroid and centring
  if (tid < D) {
    float s = 0.f;
    for (int i = 0; i < B; ++i) s += sD[i][tid];
    sMu[tid] = s * (1.0f / B);
  }
  __syncthreads();
  {
    const int row = tid >> 2;
    const int c0 = (tid & 3) * 32;
#pragma unroll
    for (int x = 0; x < 32; ++x) sD[row][c0 + x] -= sMu[c0 + x];
  }
  __syncthreads();

  // 3) Gram A = D D^T (each thread a 4 x 4 tile), U = I
  {
    const int bi = tid >> 4, bj = tid & 15;
    float acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = 0.f;
    for (int c = 0; c < D; ++c) {
      float av[4], bv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) { av[x] = sD[4 * bi + x][c]; bv[x] = sD[4 * bj + x][c]; }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(av[x], bv[y], acc[x][y]);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        sA[4 * bi + x][4 * bj + y] = acc[x][y];
        sU[4 * bi + x][4 * bj + y] = (4 * bi + x == 4 * bj + y) ? 1.f : 0.f;
      }
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
        sRp[k] = p; sRq[k] = q; sRc[k] = c; sRs[k] = s; sRt[k] = t;
      }
      __syncthreads();
      for (int b = tid; b < NBLK; b += kBuildThreads) {
        const int k1 = sBlk[b] >> 8, k2 = sBlk[b] & 0xff;
        const int p1 = sRp[k1], q1 = sRq[k1];
        if (k1 == k2) {
          const float apq = sA[p1][q1], t1 = sRt[k1];
          sA[p1][p1] -= t1 * apq;
          sA[q1][q1] += t1 * apq;
          sA[p1][q1] = 0.f;
          sA[q1][p1] = 0.f;
          continue;
        }
        const int p2 = sRp[k2], q2 = sRq[k2];
        const float c1 = sRc[k1], s1 = sRs[k1], c2 = sRc[k2], s2 = sRs[k2];
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
      // U <- U J (columns p, q of every row)
      for (int w = tid; w < B * NP; w += kBuildThreads) {
        const int i = w / NP, k = w % NP;
        const int p = sRp[k], q = sRq[k];
        const float c = sRc[k], s = sRs[k];
        const float up = sU[i][p], uq = sU[i][q];
        sU[i][p] = c * up - s * uq;
        sU[i][q] = s * up + c * uq;
      }
      __syncthreads();
    }
    // convergence: off-diagonal energy vs total
    float off = 0.f, tot = 0.f;
    for (int w = tid; w < B * B; w += kBuildThreads) {
      const int i = w / B, j = w % B;
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
    for (int w = 0; w < kBuildThreads / kWave; ++w) { o += sRed[0][w]; tt += sRed[1][w]; }
    __syncthreads();
    if (o <= 1e-13f * tt) break;
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
    const float thresh = fmaxf(kZeroModeRtol * lam1, kZeroModeFloor * sEnergy);
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
  {
    const int c = tid & (D - 1);
    for (int k = tid / D; k < KEPT; k += kBuildThreads / D) {
      float v = 0.f;
      if (sNz[k]) {
        const int col = sCol[k];
        for (int i = 0; i < B; ++i) v = fmaf(sD[i][c], sU[i][col], v);
        v /= sSigma[k];
      }
      sV[k * D + c] = v;
    }
  }
  __syncthreads();
  // sign: largest |entry| positive (ties to the lower dim)
  for (int k = wave; k < KEPT; k += kBuildThreads / kWave) {
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
