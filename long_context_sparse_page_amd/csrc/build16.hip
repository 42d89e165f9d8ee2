// Page summary builder for pages of B = 16 tokens: one wave per (page, KV
// head), four per workgroup.
//
// [Locks] §4 "Build (once, when a page completes)": centre the page,
// eigendecompose the B x B Gram D D^T = U Sigma^2 U^T (eigenvalues
// descending), keep r components: coefficients C = U_r Sigma_r and basis
// V = D^T U_r Sigma_r^{-1}; zero modes are dropped with zero coefficients.
// Same zero-mode rule, sign convention and record formats as the 64-token
// builder.
//
// The Gram is one 16 x 16 tile on the matrix cores (each fp32 entry of D as
// three bf16 terms, six products, mirrored for exact symmetry).  A 16 x 16
// eigenproblem suits the cyclic Jacobi method (Golub & Van Loan, Matrix
// Computations, §8.5): the round-robin ordering pairs the 16 indices into 8
// disjoint pairs per round (15 rounds per sweep); each round applies its 8
// symmetric Schur rotations at once (disjoint rotations commute), with the
// rotated diagonal pair set to a_pp - t a_pq, a_qq + t a_pq and a_pq to 0.
// Sweeps stop once the off-diagonal energy is below 1e-13 of the total, or
// after 12.

#include "common.cuh"
#include "kernels.h"

namespace lk {

constexpr int kB16 = 16;
constexpr int kB16Waves = 4;
constexpr int kB16Ld = 17;   // padded row of the 16 x 16 matrices
constexpr int kB16DLd = 132; // padded row of D (16 x 128)

__device__ __forceinline__ float b16_q_scale(float amax, float levels) { return (float)(_Float16)(amax / levels); }
__device__ __forceinline__ int b16_q_code(float x, float s, float levels) {
  if (!(s > 0.f)) return 0;
  return (int)fminf(fmaxf(rintf(x / s), -levels), levels);
}

template <typename T, int R>
__global__ __launch_bounds__(kB16Waves * kWave) void build16_kernel(BuildArgs a) {
  constexpr int B = kB16;
  constexpr int D = kHeadDim;
  constexpr int KEPT = R < B ? R : B;
  __shared__ float sD[kB16Waves][B][kB16DLd];       // centred keys, row i = delta_i
  __shared__ float sA[kB16Waves][2][B][kB16Ld];     // Gram / rotated matrix (ping-pong)
  __shared__ float sU[kB16Waves][2][B][kB16Ld];     // accumulated rotations
  __shared__ float sMu[kB16Waves][D];
  __shared__ float sRot[kB16Waves][B][2];           // per index: J[i][i], J[partner][i]
  __shared__ int sPart[kB16Waves][B];
  __shared__ float sV[kB16Waves][KEPT][D];          // basis rows (before the sign)
  __shared__ float sSign[kB16Waves][KEPT];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int item = blockIdx.x * kB16Waves + wave;   // (page, KV head) pair
  if (item >= a.n * a.hkv) return;
  const int idx = item / a.hkv, kvh = item % a.hkv;
  const int phys = a.phys_ids[idx];
  if (phys < 0 || phys >= a.num_phys) return;

  // 1) K tile (16 x 128), energy sum ||k_i||^2, centroid, centring
  const T* K = reinterpret_cast<const T*>(a.k_pool) + (((size_t)phys * a.hkv + kvh) * B) * D;
  float en = 0.f;
#pragma unroll
  for (int x = 0; x < B * D / kWave / 8; ++x) {  // 4 chunks of 8 elements per lane
    const int e = (lane + kWave * x) * 8;
    const int row = e / D, c0 = e % D;
    float v[8];
    load8(K + (size_t)row * D + c0, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) { sD[wave][row][c0 + t] = v[t]; en = fmaf(v[t], v[t], en); }
  }
  const float energy = group_sum<kWave>(en);
  wave_lds_fence();
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) {
    const int c = lane + kWave * x;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < B; ++i) s += sD[wave][i][c];
    const float mu = s * (1.0f / B);
    sMu[wave][c] = mu;
#pragma unroll
    for (int i = 0; i < B; ++i) sD[wave][i][c] -= mu;
  }
  wave_lds_fence();

  // 2) Gram on the matrix cores: A = B = rows of D (lane (col, kg), K-step t:
  //    dims 32 t + 8 kg .. +7), three bf16 terms per entry
  {
    const int col = lane & 15, kg = lane >> 4;
    bf16x8_t op[4][3];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t w[3][4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float x[2] = {sD[wave][col][32 * t + 8 * kg + 2 * p], sD[wave][col][32 * t + 8 * kg + 2 * p + 1]};
        uint32_t h[3][2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            const __bf16 v = (__bf16)x[e];
            h[q][e] = __builtin_bit_cast(uint16_t, v);
            x[e] -= (float)v;  // exact: the remainder of a bf16 rounding
          }
#pragma unroll
        for (int q = 0; q < 3; ++q) w[q][p] = h[q][0] | (h[q][1] << 16);
      }
#pragma unroll
      for (int q = 0; q < 3; ++q) op[t][q] = __builtin_bit_cast(bf16x8_t, make_uint4(w[q][0], w[q][1], w[q][2], w[q][3]));
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[t][0], op[t][0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[t][0], op[t][1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[t][1], op[t][0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[t][1], op[t][1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[t][0], op[t][2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[t][2], op[t][0], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * kg + i;
      if (r <= col) {
        sA[wave][0][r][col] = acc[i];
        sA[wave][0][col][r] = acc[i];
      }
    }
    // U = I
#pragma unroll
    for (int x = 0; x < B * B / kWave; ++x) {
      const int e = lane + kWave * x;
      sU[wave][0][e / B][e % B] = (e / B == e % B) ? 1.f : 0.f;
    }
  }
  wave_lds_fence();

  // 3) cyclic Jacobi.  Round t pairs index 15 with t and (t + m) mod 15 with
  //    (t - m) mod 15 for m = 1..7 (every pair once per 15 rounds).
  int cur = 0;
  for (int sweep = 0; sweep < 12; ++sweep) {
    float off = 0.f, tot = 0.f;
#pragma unroll
    for (int x = 0; x < B * B / kWave; ++x) {
      const int e = lane + kWave * x;
      const float v = sA[wave][cur][e / B][e % B];
      tot = fmaf(v, v, tot);
      if (e / B != e % B) off = fmaf(v, v, off);
    }
    off = group_sum<kWave>(off);
    tot = group_sum<kWave>(tot);
    if (!(off > 1e-13f * tot)) break;
    for (int t = 0; t < B - 1; ++t) {
      if (lane < B / 2) {  // the Schur rotation of pair m = lane
        const int m = lane;
        int p = m == 0 ? B - 1 : (t + m) % (B - 1);
        int q = m == 0 ? t : (t - m + (B - 1)) % (B - 1);
        if (p > q) { const int tmp = p; p = q; q = tmp; }
        const float app = sA[wave][cur][p][p], aqq = sA[wave][cur][q][q], apq = sA[wave][cur][p][q];
        float c = 1.f, s = 0.f, tt = 0.f;
        if (apq != 0.f) {
          const float tau = (aqq - app) / (2.f * apq);
          tt = (tau >= 0.f ? 1.f : -1.f) / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + tt * tt);
          s = tt * c;
        }
        // J = [[c, s], [-s, c]] on (p, q): column p is (c, -s), column q is (s, c)
        sRot[wave][p][0] = c; sRot[wave][p][1] = -s; sPart[wave][p] = q;
        sRot[wave][q][0] = c; sRot[wave][q][1] = s;  sPart[wave][q] = p;
        // the rotated pair's diagonal, in the exact form of the Schur rotation
        sA[wave][cur ^ 1][p][p] = app - tt * apq;
        sA[wave][cur ^ 1][q][q] = aqq + tt * apq;
      }
      wave_lds_fence();
      // A' = J^T A J (entry (a, b) with a <= b, mirrored), U' = U J
      const int nxt = cur ^ 1;
#pragma unroll
      for (int x = 0; x < B * B / kWave; ++x) {
        const int e = lane + kWave * x;
        const int i = e / B, j = e % B;
        const int ia = min(i, j), jb = max(i, j);
        const int pa = sPart[wave][ia], pb = sPart[wave][jb];
        const float ca = sRot[wave][ia][0], sa = sRot[wave][ia][1];
        const float cb = sRot[wave][jb][0], sb = sRot[wave][jb][1];
        float v;
        if (ia == jb) {
          v = sA[wave][nxt][ia][ia];  // set by the pair's lane above
        } else if (pa == jb) {
          v = 0.f;                    // the rotated pair
        } else {
          v = ca * cb * sA[wave][cur][ia][jb] + sa * cb * sA[wave][cur][pa][jb] +
              ca * sb * sA[wave][cur][ia][pb] + sa * sb * sA[wave][cur][pa][pb];
        }
        const float u = sU[wave][cur][i][j] * sRot[wave][j][0] + sU[wave][cur][i][sPart[wave][j]] * sRot[wave][j][1];
        sU[wave][nxt][i][j] = u;
        if (ia != jb) sA[wave][nxt][i][j] = v;
      }
      wave_lds_fence();
      cur = nxt;
    }
  }

  // 4) eigenvalues (diagonal), descending order by rank counting (ties to the
  //    lower index); the kept modes' indices
  __shared__ int sOrder[kB16Waves][B];
  __shared__ float sLam[kB16Waves][B];
  if (lane < B) {
    const float li = sA[wave][cur][lane][lane];
    int rank = 0;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const float lj = sA[wave][cur][j][j];
      rank += (lj > li || (lj == li && j < lane)) ? 1 : 0;
    }
    sOrder[wave][rank] = lane;
    sLam[wave][rank] = li;
  }
  wave_lds_fence();
  const float lam1 = sLam[wave][0];
  const float thresh = fmaxf(1e-5f * lam1, 1e-10f * energy);
  if (a.eigvals_out && lane < B) a.eigvals_out[((size_t)idx * a.hkv + kvh) * B + lane] = fmaxf(sLam[wave][lane], 0.f);

  // 5) basis V[k][c] = sum_i D[i][c] U[i][idx_k] / sigma_k, then signs
#pragma unroll
  for (int k = 0; k < KEPT; ++k) {
    const int ik = sOrder[wave][k];
    const bool nz = lam1 > 0.f && sLam[wave][k] > thresh;
    const float inv = nz ? 1.f / sqrtf(sLam[wave][k]) : 0.f;
#pragma unroll
    for (int x = 0; x < D / kWave; ++x) {
      const int c = lane + kWave * x;
      float v = 0.f;
#pragma unroll
      for (int i = 0; i < B; ++i) v = fmaf(sD[wave][i][c], sU[wave][cur][i][ik], v);
      sV[wave][k][c] = v * inv;
    }
  }
  wave_lds_fence();
#pragma unroll
  for (int k = 0; k < KEPT; ++k) {
    float best = -1.f, val = 0.f;
    int bidx = D;
#pragma unroll
    for (int x = 0; x < D / kWave; ++x) {
      const int c = lane + kWave * x;
      const float v = sV[wave][k][c];
      if (fabsf(v) > best || (fabsf(v) == best && c < bidx)) { best = fabsf(v); val = v; bidx = c; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float b2 = __shfl_xor(best, o);
      const float v2 = __shfl_xor(val, o);
      const int i2 = __shfl_xor(bidx, o);
      if (b2 > best || (b2 == best && i2 < bidx)) { best = b2; val = v2; bidx = i2; }
    }
    if (lane == 0) sSign[wave][k] = val < 0.f ? -1.f : 1.f;
  }
  wave_lds_fence();
  auto basis_at = [&](int k, int c) { return k < KEPT ? sV[wave][k][c] * sSign[wave][k] : 0.f; };
  auto coef_at = [&](int i, int k) -> float {
    if (k >= KEPT) return 0.f;
    const bool nz = lam1 > 0.f && sLam[wave][k] > thresh;
    return nz ? sU[wave][cur][i][sOrder[wave][k]] * sqrtf(sLam[wave][k]) * sSign[wave][k] : 0.f;
  };

  // 6) record
  if (!a.q4) {
    constexpr int REC = D + R * D + B * R;
    T* rec = reinterpret_cast<T*>(a.summary) + ((size_t)phys * a.hkv + kvh) * REC;
    for (int x = lane; x < REC; x += kWave) {
      float v;
      if (x < D) v = sMu[wave][x];
      else if (x < D + R * D) v = basis_at((x - D) / D, (x - D) % D);
      else v = coef_at((x - D - R * D) / R, (x - D - R * D) % R);
      Elem<T>::store(rec + x, v);
    }
    return;
  }
  // int4 basis / int8 coefficients and centroid (same rule as the 64-token builder)
  constexpr Q4Layout L{R, B};
  uint8_t* rec = reinterpret_cast<uint8_t*>(a.summary) + ((size_t)phys * a.hkv + kvh) * L.bytes();
  float bsc[R];
#pragma unroll
  for (int k = 0; k < R; ++k)
    bsc[k] = b16_q_scale(group_max<kWave>(fmaxf(fabsf(basis_at(k, lane)), fabsf(basis_at(k, lane + kWave)))), 7.f);
  const float msc = b16_q_scale(group_max<kWave>(fmaxf(fabsf(sMu[wave][lane]), fabsf(sMu[wave][lane + kWave]))), 127.f);
  float csc = 0.f;  // lane i < B: token i's coefficient scale
  if (lane < B) {
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) m = fmaxf(m, fabsf(coef_at(lane, k)));
    csc = b16_q_scale(m, 127.f);
  }
  for (int x = lane; x < D; x += kWave) rec[x] = (uint8_t)(int8_t)b16_q_code(sMu[wave][x], msc, 127.f);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int c = 2 * lane;  // D / 2 = 64 bytes per row: one per lane
    const int lo = b16_q_code(basis_at(k, c), bsc[k], 7.f), hi = b16_q_code(basis_at(k, c + 1), bsc[k], 7.f);
    rec[L.basis() + k * (D / 2) + lane] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
  }
  if (lane < B) {
#pragma unroll
    for (int k = 0; k < R; ++k) rec[L.coef() + lane * R + k] = (uint8_t)(int8_t)b16_q_code(coef_at(lane, k), csc, 127.f);
    reinterpret_cast<uint16_t*>(rec + L.cscale())[lane] = __builtin_bit_cast(uint16_t, (_Float16)csc);
  }
  if (lane < R) {
    float s = bsc[0];
#pragma unroll
    for (int k = 1; k < R; ++k)
      if (lane == k) s = bsc[k];
    reinterpret_cast<uint16_t*>(rec + L.bscale())[lane] = __builtin_bit_cast(uint16_t, (_Float16)s);
  }
  if (lane == 0) *reinterpret_cast<uint16_t*>(rec + L.mscale()) = __builtin_bit_cast(uint16_t, (_Float16)msc);
  for (int x = L.mscale() + 2 + lane; x < L.bytes(); x += kWave) rec[x] = 0;
}

template <typename T>
static hipError_t launch_build16_t(int rank, const BuildArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const long long items = (long long)a.n * a.hkv;
  dim3 grid((unsigned)((items + kB16Waves - 1) / kB16Waves));
  dim3 block(kB16Waves * kWave);
  switch (rank) {
    case 1: hipLaunchKernelGGL((build16_kernel<T, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((build16_kernel<T, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((build16_kernel<T, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((build16_kernel<T, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((build16_kernel<T, 16>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_build16(DType dt, int rank, const BuildArgs& a, hipStream_t s) {
  if (a.merge.part_o || a.commit_seq_lens) return hipErrorInvalidValue;  // bulk builds only
  return dt == kBF16 ? launch_build16_t<bf16_t>(rank, a, s) : launch_build16_t<float>(rank, a, s);
}

}  // namespace lk
