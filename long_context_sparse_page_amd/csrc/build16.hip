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
//
// The rounds are bound by LDS latency, so the wave keeps little else in LDS
// (about 6 KB: the 16 x 16 matrices, the centroid, a round's rotations) and
// many waves share a CU.  The key tile is read twice, both times straight
// into registers: in the matrix-core operand layout for the Gram (the
// centroid of a lane's dimensions is a sum over the 16 lanes of its DPP row,
// which hold those dimensions of the 16 tokens) and, from L2, with two
// dimensions per lane for the basis, which is formed, signed and written from
// registers.

#include "common.cuh"
#include "kernels.h"
#include "merge_impl.cuh"

namespace lk {

constexpr int kB16 = 16;
constexpr int kB16Waves = 4;
constexpr int kB16Ld = 17;  // padded row of the 16 x 16 matrices

__device__ __forceinline__ float b16_q_scale(float amax, float levels) { return (float)(_Float16)(amax / levels); }
__device__ __forceinline__ int b16_q_code(float x, float s, float levels) {
  if (!(s > 0.f)) return 0;
  return (int)fminf(fmaxf(rintf(x / s), -levels), levels);
}
// two consecutive elements
__device__ __forceinline__ void load2(const bf16_t* p, float& a, float& b) {
  const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
  a = bf16_lo(v);
  b = bf16_hi(v);
}
__device__ __forceinline__ void load2(const float* p, float& a, float& b) {
  const float2 v = *reinterpret_cast<const float2*>(p);
  a = v.x;
  b = v.y;
}

// DS: the decode step's launch (merge and length commit before the build);
// the bulk build is compiled without them (fewer registers, more waves).
template <typename T, int R, bool DS>
__global__ __launch_bounds__(kB16Waves * kWave) void build16_kernel(BuildArgs a) {
  constexpr int B = kB16;
  constexpr int D = kHeadDim;
  constexpr int KEPT = R < B ? R : B;
  __shared__ float sA[kB16Waves][2][B][kB16Ld];   // Gram / rotated matrix (ping-pong)
  __shared__ float sU[kB16Waves][2][B][kB16Ld];   // accumulated rotations
  __shared__ float sMu[kB16Waves][D];
  __shared__ float sRot[kB16Waves][B][2];         // per index: J[i][i], J[partner][i]
  __shared__ int sPart[kB16Waves][B];
  __shared__ int sOrder[kB16Waves][B];
  __shared__ float sLam[kB16Waves][B];
  __shared__ float sSign[kB16Waves][KEPT];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int item = blockIdx.x * kB16Waves + wave;  // (page, KV head) pair
  if (item >= a.n * a.hkv) return;
  const int idx = item / a.hkv, kvh = item % a.hkv;
  const int phys = a.phys_ids[idx];
  // decode step (idx = sequence): merge the attention partials of (idx, kvh),
  // then advance the sequence's length when its append was valid
  if constexpr (DS) {
    const bool commit = a.commit_seq_lens && kvh == 0 && lane == 0;
    const int len = commit ? a.commit_seq_lens[idx] : 0;
    if (a.merge.part_o) {
      switch (a.merge.group) {
        case 1: merge_partials_wave<T, 1>(a, idx, kvh, lane); break;
        case 2: merge_partials_wave<T, 2>(a, idx, kvh, lane); break;
        case 4: merge_partials_wave<T, 4>(a, idx, kvh, lane); break;
        default: merge_partials_wave<T, 8>(a, idx, kvh, lane); break;
      }
    }
    if (commit && phys != -2) a.commit_seq_lens[idx] = len + 1;
  }
  if (phys < 0 || phys >= a.num_phys) return;
  const T* K = reinterpret_cast<const T*>(a.k_pool) + (((size_t)phys * a.hkv + kvh) * B) * D;

  // 1) Gram operand layout: lane (row col, kg) holds dims 32 t + 8 kg .. +7 of
  //    row col for the K-steps t; the basis layout: dims 2 lane, 2 lane + 1 of
  //    every row (requested now, used after the eigensolver)
  const int col = lane & 15, kg = lane >> 4;
  float x[4][8];
#pragma unroll
  for (int t = 0; t < 4; ++t) load8(K + (size_t)col * D + 32 * t + 8 * kg, x[t]);
  float db[B][2];
#pragma unroll
  for (int i = 0; i < B; ++i) load2(K + (size_t)i * D + 2 * lane, db[i][0], db[i][1]);

  // energy sum_i ||k_i||^2; centroid (a sum over the 16 lanes of a DPP row);
  // centring
  float en = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) en = fmaf(x[t][e], x[t][e], en);
  const float energy = group_sum<kWave>(en);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float mu = group_sum<16>(x[t][e]) * (1.0f / B);
      if (col == 0) sMu[wave][32 * t + 8 * kg + e] = mu;
      x[t][e] -= mu;
    }

  // 2) Gram D D^T on the matrix cores: three bf16 terms per entry
  {
    bf16x8_t op[4][3];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t w[3][4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float v2[2] = {x[t][2 * p], x[t][2 * p + 1]};
        uint32_t h[3][2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            const __bf16 v = (__bf16)v2[e];
            h[q][e] = __builtin_bit_cast(uint16_t, v);
            v2[e] -= (float)v;  // exact: the remainder of a bf16 rounding
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
    for (int y = 0; y < B * B / kWave; ++y) {
      const int e = lane + kWave * y;
      sU[wave][0][e / B][e % B] = (e / B == e % B) ? 1.f : 0.f;
    }
  }
  wave_lds_fence();

  // 3) cyclic Jacobi.  Round t pairs index 15 with t and (t + m) mod 15 with
  //    (t - m) mod 15 for m = 1..7 (every pair once per 15 rounds).  The
  //    matrices alternate between two LDS buffers; lane l owns entries
  //    (l / 16 + 4 y, l % 16), y < 4, and their upper-triangle positions.
  constexpr int LD = kB16Ld;
  int cur = 0;
  const int m_pair = lane & 7;
  const int jl = lane & (B - 1);
  int ia[4], jb[4];
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int i = (lane >> 4) + 4 * y;
    ia[y] = min(i, jl);
    jb[y] = max(i, jl);
  }
  float* const Rw = &sRot[wave][0][0];  // [B][2]: J[i][i], J[partner][i]
  int* const Pw = &sPart[wave][0];
  for (int sweep = 0; sweep < 12; ++sweep) {
    const float* Ac0 = &sA[wave][cur][0][0];
    float off = 0.f, tot = 0.f;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int i = (lane >> 4) + 4 * y;
      const float v = Ac0[i * LD + jl];
      tot = fmaf(v, v, tot);
      if (i != jl) off = fmaf(v, v, off);
    }
    off = group_sum<kWave>(off);
    tot = group_sum<kWave>(tot);
    if (!(off > 1e-13f * tot)) break;
    for (int t = 0; t < B - 1; ++t) {
      const float* Ac = &sA[wave][cur][0][0];
      float* An = &sA[wave][cur ^ 1][0][0];
      const float* Uc = &sU[wave][cur][0][0];
      float* Un = &sU[wave][cur ^ 1][0][0];
      if (lane < B / 2) {  // the Schur rotation of pair m = lane
        // (t + m) mod 15 and (t - m) mod 15 with 0 <= t, m < 15, without a division
        const int tp = t + m_pair, tm = t - m_pair + (B - 1);
        const int r0 = m_pair == 0 ? B - 1 : (tp >= B - 1 ? tp - (B - 1) : tp);
        const int r1 = m_pair == 0 ? t : (tm >= B - 1 ? tm - (B - 1) : tm);
        const int p = min(r0, r1), q = max(r0, r1);
        const float app = Ac[p * LD + p], aqq = Ac[q * LD + q], apq = Ac[p * LD + q];
        float c = 1.f, s = 0.f, tt = 0.f;
        if (apq != 0.f) {
          // t = sign(tau) / (|tau| + sqrt(1 + tau^2)), c = 1 / sqrt(1 + t^2), s = t c;
          // any rotation orthogonal to rounding serves (the pair's entry is
          // then set to zero), so the single-instruction rcp / sqrt / rsq
          const float tau = (aqq - app) * __builtin_amdgcn_rcpf(2.f * apq);
          tt = (tau >= 0.f ? 1.f : -1.f) * __builtin_amdgcn_rcpf(fabsf(tau) + __builtin_amdgcn_sqrtf(fmaf(tau, tau, 1.f)));
          c = __builtin_amdgcn_rsqf(fmaf(tt, tt, 1.f));
          s = tt * c;
        }
        // J = [[c, s], [-s, c]] on (p, q): column p is (c, -s), column q is (s, c)
        Rw[2 * p] = c; Rw[2 * p + 1] = -s; Pw[p] = q;
        Rw[2 * q] = c; Rw[2 * q + 1] = s;  Pw[q] = p;
        // the rotated pair's diagonal, in the exact form of the Schur rotation
        An[p * LD + p] = app - tt * apq;
        An[q * LD + q] = aqq + tt * apq;
      }
      wave_lds_fence();
      // A' = J^T A J (entry (a, b) from the upper triangle a <= b; the
      // diagonal was set above, the rotated pair's entry is zero), U' = U J;
      // every index read is in 0 .. 15, so the reads are unconditional
      const int pj = Pw[jl];
      const float cj = Rw[2 * jl], sj = Rw[2 * jl + 1];
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int i = (lane >> 4) + 4 * y;
        const int pa = Pw[ia[y]], pb = Pw[jb[y]];
        const float ca = Rw[2 * ia[y]], sa = Rw[2 * ia[y] + 1];
        const float cb = Rw[2 * jb[y]], sb = Rw[2 * jb[y] + 1];
        const float v = ca * cb * Ac[ia[y] * LD + jb[y]] + sa * cb * Ac[pa * LD + jb[y]] +
                        ca * sb * Ac[ia[y] * LD + pb] + sa * sb * Ac[pa * LD + pb];
        // one basic block for all four entries (their LDS reads overlap): the
        // diagonal entry is stored again with the value the pair's lane set
        const float dg = An[i * LD + jl];
        An[i * LD + jl] = i == jl ? dg : (pa == jb[y] ? 0.f : v);
        Un[i * LD + jl] = Uc[i * LD + jl] * cj + Uc[i * LD + pj] * sj;
      }
      wave_lds_fence();
      cur ^= 1;
    }
  }

  // 4) eigenvalues (diagonal), descending order by rank counting (ties to the
  //    lower index)
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
  const float thresh = fmaxf(kZeroModeRtol * lam1, kZeroModeFloor * energy);
  if (a.eigvals_out && lane < B) a.eigvals_out[((size_t)idx * a.hkv + kvh) * B + lane] = fmaxf(sLam[wave][lane], 0.f);

  // 5) basis rows V[k][c] = sum_i D[i][c] U[i][idx_k] / sigma_k for this lane's
  //    dims c = 2 lane, 2 lane + 1, then the signs (largest |entry| positive,
  //    ties to the lower dim)
  const float mu0 = sMu[wave][2 * lane], mu1 = sMu[wave][2 * lane + 1];
#pragma unroll
  for (int i = 0; i < B; ++i) { db[i][0] -= mu0; db[i][1] -= mu1; }
  float vb[KEPT][2];
#pragma unroll
  for (int k = 0; k < KEPT; ++k) {
    const int ik = sOrder[wave][k];
    const bool nz = lam1 > 0.f && sLam[wave][k] > thresh;
    const float inv = nz ? 1.f / sqrtf(sLam[wave][k]) : 0.f;
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const float uik = sU[wave][cur][i][ik];
      v0 = fmaf(db[i][0], uik, v0);
      v1 = fmaf(db[i][1], uik, v1);
    }
    v0 *= inv;
    v1 *= inv;
    // this lane's candidate: the larger |entry| of its two dims (ties: the lower)
    float best = fabsf(v0), val = v0;
    int bidx = 2 * lane;
    if (fabsf(v1) > best) { best = fabsf(v1); val = v1; bidx = 2 * lane + 1; }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float b2 = __shfl_xor(best, o);
      const float v2 = __shfl_xor(val, o);
      const int i2 = __shfl_xor(bidx, o);
      if (b2 > best || (b2 == best && i2 < bidx)) { best = b2; val = v2; bidx = i2; }
    }
    const float sg = val < 0.f ? -1.f : 1.f;
    vb[k][0] = v0 * sg;
    vb[k][1] = v1 * sg;
    if (lane == 0) sSign[wave][k] = sg;
  }
  wave_lds_fence();
  auto coef_at = [&](int i, int k) -> float {
    if (k >= KEPT) return 0.f;
    const bool nz = lam1 > 0.f && sLam[wave][k] > thresh;
    return nz ? sU[wave][cur][i][sOrder[wave][k]] * sqrtf(sLam[wave][k]) * sSign[wave][k] : 0.f;
  };

  // 6) record
  if (!a.q4) {
    constexpr int REC = D + R * D + B * R;
    T* rec = reinterpret_cast<T*>(a.summary) + ((size_t)phys * a.hkv + kvh) * REC;
    Elem<T>::store(rec + 2 * lane, mu0);
    Elem<T>::store(rec + 2 * lane + 1, mu1);
#pragma unroll
    for (int k = 0; k < R; ++k) {
      Elem<T>::store(rec + D + k * D + 2 * lane, k < KEPT ? vb[k][0] : 0.f);
      Elem<T>::store(rec + D + k * D + 2 * lane + 1, k < KEPT ? vb[k][1] : 0.f);
    }
    for (int y = lane; y < B * R; y += kWave) Elem<T>::store(rec + D + R * D + y, coef_at(y / R, y % R));
    return;
  }
  // int4 basis / int8 coefficients and centroid (the 64-token builder's rule)
  constexpr Q4Layout L{R, B};
  uint8_t* rec = reinterpret_cast<uint8_t*>(a.summary) + ((size_t)phys * a.hkv + kvh) * L.bytes();
  const float msc = b16_q_scale(group_max<kWave>(fmaxf(fabsf(mu0), fabsf(mu1))), 127.f);
  rec[2 * lane] = (uint8_t)(int8_t)b16_q_code(mu0, msc, 127.f);
  rec[2 * lane + 1] = (uint8_t)(int8_t)b16_q_code(mu1, msc, 127.f);
  float bsc_lane = 0.f;  // lane k < R: basis row k's scale
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const float v0 = k < KEPT ? vb[k][0] : 0.f, v1 = k < KEPT ? vb[k][1] : 0.f;
    const float bs = b16_q_scale(group_max<kWave>(fmaxf(fabsf(v0), fabsf(v1))), 7.f);
    const int lo = b16_q_code(v0, bs, 7.f), hi = b16_q_code(v1, bs, 7.f);
    rec[L.basis() + k * (D / 2) + lane] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
    if (lane == k) bsc_lane = bs;
  }
  if (lane < B) {
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) m = fmaxf(m, fabsf(coef_at(lane, k)));
    const float csc = b16_q_scale(m, 127.f);
#pragma unroll
    for (int k = 0; k < R; ++k) rec[L.coef() + lane * R + k] = (uint8_t)(int8_t)b16_q_code(coef_at(lane, k), csc, 127.f);
    reinterpret_cast<uint16_t*>(rec + L.cscale())[lane] = __builtin_bit_cast(uint16_t, (_Float16)csc);
  }
  if (lane < R) reinterpret_cast<uint16_t*>(rec + L.bscale())[lane] = __builtin_bit_cast(uint16_t, (_Float16)bsc_lane);
  if (lane == 0) *reinterpret_cast<uint16_t*>(rec + L.mscale()) = __builtin_bit_cast(uint16_t, (_Float16)msc);
  for (int y = L.mscale() + 2 + lane; y < L.bytes(); y += kWave) rec[y] = 0;
}

template <typename T, int R>
static void launch_b16(bool ds, dim3 grid, dim3 block, hipStream_t s, const BuildArgs& a) {
  if (ds) hipLaunchKernelGGL((build16_kernel<T, R, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((build16_kernel<T, R, false>), grid, block, 0, s, a);
}

template <typename T>
static hipError_t launch_build16_t(int rank, const BuildArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const long long items = (long long)a.n * a.hkv;
  dim3 grid((unsigned)((items + kB16Waves - 1) / kB16Waves));
  const bool ds = a.merge.part_o != nullptr || a.commit_seq_lens != nullptr;
  dim3 block(kB16Waves * kWave);
  switch (rank) {
    case 1: launch_b16<T, 1>(ds, grid, block, s, a); break;
    case 2: launch_b16<T, 2>(ds, grid, block, s, a); break;
    case 4: launch_b16<T, 4>(ds, grid, block, s, a); break;
    case 8: launch_b16<T, 8>(ds, grid, block, s, a); break;
    case 16: launch_b16<T, 16>(ds, grid, block, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_build16(DType dt, int rank, const BuildArgs& a, hipStream_t s) {
  return dt == kBF16 ? launch_build16_t<bf16_t>(rank, a, s) : launch_build16_t<float>(rank, a, s);
}

}  // namespace lk
