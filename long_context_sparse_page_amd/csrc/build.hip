// Page summary builder: one workgroup of 256 threads per (page, KV head).
//
// [Locks] §4 "Build (once, when a page completes)": centre the page,
// k_i = mu + delta_i; stack the deviations as rows of D (B x d); eigendecompose
// the B x B Gram D D^T = U Sigma^2 U^T with eigenvalues descending; keep r
// components, C = U_r Sigma_r (coefficients c_i = rows of C) and the
// orthonormal basis V = D^T U_r Sigma_r^{-1}; zero modes are dropped with
// zero coefficients.
//
// Only the top r eigenpairs of the Gram are needed, so the symmetric
// eigenproblem is solved the way one computes a few eigenpairs of a dense
// symmetric matrix (Golub & Van Loan, Matrix Computations, ch. 8):
//   1. Householder reduction to tridiagonal form T = Q^T A Q (62 reflections;
//      reflector k is kept as row k of the LDS copy of A);
//   2. the r largest eigenvalues of T by Sturm-sequence multisection (a
//      wave's eigenvalues at once on lane segments: each lane counts the
//      eigenvalues below its own shift, so an interval shrinks (SL + 1)-fold
//      per pass with SL lanes per eigenvalue);
//   3. their eigenvectors of T by inverse iteration with partial pivoting,
//      re-orthogonalized within clusters of close eigenvalues;
//   4. back-transformation by the reflectors.
// All B eigenvalues (for the optional eigenvalue output) are found by plain
// bisection, one lane per eigenvalue.  The K tile takes no LDS: it is read
// from global memory (then L2) where it is needed, for the centroid, as the
// Gram's operands and for the basis, and centred in registers; the Gram D D^T
// runs on the matrix cores with each fp32 entry split into three bf16 terms.
//
// Zero-mode rule: eigenvalue <= 1e-5 * lambda_1 or <= 1e-10 * sum_i ||k_i||^2.
// Sign rule: each basis vector's largest-magnitude entry is made positive.

#include "common.cuh"
#include "kernels.h"
#include "merge_impl.cuh"

namespace lk {

constexpr int kBuildThreads = 256;
constexpr int kMergeThreads = 512;      // decode-step launch: one merged output per thread for G <= 4
constexpr int kBuildWaves = kBuildThreads / kWave;
constexpr int kInvIters = 2;         // inverse-iteration passes per eigenvector
constexpr float kClusterTol = 1e-3f; // eigenvalues this close (relative to lambda_1) are re-orthogonalized

// Number of eigenvalues of the symmetric tridiagonal (d, e) below sigma: the
// negative pivots of the LDL^T factorization of T - sigma I (Sturm count).
// e2[i] = e[i]^2; pivots smaller than pivmin are replaced by -pivmin.
__device__ __forceinline__ int sturm_count(const float* sd, const float* se2, float sigma, float pivmin) {
  constexpr int B = 64;
  float q = sd[0] - sigma;
  if (fabsf(q) < pivmin) q = -pivmin;
  int c = q < 0.f ? 1 : 0;
#pragma unroll 8
  for (int i = 1; i < B; ++i) {
    q = (sd[i] - sigma) - se2[i - 1] * __builtin_amdgcn_rcpf(q);
    if (fabsf(q) < pivmin) q = -pivmin;
    c += q < 0.f ? 1 : 0;
  }
  return c;
}
// The same count with T in registers (every lane holds all of d and e^2).
__device__ __forceinline__ int sturm_count_reg(const float (&d)[64], const float (&e2)[64], float sigma, float pivmin) {
  float q = d[0] - sigma;
  if (fabsf(q) < pivmin) q = -pivmin;
  int c = q < 0.f ? 1 : 0;
#pragma unroll
  for (int i = 1; i < 64; ++i) {
    q = (d[i] - sigma) - e2[i - 1] * __builtin_amdgcn_rcpf(q);
    if (fabsf(q) < pivmin) q = -pivmin;
    c += q < 0.f ? 1 : 0;
  }
  return c;
}

// Quantized record (Q4Layout): symmetric absmax quantization per row, the
// scale rounded to fp16 and the codes taken against that stored scale,
// rounding half to even: s = fp16(max |x| / L), code = clamp(rint(x / s), -L, L)
// with L = 7 for the basis (one scale per basis vector) and L = 127 for the
// centroid and for each token's coefficients; an all-zero row has s = 0.
__device__ __forceinline__ float q4_scale(float amax, float levels) {
  return (float)(_Float16)(amax / levels);
}
__device__ __forceinline__ int q4_code(float x, float s, float levels) {
  if (!(s > 0.f)) return 0;
  return (int)fminf(fmaxf(rintf(x / s), -levels), levels);
}

// The final record values: centroid sMu[c]; basis row k < KEPT is
// sV[k][c] * sSign[k]; coefficient (i, k) is sZ[i][k] * sigma_k * sign_k on
// nonzero modes.  Runs on the builder's kBuildThreads threads.
template <int R, int KEPT>
__device__ __forceinline__ void write_q4_record(const BuildArgs& a, int phys, int kvh, const float* sMu,
                                                const float* sV, const float* sSign, const float* sZ,
                                                const float* sSigma, const int* sNz) {
  constexpr int D = kHeadDim;
  constexpr int B = 64;
  constexpr Q4Layout L{R};
  __shared__ float sBs[R], sCs[B], sMs;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  auto basis_at = [&](int k, int c) { return k < KEPT ? sV[k * D + c] * sSign[k] : 0.f; };
  auto coef_at = [&](int i, int k) { return (k < KEPT && sNz[k]) ? sZ[i * KEPT + k] * sSigma[k] * sSign[k] : 0.f; };
  // scales: basis rows by waves (two dims per lane), the centroid by wave 0,
  // each token's coefficients by one thread
  for (int k = wave; k < R; k += kBuildWaves) {
    const float m = group_max<kWave>(fmaxf(fabsf(basis_at(k, lane)), fabsf(basis_at(k, lane + kWave))));
    if (lane == 0) sBs[k] = q4_scale(m, 7.f);
  }
  if (wave == 0) {
    const float m = group_max<kWave>(fmaxf(fabsf(sMu[lane]), fabsf(sMu[lane + kWave])));
    if (lane == 0) sMs = q4_scale(m, 127.f);
  }
  if (tid < B) {
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) m = fmaxf(m, fabsf(coef_at(tid, k)));
    sCs[tid] = q4_scale(m, 127.f);
  }
  __syncthreads();
  uint8_t* rec = reinterpret_cast<uint8_t*>(a.summary) + ((size_t)phys * a.hkv + kvh) * L.bytes();
  for (int x = tid; x < D; x += kBuildThreads) rec[x] = (uint8_t)(int8_t)q4_code(sMu[x], sMs, 127.f);
  // basis byte 4 g + b of a row holds dims 8 g + e and 8 g + e + 2 with
  // e = 4 (b & 1) + (b >> 1): even dims in the low half-word, odd dims in the high
  for (int x = tid; x < R * D / 2; x += kBuildThreads) {
    const int k = x / (D / 2), p = x % (D / 2);
    const int c = 8 * (p >> 2) + 4 * (p & 1) + ((p >> 1) & 1);
    const int lo = q4_code(basis_at(k, c), sBs[k], 7.f), hi = q4_code(basis_at(k, c + 2), sBs[k], 7.f);
    rec[L.basis() + x] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
  }
  for (int x = tid; x < B * R; x += kBuildThreads)
    rec[L.coef() + x] = (uint8_t)(int8_t)q4_code(coef_at(x / R, x % R), sCs[x / R], 127.f);
  uint16_t* cs = reinterpret_cast<uint16_t*>(rec + L.cscale());
  uint16_t* bs = reinterpret_cast<uint16_t*>(rec + L.bscale());
  if (tid < B) cs[tid] = __builtin_bit_cast(uint16_t, (_Float16)sCs[tid]);
  if (tid < R) bs[tid] = __builtin_bit_cast(uint16_t, (_Float16)sBs[tid]);
  if (tid == 0) *reinterpret_cast<uint16_t*>(rec + L.mscale()) = __builtin_bit_cast(uint16_t, (_Float16)sMs);
  for (int x = L.mscale() + 2 + tid; x < L.bytes(); x += kBuildThreads) rec[x] = 0;
}

template <typename T, int R>
__global__ __launch_bounds__(kMergeThreads) __attribute__((amdgpu_waves_per_eu(3))) void build_kernel(BuildArgs a) {
  constexpr int B = 64;
  constexpr int D = kHeadDim;
  constexpr int KEPT = R < B ? R : B;
  constexpr int KW = (KEPT + kBuildWaves - 1) / kBuildWaves;  // eigenvectors per wave
  constexpr int LA = B + 4;                // 16-byte aligned rows
  static_assert(KEPT <= 16, "rank above 16");

  __shared__ float sHalf[2][D];            // column sums of K over rows 0..31 and 32..63
  __shared__ __attribute__((aligned(16))) float sA[B + 1][LA];  // Gram; then reflector k in row k (zero in columns <= k); later the basis
  __shared__ float sMu[D];
  __shared__ float sd[B], se[B], se2[B];   // tridiagonal T (e[i] couples i, i + 1)
  __shared__ float sp4[2][kBuildWaves][B]; // partial sums of A u, one row per wave (by step parity)
  __shared__ float scol[2][B];             // the column after next, published by its owner
  __shared__ float sRed[kBuildWaves];
  __shared__ float sLam[KEPT];             // top eigenvalues, descending
  __shared__ float sZ[B][KEPT];            // eigenvectors (of T, then of A)
  __shared__ float4 sF[B][KEPT];           // inverse-iteration factors, one float4 per row
  __shared__ float sSigma[KEPT], sSign[KEPT];
  __shared__ int sNz[KEPT];
  __shared__ float sBound[2];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int idx = blockIdx.x;
  const int kvh = blockIdx.y;
  // loaded before the merge's loads and stores, which the compiler may not
  // move them across
  const int phys = a.phys_ids[idx];
  const bool commit = a.commit_seq_lens && kvh == 0 && tid == 0;
  const int len = commit ? a.commit_seq_lens[idx] : 0;
  if (a.merge.part_o) merge_partials<T>(a, idx, kvh, threadIdx.x, blockDim.x);
  // decode step: the append of sequence idx was valid -> advance its length
  if (commit && phys != -2) a.commit_seq_lens[idx] = len + 1;
  // The decode step launches kMergeThreads threads for the merge; the build
  // below runs on the first kBuildThreads (a barrier waits only for waves
  // that have not ended).
  if (tid >= kBuildThreads) return;
  if (phys < 0 || phys >= a.num_phys) return;

  // 1) centroid and energy sum ||k_i||^2 straight from the K tile: thread
  //    (column c, half h) sums rows 32 h .. 32 h + 31 of column c (the tile is
  //    read again from L2 where D is needed, so it takes no LDS)
  const T* K = reinterpret_cast<const T*>(a.k_pool) + (((size_t)phys * a.hkv + kvh) * B) * D;
  {
    const int c = tid & (D - 1), h = tid >> 7;
    float sum = 0.f, en = 0.f;
#pragma unroll 8
    for (int i = 0; i < B / 2; ++i) {
      const float v = Elem<T>::load(K + (size_t)(32 * h + i) * D + c);
      sum += v;
      en = fmaf(v, v, en);
    }
    sHalf[h][c] = sum;
    en = group_sum<kWave>(en);
    if (lane == 0) sRed[wave] = en;
  }
  __syncthreads();
  float energy = 0.f;
#pragma unroll
  for (int w = 0; w < kBuildWaves; ++w) energy += sRed[w];
  if (tid < D) sMu[tid] = (sHalf[0][tid] + sHalf[1][tid]) * (1.0f / B);
  __syncthreads();

  // 2) Gram A = D D^T on the matrix cores (v_mfma_f32_16x16x32_bf16): each
  //    fp32 entry of D is the sum of three bf16 terms d1 + d2 + d3 (each the
  //    bf16 rounding of what the previous ones leave), and the six products
  //    d_a d_b^T with a + b <= 4 are accumulated in fp32 (the dropped ones lie
  //    below fp32 rounding).  Wave w computes the 16 x 16 tiles (w, J) for
  //    J >= w and writes them with their mirror images (on diagonal tiles the
  //    entries with row <= col), so the Gram is exactly symmetric.  The rows
  //    come straight from the K tile (L2), centred with the centroid.
  {
    const int col = lane & 15, kg = lane >> 4;
    // operand of K-step t from K's dims 32 t + 8 kg .. +7 of one row: the
    // centred values as three bf16 terms
    auto split_operand = [&](const float (&k8)[8], int t, bf16x8_t (&o)[3]) {
      uint32_t w[3][4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int c = 32 * t + 8 * kg + 2 * p;
        float x[2] = {k8[2 * p] - sMu[c], k8[2 * p + 1] - sMu[c + 1]};
        uint32_t h[3][2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            const __bf16 v = (__bf16)x[e];
            h[q][e] = __builtin_bit_cast(uint16_t, v);
            x[e] -= (float)v;  // exact: the remainder of a bf16 rounding
          }
        }
#pragma unroll
        for (int q = 0; q < 3; ++q) w[q][p] = h[q][0] | (h[q][1] << 16);
      }
#pragma unroll
      for (int q = 0; q < 3; ++q) o[q] = __builtin_bit_cast(bf16x8_t, make_uint4(w[q][0], w[q][1], w[q][2], w[q][3]));
    };
    bf16x8_t ar[4][3];
    {
      float k8[4][8];
#pragma unroll
      for (int t = 0; t < 4; ++t) load8(K + (size_t)(16 * wave + col) * D + 32 * t + 8 * kg, k8[t]);
#pragma unroll
      for (int t = 0; t < 4; ++t) split_operand(k8[t], t, ar[t]);
    }
    for (int J = wave; J < 4; ++J) {
      float k8[4][8];
#pragma unroll
      for (int t = 0; t < 4; ++t) load8(K + (size_t)(16 * J + col) * D + 32 * t + 8 * kg, k8[t]);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x8_t br[3];
        split_operand(k8[t], t, br);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[t][0], br[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[t][0], br[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[t][1], br[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[t][1], br[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[t][0], br[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[t][2], br[0], acc, 0, 0, 0);
      }
      // lane holds rows 16 w + 4 kg + i, column 16 J + col
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * kg + i, c = 16 * J + col;
        if (wave < J || r <= c) {
          sA[r][c] = acc[i];
          sA[c][r] = acc[i];
        }
      }
    }
  }
  __syncthreads();

  // 3) Householder tridiagonalization with A in registers: wave q keeps
  //    columns 16 q .. 16 q + 15 of every row (lane = row).  Step k zeroes
  //    column k below the subdiagonal with H = I - 2 u u^T (||u|| = 1, u_r = 0
  //    for r <= k; u is also stored as row k of sA for the back-transformation).  With p = 2 A u (the sum of the four waves'
  //    partial sums), K = u.p and w = p - K u (rows > k), every wave applies
  //    A <- A - u w^T - w u^T to its own columns.  One barrier per step: at
  //    it the waves exchange their partial sums of p and the owner of column
  //    k + 2 publishes that column; every wave then brings its copy of the
  //    next column up to date itself and forms the next reflector from it
  //    (the same arithmetic in every wave), so the next products start
  //    without a second barrier.  LDS buffers alternate by step parity.
  const int q0 = 16 * wave;  // first column of this wave
  // wave 0, as a per-lane predicate: its stores below are exec-masked rather
  // than branched around, so the step body stays one basic block
  const bool wave0 = tid < kWave;
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  f32x16_t Ar;  // a vector, so that the uniform column index below stays in registers
#pragma unroll
  for (int t = 0; t < 16; ++t) Ar[t] = sA[lane][q0 + t];
  float colnext = sA[lane][1];  // column k + 1 as of the start of step k
  float ur;                     // u_k of this row
  {
    const float x = sA[lane][0];
    __syncthreads();  // every wave has read the Gram columns that the reflectors overwrite
    // reflector of column k from x = A[lane][k] (zero for lane <= k), formed
    // by every wave with selects only (a zero column gives u = 0, alpha = 0)
    auto reflector = [&](int k, float xk, float& alpha) {
      const float nrm2 = group_sum<kWave>(xk * xk);
      const float x0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xk), k + 1));
      const float nrm = __builtin_amdgcn_sqrtf(nrm2);
      const bool nz = nrm2 > 0.f;
      alpha = nz ? (x0 >= 0.f ? -nrm : nrm) : 0.f;
      const float inv = __builtin_amdgcn_rsqf(2.f * (nrm2 + nrm * fabsf(x0)));  // 1 / ||x - alpha e_{k+1}||
      return nz ? (lane == k + 1 ? xk - alpha : xk) * inv : 0.f;
    };
    // wave 0 keeps reflector k as row k of sA (zero in columns <= k) and the
    // subdiagonal entry alpha
    auto keep = [&](int k, float u, float alpha) {
      if (wave0) {
        sA[k][lane] = u;
        if (lane == 0) se[k] = alpha;
      }
    };
    if (wave0 && lane == 0) sd[0] = x;
    if (wave0) scol[0][lane] = colnext;  // column 1, read by every wave at step 0
    {
      float alpha;
      ur = reflector(0, lane > 0 ? x : 0.f, alpha);
      keep(0, ur, alpha);
    }
    float uj[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) uj[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ur), q0 + t));
    float pp = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) pp = fmaf(Ar[t], uj[t], pp);
    sp4[0][wave][lane] = pp;
    __syncthreads();
    // p = 2 A u_k, K = u_k.p and w = p - K u_k (zero in rows <= k)
    auto step_w = [&](int k) {
      const int buf = k & 1;
      const float p = 2.f * ((sp4[buf][0][lane] + sp4[buf][1][lane]) + (sp4[buf][2][lane] + sp4[buf][3][lane]));
      const float Kup = group_sum<kWave>(ur * p);
      return lane > k ? p - Kup * ur : 0.f;
    };
    // A <- A - u w^T - w u^T on this wave's columns.  Columns at or left of k
    // take exact zero updates (u_k and w vanish in rows <= k), so every wave
    // runs it unguarded.
    auto update = [&](float wr) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wr), q0 + t));
        Ar[t] = fmaf(-wr, uj[t], fmaf(-ur, wj, Ar[t]));
      }
    };
    // Steps 0 .. B - 4 also form the next reflector; the body has no branch
    // before the barrier's stores, so the column updates can be scheduled
    // into the latency of the reflector's reduction.
    for (int k = 0; k < B - 3; ++k) {
      const int buf = k & 1;
      const float wr = step_w(k);
      const int c = k + 1;
      // the next reflector first: column c, brought up to date with this
      // step, gives u_c (independent of this wave's own column updates)
      colnext = scol[buf][lane];
      const float uc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ur), c));
      const float wc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wr), c));
      colnext = colnext - (ur * wc + wr * uc);
      if (wave0 && lane == c) sd[c] = colnext;
      float alpha;
      const float un = reflector(c, lane > c ? colnext : 0.f, alpha);
      update(wr);
      ur = un;
#pragma unroll
      for (int t = 0; t < 16; ++t) uj[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ur), q0 + t));
      // columns <= c meet u_c's zeros: their terms are exact zeros
      float pq[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains
#pragma unroll
      for (int t = 0; t < 16; ++t) pq[t & 3] = fmaf(Ar[t], uj[t], pq[t & 3]);
      sp4[buf ^ 1][wave][lane] = (pq[0] + pq[1]) + (pq[2] + pq[3]);
      keep(c, ur, alpha);
      if (c + 1 < B - 2 && wave == (c + 1) / 16) scol[buf ^ 1][lane] = Ar[c + 1 - q0];  // column c + 1, for the next step
      __syncthreads();
    }
    update(step_w(B - 3));  // the last reflector u_{B-3}: update only
  }
  if (wave == kBuildWaves - 1) {  // the last 2 x 2 block (columns 62, 63)
    const float a62 = Ar[14], a63 = Ar[15];
    if (lane == B - 2) sd[B - 2] = a62;
    if (lane == B - 1) { sd[B - 1] = a63; se[B - 2] = a62; se[B - 1] = 0.f; }
  }
  __syncthreads();
  if (tid < B) se2[tid] = se[tid] * se[tid];
  // Gershgorin interval of T
  if (wave == 0) {
    const float em = lane > 0 ? fabsf(se[lane - 1]) : 0.f;
    const float ep = fabsf(se[lane]);
    float lo = sd[lane] - em - ep, hi = sd[lane] + em + ep;
    lo = -group_max<kWave>(-lo);
    hi = group_max<kWave>(hi);
    if (lane == 0) { sBound[0] = lo; sBound[1] = hi; }
  }
  __syncthreads();
  const float glo = sBound[0], ghi = sBound[1];
  const float tnorm = fmaxf(fabsf(glo), fabsf(ghi));
  const float pivmin = fmaxf(tnorm * 1e-30f, 1e-30f);
  const float tol = 2.f * 1.19209290e-7f * tnorm;

  // 4) the KEPT largest eigenvalues: wave w takes the w-th, (w+4)-th, ...
  //    (KW of them) at once, each on its own segment of SL = 64 / KW lanes;
  //    a pass counts the eigenvalues below SL shifts spread over the
  //    segment's interval, which shrinks (SL + 1)-fold.  T is read into
  //    registers once.
  {
    float dreg[B], e2reg[B];
#pragma unroll
    for (int i = 0; i < B; ++i) { dreg[i] = sd[i]; e2reg[i] = se2[i]; }
    constexpr int SL = kWave / KW;
    const int seg = lane / SL, sl = lane % SL;
    const int kk = wave + kBuildWaves * seg;
    const int target = B - 1 - kk;          // ascending index of the kk-th largest
    const uint64_t segmask = SL == kWave ? ~0ull : (((1ull << SL) - 1ull) << (seg * SL));
    float lo = glo, hi = ghi;
    bool more = kk < KEPT;
    for (int it = 0; it < 16; ++it) {
      more = more && hi - lo > tol;
      if (!__ballot(more)) break;
      const float width = hi - lo;
      const float sig = lo + width * (float)(sl + 1) * (1.f / (float)(SL + 1));
      const int cnt = sturm_count_reg(dreg, e2reg, sig, pivmin);
      const uint64_t below = __ballot(cnt <= target) & segmask;      // shifts at or below the eigenvalue
      const int nl = below ? 64 - __clzll(below) - seg * SL : 0;      // highest such lane of the segment + 1
      const float nlo = nl > 0 ? lo + width * (float)nl * (1.f / (float)(SL + 1)) : lo;
      const float nhi = nl < SL ? lo + width * (float)(nl + 1) * (1.f / (float)(SL + 1)) : hi;
      if (nlo == lo && nhi == hi) more = false;  // below the resolution of fp32
      if (more) { lo = nlo; hi = nhi; }
    }
    if (kk < KEPT && sl == 0) sLam[kk] = 0.5f * (lo + hi);
  }
  __syncthreads();

  // 5) inverse iteration on T: lane kk of wave 0 factors T - lambda_kk I once
  //    with partial pivoting (row i swaps with row i + 1 when |e_i| > |pivot|),
  //    then solves kInvIters times from a fixed varied start.  Without
  //    branches: the right-hand side and the swap flags stay in registers,
  //    and row i of the factors is one float4 in LDS (reciprocal pivot, the
  //    two entries right of the pivot, multiplier).
  if (wave == 0 && lane < KEPT) {
    const int kk = lane;
    const float lam = sLam[kk];
    uint64_t swm = 0ull;  // bit i: rows i and i + 1 swapped
    {
      // T in registers first, so the factorization's dependent chain waits
      // on no LDS read (its factor stores would otherwise hold each read up)
      float dT[B], eT[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        dT[i] = sd[i];
        eT[i] = se[i];
      }
      float ddc = dT[0] - lam, duc = eT[0];
#pragma unroll
      for (int i = 0; i < B - 1; ++i) {
        const float dl = eT[i];
        const float ddn = dT[i + 1] - lam;
        const float dun = i + 1 < B - 1 ? eT[i + 1] : 0.f;
        // both pivot choices are carried through and the row with the larger
        // pivot is selected at the end (a discarded choice may be inf/NaN):
        // the dependent chain per row is clamp, reciprocal, product, select
        const bool keep = fabsf(ddc) >= fabsf(dl);
        const float rk = __builtin_amdgcn_rcpf(fabsf(ddc) < pivmin ? pivmin : ddc);
        const float rs = __builtin_amdgcn_rcpf(dl);
        const float mk = dl * rk, ms = ddc * rs;
        const float nk = ddn - mk * duc, ns = duc - ms * ddn;
        sF[i][kk] = make_float4(keep ? rk : rs, keep ? duc : ddn, keep ? 0.f : dun, keep ? mk : ms);
        if (!keep) swm |= 1ull << i;
        duc = keep ? dun : -ms * dun;
        ddc = keep ? nk : ns;
      }
      sF[B - 1][kk] = make_float4(__builtin_amdgcn_rcpf(fabsf(ddc) < pivmin ? pivmin : ddc), 0.f, 0.f, 0.f);
    }
    float z[B];
    float nrm2 = 0.f;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const uint32_t hsh = (uint32_t)(i * 2654435761u) ^ (uint32_t)((kk + 1) * 40503u);
      z[i] = 0.5f + (float)((hsh >> 9) & 1023) * (1.f / 1024.f);
      nrm2 = fmaf(z[i], z[i], nrm2);
    }
    float scale = __builtin_amdgcn_rsqf(nrm2);
    for (int itr = 0; itr < kInvIters; ++itr) {
      // forward: the row swaps and multipliers applied to the right-hand side
      // (the multipliers are read first, so no LDS read waits inside the chain)
      float mw[B - 1];
#pragma unroll
      for (int i = 0; i < B - 1; ++i) mw[i] = sF[i][kk].w;
      float zc = z[0] * scale;
#pragma unroll
      for (int i = 0; i < B - 1; ++i) {
        const float zn = z[i + 1] * scale;
        const float mlt = mw[i];
        const bool sw = (swm >> i) & 1ull;
        z[i] = sw ? zn : zc;
        zc = sw ? zc - mlt * zn : zn - mlt * zc;
      }
      // back substitution, in place
      float x1 = zc * sF[B - 1][kk].x, x2 = 0.f;
      z[B - 1] = x1;
      nrm2 = x1 * x1;
#pragma unroll
      for (int i = B - 2; i >= 0; --i) {
        if (i % 16 == 14) asm volatile("" ::: "memory");  // factor reads run at most 16 rows ahead
        const float4 f = sF[i][kk];
        const float x = (z[i] - f.y * x1 - f.z * x2) * f.x;
        z[i] = x;
        nrm2 = fmaf(x, x, nrm2);
        x2 = x1;
        x1 = x;
      }
      scale = __builtin_amdgcn_rsqf(nrm2);
    }
#pragma unroll
    for (int i = 0; i < B; ++i) sZ[i][kk] = z[i] * scale;
  }
  __syncthreads();
  // re-orthogonalize within clusters of close eigenvalues (wave 0, lane =
  // row); all pairs (j, kk), j < kk, are first tested across the lanes (x =
  // 16 kk + j, one per lane and pass), so a page without close pairs (the
  // usual case) spends one LDS round trip here, not a chain of them
  bool close = false;
  if (wave == 0) {
    const float ctol = kClusterTol * fabsf(sLam[0]);
#pragma unroll
    for (int t = 0; t < (16 * KEPT + kWave - 1) / kWave; ++t) {
      const int x = t * kWave + lane, kk = x >> 4, j = x & 15;
      if (j < kk && kk < KEPT) close |= fabsf(sLam[j] - sLam[kk]) <= ctol;
    }
  }
  if (wave == 0 && __builtin_amdgcn_ballot_w64(close) != 0) {
    const float ctol = kClusterTol * fabsf(sLam[0]);
    for (int kk = 1; kk < KEPT; ++kk) {
      bool touched = false;
      float zk = sZ[lane][kk];
      for (int j = 0; j < kk; ++j) {
        if (fabsf(sLam[j] - sLam[kk]) > ctol) continue;
        const float zj = sZ[lane][j];
        zk -= group_sum<kWave>(zj * zk) * zj;
        touched = true;
      }
      if (touched) {
        zk *= __builtin_amdgcn_rsqf(group_sum<kWave>(zk * zk));
        sZ[lane][kk] = zk;
      }
    }
  }
  __syncthreads();

  // 6) back-transformation y = H_0 H_1 ... H_{B-3} z: eight eigenvectors per
  //    wave, lane 8 v + b holding rows 8 b .. 8 b + 7 of eigenvector 8 w + v,
  //    so each reflector costs a partial dot product of 8 rows and a sum over
  //    8 lanes; reflector k is row k of sA (16-byte reads)
  {
    constexpr int VW = 8;
    const int v = lane >> 3, b = lane & 7;
    const int kk = VW * wave + v;
    const bool act = VW * wave < KEPT;  // uniform
    float y[8];
    if (act) {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = kk < KEPT ? sZ[8 * b + i][kk] : 0.f;
      for (int k = B - 3; k >= 0; --k) {
        const float4 ua = *reinterpret_cast<const float4*>(&sA[k][8 * b]);
        const float4 ub = *reinterpret_cast<const float4*>(&sA[k][8 * b + 4]);
        const float u[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          d0 = fmaf(u[i], y[i], d0);
          d1 = fmaf(u[i + 1], y[i + 1], d1);
        }
        const float f = -2.f * group_sum<VW>(d0 + d1);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = fmaf(f, u[i], y[i]);
      }
    }
    __syncthreads();  // every wave is done with sZ
    if (act && kk < KEPT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sZ[8 * b + i][kk] = y[i];
    }
  }

  // zero modes, sigma
  if (tid < KEPT) {
    const float lam1 = sLam[0];
    const float lam = sLam[tid];
    const float thresh = fmaxf(kZeroModeRtol * lam1, kZeroModeFloor * energy);
    const int nz = (lam1 > 0.f && lam > thresh) ? 1 : 0;
    sNz[tid] = nz;
    sSigma[tid] = nz ? sqrtf(lam) : 1.f;
  }
  // optional: every eigenvalue (descending), bisection with one lane per eigenvalue
  if (a.eigvals_out && wave == kBuildWaves - 1) {
    const int target = B - 1 - lane;
    float lo = glo, hi = ghi;
    for (int it = 0; it < 64 && hi - lo > tol; ++it) {
      const float mid = 0.5f * (lo + hi);
      if (mid == lo || mid == hi) break;
      if (sturm_count(sd, se2, mid, pivmin) <= target) lo = mid;
      else hi = mid;
    }
    const float lam = lane < KEPT ? sLam[lane] : 0.5f * (lo + hi);
    a.eigvals_out[((size_t)idx * a.hkv + kvh) * B + lane] = fmaxf(lam, 0.f);
  }
  __syncthreads();

  // 7) basis V[k][c] = sum_i D[i][c] Y[i][k] / sigma_k (stored in sA): thread
  //    (column c, half h) reads column c of the K tile again (L2), centres it
  //    and forms rows k = h, h + 2, ...
  float* sV = &sA[0][0];
  {
    const int c = tid & (D - 1), h = tid >> 7;
    const float mu = sMu[c];
    float dc[B];
#pragma unroll
    for (int i = 0; i < B; ++i) dc[i] = Elem<T>::load(K + (size_t)i * D + c) - mu;
    for (int k = h; k < KEPT; k += 2) {
      float v = 0.f;
      if (sNz[k]) {
#pragma unroll
        for (int i = 0; i < B; ++i) v = fmaf(dc[i], sZ[i][k], v);
        v /= sSigma[k];
      }
      sV[k * D + c] = v;
    }
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

  // 8) write the record: centroid | basis rows | coefficients
  if (a.q4) {
    write_q4_record<R, KEPT>(a, phys, kvh, sMu, sV, sSign, &sZ[0][0], sSigma, sNz);
    return;
  }
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
      v = (k < KEPT && sNz[k]) ? sZ[i][k] * sSigma[k] * sSign[k] : 0.f;
    }
    Elem<T>::store(rec + x, v);
  }
}

template <typename T>
static hipError_t launch_build_t(int rank, const BuildArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  dim3 grid(a.n, a.hkv);
  dim3 block(a.merge.part_o ? kMergeThreads : kBuildThreads);
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
