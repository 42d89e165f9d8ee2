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
// three bf16 terms, six products, mirrored for exact symmetry).  Only the
// top r eigenpairs are needed, so the eigenproblem is solved as the 64-token
// builder solves its own (Golub & Van Loan, Matrix Computations, ch. 8), here
// on one wave: Householder reduction to tridiagonal form with the matrix in
// registers (lane (row, g) holds columns 4 g .. 4 g + 3 of its row, read from
// the mirrored LDS copy of the Gram), the wanted eigenvalues of T by
// Sturm-sequence multisection on lane segments, their eigenvectors by inverse
// iteration with partial pivoting (re-orthogonalized within clusters of close
// eigenvalues), and back-transformation by the 14 reflectors.  A step or a
// pass is a few dozen instructions of one wave, so a page takes a few
// microseconds; many waves share a CU.
//
// The key tile is read twice, both times straight into registers: in the
// matrix-core operand layout for the Gram (the centroid of a lane's
// dimensions is a sum over the 16 lanes of its DPP row, which hold those
// dimensions of the 16 tokens) and, from L2, with two dimensions per lane for
// the basis, which is formed, signed and written from registers.

#include "common.cuh"
#include "kernels.h"
#include "merge_impl.cuh"

namespace lk {

constexpr int kB16 = 16;
constexpr int kB16Waves = 4;
constexpr int kB16StepThreads = 512;  // decode-step launch: one merged output per thread for G <= 4
constexpr int kB16Ld = 17;  // padded row of the 16 x 16 matrices
constexpr int kB16InvIters = 2;          // inverse-iteration passes per eigenvector
constexpr float kB16ClusterTol = 1e-3f;  // eigenvalues this close (relative to lambda_1) are re-orthogonalized

// Number of eigenvalues of the symmetric tridiagonal T = (d, e) below sigma:
// the negative pivots of the LDL^T factorization of T - sigma I (Sturm
// count); e2[i] = e[i]^2, pivots smaller than pivmin are replaced by -pivmin.
__device__ __forceinline__ int sturm_count16(const float (&d)[kB16], const float (&e2)[kB16], float sigma,
                                             float pivmin) {
  float q = d[0] - sigma;
  if (fabsf(q) < pivmin) q = -pivmin;
  int c = q < 0.f ? 1 : 0;
#pragma unroll
  for (int i = 1; i < kB16; ++i) {
    q = (d[i] - sigma) - e2[i - 1] * __builtin_amdgcn_rcpf(q);
    if (fabsf(q) < pivmin) q = -pivmin;
    c += q < 0.f ? 1 : 0;
  }
  return c;
}

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

// DS: the decode step's launch, one workgroup of kB16StepThreads threads per
// (sequence, KV head): all threads merge the pair's attention partials (one
// output each), thread 0 of KV head 0 commits the length, and wave 0 then
// builds the page the step's append completed, if any.  The bulk build is
// compiled without them (one (page, KV head) per wave; fewer registers, more
// waves).
template <typename T, int R, bool DS>
__global__ __launch_bounds__(DS ? kB16StepThreads : kB16Waves * kWave) void build16_kernel(BuildArgs a) {
  constexpr int B = kB16;
  constexpr int D = kHeadDim;
  constexpr int KEPT = R < B ? R : B;
  __shared__ float sA[kB16Waves][2][B][kB16Ld];   // the Gram; the reflectors (row k = reflector k)
  __shared__ float sZ[kB16Waves][B][kB16Ld];      // eigenvector of the k-th largest eigenvalue = column k
  __shared__ float4 sF[kB16Waves][B][KEPT];       // inverse iteration: row i of the factors of T - lambda_k I
  __shared__ float sMu[kB16Waves][D];
  __shared__ float sT[kB16Waves][3][B];           // T: diagonal d, subdiagonal e (e[i] couples i, i + 1), e^2
  __shared__ float sVec[kB16Waves][2][B];         // u and w of a Householder step
  __shared__ float sLam[kB16Waves][B];            // eigenvalues, descending
  __shared__ float sSign[kB16Waves][KEPT];

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int idx, kvh;
  if constexpr (DS) {
    idx = blockIdx.x / a.hkv;  // idx = sequence
    kvh = blockIdx.x % a.hkv;
  } else {
    const int item = blockIdx.x * kB16Waves + wv;  // (page, KV head) pair
    if (item >= a.n * a.hkv) return;
    idx = item / a.hkv;
    kvh = item % a.hkv;
  }
  const int wave = DS ? 0 : wv;  // this wave's slot of the LDS arrays
  const int phys = a.phys_ids[idx];
  if constexpr (DS) {
    const bool commit = a.commit_seq_lens && kvh == 0 && threadIdx.x == 0;
    const int len = commit ? a.commit_seq_lens[idx] : 0;
    if (a.merge.part_o) merge_partials<T>(a, idx, kvh, threadIdx.x, blockDim.x);
    if (commit && phys != -2) a.commit_seq_lens[idx] = len + 1;
    if (wv != 0) return;
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
  }
  wave_lds_fence();

  // 3) eigenpairs of the Gram A.
  constexpr int LD = kB16Ld;
  float* const Rf = &sA[wave][1][0][0];  // reflector k = row k
  float* const Zw = &sZ[wave][0][0];
  float* const Td = sT[wave][0];
  float* const Te = sT[wave][1];
  float* const Te2 = sT[wave][2];
  float* const Vu = sVec[wave][0];
  float* const Vw = sVec[wave][1];
  const int rr = lane & (B - 1), gg = lane >> 4;  // lane (row, column group)
  // (a) Householder tridiagonalization: step k zeroes column k below the
  //     subdiagonal with H = I - 2 u u^T (||u|| = 1, u_r = 0 for r <= k);
  //     with p = 2 A u, K = u.p and w = p - K u, A <- A - u w^T - w u^T.
  //     Lane (r, g) holds A[r][4 g .. 4 g + 3]; u and w reach the lanes that
  //     hold their columns through LDS.  A zero column gives u = 0.
  {
    float Ar[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) Ar[t] = sA[wave][0][rr][4 * gg + t];
#pragma unroll
    for (int k = 0; k < B - 2; ++k) {
      const float ak = xor32_sum(xor16_sum(gg == (k >> 2) ? Ar[k & 3] : 0.f));  // A[r][k] in every group
      const float x = rr > k ? ak : 0.f;
      const float nrm2 = group_sum<16>(x * x);
      const float x0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k + 1));
      const float nrm = __builtin_amdgcn_sqrtf(nrm2);
      const bool nz = nrm2 > 0.f;
      const float alpha = nz ? (x0 >= 0.f ? -nrm : nrm) : 0.f;
      const float inv = __builtin_amdgcn_rsqf(2.f * (nrm2 + nrm * fabsf(x0)));  // 1 / ||x - alpha e_{k+1}||
      const float u = nz ? (rr == k + 1 ? x - alpha : x) * inv : 0.f;
      if (lane == k) Td[k] = ak;
      if (lane == 0) Te[k] = alpha;
      if (gg == 0) {
        Rf[k * LD + rr] = u;
        Vu[rr] = u;
      }
      wave_lds_fence();
      float uc[4], pp = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uc[t] = Vu[4 * gg + t];
        pp = fmaf(Ar[t], uc[t], pp);
      }
      const float p = 2.f * xor32_sum(xor16_sum(pp));
      const float K = group_sum<16>(u * p);
      const float w = rr > k ? p - K * u : 0.f;
      if (gg == 0) Vw[rr] = w;
      wave_lds_fence();
#pragma unroll
      for (int t = 0; t < 4; ++t) Ar[t] = fmaf(-u, Vw[4 * gg + t], fmaf(-w, uc[t], Ar[t]));
    }
    // the trailing 2 x 2 block (rows and columns 14, 15: lanes (14, 3), (15, 3))
    if (gg == 3 && rr == B - 2) Td[B - 2] = Ar[2];
    if (gg == 3 && rr == B - 1) {
      Td[B - 1] = Ar[3];
      Te[B - 2] = Ar[2];
      Te[B - 1] = 0.f;
    }
    wave_lds_fence();
    if (lane < B) Te2[lane] = Te[lane] * Te[lane];
    wave_lds_fence();
  }
  // (b) eigenvalues of T, descending: the NK largest at once (every
  //     eigenvalue when they are an output, else the kept ones), each on a
  //     segment of SL = 64 / NK lanes; a pass counts the eigenvalues below SL
  //     shifts spread over the segment's interval, which shrinks
  //     (SL + 1)-fold.
  float lam1, thresh;
  {
    float dreg[B], e2reg[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      dreg[i] = Td[i];
      e2reg[i] = Te2[i];
    }
    const float em = rr > 0 ? fabsf(Te[rr - 1]) : 0.f, ep = fabsf(Te[rr]);
    const float glo = -group_max<16>(-(Td[rr] - em - ep)), ghi = group_max<16>(Td[rr] + em + ep);
    const float tnorm = fmaxf(fabsf(glo), fabsf(ghi));
    const float pivmin = fmaxf(tnorm * 1e-30f, 1e-30f);
    const float tol = 2.f * 1.19209290e-7f * tnorm;
    const int NK = a.eigvals_out ? B : KEPT;  // a power of two
    const int SL = kWave / NK;
    const int seg = lane / SL, sl = lane % SL;
    const int target = B - 1 - seg;  // ascending index of the seg-th largest
    const uint64_t segmask = SL == kWave ? ~0ull : (((1ull << SL) - 1ull) << (seg * SL));
    float lo = glo, hi = ghi;
    bool more = true;
    for (int it = 0; it < 40; ++it) {
      more = more && hi - lo > tol;
      if (!__ballot(more)) break;
      const float width = hi - lo;
      const float sig = lo + width * (float)(sl + 1) * __builtin_amdgcn_rcpf((float)(SL + 1));
      const int cnt = sturm_count16(dreg, e2reg, sig, pivmin);
      const uint64_t below = __ballot(cnt <= target) & segmask;  // shifts at or below the eigenvalue
      const int nl = below ? 64 - __clzll(below) - seg * SL : 0;  // highest such lane of the segment + 1
      const float nlo = nl > 0 ? lo + width * (float)nl * __builtin_amdgcn_rcpf((float)(SL + 1)) : lo;
      const float nhi = nl < SL ? lo + width * (float)(nl + 1) * __builtin_amdgcn_rcpf((float)(SL + 1)) : hi;
      if (nlo == lo && nhi == hi) more = false;  // below the resolution of fp32
      if (more) { lo = nlo; hi = nhi; }
    }
    if (sl == 0) sLam[wave][seg] = 0.5f * (lo + hi);
    wave_lds_fence();
    lam1 = sLam[wave][0];
    thresh = fmaxf(kZeroModeRtol * lam1, kZeroModeFloor * energy);
    if (a.eigvals_out && lane < B) a.eigvals_out[((size_t)idx * a.hkv + kvh) * B + lane] = fmaxf(sLam[wave][lane], 0.f);

    // (c) inverse iteration on T: lane kk factors T - lambda_kk I once with
    //     partial pivoting (rows i and i + 1 swap when |e_i| > |pivot|; both
    //     choices are carried and one selected, so the chain has no branch),
    //     then solves kB16InvIters times from a fixed varied start.
    if (lane < KEPT) {
      const int kk = lane;
      const float lam = sLam[wave][kk];
      uint32_t swm = 0u;  // bit i: rows i and i + 1 swapped
      float ddc = dreg[0] - lam, duc = Te[0];
#pragma unroll
      for (int i = 0; i < B - 1; ++i) {
        const float dl = Te[i];
        const float ddn = dreg[i + 1] - lam;
        const float dun = i + 1 < B - 1 ? Te[i + 1] : 0.f;
        const bool keep = fabsf(ddc) >= fabsf(dl);
        const float rk = __builtin_amdgcn_rcpf(fabsf(ddc) < pivmin ? pivmin : ddc);
        const float rs = __builtin_amdgcn_rcpf(dl);
        const float mk = dl * rk, ms = ddc * rs;
        const float nk = ddn - mk * duc, ns = duc - ms * ddn;
        sF[wave][i][kk] = make_float4(keep ? rk : rs, keep ? duc : ddn, keep ? 0.f : dun, keep ? mk : ms);
        if (!keep) swm |= 1u << i;
        duc = keep ? dun : -ms * dun;
        ddc = keep ? nk : ns;
      }
      sF[wave][B - 1][kk] = make_float4(__builtin_amdgcn_rcpf(fabsf(ddc) < pivmin ? pivmin : ddc), 0.f, 0.f, 0.f);
      float z[B];
      float nrm2 = 0.f;
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const uint32_t hsh = (uint32_t)(i * 2654435761u) ^ (uint32_t)((kk + 1) * 40503u);
        z[i] = 0.5f + (float)((hsh >> 9) & 1023) * (1.f / 1024.f);
        nrm2 = fmaf(z[i], z[i], nrm2);
      }
      float scale = __builtin_amdgcn_rsqf(nrm2);
      for (int itr = 0; itr < kB16InvIters; ++itr) {
        // forward: the row swaps and multipliers applied to the right-hand side
        float zc = z[0] * scale;
#pragma unroll
        for (int i = 0; i < B - 1; ++i) {
          const float zn = z[i + 1] * scale;
          const float mlt = sF[wave][i][kk].w;
          const bool sw = (swm >> i) & 1u;
          z[i] = sw ? zn : zc;
          zc = sw ? zc - mlt * zn : zn - mlt * zc;
        }
        // back substitution, in place
        float x1 = zc * sF[wave][B - 1][kk].x, x2 = 0.f;
        z[B - 1] = x1;
        nrm2 = x1 * x1;
#pragma unroll
        for (int i = B - 2; i >= 0; --i) {
          const float4 f = sF[wave][i][kk];
          const float xv = (z[i] - f.y * x1 - f.z * x2) * f.x;
          z[i] = xv;
          nrm2 = fmaf(xv, xv, nrm2);
          x2 = x1;
          x1 = xv;
        }
        scale = __builtin_amdgcn_rsqf(nrm2);
      }
#pragma unroll
      for (int i = 0; i < B; ++i) Zw[i * LD + kk] = z[i] * scale;
    }
    wave_lds_fence();
  }
  // (d) re-orthogonalize within clusters of close eigenvalues (lane = row;
  //     the four groups compute alike, group 0 stores)
  //     All pairs are tested at once across the lanes, so a page without
  //     close pairs (the usual case) spends one LDS round trip here, not a
  //     chain of them.
  {
    const float ctol = kB16ClusterTol * fabsf(lam1);
    // pairs (j, kk), j < kk < KEPT, as x = 16 kk + j, one per lane and pass
    bool close = false;
#pragma unroll
    for (int t = 0; t < (16 * KEPT + kWave - 1) / kWave; ++t) {
      const int x = t * kWave + lane, kk = x >> 4, j = x & 15;
      if (j < kk && kk < KEPT) close |= fabsf(sLam[wave][j] - sLam[wave][kk]) <= ctol;
    }
    if (__builtin_amdgcn_ballot_w64(close) != 0) {
      for (int kk = 1; kk < KEPT; ++kk) {
        bool touched = false;
        float zk = Zw[rr * LD + kk];
        for (int j = 0; j < kk; ++j) {
          if (fabsf(sLam[wave][j] - sLam[wave][kk]) > ctol) continue;
          const float zj = Zw[rr * LD + j];
          zk -= group_sum<16>(zj * zk) * zj;
          touched = true;
        }
        if (touched) {
          zk *= __builtin_amdgcn_rsqf(group_sum<16>(zk * zk));
          if (gg == 0) Zw[rr * LD + kk] = zk;
          wave_lds_fence();
        }
      }
    }
  }
  // (e) back-transformation y = H_0 H_1 ... H_13 z: lane (kk, b) = (lane / 4,
  //     lane % 4) holds rows 4 b .. 4 b + 3 of eigenvector kk
  {
    const int kk = lane >> 2, b = lane & 3;
    float y[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) y[t] = kk < KEPT ? Zw[(4 * b + t) * LD + kk] : 0.f;
#pragma unroll
    for (int k = B - 3; k >= 0; --k) {
      float uk[4], d = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uk[t] = Rf[k * LD + 4 * b + t];
        d = fmaf(uk[t], y[t], d);
      }
      const float f = -2.f * group_sum<4>(d);
#pragma unroll
      for (int t = 0; t < 4; ++t) y[t] = fmaf(f, uk[t], y[t]);
    }
    wave_lds_fence();
    if (kk < KEPT) {
#pragma unroll
      for (int t = 0; t < 4; ++t) Zw[(4 * b + t) * LD + kk] = y[t];
    }
    wave_lds_fence();
  }

  // 5) basis rows V[k][c] = sum_i D[i][c] U[i][idx_k] / sigma_k for this lane's
  //    dims c = 2 lane, 2 lane + 1, then the signs (largest |entry| positive,
  //    ties to the lower dim)
  const float mu0 = sMu[wave][2 * lane], mu1 = sMu[wave][2 * lane + 1];
#pragma unroll
  for (int i = 0; i < B; ++i) { db[i][0] -= mu0; db[i][1] -= mu1; }
  float vb[KEPT][2];
  if constexpr (KEPT <= 8) {
    // products one vector at a time, then the signs four vectors at a time with
    // independent cross-lane reductions and no LDS: the largest magnitude over
    // the wave, the lowest dim holding it (a maximum of minus the dim), then
    // that entry's sign from its lane
#pragma unroll
    for (int k = 0; k < KEPT; ++k) {
      const bool nz = lam1 > 0.f && sLam[wave][k] > thresh;
      const float inv = nz ? 1.f / sqrtf(sLam[wave][k]) : 0.f;
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const float uik = Zw[i * LD + k];
        v0 = fmaf(db[i][0], uik, v0);
        v1 = fmaf(db[i][1], uik, v1);
      }
      // zero modes: no basis row (their eigenvector may be anything, even inf)
      vb[k][0] = nz ? v0 * inv : 0.f;
      vb[k][1] = nz ? v1 * inv : 0.f;
      wave_lds_fence();  // one vector's loads and products at a time (registers)
    }
    constexpr int SG = 4;
#pragma unroll
    for (int k0 = 0; k0 < KEPT; k0 += SG) {
      float amax[SG], cand[SG];
#pragma unroll
      for (int c = 0; c < SG; ++c)
        if (k0 + c < KEPT) amax[c] = group_max<kWave>(fmaxf(fabsf(vb[k0 + c][0]), fabsf(vb[k0 + c][1])));
#pragma unroll
      for (int c = 0; c < SG; ++c)
        if (k0 + c < KEPT) {
          const float* v = vb[k0 + c];
          cand[c] = group_max<kWave>(fabsf(v[0]) == amax[c] ? -(float)(2 * lane)
                                     : (fabsf(v[1]) == amax[c] ? -(float)(2 * lane + 1) : -1024.f));
        }
#pragma unroll
      for (int c = 0; c < SG; ++c)
        if (k0 + c < KEPT) {
          const int k = k0 + c;
          const int dim = __builtin_amdgcn_readfirstlane((int)(-cand[c]));
          const float at =
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int((dim & 1) ? vb[k][1] : vb[k][0]), dim >> 1));
          const float sg = at < 0.f ? -1.f : 1.f;
          vb[k][0] *= sg;
          vb[k][1] *= sg;
          if (lane == 0) sSign[wave][k] = sg;
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // 16 vectors: products and sign one vector at a time (the sign by
    // shuffles), which holds fewer registers
#pragma unroll
    for (int k = 0; k < KEPT; ++k) {
      const bool nz = lam1 > 0.f && sLam[wave][k] > thresh;
      const float inv = nz ? 1.f / sqrtf(sLam[wave][k]) : 0.f;
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const float uik = Zw[i * LD + k];
        v0 = fmaf(db[i][0], uik, v0);
        v1 = fmaf(db[i][1], uik, v1);
      }
      // zero modes: no basis row (their eigenvector may be anything, even inf)
      v0 = nz ? v0 * inv : 0.f;
      v1 = nz ? v1 * inv : 0.f;
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
  }
  wave_lds_fence();
  auto coef_at = [&](int i, int k) -> float {
    if (k >= KEPT) return 0.f;
    const bool nz = lam1 > 0.f && sLam[wave][k] > thresh;
    return nz ? Zw[i * LD + k] * sqrtf(sLam[wave][k]) * sSign[wave][k] : 0.f;
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
    // this lane holds dims 2 lane, 2 lane + 1; a basis byte takes dims 8 g + e
    // and 8 g + e + 2 (even dims in a word's low half-word, odd in its high), so
    // lanes 4 g + x pair with lane 4 g + (x ^ 1) and write byte 4 g + (x >> 1) +
    // 2 (x & 1): the two low codes when x is even, the two high codes when odd
    const int lo = b16_q_code(v0, bs, 7.f), hi = b16_q_code(v1, bs, 7.f);
    const int mine = (lo & 0xF) | ((hi & 0xF) << 4);
    const int other = __builtin_amdgcn_mov_dpp(mine, kDppXor1, 0xf, 0xf, true);
    const int byte = (lane & 1) ? ((other >> 4) | (mine & 0xF0)) : ((mine & 0xF) | ((other & 0xF) << 4));
    rec[L.basis() + k * (D / 2) + 4 * (lane >> 2) + ((lane >> 1) & 1) + 2 * (lane & 1)] = (uint8_t)byte;
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
  const bool ds = a.merge.part_o != nullptr || a.commit_seq_lens != nullptr;
  const long long items = (long long)a.n * a.hkv;
  dim3 grid((unsigned)(ds ? items : (items + kB16Waves - 1) / kB16Waves));
  dim3 block(ds ? kB16StepThreads : kB16Waves * kWave);
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
