// Page scorer: reconstructed log-sum-exp of every complete page.
//
// [Locks] §4 "Score", Eq. (1): for page j with centroid mu_j, basis V_j (d x r)
// and coefficients c_i, and query head g,
//   s_hat_j(q_g) = log sum_i exp(scale * (q_g . mu_j + (V_j^T q_g) . c_i)).
// The record stores centroid | basis rows | coeffs, so rows 0..r of the
// record form W = [mu; v_1; ...; v_r] and the projection is P = W q_g.
//
// fp32 records (below, VALU; one wave per page at a time, pages of one
// (sequence, KV head) per workgroup):
//   projection: lane (s = lane / 16, e = lane % 16) owns dims 8e..8e+7 of rows
//     s, s+4, s+8, ...; partial dots are summed over the 16 lanes of a row
//     group with DPP, giving P[row][g] for every query head of the group;
//   reconstruction: lane i = token i computes z_i(g) = P[0][g] + sum_m c_i[m] P[m+1][g]
//     (P broadcast from LDS);
//   LSE: z is transposed through LDS so that each query head's B logits sit
//     on a group of 64/G lanes, reduced with DPP (max, then sum of exp2).
// The page's bytes are read once, with 16-byte loads.
//
// Pages of B = 64 or B = 16 tokens.  With B = 16 a wave's lanes cover four
// records' tokens at once (lane = 16 * record + token), so each page's
// log-sum-exp is reduced within one 16-lane row, with no transpose.

#include "common.cuh"
#include "kernels.h"

namespace lk {

// One wave per workgroup: waves finish at different times, and a workgroup's
// LDS and slot are released only when all its waves are done (alternating
// timings at 128K x 4, records rotated through HBM: bf16 scorer 41.2 -> 40.7
// us, int4 26.7 -> 25.9 us, 16-token int4 56.2 -> 55.4 us against four waves).
constexpr int kScoreWaves = 1;
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

// Decode-step cache append (AppendDuty), done by the workgroup of page chunk
// 0 of every (sequence, KV head) before anything else: 16-byte copies of the
// new key and value rows into slot T mod B of page T / B, and the build-list
// entry.
template <typename T, int B>
__device__ __forceinline__ void append_duty(const ScoreArgs& a, int seq, int kvh, int chunk) {
  if (a.app.k_new == nullptr || chunk != 0) return;
  constexpr int D = kHeadDim;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CH = D / VEC;  // 16-byte chunks per row
  const int len = a.seq_lens[seq];
  const int page = len / B, slot = len % B;
  int phys = -1;
  if (len >= 0 && page < a.max_pages) phys = a.block_table[(size_t)seq * a.max_pages + page];
  const bool ok = phys >= 0 && phys < a.num_phys;
  const int t = threadIdx.x;
  if (ok && t < 2 * CH) {
    const int which = t / CH, ch = t % CH;
    const T* src = reinterpret_cast<const T*>(which ? a.app.v_new : a.app.k_new) +
                   ((size_t)seq * a.hkv + kvh) * D + ch * VEC;
    T* dst = reinterpret_cast<T*>(which ? a.app.v_pool : a.app.k_pool) +
             (((size_t)phys * a.hkv + kvh) * B + slot) * D + ch * VEC;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
  if (kvh == 0 && t == 0) a.app.build_list[seq] = !ok ? -2 : (slot == B - 1 ? phys : -1);
}

template <typename T, int R, int G, int B>
__global__ __launch_bounds__(kScoreWaves * kWave) void score_kernel(ScoreArgs a) {
  constexpr int D = kHeadDim;
  constexpr int ROWS = R + 1;                 // centroid + r basis rows
  constexpr int RG = (ROWS + 3) / 4;          // rows per lane group
  constexpr int LPH = kWave / G;              // lanes per query head in the LSE
  constexpr int TPL = B >= LPH ? B / LPH : 1;  // logits per lane in the LSE (B = 64)
  constexpr size_t REC = (size_t)ROWS * D + (size_t)B * R;

  __shared__ float sP[kScoreWaves][ROWS * G];
  __shared__ float sZ[kScoreWaves][G * B];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int seq = blockIdx.z;
  const int kvh = blockIdx.y;
  append_duty<T, B>(a, seq, kvh, blockIdx.x);
  const int len = a.seq_lens[seq] + a.len_add;
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

    // reconstructed logits, lane = token (B = 16: lanes past the page repeat
    // its tokens, and only the first row of 16 lanes is reduced)
    float c[R];
    load_coeffs<T, R>(rec + (size_t)ROWS * D + (size_t)(lane % B) * R, c);
    float zr[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float z = P[g];
#pragma unroll
      for (int m = 0; m < R; ++m) z = fmaf(c[m], P[(m + 1) * G + g], z);
      zr[g] = z * zscale;
    }
    if constexpr (B == 16) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mx = group_max<16>(zr[g]);
        const float sum = group_sum<16>(fast_exp2(zr[g] - mx));
        if (lane == g) out[(size_t)g * a.max_pages + j] = (mx + fast_log2(sum)) * kLn2;
      }
      wave_lds_fence();  // P is rewritten by the next page
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) Z[g * B + lane] = zr[g];
      wave_lds_fence();

      // per-head log-sum-exp over the page's B logits
      const int hg = lane / LPH;
      const int t0 = (lane % LPH) * TPL;
      float v[TPL];
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < TPL; ++t) {
        v[t] = Z[hg * B + t0 + t];
        mx = vmax(mx, v[t]);
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
}

// ---------------------------------------------------------------------------
// bf16 records: the projection on the matrix cores.
//
// A wave takes NR records at a time.  Their (r + 1) rows (centroid, basis)
// are the 16-wide columns of B in v_mfma_f32_16x16x32_bf16 (row slot
// s = record * (r + 1) + row), the group's G queries are the rows of A (rows
// >= G repeat the last query and are ignored), and four K-steps of 32 cover d = 128: the product holds
// P[slot][g] = W_slot . q_g.  Lane l of B supplies column l % 16 and 8
// consecutive dims of K-step t at group l / 16, i.e. one 16-byte load; lane l
// of A supplies the same dims of query l % 16.  The accumulator of lane l
// holds rows 4 (l / 16) .. +3 of column l % 16.
//
// Every record byte a wave needs is requested in its prologue, before any
// arithmetic, and waves are short (one group of NR records by default): on
// this part a scattered read of many short-lived waves, each with one batch
// of loads in flight, streams faster than fewer waves that loop over several
// batches.
// Records per wave: their (r + 1) rows fill up to 5 matrix-core tiles; at
// B = 16 a wave takes twice as many records (each covers a quarter of the
// tokens), amortizing the wave's fixed work over more of them.
template <int R, int B = 64> struct ScoreGroup {
  static constexpr int NR = B == 64 ? (R >= 16 ? 2 : (R >= 8 ? 4 : (R >= 4 ? 8 : 16)))
                                    : (R >= 16 ? 4 : (R >= 8 ? 8 : 16));  // records per group
  static constexpr int SLOTS = NR * (R + 1);
  static constexpr int TILES = (SLOTS + 15) / 16;
  static constexpr int CW = (R + 1) / 2;        // 32-bit words of one token's coefficients
  // coefficient sets a lane holds: its token of every record (B = 64), or
  // token lane % 16 of record 4 p + lane / 16 for each pass p (B = 16)
  static constexpr int CSETS = B == 64 ? NR : (NR + 3) / 4;
};

// One group's loads, held in registers until the group is computed.
template <int R, int B> struct GroupLoads {
  uint4 wb[ScoreGroup<R, B>::TILES][4];                    // B operand tiles
  uint32_t cw[ScoreGroup<R, B>::CSETS][ScoreGroup<R, B>::CW];  // token coefficients (bf16 pairs)
  uint32_t vbits;                                          // bit r: record r present in the pool (else the page scores -inf)
};

// v[x] for a lane-dependent x in [LO, LO + CNT) from uniform values, by
// masks: a select chain on x == y lets the compiler turn it into an indexed
// load of the array, which then lives in scratch memory.
template <int LO, int CNT, int N>
__device__ __forceinline__ int pick_uniform(const int (&v)[N], int x) {
  int r = 0;
#pragma unroll
  for (int y = LO; y < LO + CNT; ++y) r |= v[y] & -(int)(x == y);
  return r;
}

// The physical page of record r of a wave's group for a lane-dependent r, at
// 16-token pages: lane x < NR of `mine` holds record x's page (clamped into
// the pool), and the cross-lane permute reads it from lane r: one
// instruction in place of a compare-and-select per record.
__device__ __forceinline__ int lane_page(int mine, int r) { return __builtin_amdgcn_ds_bpermute(r << 2, mine); }

// Every load is unconditional, so the compiler keeps them in one batch with no
// wait in between: a record that is not in the pool is read from physical
// page 0 instead (always allocated) and its result discarded, and B columns
// past the group's slots repeat its last slot (their products are unused).
template <int R, int B>
__device__ __forceinline__ void load_group(GroupLoads<R, B>& L, const bf16_t* summ,
                                           const int (&phys_g)[ScoreGroup<R, B>::NR], int num_phys, int hkv, int kvh,
                                           int col, int kg, int lane) {
  constexpr int D = kHeadDim;
  constexpr int ROWS = R + 1;
  constexpr int NR = ScoreGroup<R, B>::NR;
  constexpr int SLOTS = ScoreGroup<R, B>::SLOTS;
  constexpr int TILES = ScoreGroup<R, B>::TILES;
  constexpr int CW = ScoreGroup<R, B>::CW;
  constexpr int CSETS = ScoreGroup<R, B>::CSETS;
  constexpr size_t REC = (size_t)ROWS * D + (size_t)B * R;
  auto rec_of = [&](int phys) {
    return summ + ((size_t)((phys >= 0 && phys < num_phys) ? phys : 0) * hkv + kvh) * REC;
  };
  const bf16_t* recp[NR];
  L.vbits = 0u;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int phys = phys_g[r];
    L.vbits |= (phys >= 0 && phys < num_phys) ? 1u << r : 0u;
    recp[r] = rec_of(phys);
  }
#pragma unroll
  for (int tau = 0; tau < TILES; ++tau) {
    const int slot = min(16 * tau + col, SLOTS - 1);
    const int r = slot / ROWS, m = slot % ROWS;
    const bf16_t* rp = recp[0];
    if constexpr (B == 64) {
#pragma unroll
      for (int x = 1; x < NR; ++x) if (x == r) rp = recp[x];
    } else {
      rp = rec_of(pick_uniform<0, NR>(phys_g, r));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
      L.wb[tau][t] = *reinterpret_cast<const uint4*>(rp + (size_t)m * D + 32 * t + 8 * kg);
  }
#pragma unroll
  for (int r = 0; r < CSETS; ++r) {
    const bf16_t* cp = B == 64 ? recp[r] + (size_t)ROWS * D + (size_t)lane * R
                               : rec_of(pick_uniform<0, NR>(phys_g, min(4 * r + (lane >> 4), NR - 1))) +
                                     (size_t)ROWS * D + (size_t)(lane & 15) * R;
    if constexpr (R % 8 == 0) {
#pragma unroll
      for (int x = 0; x < CW; x += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(cp + 2 * x);
        L.cw[r][x] = v.x; L.cw[r][x + 1] = v.y; L.cw[r][x + 2] = v.z; L.cw[r][x + 3] = v.w;
      }
    } else if constexpr (R == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(cp);
      L.cw[r][0] = v.x; L.cw[r][1] = v.y;
    } else if constexpr (R == 2) {
      L.cw[r][0] = *reinterpret_cast<const uint32_t*>(cp);
    } else {
      L.cw[r][0] = (uint32_t)*cp;
    }
  }
}

// 64-token pages: a page's logits z_i = z_c + d_i split into the centroid
// logit z_c (row 0 of P) and the deviation d_i = s_i * sum_m c_i[m] P[m + 1]
// (s_i = 1 unless SCALED), so LSE = z_c + log sum_i exp(d_i).  The
// deviations of a centred page straddle zero (their coefficients sum to
// zero), so sum_i 2^d_i needs no running maximum unless a deviation is
// extreme: a wave whose sums leave [2^-64, 2^64] (or are not finite) takes
// the page maxima and sums again.  In both forms the largest term that
// matters is at least 2^-64 of the total and no term overflows, so the two
// agree to rounding.  (At 16-token pages the maxima are always taken: the
// two-pass form there needs more registers than the row reductions it saves.)
__device__ __forceinline__ bool lse_sum_ok(float s) { return s >= 0x1p-64f && s <= 0x1p64f; }

// Reconstruction and per-head LSE of a group of NR records whose projections
// P[slot * G + g] (slot = record * (R + 1) + row; row 0 = centroid) are in
// LDS, RC records at a time: every record's deviations (lane = token) in one
// pass, one transpose through LDS, then the records' sums side by side
// (independent chains), and one store per head group.  coef(r, c, s) gives
// this lane's token coefficients of record r and their scale.
template <int R, int G, int NR, bool SCALED, typename Coef>
__device__ __forceinline__ void group_lse(const float* P, float* Z, Coef coef, uint32_t vbits, float* out,
                                          int max_pages, int g0, int j_end, int lane, float zscale) {
  constexpr int B = 64;
  constexpr int ROWS = R + 1;
  constexpr int LPH = kWave / G;
  constexpr int TPL = B / LPH;
  constexpr int RC = (16 / G) < NR ? (16 / G) : NR;  // records per LDS transpose (RC * G <= 16)
#pragma unroll
  for (int c0 = 0; c0 < NR; c0 += RC) {
    float z[RC][G];
#pragma unroll
    for (int rr = 0; rr < RC; ++rr) {
      const int r = c0 + rr;
      float c[R], cs;
      coef(r, c, cs);
      const float* Pr = P + r * ROWS * G;
      const float dscale = SCALED ? cs * zscale : zscale;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < R; ++m) acc = fmaf(c[m], Pr[(m + 1) * G + g], acc);
        z[rr][g] = acc * dscale;
      }
    }
#pragma unroll
    for (int rr = 0; rr < RC; ++rr)
#pragma unroll
      for (int g = 0; g < G; ++g) Z[(rr * G + g) * B + lane] = z[rr][g];
    wave_lds_fence();
    const int hg = lane / LPH;
    const int t0 = (lane % LPH) * TPL;
    float v[RC][TPL], res[RC];
    float lo_s = 0x1p64f, hi_s = 0x1p-64f;  // range of this head group's sums
#pragma unroll
    for (int rr = 0; rr < RC; ++rr) {
      float sl = 0.f;
#pragma unroll
      for (int t = 0; t < TPL; ++t) {
        v[rr][t] = Z[(rr * G + hg) * B + t0 + t];
        sl += fast_exp2(v[rr][t]);
      }
      const float sum = group_sum<LPH>(sl);
      lo_s = vmin(lo_s, sum);
      hi_s = vmax(hi_s, sum);
      res[rr] = P[(c0 + rr) * ROWS * G + hg] * zscale + fast_log2(sum);
    }
    if (__ballot(!(lse_sum_ok(lo_s) && lse_sum_ok(hi_s))) != 0ull) {  // wave-uniform: exact page maxima
#pragma unroll
      for (int rr = 0; rr < RC; ++rr) {
        float m = -INFINITY;
#pragma unroll
        for (int t = 0; t < TPL; ++t) m = vmax(m, v[rr][t]);
        m = group_max<LPH>(m);
        float sl = 0.f;
#pragma unroll
        for (int t = 0; t < TPL; ++t) sl += fast_exp2(v[rr][t] - m);
        res[rr] = P[(c0 + rr) * ROWS * G + hg] * zscale + m + fast_log2(group_sum<LPH>(sl));
      }
    }
#pragma unroll
    for (int rr = 0; rr < RC; ++rr) res[rr] = ((vbits >> (c0 + rr)) & 1u) ? res[rr] * kLn2 : -INFINITY;
    // lane hg * LPH + rr of head group hg writes record c0 + rr
    const int rsel = lane % LPH;
    if constexpr (RC <= LPH) {
      float val = res[0];
#pragma unroll
      for (int rr = 1; rr < RC; ++rr)
        if (rsel == rr) val = res[rr];
      const int j = g0 + c0 + rsel;
      if (rsel < RC && j < j_end) out[(size_t)hg * max_pages + j] = val;
    } else {
#pragma unroll
      for (int rr = 0; rr < RC; ++rr) {
        const int j = g0 + c0 + rr;
        if (rr % LPH == rsel && j < j_end) out[(size_t)hg * max_pages + j] = res[rr];
      }
    }
    if (c0 + RC < NR) wave_lds_fence();  // Z is rewritten by the next records
  }
}

// The same at B = 16: lane 16 q + t holds token t of record 4 p + q in pass p
// and forms its G logits; one transpose through LDS (Z[(q * G + g) * 16 + t])
// then gives each (record, head) pair of the pass 16 / G lanes with G tokens
// each, so a pair's LSE is G - 1 local steps and log2(16 / G) lane steps
// instead of four lane steps per head; the first lane of a pair writes it.
// coef(p, c, s) gives the lane's coefficients of pass p and their scale.
template <int R, int G, int NR, bool SCALED, typename Coef>
__device__ __forceinline__ void group_lse16(const float* P, float* Z, Coef coef, uint32_t vbits, float* out,
                                            int max_pages, int g0, int j_end, int lane, float zscale) {
  constexpr int ROWS = R + 1;
  constexpr int LPP = 16 / G;  // lanes per (record, head) pair after the transpose
  const int q = lane >> 4, t = lane & 15;
  const int pr = lane / LPP;             // pair of this lane: record 4 p + pr / G, head pr % G
  const int t0 = (lane % LPP) * G;       // its first token
#pragma unroll
  for (int p = 0; p < (NR + 3) / 4; ++p) {
    const int rc = min(4 * p + q, NR - 1);
    float c[R], cs;
    coef(p, c, cs);
    const float* Pr = P + rc * ROWS * G;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc;
      if constexpr (SCALED) {
        acc = 0.f;
#pragma unroll
        for (int m = 0; m < R; ++m) acc = fmaf(c[m], Pr[(m + 1) * G + g], acc);
        acc = fmaf(cs, acc, Pr[g]);
      } else {
        acc = Pr[g];
#pragma unroll
        for (int m = 0; m < R; ++m) acc = fmaf(c[m], Pr[(m + 1) * G + g], acc);
      }
      Z[(q * G + g) * 16 + t] = acc * zscale;
    }
    wave_lds_fence();
    float v[G];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      v[i] = Z[pr * 16 + t0 + i];
      mx = vmax(mx, v[i]);
    }
    mx = group_max<LPP>(mx);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) sum += fast_exp2(v[i] - mx);
    sum = group_sum<LPP>(sum);
    const int r = 4 * p + pr / G, g = pr % G;
    const int j = g0 + r;
    if (lane % LPP == 0 && r < NR && j < j_end)
      out[(size_t)g * max_pages + j] = ((vbits >> r) & 1u) ? (mx + fast_log2(sum)) * kLn2 : -INFINITY;
    if (4 * (p + 1) < NR) wave_lds_fence();  // Z is rewritten by the next pass
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int R, int G, int B>
__global__ __launch_bounds__(kScoreWaves * kWave) void score_mfma_kernel(ScoreArgs a) {
  constexpr int D = kHeadDim;
  constexpr int NR = ScoreGroup<R, B>::NR;
  constexpr int SLOTS = ScoreGroup<R, B>::SLOTS;
  constexpr int TILES = ScoreGroup<R, B>::TILES;
  constexpr int PAGES_PER_WAVE = NR;
  static_assert(G <= 8, "at most 8 query heads per KV head");

  __shared__ float sP[kScoreWaves][SLOTS * G];
  constexpr int RC = (16 / G) < NR ? (16 / G) : NR;  // records per LDS transpose (RC * G <= 16)
  __shared__ float sZ[kScoreWaves][B == 64 ? RC * G * B : 4 * G * 16];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar table loads
  // grid (KV head, page chunk, sequence): the KV heads of a page, whose
  // records sit side by side, are dispatched together
  const int seq = blockIdx.z;
  const int kvh = blockIdx.x;
  append_duty<bf16_t, B>(a, seq, kvh, blockIdx.y);
  const int j0 = (blockIdx.y * kScoreWaves + wave) * PAGES_PER_WAVE;
  if (j0 >= a.max_pages) return;
  const int col = lane & 15;       // B column / A row of this lane
  const int kg = lane >> 4;        // K group (8 dims) within a K-step
  const bf16_t* summ = reinterpret_cast<const bf16_t*>(a.summary);
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;

  // The wave's block-table slice (clamped in bounds), the sequence length and
  // the group's queries are requested first; a wave wholly past the scored
  // pages (ragged batches: the grid covers max_pages for every sequence)
  // leaves once the length is in, before any record load; the others then
  // request every record of the wave at once (pages past the sequence end are
  // masked when results are written).
  int phys_all[PAGES_PER_WAVE];
#pragma unroll
  for (int x = 0; x < PAGES_PER_WAVE; ++x) phys_all[x] = bt[min(j0 + x, a.max_pages - 1)];
  const int len_raw = a.seq_lens[seq] + a.len_add;
  bf16x8_t qa[4];  // A operand: query `col`, 4 K-steps
  {
    const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q) + ((size_t)seq * a.hq + (size_t)kvh * G) * D;
    // rows >= G repeat query G-1 (their products are unused)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      qa[t] = __builtin_bit_cast(bf16x8_t,
                                 *reinterpret_cast<const uint4*>(q + (size_t)min(col, G - 1) * D + 32 * t + 8 * kg));
  }
  int n_scored = len_raw <= 0 ? 0 : (len_raw - 1) / B;
  if (n_scored > a.max_pages - 1) n_scored = a.max_pages - 1;
  if (j0 >= n_scored) return;
  GroupLoads<R, B> cur;
  load_group<R, B>(cur, summ, phys_all, a.num_phys, a.hkv, kvh, col, kg, lane);
  // The loads above have no side effects, so without this fence the compiler
  // would move them between the products (each move adds a wait for earlier
  // loads before later ones are issued).
  asm volatile("" ::: "memory");
  const int j_end = min(j0 + PAGES_PER_WAVE, n_scored);

  const float zscale = a.scale * kLog2e;
  float* out = a.page_lse + ((size_t)seq * a.hq + (size_t)kvh * G) * a.max_pages;
  float* P = sP[wave];
  float* Z = sZ[wave];
  // lanes whose product rows are not query heads of the group (or whose
  // column is past the last slot) store to discard slots in Z, which the LSE
  // overwrites before reading: no exec-mask branches around the stores
  float* const Pdiscard = Z + (G < 4 ? G : 4) * lane;

  {
    const int g0 = j0;
    // projection on the matrix cores
#pragma unroll
    for (int tau = 0; tau < TILES; ++tau) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], __builtin_bit_cast(bf16x8_t, cur.wb[tau][t]), acc, 0, 0, 0);
      const int slot = 16 * tau + col;
      // rows 4 kg + i are query heads g < G: i < G is known here, 4 kg < G per lane
      float* const dst = 4 * kg < G && slot < SLOTS ? P + slot * G + 4 * kg : Pdiscard;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < G) dst[i] = acc[i];
    }
    wave_lds_fence();
    auto coef = [&](int r, float (&c)[R], float& cs) {
#pragma unroll
      for (int m = 0; m < R; ++m) c[m] = (m & 1) ? bf16_hi(cur.cw[r][m >> 1]) : bf16_lo(cur.cw[r][m >> 1]);
      cs = 1.f;
    };
    if constexpr (B == 64) group_lse<R, G, NR, false>(P, Z, coef, cur.vbits, out, a.max_pages, g0, j_end, lane, zscale);
    else group_lse16<R, G, NR, false>(P, Z, coef, cur.vbits, out, a.max_pages, g0, j_end, lane, zscale);
  }
}

template <int R, int B>
static hipError_t launch_score_mfma(int group, const ScoreArgs& a, hipStream_t s) {
  constexpr int per_block = kScoreWaves * ScoreGroup<R, B>::NR;
  dim3 grid(a.hkv, (a.max_pages + per_block - 1) / per_block, a.batch);
  dim3 block(kScoreWaves * kWave);
  switch (group) {
    case 1: hipLaunchKernelGGL((score_mfma_kernel<R, 1, B>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((score_mfma_kernel<R, 2, B>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((score_mfma_kernel<R, 4, B>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((score_mfma_kernel<R, 8, B>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantized records (Q4Layout) with bf16 queries: the projection on the matrix
// cores with the integer codes as bf16 operands (small integers are exact in
// bf16), scales applied to the fp32 products.
//
// K mapping: lane (col, kg) of K-step t covers dims 32 kg + 8 t .. +7, so a
// lane reads 32 consecutive dims of its row over the four K-steps: one
// 16-byte load of an int4 basis row, two of the int8 centroid (the queries use
// the same mapping).  Codes are converted biased (int4 + 8, int8 + 128: plain
// byte-to-float conversions) and the bias is removed from the products,
// sum_c q_c code_c = sum_c q_c (code_c + bias) - bias * S_g with S_g = sum_c q_c.
// Tiles: one tile of the NR centroids, and beside it the product of the
// queries with an all-ones operand (every column holds the S_g), then
// NR * R / 16 tiles of basis rows (column = record * R + row).  The reconstruction and LSE are those of the
// bf16 records, with the per-token coefficient scale.
template <int R, int B = 64> struct Q4Group {
  // records per wave (the centroid tile holds the NR centroids)
  static constexpr int NR = B == 64 ? (R >= 16 ? 2 : (R >= 8 ? 4 : 8)) : (R >= 16 ? 4 : 8);
  static constexpr int BT = NR * R / 16;                       // basis tiles
  static constexpr int SLOTS = NR * (R + 1);
  static constexpr int CSETS = B == 64 ? NR : (NR + 3) / 4;    // coefficient sets per lane (as ScoreGroup)
};

__device__ __forceinline__ uint32_t bf16x2_of(float lo, float hi) {  // both exact in bf16: the high halves
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ float ubyte_f(uint32_t x, int b) { return (float)((x >> (8 * b)) & 0xffu); }

// K-step operand of 8 int4 codes as bf16 values of code + 136.  The record's
// 32-bit word for 8 dims holds the even dims in its low half-word and the odd
// dims in its high half-word (element 2 j in nibble j, element 2 j + 1 in
// nibble j + 4), so (w >> 4 j) & 0x000f000f puts elements 2 j and 2 j + 1 in
// the low mantissa bits of the two halves of dword j; XOR with 0x43084308
// then sets bf16 128's exponent and flips the sign bit of the code
// (two's complement c becomes n = c + 8, and 0x4300 | n is exactly 128 + n).
// One shift and one three-input bit operation per two codes.
constexpr float kQ4Bias = 136.f;
__device__ __forceinline__ bf16x8_t q4_operand(uint32_t w) {
  uint4 o;
  o.x = (w & 0x000f000fu) ^ 0x43084308u;
  o.y = ((w >> 4) & 0x000f000fu) ^ 0x43084308u;
  o.z = ((w >> 8) & 0x000f000fu) ^ 0x43084308u;
  o.w = ((w >> 12) & 0x000f000fu) ^ 0x43084308u;
  return __builtin_bit_cast(bf16x8_t, o);
}
// K-step operand of 8 int8 codes (two 32-bit words) as bf16 values of code + 128.
__device__ __forceinline__ bf16x8_t q8_operand(uint32_t w0, uint32_t w1) {
  w0 ^= 0x80808080u;
  w1 ^= 0x80808080u;
  uint4 o;
  o.x = bf16x2_of(ubyte_f(w0, 0), ubyte_f(w0, 1));
  o.y = bf16x2_of(ubyte_f(w0, 2), ubyte_f(w0, 3));
  o.z = bf16x2_of(ubyte_f(w1, 0), ubyte_f(w1, 1));
  o.w = bf16x2_of(ubyte_f(w1, 2), ubyte_f(w1, 3));
  return __builtin_bit_cast(bf16x8_t, o);
}
__device__ __forceinline__ float half_bits_f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// At 16-token pages six waves per SIMD (registers capped accordingly) run
// ahead of the five the unconstrained allocation gives (51.5 against 53.2 us
// at 128K x 4); eight spill.
template <int B> constexpr int kQ4WavesPerEu = B == 16 ? 6 : 1;
template <int R, int G, int B>
__global__ __launch_bounds__(kScoreWaves * kWave) __attribute__((amdgpu_waves_per_eu(kQ4WavesPerEu<B>)))
void score_q4_kernel(ScoreArgs a) {
  constexpr int D = kHeadDim;
  constexpr int ROWS = R + 1;
  constexpr int NR = Q4Group<R, B>::NR;
  constexpr int BT = Q4Group<R, B>::BT;
  constexpr int SLOTS = Q4Group<R, B>::SLOTS;
  constexpr int CSETS = Q4Group<R, B>::CSETS;
  constexpr Q4Layout L{R, B};
  constexpr int REC = L.bytes();
  static_assert(G <= 8 && NR <= 16 && BT * 16 == NR * R, "tile shapes");

  __shared__ float sP[kScoreWaves][SLOTS * G];
  constexpr int RC = (16 / G) < NR ? (16 / G) : NR;
  __shared__ float sZ[kScoreWaves][B == 64 ? RC * G * B : 4 * G * 16];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // Workgroups over (KV head, page chunk, sequence), KV head fastest, dealt to
  // the XCDs in contiguous ranges: records of one page's KV heads lie side by
  // side and share 128-byte lines, which one L2 then fetches once.
  // 64-token pages: grid x = (KV head, page chunk) of sequence y, x padded to
  // a multiple of the XCD count (a workgroup's XCD then follows from x alone),
  // split with a mask and a shift for a power-of-two KV head count (int4
  // scorer 23.6 -> 22.3 us against one remapped 1-D range split by three
  // divisions).  The 16-token scorer keeps the 1-D range (49.9 against 50.5 us
  // with the 2-D grid), split by a mask, a shift and one division (49.5 ->
  // 49.2 us).
  const int n_chunks = (a.max_pages + kScoreWaves * NR - 1) / (kScoreWaves * NR);
  int seq, kvh, chunk;
  if constexpr (B == 64) {
    seq = blockIdx.y;
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    if (lin >= a.hkv * n_chunks) return;
    if ((a.hkv & (a.hkv - 1)) == 0) {
      kvh = lin & (a.hkv - 1);
      chunk = lin >> __builtin_ctz(a.hkv);
    } else {
      chunk = lin / a.hkv;
      kvh = lin - chunk * a.hkv;
    }
  } else {
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    int rest;
    if ((a.hkv & (a.hkv - 1)) == 0) {
      kvh = lin & (a.hkv - 1);
      rest = lin >> __builtin_ctz(a.hkv);
    } else {
      rest = lin / a.hkv;
      kvh = lin - rest * a.hkv;
    }
    seq = rest / n_chunks;
    chunk = rest - seq * n_chunks;
  }
  append_duty<bf16_t, B>(a, seq, kvh, chunk);
  const int j0 = (chunk * kScoreWaves + wave) * NR;
  if (j0 >= a.max_pages) return;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const uint8_t* summ = reinterpret_cast<const uint8_t*>(a.summary);
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;

  // Block-table slice, sequence length and queries first; waves wholly past
  // the scored pages leave before any record load; then every record byte at
  // once (as for bf16 records).
  int phys_all[NR];
#pragma unroll
  for (int x = 0; x < NR; ++x) phys_all[x] = __builtin_amdgcn_readfirstlane(bt[min(j0 + x, a.max_pages - 1)]);
  const int len_raw = a.seq_lens[seq] + a.len_add;
  uint4 qw[4];  // query min(col, G - 1), dims 32 kg .. 32 kg + 31
  {
    const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q) + ((size_t)seq * a.hq + (size_t)kvh * G) * D;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      qw[t] = *reinterpret_cast<const uint4*>(q + (size_t)min(col, G - 1) * D + 32 * kg + 8 * t);
  }
  int n_scored = len_raw <= 0 ? 0 : (len_raw - 1) / B;
  if (n_scored > a.max_pages - 1) n_scored = a.max_pages - 1;
  if (j0 >= n_scored) return;
  // 16-token pages: lane x < NR holds record x's physical page (clamped)
  int mine = 0;
  if constexpr (B == 16) {
    mine = bt[min(j0 + min(lane, NR - 1), a.max_pages - 1)];
    mine = (mine >= 0 && mine < a.num_phys) ? mine : 0;
  }
  const uint8_t* summ_h = summ + (size_t)kvh * REC;
  const size_t rec_stride = (size_t)a.hkv * REC;
  auto rec_of_lane = [&](int r) { return summ_h + (size_t)(uint32_t)lane_page(mine, r) * rec_stride; };
  uint32_t vbits = 0u;  // bit r: record r present in the pool
  const uint8_t* recp[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const bool valid = phys_all[r] >= 0 && phys_all[r] < a.num_phys;
    vbits |= valid ? 1u << r : 0u;
    recp[r] = summ + ((size_t)(valid ? phys_all[r] : 0) * a.hkv + kvh) * REC;
  }
  uint4 wb[BT];     // basis row (record, row) = column of tile tau: 32 codes
  uint32_t bsc[BT]; // its scale (fp16 bits)
#pragma unroll
  for (int tau = 0; tau < BT; ++tau) {
    const int slot = 16 * tau + col;
    const int r = slot / R, m = slot % R;
    constexpr int RPT = 16 / R;  // records of one tile
    const uint8_t* rp = recp[tau * RPT];
#pragma unroll
    for (int x = 1; x < RPT; ++x) if (r == tau * RPT + x) rp = recp[tau * RPT + x];
    wb[tau] = *reinterpret_cast<const uint4*>(rp + L.basis() + m * (D / 2) + 16 * kg);
    bsc[tau] = *reinterpret_cast<const uint16_t*>(rp + L.bscale() + 2 * m);
  }
  uint4 wm[2];      // centroid of record min(col, NR - 1): 32 codes
  uint32_t msc;
  {
    const int r = min(col, NR - 1);
    const uint8_t* rp = recp[0];
    if constexpr (B == 64) {
#pragma unroll
      for (int x = 1; x < NR; ++x) if (x == r) rp = recp[x];
    } else {
      rp = rec_of_lane(r);
    }
    wm[0] = *reinterpret_cast<const uint4*>(rp + 32 * kg);
    wm[1] = *reinterpret_cast<const uint4*>(rp + 32 * kg + 16);
    msc = *reinterpret_cast<const uint16_t*>(rp + L.mscale());
  }
  uint32_t cw[CSETS][(R + 3) / 4];  // a token's R int8 codes (lane's token of record r, or of pass r at B = 16)
  uint32_t csc[CSETS];              // and their scale (fp16 bits)
#pragma unroll
  for (int r = 0; r < CSETS; ++r) {
    const uint8_t* rp = B == 64 ? recp[r] : rec_of_lane(min(4 * r + (lane >> 4), NR - 1));
    const int tok = B == 64 ? lane : (lane & 15);
    const uint8_t* cp = rp + L.coef() + (size_t)tok * R;
    if constexpr (R == 16) {
      const uint4 v = *reinterpret_cast<const uint4*>(cp);
      cw[r][0] = v.x; cw[r][1] = v.y; cw[r][2] = v.z; cw[r][3] = v.w;
    } else if constexpr (R == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(cp);
      cw[r][0] = v.x; cw[r][1] = v.y;
    } else {
      cw[r][0] = *reinterpret_cast<const uint32_t*>(cp);
    }
    csc[r] = *reinterpret_cast<const uint16_t*>(rp + L.cscale() + 2 * tok);
  }
  asm volatile("" ::: "memory");  // keep the loads above in one batch (as for bf16 records)
  const int j_end = min(j0 + NR, n_scored);

  const float zscale = a.scale * kLog2e;
  float* out = a.page_lse + ((size_t)seq * a.hq + (size_t)kvh * G) * a.max_pages;
  float* P = sP[wave];
  float* Z = sZ[wave];
  // 16-token pages: lanes whose product rows are not query heads of the group
  // store to discard slots in Z, which the LSE overwrites before reading, so
  // the stores below take no exec-mask branches (rows 4 kg + i are query heads
  // g < G: i < G is known at compile time, 4 kg < G per lane).  At 64-token
  // pages the masked stores are kept (22.6 against 21.9 us with discard slots).
  float* const Pdiscard = Z + (G < 4 ? G : 4) * lane;
  const bool head_rows = 4 * kg < G;
  bf16x8_t qa[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) qa[t] = __builtin_bit_cast(bf16x8_t, qw[t]);

  // centroid tile first: columns 0 .. NR-1 are the centroids; a second
  // product with an all-ones operand holds S_g = sum of query g over all dims
  // in every column
  float Sg[4];  // S of the queries whose products this lane holds (rows 4 kg + i)
  {
    const uint32_t w[8] = {wm[0].x, wm[0].y, wm[0].z, wm[0].w, wm[1].x, wm[1].y, wm[1].z, wm[1].w};
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, accs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], q8_operand(w[2 * t], w[2 * t + 1]), acc, 0, 0, 0);
      accs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], ones, accs, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) Sg[i] = accs[i];
    const float sc = half_bits_f(msc);
    if constexpr (B == 16) {
      float* const dst = head_rows && col < NR ? P + (col * ROWS) * G + 4 * kg : Pdiscard;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < G) dst[i] = sc * (acc[i] - 128.f * Sg[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = 4 * kg + i;
        if (g < G && col < NR) P[(col * ROWS) * G + g] = sc * (acc[i] - 128.f * Sg[i]);
      }
    }
  }
  // basis tiles: P[record * ROWS + 1 + row][g] = scale * (acc - 136 S_g)
#pragma unroll
  for (int tau = 0; tau < BT; ++tau) {
    const uint32_t w[4] = {wb[tau].x, wb[tau].y, wb[tau].z, wb[tau].w};
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], q4_operand(w[t]), acc, 0, 0, 0);
    const int slot = 16 * tau + col;
    const int r = slot / R, m = slot % R;
    const float sc = half_bits_f(bsc[tau]);
    if constexpr (B == 16) {
      float* const dst = head_rows ? P + (r * ROWS + 1 + m) * G + 4 * kg : Pdiscard;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < G) dst[i] = sc * (acc[i] - kQ4Bias * Sg[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = 4 * kg + i;
        if (g < G) P[(r * ROWS + 1 + m) * G + g] = sc * (acc[i] - kQ4Bias * Sg[i]);
      }
    }
  }
  wave_lds_fence();
  auto coef = [&](int r, float (&c)[R], float& cs) {
#pragma unroll
    for (int m = 0; m < R; ++m) c[m] = (float)(int8_t)((cw[r][m >> 2] >> (8 * (m & 3))) & 0xffu);
    cs = half_bits_f(csc[r]);
  };
  if constexpr (B == 64) group_lse<R, G, NR, true>(P, Z, coef, vbits, out, a.max_pages, j0, j_end, lane, zscale);
  else group_lse16<R, G, NR, true>(P, Z, coef, vbits, out, a.max_pages, j0, j_end, lane, zscale);
}

template <int R, int B>
static hipError_t launch_score_q4(int group, const ScoreArgs& a, hipStream_t s) {
  constexpr int per_block = kScoreWaves * Q4Group<R, B>::NR;
  const int per_seq = a.hkv * ((a.max_pages + per_block - 1) / per_block);
  const dim3 grid = B == 64 ? dim3((per_seq + kXcds - 1) / kXcds * kXcds, a.batch) : dim3(per_seq * a.batch);
  dim3 block(kScoreWaves * kWave);
  switch (group) {
    case 1: hipLaunchKernelGGL((score_q4_kernel<R, 1, B>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((score_q4_kernel<R, 2, B>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((score_q4_kernel<R, 4, B>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((score_q4_kernel<R, 8, B>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int R, int B>
static hipError_t launch_score_rg(int group, const ScoreArgs& a, hipStream_t s) {
  dim3 grid((a.max_pages + kScorePagesPerBlock - 1) / kScorePagesPerBlock, a.hkv, a.batch);
  dim3 block(kScoreWaves * kWave);
  switch (group) {
    case 1: hipLaunchKernelGGL((score_kernel<T, R, 1, B>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((score_kernel<T, R, 2, B>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((score_kernel<T, R, 4, B>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((score_kernel<T, R, 8, B>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int B>
static hipError_t launch_score_b(DType dt, int rank, int group, bool q4, const ScoreArgs& a, hipStream_t s) {
  if (q4) {
    if (dt != kBF16) return hipErrorInvalidValue;
    switch (rank) {
      case 4: return launch_score_q4<4, B>(group, a, s);
      case 8: return launch_score_q4<8, B>(group, a, s);
      case 16: return launch_score_q4<16, B>(group, a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (dt == kBF16) {
    switch (rank) {
      case 1: return launch_score_mfma<1, B>(group, a, s);
      case 2: return launch_score_mfma<2, B>(group, a, s);
      case 4: return launch_score_mfma<4, B>(group, a, s);
      case 8: return launch_score_mfma<8, B>(group, a, s);
      case 16: return launch_score_mfma<16, B>(group, a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (rank) {
    case 1: return launch_score_rg<float, 1, B>(group, a, s);
    case 2: return launch_score_rg<float, 2, B>(group, a, s);
    case 4: return launch_score_rg<float, 4, B>(group, a, s);
    case 8: return launch_score_rg<float, 8, B>(group, a, s);
    case 16: return launch_score_rg<float, 16, B>(group, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_score(DType dt, int page_size, int rank, int group, bool q4, const ScoreArgs& a, hipStream_t s) {
  if (page_size == 64) return launch_score_b<64>(dt, rank, group, q4, a, s);
  if (page_size == 16) return launch_score_b<16>(dt, rank, group, q4, a, s);
  return hipErrorInvalidValue;
}

}  // namespace lk
