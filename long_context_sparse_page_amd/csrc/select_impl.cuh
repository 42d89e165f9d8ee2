// Share-average and top-k page selection for one (sequence, KV head) by one
// workgroup: the device code shared by the selection kernel and the decode
// step's fused selection + attention kernel.
//
// [Locks] §4 (after Eq. (1)) and Cor. 3: query head g's page-mass share is
//   m_hat_g(j) = exp(s_hat_j(q_g)) / sum_{j'} exp(s_hat_j'(q_g))
// over the scored pages j' < n_mr (sink included); the group average
//   m_bar_j = (1/G) sum_g m_hat_g(j)
// ranks the candidates 1 .. n_mr-1, and the selection is the sink page 0, the
// most recent page n_mr and the top-(k-2) candidates (ties to the lower page
// index), written in ascending page order.
//
// Thread t holds the scores of pages j = t + BS*i (i < NPT): coalesced
// loads, and page order is slot i first, then thread.
//  1. Per-head normalizer S_g = sum_j 2^(s2_j(g) - M_g) (scores in log2 units;
//     per-thread max and sum, combined over the block with one barrier).
//  2. m_bar_j = (1/G) sum_g 2^(s2_j(g) - M_g) / S_g; the ranking key is an
//     order-preserving uint32 of log2 m_bar_j (a share below 2^-120 is
//     evaluated in the log domain instead, so keys never underflow).
//  3. Pivot: the (k-2)-th largest of the maxima of disjoint groups of keys
//     (4 threads per group, else 1), found by one wave by bisection on its
//     bits (ballot counts, no barrier).  At least k-2 keys reach the pivot,
//     so the top k-2 keys are among them.
//  4. The keys >= pivot (typically a few more than k-2) are compacted into
//     LDS in page order (ballots per slot, wave counts through LDS).
//  5. One wave finds the exact (k-2)-th largest key of that list by the same
//     bisection and writes the selected pages in list order, i.e. ascending
//     page order; ties at the cut go to the earliest (lowest-index) pages.
// When the list would not fit (massive ties), the exact cut is instead found
// by block-wide bisection over all keys and the selection written in page
// order through the same per-slot counts.

#pragma once

#include "common.cuh"
#include "kernels.h"

namespace lk {

constexpr int kMaxGroup = 8;
constexpr int kMaxSelect = 1024;
constexpr int kListFast = 256;  // compacted keys handled in registers by one wave

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of set bits of m in lanes below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
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
  return vmax(vmax(a, b), vmax(c, d));
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

// The n-th largest of the wave's nonzero values x (R per lane): the largest t
// with #{x >= t} >= n.  Needs at least n nonzero values.  Bits above the
// highest bit where the largest and smallest nonzero values differ are common
// to the answer; the rest are set greedily from the top, one ballot count per
// bit.  With lowbit > 0 the bits below it are left clear: t is then a lower
// bound of the n-th largest value (still #{x >= t} >= n), in fewer steps.
template <int R>
__device__ __forceinline__ uint32_t wave_nth_largest(const uint32_t (&x)[R], int n, int lowbit = 0) {
  uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (x[r]) { mx = max(mx, x[r]); mn = min(mn, x[r]); }
  wave_minmax_u32(mx, mn);
  uint32_t t = mx;
  const uint32_t diff = mx ^ mn;
  if (diff) {
    const int hb = 31 - __clz(diff);
    t = mx & ~((hb == 31) ? 0xffffffffu : ((2u << hb) - 1u));
    for (int bit = hb; bit >= lowbit; --bit) {
      const uint32_t c = t | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) cnt += __popcll(__ballot(x[r] >= c));
      if (cnt >= n) t = c;
    }
  }
  return t;
}

// One wave: the n largest of the list keys ck (CR per lane, entry lane + 64 r,
// 0 = no entry; at least n nonzero), ties to the earlier entries; emit(slot, r)
// for each taken entry of this lane, slot = its rank in list order.  Returns
// how many entries of row 0 (entries 0 .. 63) were taken.
template <int CR, typename Emit>
__device__ __forceinline__ int wave_take_in_order(const uint32_t (&ck)[CR], int n, Emit emit) {
  const uint32_t t = wave_nth_largest<CR>(ck, n);
  int n_gt = 0;
#pragma unroll
  for (int r = 0; r < CR; ++r) n_gt += __popcll(__ballot(ck[r] > t));
  const int take_eq = n - n_gt;
  int eq_before = 0, out_before = 0, row0 = 0;
#pragma unroll
  for (int r = 0; r < CR; ++r) {
    const bool eq = ck[r] == t;
    const uint64_t be = __ballot(eq);
    const bool take = ck[r] > t || (eq && eq_before + lanes_below(be) < take_eq);
    eq_before += __popcll(be);
    const uint64_t bs = __ballot(take);
    if (take) emit(out_before + lanes_below(bs), r);
    out_before += __popcll(bs);
    if (r == 0) row0 = out_before;
  }
  return row0;
}

// Page-order positions of the entries flagged by pred(i), thread t holding
// pages t + BS*i (i < NPT <= 64): one ballot per slot, the [NPT][NW] wave
// counts through LDS (one barrier); lane l of each wave then sums column l
// and the slot offsets follow from a bit-sliced prefix over lanes.  Returns
// the block total.  s_cnt must not be written again before another barrier
// has passed (callers alternate two buffers).
template <int NPT, int NW, typename Pred>
__device__ __forceinline__ int page_order_positions(Pred pred, int (&pos)[NPT], int* s_cnt) {
  static_assert(NPT <= kWave, "one lane per slot");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const uint64_t m = __ballot(pred(i));
    if (lane == 0) s_cnt[i * NW + wave] = __popcll(m);
  }
  __syncthreads();
  int before = 0, tot = 0;  // lane l: slot l's entries in earlier waves, and in all
  if (lane < NPT) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = s_cnt[lane * NW + w];
      before += (w < wave) ? c : 0;
      tot += c;
    }
  }
  int excl = 0, total = 0;  // sum of tot over lanes below, and over all lanes
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const uint64_t m = __ballot((tot >> b) & 1);
    excl += lanes_below(m) << b;
    total += __popcll(m) << b;
  }
  const int base = excl + before;
#pragma unroll
  for (int i = 0; i < NPT; ++i)
    pos[i] = __builtin_amdgcn_readlane(base, i) + lanes_below(__ballot(pred(i)));
  return total;
}

// One wave: the n_top largest keys of the compacted list (c entries in page
// order, CR per lane), ties to the earliest entries, written in list order to
// selection slots 1 .. n_top.
template <int CR>
__device__ __forceinline__ void select_from_list(const uint32_t* s_ckey, const int* s_cidx, const int* s_cphys,
                                                 int c, int n_top, int32_t* sel, int32_t* selp, int num_phys) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t ck[CR];
#pragma unroll
  for (int r = 0; r < CR; ++r) {
    const int x = lane + kWave * r;
    ck[r] = x < c ? s_ckey[x] : 0u;
  }
  const uint32_t t = wave_nth_largest<CR>(ck, n_top);
  int n_gt = 0;
#pragma unroll
  for (int r = 0; r < CR; ++r) n_gt += __popcll(__ballot(ck[r] > t));
  const int take_eq = n_top - n_gt;
  int eq_before = 0, out_before = 0;
#pragma unroll
  for (int r = 0; r < CR; ++r) {
    const bool eq = ck[r] == t;
    const uint64_t be = __ballot(eq);
    const bool take = ck[r] > t || (eq && eq_before + lanes_below(be) < take_eq);
    eq_before += __popcll(be);
    const uint64_t bs = __ballot(take);
    if (take) {
      const int x = lane + kWave * r;
      const int slot = 1 + out_before + lanes_below(bs);
      sel[slot] = s_cidx[x];
      if (selp) {
        const int ph = s_cphys[x];
        selp[slot] = (ph >= 0 && ph < num_phys) ? ph : -1;
      }
    }
    out_before += __popcll(bs);
  }
}

// log2 m_bar_j of a page whose share is below 2^-120, from its G scores in
// log2 units (see share_log2), evaluated in the log domain:
// log2 m_bar = log2 sum_g 2^(x[g] - M_g - log2 S_g) - log2 G.
template <int G>
__device__ __forceinline__ float share_log2_small(const float (&x)[G], const float (&Mg)[G], const float (&log2S)[G],
                                                 float log2G, float& mb) {
  float d[G], mx = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    d[g] = (Mg[g] == -INFINITY) ? -INFINITY : x[g] - Mg[g] - log2S[g];
    mx = fmaxf(mx, d[g]);
  }
  float lm = -INFINITY;
  if (mx != -INFINITY) {
    float sm = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) sm += fast_exp2(d[g] - mx);
    lm = mx + fast_log2(sm) - log2G;
  }
  mb = fast_exp2(lm);
  return lm;
}

// log2 m_bar_j of one page from its G scores in log2 units x[g], with
// e[g] = 2^(x[g] - m_g) (m_g: the thread's running maximum of head g) and
// scale[g] = 2^(m_g - M_g) / S_g; m_bar_j itself is returned in mb.  A share
// below 2^-120 is evaluated in the log domain,
// log2 m_bar = log2 sum_g 2^(x[g] - M_g - log2 S_g) - log2 G.
template <int G>
__device__ __forceinline__ float share_log2(const float (&x)[G], const float (&e)[G], const float (&scale)[G],
                                           const float (&Mg)[G], const float (&log2S)[G], float invG, float log2G,
                                           float& mb) {
  mb = 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) mb = fmaf(e[g], scale[g], mb);
  mb *= invG;
  if (mb >= 0x1p-120f) return fast_log2(mb);
  return share_log2_small<G>(x, Mg, log2S, log2G, mb);
}

// One workgroup of BS threads selects for (seq, kvh); sel / cnt_out / selp
// may point to global memory or LDS (selp nullptr: no physical pages);
// seq_len is a.seq_lens[seq], loaded by the caller.
template <int BS, int NPT, int G>
__device__ __forceinline__ void select_block(const SelectArgs& a, int seq, int kvh, int seq_len, int32_t* sel,
                                             int32_t* cnt_out, int32_t* selp) {
  constexpr int NW = BS / kWave;
  // Up to 256 threads the scores stay in registers from one early load; larger
  // blocks (128 registers per thread) load them again for the keys (L2 hits).
  constexpr bool kTwoPass = BS > 256;
  constexpr bool kKeepE = !kTwoPass && G * NPT <= 48;  // keep 2^(s2 - m) in registers
  constexpr bool kPrefetchPhys = !kTwoPass;            // block-table entries fetched with the scores
  __shared__ float s_gred[2 * 8 * NW];
  __shared__ uint32_t s_tmax[BS];
  __shared__ int s_cnt[2][NPT * NW];
  __shared__ uint32_t s_ckey[kListFast];
  __shared__ int s_cidx[kListFast];
  __shared__ int s_cphys[kListFast];
  __shared__ uint32_t s_pivot;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int k = a.k;
  auto page = [&](int i) { return tid + BS * i; };
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;
  const size_t hq = (size_t)a.hkv * G;
  const float* lse = a.page_lse + ((size_t)seq * hq + (size_t)kvh * G) * a.max_pages;

  // Loads that need no sequence length go out first: this thread's page
  // scores (entries past the scored pages are masked below) and, for the
  // physical-page output, its block-table entries.
  float v[kTwoPass ? 1 : G][kTwoPass ? 1 : NPT];
  if constexpr (!kTwoPass) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int j = page(i);
        v[g][i] = lse[(size_t)g * a.max_pages + min(j, a.max_pages - 1)];  // unconditional: no waits between loads
      }
  }
  int ph[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = page(i);
    ph[i] = (kPrefetchPhys && selp) ? bt[min(j, a.max_pages - 1)] : -1;
  }
  auto phys_of = [&](int i) -> int {
    if (!selp) return -1;
    return kPrefetchPhys ? ph[i] : bt[page(i)];
  };
  // write selection slot s: logical page and, when asked for, its physical page
  auto emit = [&](int s, int page, int phys) {
    sel[s] = page;
    if (selp) selp[s] = (page >= 0 && phys >= 0 && phys < a.num_phys) ? phys : -1;
  };

  const int len = seq_len + a.len_add;
  if (len <= 0) {
    for (int s = tid; s < k; s += BS) emit(s, -1, -1);
    if (tid == 0) *cnt_out = 0;
    return;
  }
  int n_mr = (len - 1) / a.page_size;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  const int n_scored = n_mr;
  const int n_cand = n_mr > 0 ? n_mr - 1 : 0;
  const int n_top = min(k - 2, n_cand);
  // every page 0 .. n_mr selected: each thread writes its own pages
  auto write_all = [&]() {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int j = page(i);
      if (j <= n_mr) emit(j, j, phys_of(i));
    }
    for (int s = n_mr + 1 + tid; s < k; s += BS) emit(s, -1, -1);
    if (tid == 0) *cnt_out = n_mr + 1;
  };
  if (n_top == n_cand && a.share_out == nullptr) {  // n_mr == 0 included
    write_all();
    return;
  }

  // score s2_j(g) in log2 units; -inf past the scored pages
  auto score_at = [&](int g, int i) -> float {
    const int j = page(i);
    float raw;
    if constexpr (kTwoPass) raw = lse[(size_t)g * a.max_pages + min(j, a.max_pages - 1)];
    else raw = v[g][i];
    return j < n_scored ? raw * kLog2e : -INFINITY;
  };

  // 1) per-head normalizers: each thread's (max m_g, sum of 2^(s2 - m_g)),
  //    combined over the block with one barrier:
  //    M_g = max m_g, S_g = sum 2^(m_g - M_g) * s_g
  float m[G], sl[G];
  float E[kKeepE ? G : 1][kKeepE ? NPT : 1];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x[NPT];
    m[g] = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      x[i] = score_at(g, i);
      m[g] = vmax(m[g], x[i]);
    }
    sl[g] = 0.f;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const float ei = m[g] == -INFINITY ? 0.f : fast_exp2(x[i] - m[g]);
      if constexpr (kKeepE) E[g][i] = ei;
      sl[g] += ei;
    }
  }
  float* s_pm = s_gred;            // [G][NW] wave maxima
  float* s_ps = s_gred + 8 * NW;   // [G][NW] wave sums relative to them
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float wm = wave_max(m[g]);
    const float ws = wave_sum(wm == -INFINITY || m[g] == -INFINITY ? 0.f : sl[g] * fast_exp2(m[g] - wm));
    if (lane == 0) { s_pm[g * NW + wave] = wm; s_ps[g * NW + wave] = ws; }
  }
  __syncthreads();
  float Mg[G], scale[G], log2S[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = vmax(M, s_pm[g * NW + w]);
    float S = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wm = s_pm[g * NW + w];
      S += wm == -INFINITY ? 0.f : s_ps[g * NW + w] * fast_exp2(wm - M);
    }
    Mg[g] = M;
    log2S[g] = fast_log2(S);
    // 2^(s2 - M_g) / S_g = E * 2^(m_g - M_g) / S_g
    scale[g] = (m[g] == -INFINITY || !(S > 0.f)) ? 0.f : fast_exp2(m[g] - M) / S;
  }

  // 2) shares and ranking keys
  const float invG = 1.f / (float)G;
  const float log2G = fast_log2((float)G);
  float* so = a.share_out ? a.share_out + ((size_t)seq * a.hkv + kvh) * a.max_pages : nullptr;
  uint32_t key[NPT];
  uint32_t tmax = 0u;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = page(i);
    key[i] = 0u;
    if (j >= n_scored) continue;
    float x[G];
#pragma unroll
    for (int g = 0; g < G; ++g) x[g] = score_at(g, i);
    float eg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if constexpr (kKeepE) eg[g] = E[g][i];
      else eg[g] = m[g] == -INFINITY ? 0.f : fast_exp2(x[g] - m[g]);
    }
    float mb;
    const float lm = share_log2<G>(x, eg, scale, Mg, log2S, invG, log2G, mb);
    if (so) so[j] = mb;
    if (j >= 1) {  // candidates: pages 1 .. n_mr - 1
      key[i] = order_key(lm);
      tmax = max(tmax, key[i]);
    }
  }
  if (n_top == n_cand) {
    write_all();
    return;
  }

  // fixed slots and padding: the sink, the most recent page, unused slots
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = page(i);
    if (j == 0) emit(0, 0, phys_of(i));
    if (j == n_mr) emit(n_top + 1, n_mr, phys_of(i));
  }
  for (int s = n_top + 2 + tid; s < k; s += BS) emit(s, -1, -1);
  if (tid == 0) *cnt_out = n_top + 2;
  if (n_top == 0) return;

  // 3) pivot: the n_top-th largest of the maxima of groups of TR threads
  //    (one value per lane), else of the per-thread maxima, else every
  //    candidate (fewer than n_top threads hold one)
  s_tmax[tid] = tmax;
  __syncthreads();
  if (wave == 0) {
    constexpr int TR = BS / kWave;
    uint32_t gm[1] = {0u};
#pragma unroll
    for (int r = 0; r < TR; ++r) gm[0] = max(gm[0], s_tmax[lane * TR + r]);
    uint32_t piv;
    if (__popcll(__ballot(gm[0] != 0u)) >= n_top) {
      piv = wave_nth_largest<1>(gm, n_top);
    } else {
      uint32_t tv[TR];
      int nz = 0;
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        tv[r] = s_tmax[lane + kWave * r];
        nz += __popcll(__ballot(tv[r] != 0u));
      }
      piv = nz >= n_top ? wave_nth_largest<TR>(tv, n_top) : 1u;
    }
    if (lane == 0) s_pivot = piv;
  }
  __syncthreads();
  const uint32_t piv = s_pivot;

  // 4) compaction of the keys >= pivot, in page order
  int pos[NPT];
  const int c_total = page_order_positions<NPT, NW>([&](int i) { return key[i] >= piv; }, pos, s_cnt[0]);

  if (c_total <= kListFast) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      if (key[i] >= piv) {
        s_ckey[pos[i]] = key[i];
        s_cidx[pos[i]] = page(i);
        s_cphys[pos[i]] = phys_of(i);
      }
    }
    __syncthreads();
    // 5) exact cut on the list by one wave; output in list (= page) order
    if (wave == 0) {
      if (c_total <= kWave) select_from_list<1>(s_ckey, s_cidx, s_cphys, c_total, n_top, sel, selp, a.num_phys);
      else select_from_list<kListFast / kWave>(s_ckey, s_cidx, s_cphys, c_total, n_top, sel, selp, a.num_phys);
    }
    return;
  }

  // Fallback: exact cut t over all keys by block-wide bisection, two bits per
  // barrier (wave counts from ballots), starting below the bits common to the
  // largest and smallest candidate keys.
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < NPT; ++i)
    if (key[i]) { kmax = max(kmax, key[i]); kmin = min(kmin, key[i]); }
  wave_minmax_u32(kmax, kmin);
  uint32_t* ib = reinterpret_cast<uint32_t*>(s_gred);
  if (lane == 0) { ib[wave] = kmax; ib[NW + wave] = kmin; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) { kmax = max(kmax, ib[w]); kmin = min(kmin, ib[NW + w]); }
  __syncthreads();
  uint32_t t = kmax;
  const uint32_t diff = kmax ^ kmin;
  if (diff) {
    const int hb = 31 - __clz(diff);
    t = kmax & ~((hb == 31) ? 0xffffffffu : ((2u << hb) - 1u));
    int par = 0;
    for (int bit = hb; bit >= 0; bit -= 2) {
      const uint32_t b1 = 1u << bit;
      const uint32_t b0 = bit > 0 ? (1u << (bit - 1)) : 0u;
      int c1 = 0, c0 = 0, c3 = 0;
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        c1 += __popcll(__ballot(key[i] >= (t | b1)));
        c0 += __popcll(__ballot(key[i] >= (t | b0)));
        c3 += __popcll(__ballot(key[i] >= (t | b1 | b0)));
      }
      int* cb = reinterpret_cast<int*>(s_gred) + par * 3 * NW;
      if (lane == 0) { cb[wave] = c1; cb[NW + wave] = c0; cb[2 * NW + wave] = c3; }
      __syncthreads();
      c1 = c0 = c3 = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) { c1 += cb[w]; c0 += cb[NW + w]; c3 += cb[2 * NW + w]; }
      par ^= 1;
      if (b0 && c3 >= n_top) t |= b1 | b0;
      else if (c1 >= n_top) t |= b1;
      else if (b0 && c0 >= n_top) t |= b0;
    }
  }
  // keys > t all selected; keys == t by page order, the first n_top - n_gt
  const int n_gt = page_order_positions<NPT, NW>([&](int i) { return key[i] > t; }, pos, s_cnt[1]);
  int eq_rank[NPT];
  page_order_positions<NPT, NW>([&](int i) { return key[i] == t; }, eq_rank, s_cnt[0]);
  const int take_eq = n_top - n_gt;
  auto take = [&](int i) { return key[i] > t || (key[i] == t && eq_rank[i] < take_eq); };
  page_order_positions<NPT, NW>(take, pos, s_cnt[1]);
#pragma unroll
  for (int i = 0; i < NPT; ++i)
    if (take(i)) emit(1 + pos[i], page(i), phys_of(i));
}

}  // namespace lk
