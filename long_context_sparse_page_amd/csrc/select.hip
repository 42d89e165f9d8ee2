// Share-average and top-k page selection kernels.  select_kernel: one
// workgroup per (sequence, KV head), the algorithm in select_impl.cuh.
//
// Chunked selection (long tables, few pairs): one workgroup per pair leaves
// most of the chip idle when a table holds thousands of pages and only a few
// pairs exist (one 1M-token sequence: 8 pairs of 16,383 candidates each), and
// one CU reads a pair's scores slowly.  There the pair's pages are split into
// chunks of kSelChunkPages, each read by one workgroup only:
//   select_part_kernel, per (chunk, pair): per-head max and sum of 2^(s2 - max)
//     over the chunk's scored pages;
//   select_chunk_kernel, per (chunk, pair): the normalizers M_g, S_g from the
//     pair's chunk partials (every workgroup combines them in the same order,
//     hence to the same values); m_bar and the ranking key of the chunk's
//     pages, as select_block; the chunk's top-(k-2) by (key descending, page
//     ascending) as select_block finds a selection (pivot from group maxima,
//     compaction, one wave's exact cut), written in page order (all
//     candidates when fewer);
//   select_merge_kernel, one wave per pair: the top-(k-2) of the concatenated
//     chunk lists, ties to the earlier entry = the lower page, written as
//     select_block writes the selection (lk_score_select; the decode step
//     instead merges the lists in its attention launch, list_attn_kernel).
// A page of a top-(k-2) under that order is within the top-(k-2) of any
// subset holding it (its chunk), so the lists hold every page the pair's
// selection needs.

#include "select_impl.cuh"

namespace lk {

namespace {
constexpr int kChunkThreads = 512;
constexpr int kChunkNPT = kSelChunkPages / kChunkThreads;  // pages per thread of its chunk
constexpr int kPartThreads = 256;
constexpr int kPartNPT = kSelChunkPages / kPartThreads;
constexpr int kChunkedFrom = 3072;                        // tables above this many pages
constexpr int kChunkMaxTop = 126;                         // k - 2 the lists hold
constexpr int kChunkMaxChunks = 12;
constexpr int kChunkMaxEntries = 12 * kWave;              // list slots one merging wave holds
constexpr int kChunkPairsBelow = 128;                     // fewer pairs than this
static_assert(kChunkNPT * kChunkThreads == kSelChunkPages, "chunk tiling");

}  // namespace

int select_chunk_capacity(int max_pages, int k) {
  if (max_pages <= kChunkedFrom || k < 3 || k - 2 > kChunkMaxTop) return 0;
  const int c = (max_pages + kSelChunkPages - 1) / kSelChunkPages;
  return (c <= kChunkMaxChunks && c * (k - 2) <= kChunkMaxEntries) ? c : 0;
}

int select_chunks(int batch, int hkv, int max_pages, int k) {
  return batch * hkv < kChunkPairsBelow ? select_chunk_capacity(max_pages, k) : 0;
}

// Scored-page range, candidate count and kept count of one (sequence, KV head).
struct PairPages {
  int n_mr, n_scored, n_cand, n_top;
};
__device__ __forceinline__ PairPages pair_pages(const SelectArgs& a, int seq) {
  const int len = a.seq_lens[seq] + a.len_add;
  int n_mr = len > 0 ? (len - 1) / a.page_size : 0;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  const int n_cand = n_mr > 1 ? n_mr - 1 : 0;
  return {n_mr, n_mr, n_cand, min(a.k - 2, n_cand)};
}

template <int G>
__global__ __launch_bounds__(kPartThreads) void select_part_kernel(SelectArgs a) {
  constexpr int BS = kPartThreads, NPT = kPartNPT, NW = BS / kWave;
  __shared__ float s_pm[G][NW], s_ps[G][NW];
  const int chunk = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const size_t pair = (size_t)seq * a.hkv + kvh;
  const float* lse = a.page_lse + ((size_t)seq * a.hkv * G + (size_t)kvh * G) * a.max_pages;
  const int p0 = chunk * kSelChunkPages;
  float x[G][NPT];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NPT; ++i) x[g][i] = lse[(size_t)g * a.max_pages + min(p0 + tid + BS * i, a.max_pages - 1)];
  const PairPages pp = pair_pages(a, seq);
  float* out = a.chunk_ms + (pair * a.n_chunks + chunk) * G * 2;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      x[g][i] = p0 + tid + BS * i < pp.n_scored ? x[g][i] * kLog2e : -INFINITY;
      m = vmax(m, x[g][i]);
    }
    float sl = 0.f;
#pragma unroll
    for (int i = 0; i < NPT; ++i) sl += x[g][i] == -INFINITY ? 0.f : fast_exp2(x[g][i] - m);
    const float wm = wave_max(m);
    const float ws = wave_sum(wm == -INFINITY || m == -INFINITY ? 0.f : sl * fast_exp2(m - wm));
    if (lane == 0) { s_pm[g][wave] = wm; s_ps[g][wave] = ws; }
  }
  __syncthreads();
  if (tid < G) {
    const int g = tid;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = vmax(M, s_pm[g][w]);
    float S = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) S += s_pm[g][w] == -INFINITY ? 0.f : s_ps[g][w] * fast_exp2(s_pm[g][w] - M);
    out[2 * g] = M;
    out[2 * g + 1] = S;
  }
}

template <int G>
__global__ __launch_bounds__(kChunkThreads) void select_chunk_kernel(SelectArgs a) {
  constexpr int BS = kChunkThreads;
  constexpr int NPT = kChunkNPT;
  constexpr int NW = BS / kWave;
  constexpr int TR = BS / kWave;  // threads per pivot group (one group per lane)
  static_assert(kChunkMaxChunks <= kWave, "one lane per chunk partial");
  __shared__ uint32_t s_tmax[BS];
  __shared__ int s_cnt[2][NPT * NW];
  __shared__ uint32_t s_ckey[kListFast];
  __shared__ int s_cidx[kListFast];
  __shared__ int s_cphys[kListFast];
  __shared__ uint32_t s_ib[2 * NW];
  __shared__ int s_cb[2][3 * NW];
  __shared__ uint32_t s_pivot;

  const int chunk = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const size_t pair = (size_t)seq * a.hkv + kvh;
  const int ktop = a.k - 2;
  const float* lse = a.page_lse + ((size_t)seq * a.hkv * G + (size_t)kvh * G) * a.max_pages;
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;
  int32_t* cc = a.cand_cnt + pair * a.n_chunks + chunk;
  uint32_t* ck_out = a.cand_key + (pair * a.n_chunks + chunk) * ktop;
  int32_t* cp_out = a.cand_page + (pair * a.n_chunks + chunk) * ktop;
  int32_t* cq_out = a.cand_phys + (pair * a.n_chunks + chunk) * ktop;
  float* so = a.share_out ? a.share_out + pair * a.max_pages : nullptr;
  const int p0 = chunk * kSelChunkPages;
  auto page = [&](int i) { return p0 + tid + BS * i; };
  // everything that needs no length first: this chunk's scores and
  // block-table entries, and the pair's chunk partials (lane c: chunk c)
  float xs[G][NPT];
  int ph[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
#pragma unroll
    for (int g = 0; g < G; ++g) xs[g][i] = lse[(size_t)g * a.max_pages + min(page(i), a.max_pages - 1)];
    ph[i] = bt[min(page(i), a.max_pages - 1)];
  }
  float pm[G], ps[G];
  {
    const float* ms = a.chunk_ms + (pair * a.n_chunks + min(lane, a.n_chunks - 1)) * G * 2;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      pm[g] = lane < a.n_chunks ? ms[2 * g] : -INFINITY;
      ps[g] = lane < a.n_chunks ? ms[2 * g + 1] : 0.f;
    }
  }
  const PairPages pp = pair_pages(a, seq);
  // nothing of this chunk is scored, or every page is selected and no shares
  // are asked for: the merge needs no list from this chunk
  if (p0 >= pp.n_scored || (pp.n_top == pp.n_cand && !so)) {
    if (tid == 0) *cc = 0;
    return;
  }

  // 1) normalizers from the chunk partials (wave reductions over lanes = chunks:
  //    the same values in every chunk workgroup of the pair)
  float Mg[G], log2S[G], inv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = wave_max(pm[g]);
    const float S = wave_sum(pm[g] == -INFINITY ? 0.f : ps[g] * fast_exp2(pm[g] - M));
    Mg[g] = M;
    log2S[g] = fast_log2(S);
    inv[g] = (M == -INFINITY || !(S > 0.f)) ? 0.f : 1.f / S;  // 2^(s2 - M_g) / S_g
  }

  // 2) shares and ranking keys of this chunk's pages
  const float invG = 1.f / (float)G;
  const float log2G = fast_log2((float)G);
  uint32_t key[NPT];
  uint32_t tmax = 0u;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = page(i);
    key[i] = 0u;
    if (j >= pp.n_scored) continue;
    float x[G], e[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      x[g] = xs[g][i] * kLog2e;
      e[g] = Mg[g] == -INFINITY ? 0.f : fast_exp2(x[g] - Mg[g]);
    }
    float mb;
    const float lm = share_log2<G>(x, e, inv, Mg, log2S, invG, log2G, mb);
    if (so) so[j] = mb;
    if (j >= 1) {  // candidates: pages 1 .. n_mr - 1
      key[i] = order_key(lm);
      tmax = max(tmax, key[i]);
    }
  }
  if (pp.n_top == pp.n_cand) {  // every page is selected; the shares are written
    if (tid == 0) *cc = 0;
    return;
  }

  // 3) the chunk's candidates: all of them when at most k - 2 (the chunk's
  //    candidate pages are the range [max(p0, 1), min(p0 + chunk, n_mr))),
  //    else its top-(k-2) by pivot, compaction and one wave's exact cut
  int pos[NPT];
  const int c_lo = max(p0, 1), c_hi = min(p0 + kSelChunkPages, pp.n_mr);
  if (c_hi - c_lo <= ktop) {
    const int n = page_order_positions<NPT, NW>([&](int i) { return key[i] != 0u; }, pos, s_cnt[0]);
#pragma unroll
    for (int i = 0; i < NPT; ++i)
      if (key[i]) { ck_out[pos[i]] = key[i]; cp_out[pos[i]] = page(i); cq_out[pos[i]] = ph[i]; }
    if (tid == 0) *cc = n;
    return;
  }
  s_tmax[tid] = tmax;
  __syncthreads();
  if (wave == 0) {
    uint32_t gm[1] = {0u};
#pragma unroll
    for (int r = 0; r < TR; ++r) gm[0] = max(gm[0], s_tmax[lane * TR + r]);
    uint32_t piv;
    if (__popcll(__ballot(gm[0] != 0u)) >= ktop) {
      piv = wave_nth_largest<1>(gm, ktop);
    } else {
      uint32_t tv[TR];
      int nz = 0;
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        tv[r] = s_tmax[lane + kWave * r];
        nz += __popcll(__ballot(tv[r] != 0u));
      }
      piv = nz >= ktop ? wave_nth_largest<TR>(tv, ktop) : 1u;
    }
    if (lane == 0) s_pivot = piv;
  }
  __syncthreads();
  const uint32_t piv = s_pivot;
  const int c_total = page_order_positions<NPT, NW>([&](int i) { return key[i] >= piv; }, pos, s_cnt[1]);
  if (c_total <= kListFast) {
#pragma unroll
    for (int i = 0; i < NPT; ++i)
      if (key[i] >= piv) { s_ckey[pos[i]] = key[i]; s_cidx[pos[i]] = page(i); s_cphys[pos[i]] = ph[i]; }
    __syncthreads();
    if (wave == 0) {
      constexpr int CR = kListFast / kWave;
      uint32_t ck[CR];
#pragma unroll
      for (int r = 0; r < CR; ++r) {
        const int x = lane + kWave * r;
        ck[r] = x < c_total ? s_ckey[x] : 0u;
      }
      const int n = min(ktop, c_total);  // fewer only when non-finite scores leave zero keys
      wave_take_in_order<CR>(ck, n, [&](int slot, int r) {
        const int x = lane + kWave * r;
        ck_out[slot] = ck[r];
        cp_out[slot] = s_cidx[x];
        cq_out[slot] = s_cphys[x];
      });
      if (lane == 0) *cc = n;
    }
    return;
  }
  //    massive ties at the pivot: the exact cut t over all the chunk's keys by
  //    block-wide bisection, two bits per barrier, as select_block
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < NPT; ++i)
    if (key[i]) { kmax = max(kmax, key[i]); kmin = min(kmin, key[i]); }
  wave_minmax_u32(kmax, kmin);
  if (lane == 0) { s_ib[wave] = kmax; s_ib[NW + wave] = kmin; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) { kmax = max(kmax, s_ib[w]); kmin = min(kmin, s_ib[NW + w]); }
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
      int* cb = s_cb[par];
      if (lane == 0) { cb[wave] = c1; cb[NW + wave] = c0; cb[2 * NW + wave] = c3; }
      __syncthreads();
      c1 = c0 = c3 = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) { c1 += cb[w]; c0 += cb[NW + w]; c3 += cb[2 * NW + w]; }
      par ^= 1;
      if (b0 && c3 >= ktop) t |= b1 | b0;
      else if (c1 >= ktop) t |= b1;
      else if (b0 && c0 >= ktop) t |= b0;
    }
  }
  // keys > t all kept; keys == t by page order, the first ktop - n_gt
  const int n_gt = page_order_positions<NPT, NW>([&](int i) { return key[i] > t; }, pos, s_cnt[0]);
  int eq_rank[NPT];
  page_order_positions<NPT, NW>([&](int i) { return key[i] == t; }, eq_rank, s_cnt[1]);
  const int take_eq = ktop - n_gt;
  auto take = [&](int i) { return key[i] > t || (key[i] == t && eq_rank[i] < take_eq); };
  page_order_positions<NPT, NW>(take, pos, s_cnt[0]);
#pragma unroll
  for (int i = 0; i < NPT; ++i)
    if (take(i)) { ck_out[pos[i]] = key[i]; cp_out[pos[i]] = page(i); cq_out[pos[i]] = ph[i]; }
  if (tid == 0) *cc = ktop;
}

template <int CR>
__global__ __launch_bounds__(kWave) void select_merge_kernel(SelectArgs a) {
  const int kvh = blockIdx.x, seq = blockIdx.y;
  const int lane = threadIdx.x;
  const size_t pair = (size_t)seq * a.hkv + kvh;
  const int k = a.k, ktop = k - 2, C = a.n_chunks;
  int32_t* sel = a.sel_pages + pair * k;
  int32_t* selp = a.sel_phys ? a.sel_phys + pair * k : nullptr;
  const int32_t* bt = a.block_table + (size_t)seq * a.max_pages;
  auto valid_phys = [&](int ph) { return (ph >= 0 && ph < a.num_phys) ? ph : -1; };
  // the list slots at their fixed places (chunk c, entry i) with the chunk
  // counts, in one round trip; slot order is page order
  uint32_t ck[CR];
  int cp[CR], cq[CR];
#pragma unroll
  for (int r = 0; r < CR; ++r) {
    const int x = lane + kWave * r;
    const int c = x / ktop, i = x - c * ktop;
    const bool in = c < C;
    const size_t at = pair * C * ktop + (in ? x : 0);
    const int n = a.cand_cnt[pair * C + (in ? c : 0)];
    const uint32_t kv = a.cand_key[at];
    ck[r] = (in && i < n) ? kv : 0u;
    cp[r] = a.cand_page[at];
    cq[r] = a.cand_phys[at];
  }
  const int len = a.seq_lens[seq] + a.len_add;
  int n_mr = len > 0 ? (len - 1) / a.page_size : 0;
  if (n_mr > a.max_pages - 1) n_mr = a.max_pages - 1;
  const int ph0 = bt[0], phr = bt[n_mr];
  if (len <= 0) {
    for (int s = lane; s < k; s += kWave) {
      sel[s] = -1;
      if (selp) selp[s] = -1;
    }
    if (lane == 0) a.sel_count[pair] = 0;
    return;
  }
  const int n_cand = n_mr > 0 ? n_mr - 1 : 0;
  if (min(ktop, n_cand) == n_cand) {  // every page 0 .. n_mr
    for (int s = lane; s < k; s += kWave) {
      sel[s] = s <= n_mr ? s : -1;
      if (selp) selp[s] = s <= n_mr ? valid_phys(bt[s]) : -1;
    }
    if (lane == 0) a.sel_count[pair] = n_mr + 1;
    return;
  }
  // k - 2 entries, fewer only if non-finite scores left keys at zero
  int nz = 0;
#pragma unroll
  for (int r = 0; r < CR; ++r) nz += __popcll(__ballot(ck[r] != 0u));
  const int n_top = min(ktop, nz);
  if (lane == 0) {
    sel[0] = 0;
    sel[n_top + 1] = n_mr;
    if (selp) { selp[0] = valid_phys(ph0); selp[n_top + 1] = valid_phys(phr); }
    a.sel_count[pair] = n_top + 2;
  }
  for (int s = n_top + 2 + lane; s < k; s += kWave) {
    sel[s] = -1;
    if (selp) selp[s] = -1;
  }
  if (n_top > 0) wave_take_in_order<CR>(ck, n_top, [&](int slot, int r) {
    sel[1 + slot] = cp[r];
    if (selp) selp[1 + slot] = valid_phys(cq[r]);
  });
}

template <int G>
static hipError_t launch_chunked_g(const SelectArgs& a, hipStream_t s, bool merge) {
  const dim3 cg(a.n_chunks, a.hkv, a.batch);
  hipLaunchKernelGGL((select_part_kernel<G>), cg, dim3(kPartThreads), 0, s, a);
  hipLaunchKernelGGL((select_chunk_kernel<G>), cg, dim3(kChunkThreads), 0, s, a);
  if (!merge) return hipGetLastError();
  const int entries = a.n_chunks * (a.k - 2);  // list slots, all read by the merge
  const dim3 mg(a.hkv, a.batch);
  if (entries <= kWave) hipLaunchKernelGGL((select_merge_kernel<1>), mg, dim3(kWave), 0, s, a);
  else if (entries <= 2 * kWave) hipLaunchKernelGGL((select_merge_kernel<2>), mg, dim3(kWave), 0, s, a);
  else if (entries <= 4 * kWave) hipLaunchKernelGGL((select_merge_kernel<4>), mg, dim3(kWave), 0, s, a);
  else if (entries <= 8 * kWave) hipLaunchKernelGGL((select_merge_kernel<8>), mg, dim3(kWave), 0, s, a);
  else if (entries <= 12 * kWave) hipLaunchKernelGGL((select_merge_kernel<12>), mg, dim3(kWave), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

static hipError_t launch_chunked(const SelectArgs& a, hipStream_t s, bool merge) {
  if (a.n_chunks != select_chunks(a.batch, a.hkv, a.max_pages, a.k) || a.n_chunks <= 0 || !a.cand_key ||
      !a.cand_page || !a.cand_phys || !a.cand_cnt || !a.chunk_ms)
    return hipErrorInvalidValue;
  switch (a.group) {
    case 1: return launch_chunked_g<1>(a, s, merge);
    case 2: return launch_chunked_g<2>(a, s, merge);
    case 4: return launch_chunked_g<4>(a, s, merge);
    case 8: return launch_chunked_g<8>(a, s, merge);
    default: return hipErrorInvalidValue;
  }
}

template <int BS, int NPT, int G>
__global__ __launch_bounds__(BS) void select_kernel(SelectArgs a) {
  const int kvh = blockIdx.x;
  const int seq = blockIdx.y;
  const size_t pair = (size_t)seq * a.hkv + kvh;
  select_block<BS, NPT, G>(a, seq, kvh, a.seq_lens[seq], a.sel_pages + pair * a.k, a.sel_count + pair,
                           a.sel_phys ? a.sel_phys + pair * a.k : nullptr);
}

template <int BS, int NPT>
static hipError_t launch_sel_g(int G, dim3 grid, const SelectArgs& a, hipStream_t s) {
  switch (G) {
    case 1: hipLaunchKernelGGL((select_kernel<BS, NPT, 1>), grid, dim3(BS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((select_kernel<BS, NPT, 2>), grid, dim3(BS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((select_kernel<BS, NPT, 4>), grid, dim3(BS), 0, s, a); break;
    case 8:
      if constexpr (NPT * 8 <= 96) {
        hipLaunchKernelGGL((select_kernel<BS, NPT, 8>), grid, dim3(BS), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_select_lists(const SelectArgs& a, hipStream_t s) {
  if (a.k > kMaxSelect || a.group > kMaxGroup || a.n_chunks <= 0) return hipErrorInvalidValue;
  return launch_chunked(a, s, false);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.k > kMaxSelect || a.group > kMaxGroup) return hipErrorInvalidValue;
  if (a.n_chunks > 0) return launch_chunked(a, s, true);
  const int n = a.max_pages;  // bound on scored pages per sequence
  const int G = a.group;
  dim3 grid(a.hkv, a.batch);
  // smallest (block, pages per thread) covering n pages with G * NPT <= 96
  if (n <= 256 * 4) return launch_sel_g<256, 4>(G, grid, a, s);
  if (n <= 256 * 8) return launch_sel_g<256, 8>(G, grid, a, s);
  if (n <= 256 * 12) return launch_sel_g<256, 12>(G, grid, a, s);
  if (n <= 1024 * 8) return launch_sel_g<1024, 8>(G, grid, a, s);
  if (n <= 1024 * 12) return launch_sel_g<1024, 12>(G, grid, a, s);
  if (n <= 1024 * 17 && G <= 4) return launch_sel_g<1024, 17>(G, grid, a, s);
  if (n <= 1024 * 24 && G <= 4) return launch_sel_g<1024, 24>(G, grid, a, s);
  return hipErrorInvalidValue;
}

}  // namespace lk
