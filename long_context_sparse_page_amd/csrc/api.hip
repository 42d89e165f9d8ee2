// C ABI of the Locks decode path (declared in include/locks.h): argument
// validation, workspace carving and kernel launches.  Host code only; every
// entry point enqueues on the caller's stream and returns without waiting.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/locks.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

// attention: a split is a workgroup of 4 waves; each wave takes this many
// 32-token units (half a 64-token page, or two 16-token pages)
constexpr int kAttnWavesPerSplit = 4;
constexpr int kUnitsPerWaveSparse = 1;
constexpr int kUnitsPerWaveDense = 32;
// the selector holds every page's G scores in registers: 1024 threads x up to
// 96 / G values (24 pages per thread for G <= 4, 12 for G = 8)
constexpr int kMaxPagesPerSeq = 1024 * 24;
int max_pages_for_group(int G) { return G == 8 ? 1024 * 12 : kMaxPagesPerSeq; }
constexpr int kMaxPageBudget = 1024;
constexpr size_t kAlign = 256;

lk_status fail(lk_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lk_status fail(lk_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

lk_status ok() {
  g_last_error.clear();
  return LK_OK;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Shape {
  int d, B, r, hq, hkv, G, k;
  lk::DType dt;
  size_t elem;
  bool q4;  // LK_SUMMARY_I4 records
};

lk_status check_config(const lk_config* cfg, Shape* sh) {
  if (!cfg) return fail(LK_ERR_INVALID_ARG, "config is null");
  if (cfg->head_dim <= 0 || cfg->page_size <= 0 || cfg->rank <= 0 || cfg->num_q_heads <= 0 ||
      cfg->num_kv_heads <= 0 || cfg->token_budget <= 0)
    return fail(LK_ERR_INVALID_ARG, "config sizes must be positive (d=%d B=%d r=%d Hq=%d Hkv=%d b=%d)",
                cfg->head_dim, cfg->page_size, cfg->rank, cfg->num_q_heads, cfg->num_kv_heads,
                cfg->token_budget);
  if (cfg->num_q_heads % cfg->num_kv_heads != 0)
    return fail(LK_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                cfg->num_q_heads, cfg->num_kv_heads);
  if (cfg->kv_dtype != LK_F32 && cfg->kv_dtype != LK_BF16)
    return fail(LK_ERR_INVALID_ARG, "kv_dtype %d is not LK_F32 or LK_BF16", cfg->kv_dtype);
  if (!std::isfinite(cfg->scale)) return fail(LK_ERR_INVALID_ARG, "scale is not finite");
  const int k = (cfg->token_budget + cfg->page_size - 1) / cfg->page_size;
  if (k < 2)
    return fail(LK_ERR_INVALID_ARG, "page budget ceil(b/B) = %d < 2 (the sink and the most recent page need two slots)", k);
  if (cfg->head_dim != 128) return fail(LK_ERR_UNSUPPORTED, "head_dim %d: only 128 is built", cfg->head_dim);
  if (cfg->page_size != 64 && cfg->page_size != 16)
    return fail(LK_ERR_UNSUPPORTED, "page_size %d: built page sizes are 64 and 16", cfg->page_size);
  const int r = cfg->rank;
  if (r != 1 && r != 2 && r != 4 && r != 8 && r != 16)
    return fail(LK_ERR_UNSUPPORTED, "rank %d: built ranks are 1, 2, 4, 8, 16", r);
  const int G = cfg->num_q_heads / cfg->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(LK_ERR_UNSUPPORTED, "GQA group %d: built groups are 1, 2, 4, 8", G);
  if (k > kMaxPageBudget) return fail(LK_ERR_UNSUPPORTED, "page budget %d exceeds %d", k, kMaxPageBudget);
  if (cfg->summary_format != LK_SUMMARY_KV && cfg->summary_format != LK_SUMMARY_I4)
    return fail(LK_ERR_INVALID_ARG, "summary_format %d is not LK_SUMMARY_KV or LK_SUMMARY_I4", cfg->summary_format);
  if (cfg->summary_format == LK_SUMMARY_I4 && cfg->kv_dtype != LK_BF16)
    return fail(LK_ERR_UNSUPPORTED, "LK_SUMMARY_I4 is built for kv_dtype LK_BF16 only");
  if (cfg->summary_format == LK_SUMMARY_I4 && r != 4 && r != 8 && r != 16)
    return fail(LK_ERR_UNSUPPORTED, "LK_SUMMARY_I4 rank %d: built ranks are 4, 8, 16", r);
  sh->d = cfg->head_dim;
  sh->B = cfg->page_size;
  sh->r = r;
  sh->hq = cfg->num_q_heads;
  sh->hkv = cfg->num_kv_heads;
  sh->G = G;
  sh->k = k;
  sh->dt = cfg->kv_dtype == LK_BF16 ? lk::kBF16 : lk::kF32;
  sh->elem = cfg->kv_dtype == LK_BF16 ? 2 : 4;
  sh->q4 = cfg->summary_format == LK_SUMMARY_I4;
  return LK_OK;
}

lk_status check_cache(const lk_cache* c, bool need_kv, bool need_summary) {
  if (!c) return fail(LK_ERR_INVALID_ARG, "cache is null");
  if (need_kv && (!c->k_pool || !c->v_pool)) return fail(LK_ERR_INVALID_ARG, "k_pool / v_pool is null");
  if (need_summary && !c->summary_pool) return fail(LK_ERR_INVALID_ARG, "summary_pool is null");
  if (c->num_phys_pages <= 0) return fail(LK_ERR_INVALID_ARG, "num_phys_pages %d <= 0", c->num_phys_pages);
  return LK_OK;
}

lk_status check_table(const lk_cache* c, const Shape& sh) {
  if (!c->block_table || !c->seq_lens) return fail(LK_ERR_INVALID_ARG, "block_table / seq_lens is null");
  if (c->max_pages_per_seq <= 0) return fail(LK_ERR_INVALID_ARG, "max_pages_per_seq %d <= 0", c->max_pages_per_seq);
  const int lim = max_pages_for_group(sh.G);
  if (c->max_pages_per_seq > lim)
    return fail(LK_ERR_UNSUPPORTED, "max_pages_per_seq %d exceeds %d (GQA group %d)", c->max_pages_per_seq, lim, sh.G);
  return LK_OK;
}

// 32-token attention units over n list entries (pages).
int attn_units(const Shape& sh, int n) { return sh.B == 64 ? 2 * n : (n + 1) / 2; }

// Workspace regions.
struct Layout {
  size_t page_lse, sel_pages, sel_count, sel_phys, part_o, part_ml, build_list, cand_key, cand_page, cand_phys,
      cand_cnt, chunk_ms, total;
  int n_splits;
};

// decode_only: the regions lk_decode_step uses (its attention has the sparse
// split count only); a workspace of the full size serves it too.
Layout layout(const Shape& sh, int batch, int max_pages, bool decode_only = false) {
  Layout L{};
  const int per_sparse = kAttnWavesPerSplit * kUnitsPerWaveSparse;
  const int per_dense = kAttnWavesPerSplit * kUnitsPerWaveDense;
  const int ns_sparse = (attn_units(sh, sh.k) + per_sparse - 1) / per_sparse;
  const int ns_dense = (attn_units(sh, max_pages) + per_dense - 1) / per_dense;
  L.n_splits = (decode_only || ns_sparse > ns_dense) ? ns_sparse : ns_dense;
  size_t off = 0;
  L.page_lse = off; off = align_up(off + sizeof(float) * (size_t)batch * sh.hq * max_pages);
  L.sel_pages = off; off = align_up(off + sizeof(int32_t) * (size_t)batch * sh.hkv * sh.k);
  L.sel_count = off; off = align_up(off + sizeof(int32_t) * (size_t)batch * sh.hkv);
  L.sel_phys = off; off = align_up(off + sizeof(int32_t) * (size_t)batch * sh.hkv * sh.k);
  L.part_o = off; off = align_up(off + sizeof(float) * (size_t)batch * sh.hkv * L.n_splits * sh.G * sh.d);
  L.part_ml = off; off = align_up(off + sizeof(float) * (size_t)batch * sh.hkv * L.n_splits * sh.G * 2);
  L.build_list = off; off = align_up(off + sizeof(int32_t) * (size_t)batch);
  // candidate lists of the chunked selection, reserved whenever the table and
  // budget admit it (whether a call uses it also depends on its pair count)
  const size_t n_lists = (size_t)batch * sh.hkv * lk::select_chunk_capacity(max_pages, sh.k);
  const size_t n_entries = n_lists * (sh.k > 2 ? sh.k - 2 : 0);
  L.cand_key = off; off = align_up(off + sizeof(uint32_t) * n_entries);
  L.cand_page = off; off = align_up(off + sizeof(int32_t) * n_entries);
  L.cand_phys = off; off = align_up(off + sizeof(int32_t) * n_entries);
  L.cand_cnt = off; off = align_up(off + sizeof(int32_t) * n_lists);
  L.chunk_ms = off; off = align_up(off + sizeof(float) * n_lists * sh.G * 2);
  L.total = off;
  return L;
}

lk_status check_ws(const Layout& L, void* ws, size_t ws_bytes) {
  if (ws_bytes < L.total) return fail(LK_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, L.total);
  if (!ws) return fail(LK_ERR_WORKSPACE, "workspace pointer is null");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return fail(LK_ERR_WORKSPACE, "workspace is not %zu-byte aligned", kAlign);
  return LK_OK;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

lk_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// The chunked selection's lists, when the call's shape uses it.
void attach_chunk_lists(lk::SelectArgs& se, void* ws, const Layout& L) {
  se.n_chunks = lk::select_chunks(se.batch, se.hkv, se.max_pages, se.k);
  if (se.n_chunks > 0) {
    se.cand_key = at<uint32_t>(ws, L.cand_key);
    se.cand_page = at<int32_t>(ws, L.cand_page);
    se.cand_phys = at<int32_t>(ws, L.cand_phys);
    se.cand_cnt = at<int32_t>(ws, L.cand_cnt);
    se.chunk_ms = at<float>(ws, L.chunk_ms);
  }
}

// Score (+ the decode step's append when app.k_new is set) and select.
lk_status enqueue_score_select(const Shape& sh, const lk_config* cfg, const lk_cache* c, int batch,
                               const void* q, float* page_lse, float* share_out, int32_t* sel,
                               int32_t* cnt, int32_t* sel_phys, int len_add, const lk::AppendDuty& app,
                               void* ws, const Layout& L, hipStream_t s) {
  lk::ScoreArgs sa{q, c->summary_pool, c->block_table, c->seq_lens, page_lse,
                   batch, c->max_pages_per_seq, c->num_phys_pages, sh.hkv, sh.hq, cfg->scale, len_add, app};
  hipError_t e = lk::launch_score(sh.dt, sh.B, sh.r, sh.G, sh.q4, sa, s);
  if (e != hipSuccess) return hip_status(e, "score launch");
  lk::SelectArgs se{page_lse, share_out, sel, cnt, c->seq_lens, batch, c->max_pages_per_seq,
                    sh.hkv, sh.G, sh.B, sh.k, len_add, c->block_table, sel_phys, c->num_phys_pages};
  attach_chunk_lists(se, ws, L);
  return hip_status(lk::launch_select(se, s), "select launch");
}

lk_status enqueue_attn(const Shape& sh, const lk_config* cfg, const lk_cache* c, int batch,
                       const void* q, const int32_t* sel, const int32_t* cnt, const int32_t* sel_phys,
                       void* out, float* lse_out, void* ws, const Layout& L, int len_add, bool merge,
                       hipStream_t s, int* n_splits_out = nullptr) {
  const bool dense = sel == nullptr;
  const int ups = dense ? kUnitsPerWaveDense : kUnitsPerWaveSparse;
  const int per = kAttnWavesPerSplit * ups;
  const int n_splits = (attn_units(sh, dense ? c->max_pages_per_seq : sh.k) + per - 1) / per;
  lk::AttnArgs aa{q, c->k_pool, c->v_pool, c->block_table, c->seq_lens, sel, cnt, sel_phys,
                  at<float>(ws, L.part_o), at<float>(ws, L.part_ml), out, lse_out,
                  batch, c->max_pages_per_seq, c->num_phys_pages, sh.hkv, sh.hq, sh.k,
                  n_splits, ups, cfg->scale, len_add, sh.B};
  if (n_splits_out) *n_splits_out = n_splits;
  return hip_status(lk::launch_attn(sh.dt, sh.G, aa, merge, s), "attention launch");
}

lk_status check_decode_step(const lk_config* cfg, const lk_cache* cache, int batch, const void* q,
                            const void* k_new, const void* v_new, const void* out, const int32_t* sel_pages,
                            const int32_t* sel_count, Shape* sh) {
  lk_status st = check_config(cfg, sh);
  if (st != LK_OK) return st;
  if ((st = check_cache(cache, true, true)) != LK_OK) return st;
  if ((st = check_table(cache, *sh)) != LK_OK) return st;
  if (batch <= 0) return fail(LK_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (!q || !k_new || !v_new || !out) return fail(LK_ERR_INVALID_ARG, "q / k_new / v_new / out is null");
  if ((sel_pages == nullptr) != (sel_count == nullptr))
    return fail(LK_ERR_INVALID_ARG, "sel_pages and sel_count must both be given or both be null");
  return LK_OK;
}

// The decode step's launches on stream s with workspace ws carved by L.
lk_status enqueue_decode_step(const Shape& sh, const lk_config* cfg, const lk_cache* cache, int batch,
                              const void* q, const void* k_new, const void* v_new, void* out, float* lse_out,
                              int32_t* sel_pages, int32_t* sel_count, void* ws, const Layout& L, hipStream_t s) {
  lk_status st;
  int32_t* build_list = at<int32_t>(ws, L.build_list);
  int32_t* sel_phys = at<int32_t>(ws, L.sel_phys);
  float* page_lse = at<float>(ws, L.page_lse);

  // 1) append (done by the scorer's prologue) + score, with T + 1
  lk::AppendDuty app{cache->k_pool, cache->v_pool, k_new, v_new, build_list};
  lk::ScoreArgs sa{q, cache->summary_pool, cache->block_table, cache->seq_lens, page_lse, batch,
                   cache->max_pages_per_seq, cache->num_phys_pages, sh.hkv, sh.hq, cfg->scale, 1, app};
  st = hip_status(lk::launch_score(sh.dt, sh.B, sh.r, sh.G, sh.q4, sa, s), "score launch");
  if (st != LK_OK) return st;
  // 2-3) selection and the attention splits: one fused launch when the table
  //      fits one workgroup's selection (64-token pages), else a selection then
  //      an attention launch
  lk::SelectArgs se{page_lse, nullptr, sel_pages, sel_count, cache->seq_lens, batch, cache->max_pages_per_seq,
                    sh.hkv, sh.G, sh.B, sh.k, 1, cache->block_table, nullptr, cache->num_phys_pages};
  const bool fused = lk::select_attn_fusable(se);
  int n_merge = fused ? lk::select_attn_splits(sh.k, sh.B) : lk::list_attn_splits(sh.k, sh.B);  // the attention's splits
  if (fused) {
    lk::AttnArgs aa{q, cache->k_pool, cache->v_pool, cache->block_table, cache->seq_lens, nullptr, nullptr, nullptr,
                    at<float>(ws, L.part_o), at<float>(ws, L.part_ml), out, lse_out,
                    batch, cache->max_pages_per_seq, cache->num_phys_pages, sh.hkv, sh.hq, sh.k,
                    n_merge, 1, cfg->scale, 1, sh.B};
    st = hip_status(lk::launch_select_attn(sh.dt, se, aa, s), "selection + attention launch");
    if (st != LK_OK) return st;
  } else {
    int32_t* sel = sel_pages ? sel_pages : at<int32_t>(ws, L.sel_pages);
    int32_t* cnt = sel_count ? sel_count : at<int32_t>(ws, L.sel_count);
    se.sel_pages = sel;
    se.sel_count = cnt;
    se.sel_phys = sel_phys;
    attach_chunk_lists(se, ws, L);
    if (se.n_chunks > 0) {
      // chunked selection: the chunk lists, then attention whose waves merge
      // them (the selection is written only when the caller asked for it)
      se.sel_pages = sel_pages;
      se.sel_count = sel_count;
      st = hip_status(lk::launch_select_lists(se, s), "select launch");
      if (st != LK_OK) return st;
      lk::AttnArgs aa{q, cache->k_pool, cache->v_pool, cache->block_table, cache->seq_lens, nullptr, nullptr, nullptr,
                      at<float>(ws, L.part_o), at<float>(ws, L.part_ml), out, lse_out,
                      batch, cache->max_pages_per_seq, cache->num_phys_pages, sh.hkv, sh.hq, sh.k,
                      n_merge, 1, cfg->scale, 1, sh.B};
      st = hip_status(lk::launch_list_attn(sh.dt, se, aa, s), "attention launch");
      if (st != LK_OK) return st;
    } else {
      st = hip_status(lk::launch_select(se, s), "select launch");
      if (st != LK_OK) return st;
      st = enqueue_attn(sh, cfg, cache, batch, q, sel, cnt, sel_phys, out, lse_out, ws, L, 1, false, s, &n_merge);
      if (st != LK_OK) return st;
    }
  }
  // 4) one launch of (sequence, KV head) workgroups: merge the attention
  //    partials, advance the stored lengths, and summarize pages the append
  //    completed
  lk::BuildArgs ba{cache->k_pool, cache->summary_pool, build_list, nullptr, batch,
                   cache->num_phys_pages, sh.hkv, cache->seq_lens, cache->block_table,
                   cache->max_pages_per_seq,
                   {at<float>(ws, L.part_o), at<float>(ws, L.part_ml), out, lse_out, n_merge, sh.G, sh.hq},
                   sh.q4 ? 1 : 0};
  if (sh.B == 16) return hip_status(lk::launch_build16(sh.dt, sh.r, ba, s), "build launch");
  return hip_status(lk::launch_build(sh.dt, sh.r, ba, s), "build launch");
}

// Workspace of lk_decode_step_noalloc: one static buffer per GPU (each device
// holds its own copy of this array while the library is loaded).  Host code
// uses the device address from hipGetSymbolAddress, taken once per device
// with that device current; the array's name itself is not a device address
// in host code.
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
__device__ __align__(256) static unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

lk_status static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LK_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(LK_ERR_HIP, "hipGetSymbolAddress(scratch) gave no address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return LK_OK;
}

}  // namespace

extern "C" {

size_t lk_summary_record_bytes(const lk_config* cfg) {
  if (!cfg || cfg->head_dim <= 0 || cfg->page_size <= 0 || cfg->rank <= 0) return 0;
  const size_t d = cfg->head_dim, B = cfg->page_size, r = cfg->rank;
  if (cfg->summary_format == LK_SUMMARY_I4) {
    if (d % 2) return 0;
    return (d + r * d / 2 + B * r + 2 * (B + r + 1) + 15) / 16 * 16;
  }
  if (cfg->summary_format != LK_SUMMARY_KV) return 0;
  const size_t e = cfg->kv_dtype == LK_BF16 ? 2 : (cfg->kv_dtype == LK_F32 ? 4 : 0);
  return (d + r * d + B * r) * e;
}

int32_t lk_page_budget(const lk_config* cfg) {
  if (!cfg || cfg->page_size <= 0 || cfg->token_budget <= 0) return 0;
  return (cfg->token_budget + cfg->page_size - 1) / cfg->page_size;
}

lk_status lk_workspace_size(const lk_config* cfg, int32_t batch, int32_t max_pages_per_seq, size_t* bytes) {
  Shape sh;
  lk_status st = check_config(cfg, &sh);
  if (st != LK_OK) return st;
  if (!bytes) return fail(LK_ERR_INVALID_ARG, "bytes is null");
  if (batch <= 0) return fail(LK_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (max_pages_per_seq <= 0) return fail(LK_ERR_INVALID_ARG, "max_pages_per_seq %d <= 0", max_pages_per_seq);
  if (max_pages_per_seq > max_pages_for_group(sh.G))
    return fail(LK_ERR_UNSUPPORTED, "max_pages_per_seq %d exceeds %d (GQA group %d)", max_pages_per_seq,
                max_pages_for_group(sh.G), sh.G);
  *bytes = layout(sh, batch, max_pages_per_seq).total;
  return ok();
}

lk_status lk_build_page_summary(const lk_config* cfg, const lk_cache* cache, const int32_t* phys_page_ids,
                                int32_t n_pages, float* eigvals_out, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  Shape sh;
  lk_status st = check_config(cfg, &sh);
  if (st != LK_OK) return st;
  if (!cache) return fail(LK_ERR_INVALID_ARG, "cache is null");
  if (!cache->k_pool || !cache->summary_pool) return fail(LK_ERR_INVALID_ARG, "k_pool / summary_pool is null");
  if (cache->num_phys_pages <= 0) return fail(LK_ERR_INVALID_ARG, "num_phys_pages %d <= 0", cache->num_phys_pages);
  if (n_pages < 0) return fail(LK_ERR_INVALID_ARG, "n_pages %d < 0", n_pages);
  if (n_pages > 0 && !phys_page_ids) return fail(LK_ERR_INVALID_ARG, "phys_page_ids is null");
  if (n_pages == 0) return ok();
  lk::BuildArgs ba{cache->k_pool, cache->summary_pool, phys_page_ids, eigvals_out, n_pages,
                   cache->num_phys_pages, sh.hkv, nullptr, nullptr, 0, {}, sh.q4 ? 1 : 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (sh.B == 16) return hip_status(lk::launch_build16(sh.dt, sh.r, ba, s), "build launch");
  return hip_status(lk::launch_build(sh.dt, sh.r, ba, s), "build launch");
}

lk_status lk_score_select(const lk_config* cfg, const lk_cache* cache, int32_t batch, const void* q,
                          float* page_lse_out, float* share_out, int32_t* sel_pages, int32_t* sel_count,
                          void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  lk_status st = check_config(cfg, &sh);
  if (st != LK_OK) return st;
  if ((st = check_cache(cache, false, true)) != LK_OK) return st;
  if ((st = check_table(cache, sh)) != LK_OK) return st;
  if (batch <= 0) return fail(LK_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (!q) return fail(LK_ERR_INVALID_ARG, "q is null");
  const bool score_only = sel_pages == nullptr && sel_count == nullptr;
  if (score_only && !page_lse_out)
    return fail(LK_ERR_INVALID_ARG, "score-only call (no sel_pages / sel_count) needs page_lse_out");
  if (!score_only && (!sel_pages || !sel_count))
    return fail(LK_ERR_INVALID_ARG, "sel_pages and sel_count must both be given or both be null");
  if (score_only && share_out)
    return fail(LK_ERR_INVALID_ARG, "share_out needs the selection outputs");
  const Layout L = layout(sh, batch, cache->max_pages_per_seq);
  if ((st = check_ws(L, ws, ws_bytes)) != LK_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (score_only) {
    lk::ScoreArgs sa{q, cache->summary_pool, cache->block_table, cache->seq_lens, page_lse_out, batch,
                     cache->max_pages_per_seq, cache->num_phys_pages, sh.hkv, sh.hq, cfg->scale, 0,
                     lk::AppendDuty{}};
    return hip_status(lk::launch_score(sh.dt, sh.B, sh.r, sh.G, sh.q4, sa, s), "score launch");
  }
  float* lse = page_lse_out ? page_lse_out : at<float>(ws, L.page_lse);
  return enqueue_score_select(sh, cfg, cache, batch, q, lse, share_out, sel_pages, sel_count, nullptr, 0,
                              lk::AppendDuty{}, ws, L, s);
}

lk_status lk_sparse_decode_attn(const lk_config* cfg, const lk_cache* cache, int32_t batch, const void* q,
                                const int32_t* sel_pages, const int32_t* sel_count, void* out,
                                float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  lk_status st = check_config(cfg, &sh);
  if (st != LK_OK) return st;
  if ((st = check_cache(cache, true, false)) != LK_OK) return st;
  if ((st = check_table(cache, sh)) != LK_OK) return st;
  if (batch <= 0) return fail(LK_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (!q || !out || !sel_pages || !sel_count) return fail(LK_ERR_INVALID_ARG, "q / out / sel_pages / sel_count is null");
  const Layout L = layout(sh, batch, cache->max_pages_per_seq);
  if ((st = check_ws(L, ws, ws_bytes)) != LK_OK) return st;
  return enqueue_attn(sh, cfg, cache, batch, q, sel_pages, sel_count, nullptr, out, lse_out, ws, L, 0, true,
                      static_cast<hipStream_t>(stream));
}

lk_status lk_dense_decode_attn(const lk_config* cfg, const lk_cache* cache, int32_t batch, const void* q,
                               void* out, float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  lk_status st = check_config(cfg, &sh);
  if (st != LK_OK) return st;
  if ((st = check_cache(cache, true, false)) != LK_OK) return st;
  if ((st = check_table(cache, sh)) != LK_OK) return st;
  if (batch <= 0) return fail(LK_ERR_INVALID_ARG, "batch %d <= 0", batch);
  if (!q || !out) return fail(LK_ERR_INVALID_ARG, "q / out is null");
  const Layout L = layout(sh, batch, cache->max_pages_per_seq);
  if ((st = check_ws(L, ws, ws_bytes)) != LK_OK) return st;
  return enqueue_attn(sh, cfg, cache, batch, q, nullptr, nullptr, nullptr, out, lse_out, ws, L, 0, true,
                      static_cast<hipStream_t>(stream));
}

lk_status lk_decode_step(const lk_config* cfg, const lk_cache* cache, int32_t batch, const void* q,
                         const void* k_new, const void* v_new, void* out, float* lse_out,
                         int32_t* sel_pages, int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  lk_status st = check_decode_step(cfg, cache, batch, q, k_new, v_new, out, sel_pages, sel_count, &sh);
  if (st != LK_OK) return st;
  const Layout L = layout(sh, batch, cache->max_pages_per_seq, true);
  if ((st = check_ws(L, ws, ws_bytes)) != LK_OK) return st;
  return enqueue_decode_step(sh, cfg, cache, batch, q, k_new, v_new, out, lse_out, sel_pages, sel_count, ws, L,
                             static_cast<hipStream_t>(stream));
}

lk_status lk_decode_step_noalloc(const lk_config* cfg, const lk_cache* cache, int32_t batch, const void* q,
                                 const void* k_new, const void* v_new, void* out, float* lse_out,
                                 int32_t* sel_pages, int32_t* sel_count, void* stream) {
  Shape sh;
  lk_status st = check_decode_step(cfg, cache, batch, q, k_new, v_new, out, sel_pages, sel_count, &sh);
  if (st != LK_OK) return st;
  const Layout L = layout(sh, batch, cache->max_pages_per_seq, true);
  if (L.total > kStaticScratchBytes)
    return fail(LK_ERR_WORKSPACE, "the step needs %zu bytes of workspace, more than the %zu of the static buffer",
                L.total, kStaticScratchBytes);
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != LK_OK) return st;
  return enqueue_decode_step(sh, cfg, cache, batch, q, k_new, v_new, out, lse_out, sel_pages, sel_count, ws, L,
                             static_cast<hipStream_t>(stream));
}

const char* lk_status_string(lk_status status) {
  switch (status) {
    case LK_OK: return "ok";
    case LK_ERR_INVALID_ARG: return "invalid argument";
    case LK_ERR_UNSUPPORTED: return "unsupported configuration";
    case LK_ERR_WORKSPACE: return "workspace missing or too small";
    case LK_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* lk_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
