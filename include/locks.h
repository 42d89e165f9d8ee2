/*
 * locks.h -- C ABI of the MI355X (gfx950) Locks decode path.
 *
 * The method is "Locks: Page-Local Compact Key Summaries for Efficient
 * Long-Context Decoding" (arXiv 2607.24555), cited here as [Locks]:
 *   - paged KV cache with pages of B consecutive tokens, per-head token
 *     budget b and page budget k = ceil(b / B), of which the sink page and
 *     the most recent page fill two slots ([Locks] §2 "Decode-time attention");
 *   - per-page summary built once when a page completes: centroid mu, basis
 *     V (d x r) and coefficients C = U_r Sigma_r (B x r) from the B x B Gram
 *     eigendecomposition ([Locks] §4 "Build");
 *   - per-step score of every completed page by the reconstructed log-sum-exp
 *     of Eq. (1), page-mass shares averaged over each GQA group, and one shared
 *     selection per KV head: sink + most recent + top-(k-2) by the averaged
 *     share ([Locks] §4 "Score", Cor. 3);
 *   - exact attention over only the selected pages ([Locks] App. E, Stage B).
 *
 * Conventions shared by every entry point
 *   - All pointers named *_pool, q, k_new, v_new, out, lse_out, page_lse_out,
 *     share_out, sel_pages, sel_count, seq_lens, block_table, phys_page_ids,
 *     eigvals_out and ws are DEVICE pointers, allocated and owned by the
 *     caller.  The library allocates nothing, never synchronizes, and keeps no
 *     pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on it; results are valid once the stream
 *     has reached that point.
 *   - Every argument is validated on the host before anything is enqueued.  On
 *     error nothing is enqueued, a status is returned and lk_last_error()
 *     gives a message (thread-local).  A launch failure returns LK_ERR_HIP.
 *     Asynchronous device faults surface at the caller's next synchronization.
 *   - Launch grids are sized from capacities (batch, max_pages_per_seq), never
 *     from device data, so identical arguments give identical launches.
 *   - Device-side content checks: a block-table entry outside
 *     [0, num_phys_pages) or a sequence length beyond the table's capacity is
 *     skipped by the kernels rather than dereferenced.
 *
 * Memory layouts (row-major, element type = kv_dtype unless stated)
 *   k_pool, v_pool   [num_phys_pages][num_kv_heads][B][d]
 *   summary_pool     [num_phys_pages][num_kv_heads][record] where one record is
 *                    centroid[d] | basis[r][d] (row m = m-th basis vector) |
 *                    coeffs[B][r] (row i = c_i) in kv_dtype; with
 *                    summary_format = LK_SUMMARY_I4 the record holds bytes:
 *                    centroid int8[d] | basis int4[r][d/2] (row m in 32-bit
 *                    little-endian words of 8 dims: word g holds dim 8g+2j in nibble j
 *                    and dim 8g+2j+1 in nibble j+4, j = 0..3, two's complement) |
 *                    coeffs int8[B][r] | coefficient scales fp16[B] | basis
 *                    scales fp16[r] | centroid scale fp16, zero-padded to a
 *                    multiple of 16 bytes.  A value is code * scale.
 *                    lk_summary_record_bytes() gives the record size
 *   block_table      int32 [batch][max_pages_per_seq], logical -> physical page
 *   seq_lens         int32 [batch], tokens held by each sequence
 *   q, out           [batch][num_q_heads][d]; query head h reads KV head h / G,
 *                    G = num_q_heads / num_kv_heads
 *   k_new, v_new     [batch][num_kv_heads][d]
 *   page_lse_out     fp32 [batch][num_q_heads][max_pages_per_seq]
 *   share_out        fp32 [batch][num_kv_heads][max_pages_per_seq]
 *   sel_pages        int32 [batch][num_kv_heads][k], logical page indices
 *   sel_count        int32 [batch][num_kv_heads]
 *   lse_out          fp32 [batch][num_q_heads], natural-log LSE of the logits
 *
 * Page roles for a sequence holding T >= 1 tokens: n_mr = (T - 1) / B is the
 * most recent page (holds the newest token, may be partial); pages
 * 0 .. n_mr - 1 are complete and must have summaries; they are the scored
 * pages, and pages 1 .. n_mr - 1 are the selection candidates.
 */
#ifndef LOCKS_H
#define LOCKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LK_OK = 0,
  LK_ERR_INVALID_ARG = 1,  /* null pointer, bad size, inconsistent shapes  */
  LK_ERR_UNSUPPORTED = 2,  /* valid but not built here (e.g. d != 128)      */
  LK_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required    */
  LK_ERR_HIP = 4           /* a HIP launch or runtime call failed           */
} lk_status;

typedef enum { LK_F32 = 0, LK_BF16 = 1 } lk_dtype;

/* Storage of the page summaries ([Locks] §4 "Build", App. D "State
 * accounting"):
 *   LK_SUMMARY_KV  centroid, basis and coefficients in kv_dtype;
 *   LK_SUMMARY_I4  the deployed compact form: int4 basis with one scale per
 *                  basis vector (a column of V), int8 coefficients with one
 *                  scale per token (a row of C) and int8 centroid with one
 *                  scale.  Scales are fp16; the quantization is symmetric,
 *                  s = fp16(max |x| / L) with L = 7 (int4) or 127 (int8),
 *                  code = round-half-even(x / s) clamped to [-L, L], and an
 *                  all-zero row has s = 0.  Needs kv_dtype LK_BF16 and rank
 *                  4, 8 or 16 (the pages quote r = 8, "r8i4"). */
typedef enum { LK_SUMMARY_KV = 0, LK_SUMMARY_I4 = 1 } lk_summary_format;

/* Problem parameters ([Locks] §2, §4): head dimension d, page size B, rank r,
 * GQA grouping, per-head token budget b, storage dtype and logit scale. */
typedef struct {
  int32_t head_dim;      /* d; 128 is supported                              */
  int32_t page_size;     /* B; 64 or 16 (the pages' deployed size)         */
  int32_t rank;          /* r in {1, 2, 4, 8, 16}; modes beyond the page's
                          * nonzero modes are stored as zeros              */
  int32_t num_q_heads;   /* Hq                                               */
  int32_t num_kv_heads;  /* Hkv; G = Hq / Hkv in {1, 2, 4, 8}                */
  int32_t token_budget;  /* b; k = ceil(b / B) must be >= 2                  */
  int32_t kv_dtype;      /* lk_dtype of K, V, q, out, k_new, v_new, summary  */
  float scale;           /* logit scale, normally 1 / sqrt(d)                */
  int32_t summary_format;  /* lk_summary_format                              */
} lk_config;

/* The paged cache of one attention layer. */
typedef struct {
  void* k_pool;
  void* v_pool;
  void* summary_pool;
  const int32_t* block_table;
  int32_t* seq_lens;          /* read by every call; lk_decode_step adds 1   */
  int32_t max_pages_per_seq;  /* columns of block_table                      */
  int32_t num_phys_pages;     /* rows of k_pool / v_pool / summary_pool      */
} lk_cache;

/* Bytes of one (page, KV head) summary record: (d + r*d + B*r) elements of
 * kv_dtype ([Locks] App. D "State accounting": basis d*r, coefficients B*r,
 * centroid d), or for LK_SUMMARY_I4 d + r*d/2 + B*r bytes of codes plus
 * 2*(B + r + 1) bytes of scales, rounded up to 16 (1312 at d = 128, B = 64,
 * r = 8).  Returns 0 for an invalid config. */
size_t lk_summary_record_bytes(const lk_config* cfg);

/* Page budget k = ceil(token_budget / page_size) ([Locks] §2); 0 if invalid. */
int32_t lk_page_budget(const lk_config* cfg);

/* Workspace bytes that every entry point below needs for `batch` sequences of
 * up to `max_pages_per_seq` pages.  One workspace of this size serves all of
 * them, and every smaller batch; it holds intermediate scores, selections,
 * the per-chunk candidate lists that long tables with few (sequence, KV head)
 * pairs are selected through, and attention partials, and its contents need
 * no initialization.  Calls that share a workspace must be ordered on one
 * stream (concurrent calls on one workspace race). */
lk_status lk_workspace_size(const lk_config* cfg, int32_t batch,
                            int32_t max_pages_per_seq, size_t* bytes);

/* Build the summary of each listed physical page for every KV head
 * ([Locks] §4 "Build"; one B x B Gram eigendecomposition per page and head):
 * mu = mean key, D = K - 1 mu^T, D D^T = U Sigma^2 U^T (eigenvalues sorted
 * descending), C = U_r Sigma_r, V = D^T U_r Sigma_r^{-1}.  A mode whose
 * eigenvalue is <= 1e-5 * lambda_1 or <= 1e-10 * sum_i ||k_i||^2 is a zero
 * mode: its basis row and coefficients are written as zeros.  Each basis
 * vector is signed so that its largest-magnitude entry is positive.  The
 * record is written in kv_dtype (round to nearest even).
 *   phys_page_ids  int32 [n_pages] device; entries < 0 are skipped.
 *   eigvals_out    optional fp32 [n_pages][Hkv][B], sorted descending, >= 0.
 * Pages must be full (all B token slots written).  B = 16 (the page-size
 * study of the Locks appendix, Table D.10) uses the same record layout and
 * every rule above, with B = 16. */
lk_status lk_build_page_summary(const lk_config* cfg, const lk_cache* cache,
                                const int32_t* phys_page_ids, int32_t n_pages,
                                float* eigvals_out, void* ws, size_t ws_bytes,
                                void* stream);

/* Score and select for one decode step ([Locks] §4 "Score", Eq. (1), Cor. 3).
 * For each sequence, KV head and scored page j < n_mr, and each query head g
 * of the group:  s_hat_j(q_g) = log sum_i exp(scale * (q_g.mu_j + (V_j^T q_g).c_i)).
 * The share m_hat_g(j) = exp(s_hat_j(q_g)) / sum_{j' < n_mr} exp(s_hat_j'(q_g))
 * is averaged over the group, m_bar_j = (1/G) sum_g m_hat_g(j), and the
 * selection is page 0, page n_mr and the top-(k-2) candidates by m_bar (ties
 * to the lower index), in ascending page order; sel_count = min(k, n_mr + 1)
 * (0 for an empty sequence).  Unused sel_pages slots are set to -1.
 *   page_lse_out  optional; s_hat for j < n_mr (other entries untouched).
 *   share_out     optional; m_bar for j < n_mr (other entries untouched).
 * Score only: with sel_pages and sel_count both NULL, only the page scores are
 * computed (page_lse_out is then required and share_out must be NULL). */
lk_status lk_score_select(const lk_config* cfg, const lk_cache* cache,
                          int32_t batch, const void* q, float* page_lse_out,
                          float* share_out, int32_t* sel_pages,
                          int32_t* sel_count, void* ws, size_t ws_bytes,
                          void* stream);

/* Exact attention of every query head over the tokens of its KV head's
 * selected pages ([Locks] §2; the most recent page contributes its T - n_mr*B
 * filled slots): o = sum_t softmax_t(scale * q.k_t) v_t, written to `out` in
 * kv_dtype, and lse = log sum_t exp(scale * q.k_t) to lse_out (optional).
 * sel_pages / sel_count as written by lk_score_select; entries outside
 * [0, n_mr] are skipped.  Split-K over the page list, merged by LSE. */
lk_status lk_sparse_decode_attn(const lk_config* cfg, const lk_cache* cache,
                                int32_t batch, const void* q,
                                const int32_t* sel_pages,
                                const int32_t* sel_count, void* out,
                                float* lse_out, void* ws, size_t ws_bytes,
                                void* stream);

/* Dense decode attention over every token of every sequence: the same-GPU
 * baseline the sparse path is compared with ([Locks] §5.3 compares against
 * dense decode).  Same outputs as lk_sparse_decode_attn with all pages. */
lk_status lk_dense_decode_attn(const lk_config* cfg, const lk_cache* cache,
                               int32_t batch, const void* q, void* out,
                               float* lse_out, void* ws, size_t ws_bytes,
                               void* stream);

/* One whole decode step on `stream` ([Locks] App. E, Fig. E.1):
 *   1. append k_new / v_new at slot T mod B of page T / B, so the sequence
 *      holds T + 1 tokens (done by the scoring kernel before it scores);
 *   2. score every complete page, share-average, select (as lk_score_select,
 *      with T + 1 tokens);
 *   3. attend over the selection (as lk_sparse_decode_attn);
 *   4. if the append completed a page, build its summary for every KV head
 *      (as lk_build_page_summary).  That page is this step's most recent page,
 *      so it is attended, not scored, and its summary is first scored by the
 *      next step; the result does not depend on when the build runs.  This
 *      last kernel also stores seq_lens[seq] = T + 1.
 * An append whose page is outside the block table (T / B >= max_pages_per_seq
 * or an invalid entry) writes nothing and leaves seq_lens unchanged.
 * sel_pages / sel_count are optional outputs of step 2. */
lk_status lk_decode_step(const lk_config* cfg, const lk_cache* cache,
                         int32_t batch, const void* q, const void* k_new,
                         const void* v_new, void* out, float* lse_out,
                         int32_t* sel_pages, int32_t* sel_count, void* ws,
                         size_t ws_bytes, void* stream);

/* lk_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops or harnesses that forbid hipMalloc): the
 * same step, with the same results, whose workspace is a library-owned static
 * buffer of 128 MiB per GPU instead of a caller's workspace.  It allocates
 * nothing.  The buffer lives while the library is loaded; every call on one
 * GPU uses that GPU's buffer, so calls that overlap on one GPU (on different
 * streams, or from different threads) race, and must be ordered by the
 * caller.  A step whose workspace (the decode-step part of
 * lk_workspace_size) exceeds 128 MiB returns LK_ERR_WORKSPACE with nothing
 * enqueued.  Every other argument is as for lk_decode_step. */
lk_status lk_decode_step_noalloc(const lk_config* cfg, const lk_cache* cache,
                                 int32_t batch, const void* q,
                                 const void* k_new, const void* v_new,
                                 void* out, float* lse_out, int32_t* sel_pages,
                                 int32_t* sel_count, void* stream);

/* Static text for a status code. */
const char* lk_status_string(lk_status status);

/* Message of the last failed call on this thread ("" if none). */
const char* lk_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LOCKS_H */
