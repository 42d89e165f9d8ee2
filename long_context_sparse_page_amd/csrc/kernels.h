// Launch wrappers of the Locks kernels (host side; each returns hipError_t).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lk {

enum DType : int { kF32 = 0, kBF16 = 1 };

// Zero-mode rule of both summary builders: a Gram eigenvalue at or below
// kZeroModeRtol * lambda_1 or kZeroModeFloor * sum_i ||k_i||^2 is a zero mode
// (zero basis row and coefficients).
constexpr float kZeroModeRtol = 1e-5f;
constexpr float kZeroModeFloor = 1e-10f;

// Byte layout of a quantized (int4 basis / int8 coefficients and centroid)
// summary record at d = 128, page size b (64 unless given) and rank r:
// centroid int8[d] | basis int4[r][d/2] (byte c of row m: dims 2c in the low
// nibble, 2c+1 in the high one) | coefficients int8[b][r] | coefficient
// scales fp16[b] | basis scales fp16[r] | centroid scale fp16, padded to 16
// bytes.
struct Q4Layout {
  static constexpr int kD = 128;
  int r;
  int b = 64;
  __host__ __device__ constexpr int basis() const { return kD; }
  __host__ __device__ constexpr int coef() const { return kD + r * kD / 2; }
  __host__ __device__ constexpr int cscale() const { return coef() + b * r; }
  __host__ __device__ constexpr int bscale() const { return cscale() + 2 * b; }
  __host__ __device__ constexpr int mscale() const { return bscale() + 2 * r; }
  __host__ __device__ constexpr int bytes() const { return (mscale() + 2 + 15) / 16 * 16; }
};

// The cache append of a decode step, carried out by the scorer's first
// workgroup of every (sequence, KV head): the new key and value go to slot
// T mod B of logical page T / B (T = seq_lens[seq] before the step), and
// build_list[seq] records the outcome: the physical page when the append
// completes it, -1 for any other valid append, -2 when page T / B has no
// physical page (nothing is written and the length is not advanced).
struct AppendDuty {
  void* k_pool;
  void* v_pool;
  const void* k_new;           // [batch][Hkv][d]; nullptr: no append
  const void* v_new;
  int32_t* build_list;         // [batch]
};

// In a decode step every kernel sees T = seq_lens[seq] + len_add (len_add = 1:
// the token appended by this step); the stored length is advanced by the
// step's last kernel.
struct ScoreArgs {
  const void* q;               // [batch][Hq][d]
  const void* summary;         // [num_phys][Hkv][record]
  const int32_t* block_table;  // [batch][max_pages]
  const int32_t* seq_lens;     // [batch]
  float* page_lse;             // [batch][Hq][max_pages]
  int32_t batch, max_pages, num_phys, hkv, hq;
  float scale;
  int32_t len_add;
  AppendDuty app;
};

struct SelectArgs {
  const float* page_lse;       // [batch][Hq][max_pages]
  float* share_out;            // optional [batch][Hkv][max_pages]
  int32_t* sel_pages;          // [batch][Hkv][k]
  int32_t* sel_count;          // [batch][Hkv]
  const int32_t* seq_lens;
  int32_t batch, max_pages, hkv, group, page_size, k;
  int32_t len_add;
  const int32_t* block_table;  // with sel_phys: physical page of every selected page
  int32_t* sel_phys;           // optional [batch][Hkv][k]
  int32_t num_phys;
  // Chunked selection (select_chunks() > 0): per chunk of kSelChunkPages pages
  // its top-(k-2) candidates, in page order, and their count.
  uint32_t* cand_key = nullptr;   // [batch][Hkv][n_chunks][k - 2]
  int32_t* cand_page = nullptr;   // [batch][Hkv][n_chunks][k - 2]
  int32_t* cand_phys = nullptr;   // [batch][Hkv][n_chunks][k - 2], their physical pages
  int32_t* cand_cnt = nullptr;    // [batch][Hkv][n_chunks]
  float* chunk_ms = nullptr;      // [batch][Hkv][n_chunks][G][2]: per-head max and sum of 2^(s2 - max)
  int32_t n_chunks = 0;
};

// Chunked selection of long tables: pages per chunk workgroup, and the chunk
// count a table of max_pages pages with page budget k uses (0: the table is
// selected by one workgroup per (sequence, KV head)).  select_chunk_capacity
// ignores how many pairs there are (it sizes the workspace); select_chunks
// also requires few pairs, where one workgroup per pair would leave most of
// the chip idle.
constexpr int kSelChunkPages = 2048;
int select_chunk_capacity(int max_pages, int k);
int select_chunks(int batch, int hkv, int max_pages, int k);

struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* sel_pages;    // null: every page of the sequence (dense)
  const int32_t* sel_count;
  const int32_t* sel_phys;     // optional: physical pages of sel_pages
  float* part_o;               // [batch][Hkv][n_splits][G][d]
  float* part_ml;              // [batch][Hkv][n_splits][G][2]  (max in log2 units, sum)
  void* out;                   // [batch][Hq][d]
  float* lse_out;              // optional [batch][Hq]
  int32_t batch, max_pages, num_phys, hkv, hq, k, n_splits;
  int32_t pages_per_split;     // 32-token units per wave (4 waves per split)
  float scale;
  int32_t len_add;
  int32_t page_size = 64;      // 64: a unit is half a page; 16: two consecutive list entries
};

struct BuildArgs {
  const void* k_pool;
  void* summary;
  const int32_t* phys_ids;     // [n]; entries < 0 are skipped
  float* eigvals_out;          // optional [n][Hkv][B]
  int32_t n, num_phys, hkv;
  // decode step: workgroup (seq, 0) advances seq_lens[seq] by one when the
  // step's append was valid, i.e. build_list[seq] != -2 (phys_ids is then the
  // build list, n = batch)
  int32_t* commit_seq_lens;
  const int32_t* block_table;
  int32_t max_pages;
  // decode step: workgroup (seq, kvh) first merges the attention partials of
  // (seq, kvh) for its G heads into out / lse_out (merge.part_o == nullptr: no merge)
  struct {
    const float* part_o;
    const float* part_ml;
    void* out;
    float* lse_out;
    int32_t n_splits, group, hq;
  } merge;
  int32_t q4;                  // records in the quantized layout (Q4Layout)
};

// q4: the summary records use Q4Layout (bf16 queries only); page_size 64 or 16
hipError_t launch_score(DType dt, int page_size, int rank, int group, bool q4, const ScoreArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
// Chunked selection without its merge (a.n_chunks > 0): the per-chunk lists
// only, for launch_list_attn.
hipError_t launch_select_lists(const SelectArgs& a, hipStream_t s);
// merge = false leaves the split partials for the decode step's build launch
hipError_t launch_attn(DType dt, int group, const AttnArgs& a, bool merge, hipStream_t s);
hipError_t launch_build(DType dt, int rank, const BuildArgs& a, hipStream_t s);
// Pages of 16 tokens: one wave per (page, KV head); in the decode step (merge
// and length commit set) one 512-thread workgroup per (seq, kvh) merges and
// commits as above, then its wave 0 builds
hipError_t launch_build16(DType dt, int rank, const BuildArgs& a, hipStream_t s);
// Decode step: selection (se) and attention splits (a) in one launch, for
// tables of up to 3,072 pages per sequence at 64-token pages and 8,704 at
// 16-token pages, G <= 4 (select_attn_fusable).
bool select_attn_fusable(const SelectArgs& se);
int select_attn_splits(int k, int page_size);  // attention splits of the fused launch
hipError_t launch_select_attn(DType dt, const SelectArgs& se, const AttnArgs& a, hipStream_t s);
// Decode step with the chunked selection: attention over the selection merged
// from the chunk lists (launch_select_lists) by every attention wave; split 0
// writes the selection when se.sel_pages is set.  One 32-token unit per wave,
// a.n_splits = list_attn_splits(k, page size).
int list_attn_splits(int k, int page_size);
hipError_t launch_list_attn(DType dt, const SelectArgs& se, const AttnArgs& a, hipStream_t s);

}  // namespace lk
