// Launch wrappers of the Locks kernels (host side; each returns hipError_t).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lk {

enum DType : int { kF32 = 0, kBF16 = 1 };

struct ScoreArgs {
  const void* q;               // [batch][Hq][d]
  const void* summary;         // [num_phys][Hkv][record]
  const int32_t* block_table;  // [batch][max_pages]
  const int32_t* seq_lens;     // [batch]
  float* page_lse;             // [batch][Hq][max_pages]
  int32_t batch, max_pages, num_phys, hkv, hq;
  float scale;
};

struct SelectArgs {
  const float* page_lse;       // [batch][Hq][max_pages]
  float* share_out;            // optional [batch][Hkv][max_pages]
  int32_t* sel_pages;          // [batch][Hkv][k]
  int32_t* sel_count;          // [batch][Hkv]
  const int32_t* seq_lens;
  int32_t batch, max_pages, hkv, group, page_size, k;
};

struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* sel_pages;    // null: every page of the sequence (dense)
  const int32_t* sel_count;
  float* part_o;               // [batch][Hkv][n_splits][G][d]
  float* part_ml;              // [batch][Hkv][n_splits][G][2]  (max in log2 units, sum)
  void* out;                   // [batch][Hq][d]
  float* lse_out;              // optional [batch][Hq]
  int32_t batch, max_pages, num_phys, hkv, hq, k, n_splits, pages_per_split;
  float scale;
};

struct BuildArgs {
  const void* k_pool;
  void* summary;
  const int32_t* phys_ids;     // [n]; entries < 0 are skipped
  float* eigvals_out;          // optional [n][Hkv][B]
  int32_t n, num_phys, hkv;
};

struct AppendArgs {
  void* k_pool;
  void* v_pool;
  const void* k_new;           // [batch][Hkv][d]
  const void* v_new;
  const int32_t* block_table;
  int32_t* seq_lens;
  int32_t* build_list;         // [batch]: physical page completed by this append, else -1
  int32_t batch, max_pages, num_phys, hkv;
};

hipError_t launch_score(DType dt, int rank, int group, const ScoreArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_attn(DType dt, int group, const AttnArgs& a, hipStream_t s);
hipError_t launch_build(DType dt, int rank, const BuildArgs& a, hipStream_t s);
hipError_t launch_append(DType dt, const AppendArgs& a, hipStream_t s);

}  // namespace lk
