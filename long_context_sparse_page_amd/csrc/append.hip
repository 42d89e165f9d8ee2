// Cache append for one decode step: the new token's key and value go to slot
// T mod B of logical page T / B ([Locks] §2: pages of B consecutive tokens),
// then T += 1.  When the append fills its page, the page's physical index is
// recorded in build_list[seq] (else -1) so the builder can summarize it.
//
// One workgroup per sequence; every KV head's row is copied with 16-byte
// stores before the single thread that owns seq_lens[seq] advances it.

#include "common.cuh"
#include "kernels.h"

namespace lk {

template <typename T>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int B = 64;
  constexpr int D = kHeadDim;
  constexpr int VEC = 16 / sizeof(T);     // elements per 16-byte chunk
  constexpr int CHUNKS = D / VEC;          // chunks per row
  const int seq = blockIdx.x;
  const int len = a.seq_lens[seq];
  const int page = len / B;
  const int slot = len % B;
  bool ok = len >= 0 && page < a.max_pages;
  int phys = -1;
  if (ok) {
    phys = a.block_table[(size_t)seq * a.max_pages + page];
    ok = phys >= 0 && phys < a.num_phys;
  }
  if (ok) {
    const int total = a.hkv * CHUNKS;
    for (int w = threadIdx.x; w < 2 * total; w += blockDim.x) {
      const int which = w / total;  // 0: key, 1: value
      const int h = (w % total) / CHUNKS;
      const int ch = w % CHUNKS;
      const T* src = reinterpret_cast<const T*>(which ? a.v_new : a.k_new) +
                     ((size_t)seq * a.hkv + h) * D + ch * VEC;
      T* dst = reinterpret_cast<T*>(which ? a.v_pool : a.k_pool) +
               ((((size_t)phys * a.hkv + h) * B) + slot) * D + ch * VEC;
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (ok) a.seq_lens[seq] = len + 1;
    a.build_list[seq] = (ok && slot == B - 1) ? phys : -1;
  }
}

hipError_t launch_append(DType dt, const AppendArgs& a, hipStream_t s) {
  if (dt == kBF16) hipLaunchKernelGGL(append_kernel<bf16_t>, dim3(a.batch), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(append_kernel<float>, dim3(a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lk
