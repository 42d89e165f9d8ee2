// Share-average and top-k page selection kernel, one workgroup per
// (sequence, KV head); the algorithm is in select_impl.cuh.

#include "select_impl.cuh"

namespace lk {

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

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.k > kMaxSelect || a.group > kMaxGroup) return hipErrorInvalidValue;
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
