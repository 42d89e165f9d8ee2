// The decode step's merge of the attention split partials, run by the
// launch that ends the step (the summary builders' decode-step launch).
#pragma once

#include "common.cuh"
#include "kernels.h"

namespace lk {

// Decode step: combine the attention split partials of (seq, kvh) for its G
// heads, o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s and
// lse = M + log sum_s e^{m_s - M} l_s (max in log2 units).
// Threads t0, t0 + nt, ... of the caller take one (head, dim) output each;
// the partials of CH splits are loaded together (one round trip).
template <typename T, int CH>
__device__ __forceinline__ void merge_partials_ch(const BuildArgs& a, int seq, int kvh, int t0, int nt) {
  constexpr int D = kHeadDim;
  const int G = a.merge.group;
  const int ns = a.merge.n_splits;
  const float* ml = a.merge.part_ml + ((size_t)seq * a.hkv + kvh) * ns * G * 2;
  const float* ob = a.merge.part_o + ((size_t)seq * a.hkv + kvh) * ns * G * D;
  for (int x = t0; x < G * D; x += nt) {
    const int g = x / D, dim = x % D;
    float M = -INFINITY, ov = 0.f, lv = 0.f;
    for (int c0 = 0; c0 < ns; c0 += CH) {
      float ms[CH], ls[CH], os[CH];
#pragma unroll
      for (int t = 0; t < CH; ++t) {  // clamped, unconditional: no waits between the loads
        const int s0 = min(c0 + t, ns - 1);
        const float2 mlv = *reinterpret_cast<const float2*>(ml + ((size_t)s0 * G + g) * 2);
        ms[t] = mlv.x;
        ls[t] = mlv.y;
        os[t] = ob[((size_t)s0 * G + g) * D + dim];
      }
      float Mc = M;
#pragma unroll
      for (int t = 0; t < CH; ++t)
        if (c0 + t < ns) Mc = vmax(Mc, ms[t]);
      if (Mc == -INFINITY) continue;
      const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mc);  // earlier chunks to the new max
      ov *= r;
      lv *= r;
#pragma unroll
      for (int t = 0; t < CH; ++t) {
        if (c0 + t >= ns) continue;
        const float f = ms[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[t] - Mc);
        ov = fmaf(f, os[t], ov);
        lv = fmaf(f, ls[t], lv);
      }
      M = Mc;
    }
    const int h = kvh * G + g;
    Elem<T>::store(reinterpret_cast<T*>(a.merge.out) + ((size_t)seq * a.merge.hq + h) * D + dim,
                   lv > 0.f ? ov / lv : 0.f);
    if (a.merge.lse_out && dim == 0)
      a.merge.lse_out[(size_t)seq * a.merge.hq + h] =
          lv > 0.f ? (M + __builtin_amdgcn_logf(lv)) * kLn2 : -INFINITY;
  }
}

// Eight splits (the fused launch's count) in one batch without the clamped
// duplicate loads a batch of 16 would issue; more splits in batches of 16.
template <typename T>
__device__ __forceinline__ void merge_partials(const BuildArgs& a, int seq, int kvh, int t0, int nt) {
  if (a.merge.n_splits <= 8) merge_partials_ch<T, 8>(a, seq, kvh, t0, nt);
  else merge_partials_ch<T, 16>(a, seq, kvh, t0, nt);
}

}  // namespace lk
