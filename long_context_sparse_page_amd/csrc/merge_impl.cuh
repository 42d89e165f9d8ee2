// The decode step's merge of the attention split partials, run by the
// launch that ends the step (the summary builders' decode-step launch).
#pragma once

#include "common.cuh"
#include "kernels.h"

namespace lk {

// Decode step: combine the attention split partials of (seq, kvh) for its G
// heads, o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s and
// lse = M + log sum_s e^{m_s - M} l_s (max in log2 units).
// Threads t0, t0 + nt, ... of the caller take one (head, dim) output each.
template <typename T>
__device__ __forceinline__ void merge_partials(const BuildArgs& a, int seq, int kvh, int t0, int nt) {
  constexpr int D = kHeadDim;
  constexpr int CH = 16;  // splits whose partials are loaded together (one round trip)
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

// The same merge by one wave for (seq, kvh): lane l holds dims W (l % 32) ..
// W (l % 32) + W - 1 of heads 2 u + l / 32, u < G / 2 (G = 1: dims 2 l, 2 l + 1
// of the one head), so every output of the pair is owned by one lane and the
// partials of CH splits are requested together with vector loads (a few
// round trips for the whole pair instead of one per output).
template <typename T, int G>
__device__ __forceinline__ void merge_partials_wave(const BuildArgs& a, int seq, int kvh, int lane) {
  constexpr int D = kHeadDim;
  constexpr int W = G == 1 ? 2 : 4;         // dims per lane and head
  constexpr int HPL = G == 1 ? 1 : G / 2;  // heads per lane
  constexpr int CH = G <= 4 ? 8 : 4;  // splits per round trip (one for the fused launch's 8 at G <= 4)
  static_assert(HPL * W * kWave == G * D, "every output owned by one lane");
  const int ns = a.merge.n_splits;
  const int hsub = G == 1 ? 0 : lane / 32;
  const int d0 = G == 1 ? W * lane : W * (lane % 32);
  const float* ml = a.merge.part_ml + ((size_t)seq * a.hkv + kvh) * ns * G * 2;
  const float* ob = a.merge.part_o + ((size_t)seq * a.hkv + kvh) * ns * G * D;
  float M[HPL], lv[HPL], ov[HPL][W];
#pragma unroll
  for (int u = 0; u < HPL; ++u) {
    M[u] = -INFINITY;
    lv[u] = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) ov[u][w] = 0.f;
  }
  for (int c0 = 0; c0 < ns; c0 += CH) {
    float ms[CH][HPL], ls[CH][HPL], os[CH][HPL][W];
#pragma unroll
    for (int t = 0; t < CH; ++t) {  // clamped, unconditional: no waits between the loads
      const int s0 = min(c0 + t, ns - 1);
#pragma unroll
      for (int u = 0; u < HPL; ++u) {
        const int g = 2 * u + hsub;
        const float2 mlv = *reinterpret_cast<const float2*>(ml + ((size_t)s0 * G + g) * 2);
        ms[t][u] = mlv.x;
        ls[t][u] = mlv.y;
        const float* op = ob + ((size_t)s0 * G + g) * D + d0;
        if constexpr (W == 4) {
          const float4 v = *reinterpret_cast<const float4*>(op);
          os[t][u][0] = v.x; os[t][u][1] = v.y; os[t][u][2] = v.z; os[t][u][3] = v.w;
        } else {
          const float2 v = *reinterpret_cast<const float2*>(op);
          os[t][u][0] = v.x; os[t][u][1] = v.y;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      float Mc = M[u];
#pragma unroll
      for (int t = 0; t < CH; ++t)
        if (c0 + t < ns) Mc = vmax(Mc, ms[t][u]);
      if (Mc == -INFINITY) continue;
      const float r = M[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[u] - Mc);  // earlier chunks to the new max
      lv[u] *= r;
#pragma unroll
      for (int w = 0; w < W; ++w) ov[u][w] *= r;
#pragma unroll
      for (int t = 0; t < CH; ++t) {
        if (c0 + t >= ns) continue;
        const float f = ms[t][u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[t][u] - Mc);
        lv[u] = fmaf(f, ls[t][u], lv[u]);
#pragma unroll
        for (int w = 0; w < W; ++w) ov[u][w] = fmaf(f, os[t][u][w], ov[u][w]);
      }
      M[u] = Mc;
    }
  }
#pragma unroll
  for (int u = 0; u < HPL; ++u) {
    const int h = kvh * G + 2 * u + hsub;
    T* out = reinterpret_cast<T*>(a.merge.out) + ((size_t)seq * a.merge.hq + h) * D + d0;
#pragma unroll
    for (int w = 0; w < W; ++w) Elem<T>::store(out + w, lv[u] > 0.f ? ov[u][w] / lv[u] : 0.f);
    if (a.merge.lse_out && d0 == 0)
      a.merge.lse_out[(size_t)seq * a.merge.hq + h] =
          lv[u] > 0.f ? (M[u] + __builtin_amdgcn_logf(lv[u])) * kLn2 : -INFINITY;
  }
}

}  // namespace lk
