// Device helpers shared by the Locks kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lk {

constexpr int kWave = 64;
constexpr int kHeadDim = 128;

typedef uint16_t bf16_t;  // bfloat16 storage
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ void load8(const bf16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// ---------------------------------------------------------------- cross-lane
// DPP row controls (rows of 16 lanes).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within 16
constexpr int kDppRor8 = 0x128;       // lane i <- (i + 8) mod 16 within 16

// Every control above reads a lane of the same row, so no lane is out of
// bounds and the bound-control zero never applies (no old value to set up).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Maximum (minimum) with NaN propagation (one v_maximum3_f32 / v_minimum3_f32).  fmaxf drops a NaN
// operand, so in IEEE mode the compiler first quiets every operand that is
// not the result of arithmetic (LDS loads, DPP and permlane moves): two
// extra instructions per maximum.  For values that are never NaN the two
// agree, up to the sign of a zero maximum.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// Exchange with lane ^ 16 / lane ^ 32 on the VALU (gfx950 permlane swaps):
// swapping a value with itself leaves x in one result and its partner in the
// other, so their sum (or max) is the pairwise combine for every lane.
__device__ __forceinline__ float xor16_sum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Sum / max over aligned groups of N lanes (N in {1,2,4,8,16,32,64}); every
// lane of the group receives the result.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  if constexpr (N >= 32) x = xor16_sum(x);
  if constexpr (N >= 64) x = xor32_sum(x);
  return x;
}
template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = vmax(x, dpp<kDppXor1>(x));
  if constexpr (N >= 4) x = vmax(x, dpp<kDppXor2>(x));
  if constexpr (N >= 8) x = vmax(x, dpp<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = vmax(x, dpp<kDppMirror>(x));
  if constexpr (N >= 32) x = xor16_max(x);
  if constexpr (N >= 64) x = xor32_max(x);
  return x;
}

// Orders this wave's earlier LDS accesses before its later ones (LDS
// instructions of one wave execute in issue order; this stops the compiler
// from moving them across).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroups of a launch are dispatched to the XCDs round-robin: linear id b
// runs on XCD b % kXcds, each XCD with its own L2.  xcd_remap(b, n) is a
// bijection of [0, n) that gives each XCD a contiguous range of logical
// indices, so logically adjacent workgroups (which read the same lines) share
// one L2.  Only locality depends on the dispatch order, not correctness.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int q = n / kXcds, r = n % kXcds;
  const int x = b % kXcds, local = b / kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace lk
