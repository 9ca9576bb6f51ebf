// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// bf16 <-> fp32.  A bf16 is the upper 16 bits of an IEEE fp32.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round-to-nearest-even fp32 -> bf16; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Unpack 8 bf16 held in a uint4 into fp32.
__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
  return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o, MOE_WAVE);
    v = w > v ? w : v;
  }
  return v;
}

// silu(u) = u / (1 + exp(-u)); gelu_tanh(u) = 0.5 u (1 + tanh(sqrt(2/pi)(u + 0.044715 u^3))).
// silu divides by one hardware reciprocal (v_rcp_f32, within 1 ulp) and a
// multiply instead of the correctly rounded division, whose expansion is
// about ten instructions per element of the SwiGLU epilogues; the results go
// to bf16 (or carry an fp32 error of a few ulp).  1 + exp(-u) >= 1, and its
// infinity (u below about -88) gives a reciprocal of 0 and silu = -0.
__device__ __forceinline__ float silu_f(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u));
}

// gelu_tanh through 0.5 (1 + tanh(z)) = 1 / (1 + exp(-2 z)): one exp and one
// hardware reciprocal, as silu, instead of tanhf (the bf16 epilogues and the
// backward's recompute of h; the fp32 layer keeps tanhf).  A large negative
// argument gives exp = inf, a reciprocal of 0 and gelu = -0.
__device__ __forceinline__ float gelu_tanh_f(float u) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  const float inner = c * (u + 0.044715f * u * u * u);
  return u * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * inner));
}

// Find the group g with base[g] <= v < base[g+1] (base is non-decreasing,
// base[0] = 0, v < base[G]); binary search over G+1 entries.
__device__ __forceinline__ int find_group(const int32_t* base, int G, int v) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace moe
