// Weight-only quantization of expert weights (the pages name INT4/INT8
// quantization of the experts, wmrh.cn section 工程优化方案, but give no
// scheme).
//
// INT8: one fp32 scale per output row (symmetric absmax, the scheme of
// Dettmers et al., "LLM.int8(): 8-bit Matrix Multiplication for Transformers
// at Scale", section 2, applied per row).  s = absmax(row) / 127 and
// q = rint(w / s), both in fp32 with correctly rounded division, clamped to
// [-127, 127]; a zero row gets s = 0 and q = 0.
//
// INT4: one fp32 scale per group of 128 consecutive input columns of a row
// (symmetric absmax round-to-nearest, the RTN baseline of GPTQ and AWQ at
// group size 128).  s = absmax(group) / 7, q = rint(w / s) clamped to
// [-7, 7], in fp32 as for INT8.  Stored as u = q + 8 in 4 bits; the codes of
// columns 8j .. 8j+7 fill one 32-bit word, column 8j + 2i in bits 4i .. 4i+3
// and column 8j + 2i + 1 in bits 16 + 4i .. 16 + 4i + 3, so that
// ((word >> 4i) & 0x000F000F) | 0x43004300 is the bf16 pair
// (128 + u_{2i}, 128 + u_{2i+1}) with no further arithmetic.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

// One wave per row; each lane takes 8 consecutive columns at a time.
__global__ __launch_bounds__(256) void quantize_int8_kernel(const uint16_t* __restrict__ w,
                                                            int64_t rows, int cols,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += nw) {
    const uint16_t* wr = w + r * cols;
    float amax = 0.f;
    for (int c = lane * 8; c < cols; c += 512) {
      const uint4 v = *(const uint4*)(wr + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        amax = fmaxf(amax, fabsf(__uint_as_float(u[i] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(u[i] & 0xffff0000u)));
      }
    }
    amax = wave_max(amax);
    const float s = __fdiv_rn(amax, 127.0f);
    int8_t* qr = q + r * cols;
    for (int c = lane * 8; c < cols; c += 512) {
      const uint4 v = *(const uint4*)(wr + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t bits = (i & 1) ? (u[i >> 1] & 0xffff0000u) : (u[i >> 1] << 16);
        float t = s > 0.f ? rintf(__fdiv_rn(__uint_as_float(bits), s)) : 0.f;
        t = fminf(fmaxf(t, -127.f), 127.f);
        packed[i >> 2] |= ((uint32_t)(int)t & 0xffu) << (8 * (i & 3));
      }
      *(uint2*)(qr + c) = make_uint2(packed[0], packed[1]);
    }
    if (lane == 0) scale[r] = s;
  }
}

// One wave per row; 16 lanes per 128-column group, each lane 8 consecutive
// columns (one packed word).
__global__ __launch_bounds__(256) void quantize_int4_kernel(const uint16_t* __restrict__ w,
                                                            int64_t rows, int cols,
                                                            uint32_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  const int ng = cols / 128;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += nw) {
    const uint16_t* wr = w + r * cols;
    for (int c0 = 0; c0 < cols; c0 += 512) {
      const int c = c0 + lane * 8;
      const bool in = c < cols;  // cols % 128 == 0: a group is wholly in or out
      const uint4 v = in ? *(const uint4*)(wr + c) : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
      // maximum over the group's 16 lanes
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
      const float s = __fdiv_rn(amax, 7.0f);
      uint32_t word = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float t = s > 0.f ? rintf(__fdiv_rn(f[i], s)) : 0.f;
        t = fminf(fmaxf(t, -7.f), 7.f);
        const uint32_t code = (uint32_t)((int)t + 8);
        word |= code << ((i & 1) ? 16 + 4 * (i >> 1) : 4 * (i >> 1));
      }
      if (in) {
        q[(r * cols + c) >> 3] = word;
        if ((lane & 15) == 0) scale[r * ng + (c >> 7)] = s;
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize_int4(const void* w, int64_t rows, int cols, uint8_t* q, float* scale,
                                hipStream_t stream) {
  int64_t grid = (rows + 3) / 4;
  if (grid > 65536) grid = 65536;
  if (grid < 1) grid = 1;
  quantize_int4_kernel<<<(unsigned)grid, 256, 0, stream>>>((const uint16_t*)w, rows, cols,
                                                             (uint32_t*)q, scale);
  return hipGetLastError();
}

hipError_t launch_quantize_int8(const void* w, int64_t rows, int cols, int8_t* q, float* scale,
                                hipStream_t stream) {
  int64_t grid = (rows + 3) / 4;
  if (grid > 65536) grid = 65536;
  if (grid < 1) grid = 1;
  quantize_int8_kernel<<<(unsigned)grid, 256, 0, stream>>>((const uint16_t*)w, rows, cols, q,
                                                             scale);
  return hipGetLastError();
}

}  // namespace moe
