// Weight-only INT8 quantization of expert weights: one fp32 scale per output
// row (symmetric absmax, the scheme of Dettmers et al., "LLM.int8(): 8-bit
// Matrix Multiplication for Transformers at Scale", section 2, applied per
// row; the pages give no scheme).  s = absmax(row) / 127 and
// q = rint(w / s), both in fp32 with correctly rounded division, clamped to
// [-127, 127]; a zero row gets s = 0 and q = 0.
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

}  // namespace

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
