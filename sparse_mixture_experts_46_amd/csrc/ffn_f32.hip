// fp32 expert FFNs (layers whose activations and weights are fp32).  One
// workgroup per expert row: the hidden vector is formed in LDS, then the
// output row; plain fp32 FMAs in a fixed order.  Used for small fp32
// layers such as the 64-wide GELU layer of the learnagent.wiki
// "混合专家模型（Mixture of Experts, MoE）" 运行示例 (Linear -> GELU -> Linear,
// with biases); SwiGLU (mzlw.cn section 三, Expert) is supported as well.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void ffn_f32_kernel(
    const float* __restrict__ a, const int32_t* __restrict__ a_rows, int a_div,
    const int32_t* __restrict__ offset, int N, int64_t T, int K, int d, int F,
    int Fs, int act, const float* __restrict__ w1, const float* __restrict__ w3,
    const float* __restrict__ w2, const float* __restrict__ b1,
    const float* __restrict__ b2, const float* __restrict__ ws1,
    const float* __restrict__ ws3, const float* __restrict__ ws2,
    const float* __restrict__ x_shared, float* __restrict__ y_perm,
    float* __restrict__ y_shared) {
  extern __shared__ float sh[];  // [max(F, Fs)] hidden, then [d] input row
  const int64_t total = offset[N];
  const int64_t nrows = total + (Fs > 0 ? T : 0);
  for (int64_t v = blockIdx.x; v < nrows; v += gridDim.x) {
    const bool shared = v >= total;
    const int64_t r = v;
    int e = 0;
    const float* xin;
    const float *W1, *W3, *W2, *B1 = nullptr, *B2 = nullptr;
    int FF;
    float* out;
    if (shared) {
      const int64_t t = v - total;
      xin = x_shared + t * d;
      W1 = ws1; W3 = ws3; W2 = ws2; FF = Fs;
      out = y_shared + t * d;
    } else {
      e = find_group(offset, N, (int)r);
      const int64_t src = a_rows ? (int64_t)(a_rows[r] / a_div) : r;
      xin = a + src * d;
      W1 = w1 + (int64_t)e * F * d;
      W3 = w3 ? w3 + (int64_t)e * F * d : nullptr;
      W2 = w2 + (int64_t)e * d * F;
      if (b1) B1 = b1 + (int64_t)e * F;
      if (b2) B2 = b2 + (int64_t)e * d;
      FF = F;
      out = y_perm + r * d;
    }
    float* hid = sh;
    float* xs = sh + (F > Fs ? F : Fs);
    for (int j = threadIdx.x; j < d; j += 256) xs[j] = xin[j];
    __syncthreads();
    for (int f = threadIdx.x; f < FF; f += 256) {
      float g = 0.f;
      const float* wr = W1 + (int64_t)f * d;
      for (int k = 0; k < d; ++k) g = fmaf(xs[k], wr[k], g);
      float hv;
      if (act == 0) {
        float u = 0.f;
        const float* ur = W3 + (int64_t)f * d;
        for (int k = 0; k < d; ++k) u = fmaf(xs[k], ur[k], u);
        hv = (g / (1.0f + expf(-g))) * u;
      } else {
        if (B1) g += B1[f];
        const float c = 0.7978845608028654f;
        hv = 0.5f * g * (1.0f + tanhf(c * (g + 0.044715f * g * g * g)));
      }
      hid[f] = hv;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < d; j += 256) {
      float o = 0.f;
      const float* wr = W2 + (int64_t)j * FF;
      for (int f = 0; f < FF; ++f) o = fmaf(hid[f], wr[f], o);
      if (B2) o += B2[j];
      out[j] = o;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_ffn_f32(const FfnProblem& p, hipStream_t stream) {
  const int Fm = p.F > p.F_shared ? p.F : p.F_shared;
  const size_t smem = (size_t)(Fm + p.d) * sizeof(float);
  int64_t rows = p.T * p.K + (p.F_shared > 0 ? p.T : 0);
  int64_t grid = rows < 4096 ? rows : 4096;
  if (grid < 1) grid = 1;
  ffn_f32_kernel<<<(unsigned)grid, 256, smem, stream>>>(
      (const float*)p.a, p.a_rows, p.K, p.offset, p.N, p.T, p.K, p.d, p.F, p.F_shared, p.act,
      (const float*)p.w1, (const float*)p.w3, (const float*)p.w2, (const float*)p.b1,
      (const float*)p.b2, (const float*)p.ws1, (const float*)p.ws3, (const float*)p.ws2,
      (const float*)p.x_shared, (float*)p.y_perm, (float*)p.y_shared);
  return hipGetLastError();
}

}  // namespace moe
