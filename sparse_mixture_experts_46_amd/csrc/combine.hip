// Gate-weighted combine: y_t = sum_k [kept] g_tk * E_{e_tk}(x_t) (+ shared).
//
// Pages (by title and section): wmrh.cn explainer ("MoE 的核心思想")
// 公式表达重点 (output = gate-weighted sum of the chosen experts' outputs);
// learnagent.wiki "混合专家模型（Mixture of Experts, MoE）" 结构 3 (same sum);
// mzlw.cn "MoE 混合专家模型稀疏激活的架构原理与负载均衡挑战" 2.3 (a dropped
// token skips the expert computation and is carried by the residual, so it
// contributes nothing here).
//
// Deterministic gather-reduce: each output element sums its K terms in slot
// order in fp32, then adds the shared expert, then rounds once.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

// bf16: each thread owns 8 consecutive columns (16 bytes) of one token at a
// time; the gridDim.y workgroups of a token cover its row (blockDim.x divides
// d / 8 where it can).  The up to KB expert rows of a token are all loaded
// before any is added, so every thread has KB loads in flight; the sum still
// runs in slot order.
template <int KB>
__global__ __launch_bounds__(256) void combine_bf16_kernel(
    const uint16_t* __restrict__ y_perm, const int32_t* __restrict__ pair_row,
    const float* __restrict__ gate, const uint16_t* __restrict__ y_shared,
    uint16_t* __restrict__ y, int64_t T, int d, int K) {
  const int chunks = d / 8;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    int32_t rows[KB];
    float gs[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      rows[k] = k < K ? pair_row[t * K + k] : -1;
      gs[k] = k < K ? gate[t * K + k] : 0.f;
    }
    for (int c = blockIdx.y * blockDim.x + threadIdx.x; c < chunks; c += gridDim.y * blockDim.x) {
      uint4 v[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k)
        if (rows[k] >= 0) v[k] = *(const uint4*)(y_perm + (int64_t)rows[k] * d + c * 8);
      uint4 vs = make_uint4(0u, 0u, 0u, 0u);
      if (y_shared) vs = *(const uint4*)(y_shared + t * d + c * 8);
      float acc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        if (rows[k] < 0) continue;
        float f[8];
        unpack_bf16x8(v[k], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(gs[k], f[j], acc[j]);
      }
      if (y_shared) {
        float f[8];
        unpack_bf16x8(vs, f);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += f[j];
      }
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      *(uint4*)(y + t * d + c * 8) = o;
    }
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(
    const float* __restrict__ y_perm, const int32_t* __restrict__ pair_row,
    const float* __restrict__ gate, const float* __restrict__ y_shared,
    float* __restrict__ y, int64_t T, int d, int K) {
  const int chunks = d / 4;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    int32_t rows[kMaxTopK];
    float gs[kMaxTopK];
    for (int k = 0; k < K; ++k) {
      rows[k] = pair_row[t * K + k];
      gs[k] = gate[t * K + k];
    }
    for (int c = threadIdx.x; c < chunks; c += 256) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k = 0; k < K; ++k) {
        if (rows[k] < 0) continue;
        const float4 v = *(const float4*)(y_perm + (int64_t)rows[k] * d + c * 4);
        acc.x = fmaf(gs[k], v.x, acc.x);
        acc.y = fmaf(gs[k], v.y, acc.y);
        acc.z = fmaf(gs[k], v.z, acc.z);
        acc.w = fmaf(gs[k], v.w, acc.w);
      }
      if (y_shared) {
        const float4 v = *(const float4*)(y_shared + t * d + c * 4);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      *(float4*)(y + t * d + c * 4) = acc;
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* y_perm, const int32_t* pair_row,
                          const float* gate, const void* y_shared, void* y,
                          int64_t T, int d, int K, bool bf16,
                          hipStream_t stream) {
  int64_t grid = T < 8192 ? T : 8192;
  if (grid < 1) grid = 1;
  if (bf16) {
    const int chunks = d / 8;
    int nt = chunks % 256 == 0 ? 256 : (chunks % 128 == 0 ? 128 : (chunks <= 64 ? 64 : 256));
    // Decode-sized batches: too few tokens to fill the GPU one workgroup per
    // token, so a token's row is cut over workgroups of 64 threads, one
    // 16-byte chunk each.
    int cs = 1;
    if (T < 1024) {
      nt = 64;
      cs = (chunks + 63) / 64;
    }
    const dim3 g((unsigned)grid, (unsigned)cs);
    const uint16_t* yp = (const uint16_t*)y_perm;
    const uint16_t* ys = (const uint16_t*)y_shared;
    if (K <= 2)
      combine_bf16_kernel<2><<<g, nt, 0, stream>>>(yp, pair_row, gate, ys, (uint16_t*)y, T, d, K);
    else if (K <= 8)
      combine_bf16_kernel<8><<<g, nt, 0, stream>>>(yp, pair_row, gate, ys, (uint16_t*)y, T, d, K);
    else
      combine_bf16_kernel<kMaxTopK><<<g, nt, 0, stream>>>(yp, pair_row, gate, ys, (uint16_t*)y, T, d, K);
  } else
    combine_f32_kernel<<<(unsigned)grid, 256, 0, stream>>>(
        (const float*)y_perm, pair_row, gate, (const float*)y_shared, (float*)y, T, d, K);
  return hipGetLastError();
}

}  // namespace moe
