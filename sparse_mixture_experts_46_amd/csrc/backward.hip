// Backward pass of the MoE layer: the vector-Jacobian product of the forward
// for the scalar  L = sum dy * y + c_aux aux + c_z z + c_zlse z_lse.
//
// Pages (by title and section):
//   mzlw.cn "MoE 混合专家模型稀疏激活的架构原理与负载均衡挑战", section 三:
//     the PyTorch modules the layer is trained through (router: top-K, then
//     softmax of the chosen logits; SwiGLU experts; gate-weighted sum), and
//     2.2: the auxiliary load-balance loss added to the training loss.
//   wmrh.cn/news/98181, Router Z-Loss: the penalty on the router logits.
//   mstx.cn "MoE 如何替代 FFN？…", the challenges list: routing is a discrete
//     choice, so gradients reach the router only through the gate values and
//     the auxiliary losses (top-K, the capacity cut and the counts carry none).
//
// Steps (each its own kernel, all on the caller's stream, no atomics, every
// reduction in a fixed order):
//   combine backward   d_perm[row(t,k)] = g_tk dy_t, dgate_tk = dy_t . y_perm[row]
//   router backward    dlogits from the gates, aux, z and z_lse (+ db_r)
//   router weights     dW_r = dlogits^T x
//   expert backward    grouped GEMMs (gemm_bwd.h): recompute u (and v), then
//                      dh -> du (dv) and h, dW2, dx_perm, dW1 (dW3), biases
//   dx                 sum over the token's kept rows of dx_perm, + the shared
//                      expert's dx, + dlogits W_r
#include <type_traits>

#include "gemm_bwd.h"
#include "gemm_bwd_tr.h"

#include "host_device.h"
#include "moe_internal.h"
#include "rng.h"

namespace moe {

namespace {

int cus() { return device_cus(); }

}  // namespace

// ============================================================ combine =====
// One wave per pair p = t*K + k.  A dropped pair gets dgate = 0.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const void* __restrict__ dy,
                                                          const void* __restrict__ y_perm,
                                                          const float* __restrict__ gate,
                                                          const int32_t* __restrict__ pair_row,
                                                          int64_t pairs, int K, int d,
                                                          void* __restrict__ d_perm,
                                                          float* __restrict__ dgate) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t pr = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); pr < pairs; pr += nw) {
    const int r = pair_row[pr];
    if (r < 0) {
      if (lane == 0) dgate[pr] = 0.f;
      continue;
    }
    const int64_t t = pr / K;
    const float g = gate[pr];
    float dot = 0.f;
    if (BF16) {
      const uint4* a = (const uint4*)((const uint16_t*)dy + t * d);
      const uint4* y = (const uint4*)((const uint16_t*)y_perm + (int64_t)r * d);
      uint4* o = (uint4*)((uint16_t*)d_perm + (int64_t)r * d);
      for (int c = lane; c < d / 8; c += 64) {
        float fa[8], fy[8];
        unpack_bf16x8(a[c], fa);
        unpack_bf16x8(y[c], fy);
#pragma unroll
        for (int i = 0; i < 8; ++i) dot += fa[i] * fy[i];
        o[c] = make_uint4(pack_bf16x2(g * fa[0], g * fa[1]), pack_bf16x2(g * fa[2], g * fa[3]),
                          pack_bf16x2(g * fa[4], g * fa[5]), pack_bf16x2(g * fa[6], g * fa[7]));
      }
    } else {
      const float4* a = (const float4*)((const float*)dy + t * d);
      const float4* y = (const float4*)((const float*)y_perm + (int64_t)r * d);
      float4* o = (float4*)((float*)d_perm + (int64_t)r * d);
      for (int c = lane; c < d / 4; c += 64) {
        const float4 va = a[c], vy = y[c];
        dot += va.x * vy.x + va.y * vy.y + va.z * vy.z + va.w * vy.w;
        o[c] = make_float4(g * va.x, g * va.y, g * va.z, g * va.w);
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) dgate[pr] = dot;
  }
}

hipError_t launch_combine_backward(const void* dy, const void* y_perm, const float* gate,
                                   const int32_t* pair_row, int64_t T, int K, int d, bool bf16,
                                   void* d_perm, float* dgate, hipStream_t s) {
  const int64_t pairs = T * K;
  if (pairs == 0) return hipSuccess;
  int64_t grid = (pairs + 3) / 4;
  if (grid > (int64_t)cus() * 16) grid = (int64_t)cus() * 16;
  if (bf16)
    combine_bwd_kernel<true><<<(unsigned)grid, 256, 0, s>>>(dy, y_perm, gate, pair_row, pairs, K,
                                                             d, d_perm, dgate);
  else
    combine_bwd_kernel<false><<<(unsigned)grid, 256, 0, s>>>(dy, y_perm, gate, pair_row, pairs, K,
                                                              d, d_perm, dgate);
  return hipGetLastError();
}

// ============================================================= router =====
constexpr int kRouterBwdTokens = 32;  // tokens per block (8 per wave)

int64_t router_bwd_num_blocks(int64_t T) { return (T + kRouterBwdTokens - 1) / kRouterBwdTokens; }

// Value held by lane e % 64 in register slot e / 64 of every lane (e uniform).
template <int NJ>
__device__ __forceinline__ float lane_value(const float (&v)[NJ], int e) {
  float x = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (j == (e >> 6)) x = v[j];
  return __shfl(x, e & 63, MOE_WAVE);
}

template <int NJ>
__device__ __forceinline__ void lane_add(float (&v)[NJ], int e, int lane, float x) {
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (j == (e >> 6) && lane == (e & 63)) v[j] += x;
}

// One wave per token.  Expert e lives in lane e % 64, slot e / 64.
//   gates (renorm_all / softmax_topk): g = softmax of the chosen logits,
//     dl[i_k] += g_k (dg_k - sum_j g_j dg_j)
//   gates (prob_no_renorm): g_k = P[i_k], dl += P * (dP - sum_k dg_k P[i_k])
//   aux: dl += c_aux alpha N / T * P * (f - sum_e f_e P_e), f = count / (T K)
//   z:   dl += c_z * 2 l / T;   z_lse: dl += c_zlse * 2 lse / T * P
// part [nblk, N]: this block's column sums of dl (for db_r).
template <int NJ>
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const float* __restrict__ logits, RouterNoise noise,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ pair_row,
    const float* __restrict__ dgate, const int32_t* __restrict__ count, int64_t T, int N, int K,
    int gate_mode, float alpha, float c_aux, float c_z, float c_zlse, float* __restrict__ dlogits,
    float* __restrict__ part) {
  __shared__ float colsum[4][NJ * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float invT = 1.f / (float)T;
  const float fscale = 1.f / ((float)T * (float)K);
  float f[NJ], cs[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    f[j] = e < N ? (float)count[e] * fscale : 0.f;
    cs[j] = 0.f;
  }
  const int64_t t0 = (int64_t)blockIdx.x * kRouterBwdTokens;
  const int64_t t1 = t0 + kRouterBwdTokens < T ? t0 + kRouterBwdTokens : T;
  for (int64_t t = t0 + wave; t < t1; t += 4) {
    float l[NJ], P[NJ], dl[NJ];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      l[j] = -INFINITY;
      if (e < N) {
        l[j] = logits[t * N + e];
        if (noise_on(noise)) l[j] += noise.std * noise_draw(noise, t * N + e);
      }
      m = fmaxf(m, l[j]);
    }
    m = wave_max(m);
    float ssum = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      P[j] = (lane + 64 * j < N) ? expf(l[j] - m) : 0.f;
      ssum += P[j];
    }
    ssum = wave_sum(ssum);
    const float inv = 1.f / ssum, lse = m + logf(ssum);
    float sfp = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      P[j] *= inv;
      sfp += f[j] * P[j];
    }
    sfp = wave_sum(sfp);
    const float ca = c_aux * alpha * (float)N * invT, cz = 2.f * c_z * invT,
                cl = 2.f * c_zlse * lse * invT;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bool in = lane + 64 * j < N;
      dl[j] = in ? ca * P[j] * (f[j] - sfp) + cz * l[j] + cl * P[j] : 0.f;
    }
    // gates
    const int32_t* it = idx + t * K;
    const int32_t* pt = pair_row + t * K;
    const float* gt = dgate + t * K;
    if (gate_mode == 2) {  // prob_no_renorm: g_k = P[i_k]
      float s = 0.f;
      for (int k = 0; k < K; ++k) {
        const int e = it[k];
        const float dg = pt[k] >= 0 ? gt[k] : 0.f;
        const float pe = lane_value<NJ>(P, e);
        s += dg * pe;
        lane_add<NJ>(dl, e, lane, pe * dg);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) dl[j] -= P[j] * s;
    } else {  // renorm_all, softmax_topk: g = softmax of the chosen logits
      float ms = -INFINITY;
      for (int k = 0; k < K; ++k) ms = fmaxf(ms, lane_value<NJ>(l, it[k]));
      float z = 0.f, s = 0.f;
      for (int k = 0; k < K; ++k) {
        const float ek = expf(lane_value<NJ>(l, it[k]) - ms);
        z += ek;
        s += ek * (pt[k] >= 0 ? gt[k] : 0.f);
      }
      const float iz = 1.f / z;
      s *= iz;
      for (int k = 0; k < K; ++k) {
        const int e = it[k];
        const float g = expf(lane_value<NJ>(l, e) - ms) * iz;
        const float dg = pt[k] >= 0 ? gt[k] : 0.f;
        lane_add<NJ>(dl, e, lane, g * (dg - s));
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (e < N) dlogits[t * N + e] = dl[j];
      cs[j] += dl[j];
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) colsum[wave][lane + 64 * j] = cs[j];
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256)
    part[(int64_t)blockIdx.x * N + e] = colsum[0][e] + colsum[1][e] + colsum[2][e] + colsum[3][e];
}

// out[e] = sum over the nb rows of part[:, e], in row order.
__global__ __launch_bounds__(256) void colsum_rows_kernel(const float* __restrict__ part,
                                                          int64_t nb, int64_t n,
                                                          float* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float s = 0.f;
  for (int64_t b = 0; b < nb; ++b) s += part[b * n + e];
  out[e] = s;
}

hipError_t launch_router_backward(const float* logits, const RouterNoise& noise,
                                  const int32_t* idx, const int32_t* pair_row, const float* dgate,
                                  const int32_t* count, int64_t T, int N, int K, int gate_mode,
                                  float alpha, float c_aux, float c_z, float c_zlse,
                                  float* dlogits, float* part, float* db_r, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t nb = router_bwd_num_blocks(T);
  const int nj = (N + 63) / 64;
#define MOE_RB(NJ)                                                                          \
  router_bwd_kernel<NJ><<<(unsigned)nb, 256, 0, s>>>(logits, noise, idx, pair_row,            \
                                                      dgate, count, T, N, K, gate_mode, alpha, \
                                                      c_aux, c_z, c_zlse, dlogits, part)
  if (nj <= 1) MOE_RB(1);
  else if (nj <= 2) MOE_RB(2);
  else if (nj <= 4) MOE_RB(4);
  else if (nj <= 8) MOE_RB(8);
  else MOE_RB(16);
#undef MOE_RB
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !db_r) return e;
  colsum_rows_kernel<<<(unsigned)((N + 255) / 256), 256, 0, s>>>(part, nb, N, db_r);
  return hipGetLastError();
}

// ----------------------------------------------------- router weights ----
// dW_r[e, i] = sum_t dl[t, e] x[t, i].  Block: 64 experts x 64 columns over
// a chunk of tokens (grid z), 4 x 4 outputs per thread, 16 tokens per step
// staged in LDS.  Partial products [nsplit, N, d] reduced in split order.
// With few experts the blocks are few, and each step waits for its loads:
// shorter chunks put more of them in flight.
int router_dw_chunk(int N) { return N <= 16 ? 128 : 512; }

int router_dw_splits(int64_t T, int N) {
  const int c = router_dw_chunk(N);
  return (int)((T + c - 1) / c);
}

template <bool BF16>
__global__ __launch_bounds__(256) void router_dw_kernel(const float* __restrict__ dl,
                                                        const void* __restrict__ x, int64_t T,
                                                        int N, int d, int chunk,
                                                        float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float sl[16][64];
  __shared__ __attribute__((aligned(16))) float sx[16][64];
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int64_t tb = (int64_t)blockIdx.z * chunk;
  const int64_t te = tb + chunk < T ? tb + chunk : T;
  const int ty = tid >> 4, tx = tid & 15;  // experts ty*4.., columns tx*4..
  float acc[4][4] = {};
  for (int64_t t0 = tb; t0 < te; t0 += 16) {
    {  // 16 tokens x 64 experts / columns: 4 values per thread each
      const int r = tid >> 4, c = (tid & 15) * 4;
      const int64_t t = t0 + r;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + c + u;
        sl[r][c + u] = (t < te && e < N) ? dl[t * N + e] : 0.f;
      }
      if (t < te && i0 + c < d) {
        if (BF16) {
          const uint2 v = *(const uint2*)((const uint16_t*)x + t * d + i0 + c);
          sx[r][c] = __uint_as_float(v.x << 16);
          sx[r][c + 1] = __uint_as_float(v.x & 0xffff0000u);
          sx[r][c + 2] = __uint_as_float(v.y << 16);
          sx[r][c + 3] = __uint_as_float(v.y & 0xffff0000u);
        } else {
          const float4 v = *(const float4*)((const float*)x + t * d + i0 + c);
          sx[r][c] = v.x; sx[r][c + 1] = v.y; sx[r][c + 2] = v.z; sx[r][c + 3] = v.w;
        }
      } else {
        sx[r][c] = sx[r][c + 1] = sx[r][c + 2] = sx[r][c + 3] = 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float4 a = *(const float4*)&sl[r][ty * 4];
      const float4 b = *(const float4*)&sx[r][tx * 4];
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] += av[u] * bv[v];
    }
    __syncthreads();
  }
  float* o = out + (int64_t)blockIdx.z * N * d;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = e0 + ty * 4 + u;
    const int i = i0 + tx * 4;
    if (e < N && i < d)
      *(float4*)(o + (int64_t)e * d + i) = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
  }
}

hipError_t launch_router_dw(const float* dl, const void* x, bool bf16, int64_t T, int N, int d,
                            float* part, float* dw_r, hipStream_t s) {
  const int ns = router_dw_splits(T, N);
  const int chunk = router_dw_chunk(N);
  if (ns == 0) return hipSuccess;  // T == 0 is handled by the caller
  float* dst = ns == 1 ? dw_r : part;
  dim3 grid((unsigned)((d + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)ns);
  if (bf16) router_dw_kernel<true><<<grid, 256, 0, s>>>(dl, x, T, N, d, chunk, dst);
  else router_dw_kernel<false><<<grid, 256, 0, s>>>(dl, x, T, N, d, chunk, dst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  const int64_t n = (int64_t)N * d;
  colsum_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, ns, n, dw_r);
  return hipGetLastError();
}

// ------------------------------------------------------------------- dx ---
// dx[t, i] = sum_k [kept] dx_perm[row(t,k), i] + dx_shared[t, i] + sum_e dl[t, e] W_r[e, i].
// Block: 64 tokens x 64 columns, 4 x 4 per thread; the router term from LDS
// tiles of 16 experts; the row gathers afterwards, in slot order.
template <bool BF16, int P2>
__global__ __launch_bounds__(256) void dx_kernel(const void* __restrict__ dx_perm,
                                                 const void* __restrict__ dx_perm2,
                                                 int64_t rows,
                                                 const int32_t* __restrict__ pair_row, int K,
                                                 const void* __restrict__ dx_shared,
                                                 const void* __restrict__ dx_shared2,
                                                 const float* __restrict__ dl,
                                                 const float* __restrict__ w_r, int N, int64_t T,
                                                 int d, void* __restrict__ dx) {
  __shared__ float sl[64][17];
  __shared__ __attribute__((aligned(16))) float sw[16][64];
  const int tid = threadIdx.x;
  const int64_t tb = (int64_t)blockIdx.x * 64;
  const int i0 = blockIdx.y * 64;
  const int ty = tid >> 4, tx = tid & 15;  // tokens ty*4.., columns tx*4..
  float acc[4][4] = {};
  if (dl) {
    for (int e0 = 0; e0 < N; e0 += 16) {
      for (int q = tid; q < 64 * 16; q += 256) {
        const int r = q >> 4, c = q & 15;
        const int64_t t = tb + r;
        sl[r][c] = (t < T && e0 + c < N) ? dl[t * N + e0 + c] : 0.f;
      }
      for (int q = tid; q < 16 * 64; q += 256) {
        const int r = q >> 6, c = q & 63;
        sw[r][c] = (e0 + r < N && i0 + c < d) ? w_r[(int64_t)(e0 + r) * d + i0 + c] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float4 b = *(const float4*)&sw[r][tx * 4];
        const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float a = sl[ty * 4 + u][r];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] += a * bv[v];
        }
      }
      __syncthreads();
    }
  }
  const int i = i0 + tx * 4;
  if (i >= d) return;
  // per output: the router term, then slot k's row of dx_perm and of each of
  // the P2 further planes for k = 0..K-1, then the shared rows; the four
  // tokens' rows of one slot are loaded together
  auto add_row = [&](float (&o)[4], const void* base, int64_t row) {
    if (BF16) {
      const uint2 v = *(const uint2*)((const uint16_t*)base + row * d + i);
      o[0] += __uint_as_float(v.x << 16);
      o[1] += __uint_as_float(v.x & 0xffff0000u);
      o[2] += __uint_as_float(v.y << 16);
      o[3] += __uint_as_float(v.y & 0xffff0000u);
    } else {
      const float4 v = *(const float4*)((const float*)base + row * d + i);
      o[0] += v.x; o[1] += v.y; o[2] += v.z; o[3] += v.w;
    }
  };
  for (int k = 0; k < K; ++k) {
    int r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t t = tb + ty * 4 + u;
      r[u] = t < T ? pair_row[t * K + k] : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (r[u] >= 0) {
        add_row(acc[u], dx_perm, r[u]);
#pragma unroll
        for (int q = 0; q < P2; ++q) add_row(acc[u], dx_perm2, q * rows + r[u]);
      }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t t = tb + ty * 4 + u;
    if (t >= T) continue;
    if (dx_shared) add_row(acc[u], dx_shared, t);
    if (dx_shared2)
#pragma unroll
      for (int q = 0; q < P2; ++q) add_row(acc[u], dx_shared2, q * T + t);
    float(&o)[4] = acc[u];
    if (BF16)
      *(uint2*)((uint16_t*)dx + t * d + i) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    else
      *(float4*)((float*)dx + t * d + i) = make_float4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_dx(const void* dx_perm, const int32_t* pair_row, int K, const void* dx_shared,
                     const float* dl, const float* w_r, int N, int64_t T, int d, bool bf16,
                     void* dx, hipStream_t s, const void* dx_perm2, const void* dx_shared2,
                     int planes2) {
  if (T == 0) return hipSuccess;
  if (!dx_perm2) planes2 = 0;
  if (planes2 != 0 && planes2 != 1 && planes2 != 3) return hipErrorInvalidValue;
  dim3 grid((unsigned)((T + 63) / 64), (unsigned)((d + 63) / 64));
  auto go = [&](auto bf, auto p2) {
    dx_kernel<decltype(bf)::value, decltype(p2)::value><<<grid, 256, 0, s>>>(
        dx_perm, dx_perm2, T * K, pair_row, K, dx_shared, dx_shared2, dl, w_r, N, T, d, dx);
  };
  using TT = std::true_type;
  using FF = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P3 = std::integral_constant<int, 3>;
  if (bf16) {
    if (planes2 == 0) go(TT{}, P0{});
    else if (planes2 == 1) go(TT{}, P1{});
    else go(TT{}, P3{});
  } else {
    if (planes2 != 0) return hipErrorInvalidValue;  // the fp32 path never splits dx_perm
    go(FF{}, P0{});
  }
  return hipGetLastError();
}

// ---------------------------------------------------------- bias grads ---
// out[g, c] = sum over group g's rows of src[row, c] (row order).
template <bool BF16>
__global__ __launch_bounds__(256) void group_colsum_kernel(const void* __restrict__ src,
                                                           const int32_t* __restrict__ offset,
                                                           int C, void* __restrict__ out) {
  const int g = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  float s = 0.f;
  for (int64_t r = offset[g]; r < offset[g + 1]; ++r)
    s += BF16 ? bf16_to_f32(((const uint16_t*)src)[r * C + c]) : ((const float*)src)[r * C + c];
  if (BF16) ((uint16_t*)out)[(int64_t)g * C + c] = f32_to_bf16(s);
  else ((float*)out)[(int64_t)g * C + c] = s;
}

// ---------------------------------------------------------------- zero ---
__global__ __launch_bounds__(256) void zero_kernel(unsigned char* __restrict__ p, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = 0;
}

hipError_t launch_zero(void* p, size_t n, hipStream_t s) {
  if (!p || n == 0) return hipSuccess;
  size_t grid = (n + 255) / 256;
  if (grid > 4096) grid = 4096;
  zero_kernel<<<(unsigned)grid, 256, 0, s>>>((unsigned char*)p, n);
  return hipGetLastError();
}

// ======================================================== expert GEMMs ====
namespace {

template <int R, bool WG, bool BS, bool DUALB, bool DUALK, int EPI>
hipError_t run_bwd(const BwdArgs& a, int64_t max_tiles, bool bf16, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (!bf16) {
    int64_t grid = max_tiles < (int64_t)cus() * 8 ? max_tiles : (int64_t)cus() * 8;
    gemm_bwd_f32_kernel<WG, BS, DUALB, DUALK, EPI><<<(unsigned)grid, 256, 0, s>>>(a, (int)max_tiles);
    return hipGetLastError();
  }
  auto kern = gemm_bwd_kernel<R, WG, BS, DUALB, DUALK, EPI>;
  constexpr size_t smem = (size_t)2 * (2 * R) * 8 * 16;  // two stages of 2R rows x 128 bytes
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = set_dynamic_lds_once((const void*)kern, (int)smem, lds_set);
  if (e != hipSuccess) return e;
  int64_t grid = (int64_t)cus() * (R == 128 ? 2 : 1);
  if (max_tiles < grid) grid = ((max_tiles + 7) / 8) * 8;
  kern<<<(unsigned)grid, 2 * R, smem, s>>>(a, (int)max_tiles);
  return hipGetLastError();
}

// The 256 x 256 DMA kernel (gemm_bwd_tr.h): one workgroup per CU.
template <bool WG, bool BS, bool DUALB, bool DUALK, int EPI, int SPLIT = 1>
hipError_t run_bwd_tr(const BwdArgs& a, int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  auto kern = gemm_bwd_tr_kernel<WG, BS, DUALB, DUALK, EPI, SPLIT>;
  constexpr size_t smem = 2 * 2 * 32768;  // two stages of A and B
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = set_dynamic_lds_once((const void*)kern, (int)smem, lds_set);
  if (e != hipSuccess) return e;
  int64_t grid = cus();
  if (max_tiles < grid) grid = ((max_tiles + 7) / 8) * 8;
  kern<<<(unsigned)grid, 512, smem, s>>>(a, (int)max_tiles);
  return hipGetLastError();
}

// Upper bound on the tiles of a row-group table: sum over groups of
// ceil(M_g / bm) * ceil(nout / bno) with sum M_g <= rows.
int64_t row_tiles_bound(int64_t rows, int G, int bm, int nout, int bno) {
  return (rows / bm + G) * (int64_t)((nout + bno - 1) / bno);
}

}  // namespace

size_t ffn_backward_workspace_bytes(int64_t T, int d, int N, int K, int F, int F_shared,
                                    bool bf16) {
  const size_t el = bf16 ? 2 : 4;
  const int64_t rows = T * K + (F_shared > 0 ? T : 0);
  size_t o = (size_t)3 * (N + 2) * 4;
  o = (o + 255) / 256 * 256;
  o += ((size_t)T * K * d * el + 255) / 256 * 256;  // x_perm
  return o + 3 * ((size_t)rows * F * el + 256);
}

namespace {
// Row-group GEMMs (the recompute, dh, dx_perm) use the 256 x 256 DMA kernel
// from 192 rows per expert on (about a third of a ~256-row expert's tiles is
// padding there, and the DMA kernel still wins), else the 128 x 128
// register-staged kernel.  The weight-gradient GEMMs tile F x d, whatever
// the rows: the DMA kernel when both are at least 256.
int rows_tile(int64_t rows, int N) { return rows >= (int64_t)192 * N ? 256 : 128; }
bool weight_tr(int F, int d) { return F >= 256 && d >= 256; }
}  // namespace

int ffn_backward_dx_parts(int64_t T, int N, int K, int F, int d, int act, bool bf16) {
  if (!(bf16 && act == 0 && rows_tile(T * K, N) == 256)) return 1;
  // expected tiles: whole row tiles plus half a tile of padding per expert;
  // with eight rounds of them on the CUs the walk is even enough whole
  const int64_t tiles = (T * K / 256 + N / 2) * (int64_t)((d + 255) / 256);
  if (tiles >= (int64_t)8 * cus()) return 1;
  return (2 * F / 64) % 4 == 0 ? 4 : 2;  // parts of whole 64-wide K steps
}

template <int RR>
hipError_t ffn_backward_gemms(const FfnBwdProblem& p, hipStream_t s);

hipError_t launch_expert_ffn_backward(const FfnBwdProblem& p, hipStream_t s) {
  if (p.bf16 && rows_tile(p.T * p.K, p.N) == 256) return ffn_backward_gemms<256>(p, s);
  return ffn_backward_gemms<128>(p, s);  // fp32: 16 x 16 tiles whatever RR
}

template <int RR>
hipError_t ffn_backward_gemms(const FfnBwdProblem& p, hipStream_t s) {
  auto mark = [&](int i) -> hipError_t {
    return (p.ev && p.ev[i]) ? hipEventRecord(p.ev[i], s) : hipSuccess;
  };
  const bool bf16 = p.bf16, swiglu = p.act == 0;
  const int64_t rows = p.T * p.K;
  const int64_t srows = p.F_shared > 0 ? p.T : 0;
  const int G = p.N + (srows > 0 ? 1 : 0);
  const size_t el = bf16 ? 2 : 4;
  const int F = p.F, d = p.d;
  // scratch: tile tables, x_perm [rows, d] (x gathered into the expert-
  // contiguous rows once, so no GEMM gathers in its K loop), then u (-> du),
  // v (-> dv), h, each [rows + srows, F]
  unsigned char* w = (unsigned char*)p.ws;
  int32_t* tb = (int32_t*)w;
  size_t o = ((size_t)3 * (p.N + 2) * 4 + 255) / 256 * 256;
  unsigned char* Xp = w + o;
  o += ((size_t)rows * d * el + 255) / 256 * 256;
  const size_t buf = ((size_t)(rows + srows) * F * el + 255) / 256 * 256;
  unsigned char* U = w + o;
  unsigned char* V = U + buf;
  unsigned char* H = V + buf;
  unsigned char* Us = U + (size_t)rows * F * el;
  unsigned char* Vs = V + (size_t)rows * F * el;
  unsigned char* Hs = H + (size_t)rows * F * el;

  constexpr bool TR = RR == 256;     // row groups on the DMA kernel
  const bool wtr = bf16 && weight_tr(F, d);
  const int bm1 = bf16 ? RR : 16;    // row-group tiles (recompute, dh, dx_perm)
  const int bm2 = bm1;
  const int bm4 = bm1;
  const int wbm = bf16 ? (wtr ? 256 : 128) : 16;  // weight-gradient tiles
  const int bno1 = (bf16 && swiglu) ? bm1 / 2 : bm1;  // dual B: half the tile's columns are outputs
  int32_t* base[3] = {tb, tb + (p.N + 2), tb + 2 * (p.N + 2)};
  TileSpecs specs = {};
  specs.s[0] = {bm1, bno1, F, p.F_shared, 0, 0};  // recompute: [rows, F]
  specs.s[1] = {bm2, bm2, F, p.F_shared, 0, 0};   // dh: [rows, F]
  specs.s[2] = {bm4, bm4, d, d, 0, 0};            // dx_perm: [rows, d]
  tile_setup_kernel<<<1, 1024, 0, s>>>(p.offset, p.N, srows, specs, 3, tb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (rows > 0 && (e = launch_permute(p.x, (int)el, p.row_pair, p.offset, p.N, p.K, d, rows, Xp,
                                      s)) != hipSuccess)
    return e;
  const int64_t all_rows = rows + srows;

  // ---- 1. recompute u = x W1^T (+ b1) and v = x W3^T, unless the forward
  // saved them
  const bool saved_uv = bf16 && swiglu && p.u_in && p.v_in;
  if (!saved_uv) {
    BwdArgs a = {};
    a.offset = p.offset; a.n_routed = p.N; a.shared_rows = srows; a.tile_base = base[0]; a.G = G;
    a.a = Xp; a.lda = d; a.a_shared = p.x;
    a.b0 = p.w1; a.b1 = p.w3; a.b_stride = (int64_t)F * d; a.ldb = d;
    a.bs0 = p.ws1; a.bs1 = p.ws3;
    a.Nout = F; a.Nout_shared = p.F_shared; a.Kdim = d;
    a.bias = p.b1;
    a.c = U; a.c2 = V; a.c_shared = Us; a.c2_shared = Vs; a.ldc = F;
    const int64_t mt = row_tiles_bound(all_rows, G, bm1, F, bno1);
    if (TR)
      e = swiglu ? run_bwd_tr<false, false, true, false, BEPI_UV>(a, mt, s)
                 : run_bwd_tr<false, false, false, false, BEPI_STORE>(a, mt, s);
    else
      e = swiglu ? run_bwd<128, false, false, true, false, BEPI_UV>(a, mt, bf16, s)
                 : run_bwd<128, false, false, false, false, BEPI_STORE>(a, mt, bf16, s);
    if (e != hipSuccess) return e;
  }
  if ((e = mark(0)) != hipSuccess) return e;  // recorded whether or not it ran
  // ---- 2. dh = d_perm W2 (W2 [d, F] read transposed); du, dv, h in the epilogue
  {
    BwdArgs a = {};
    a.offset = p.offset; a.n_routed = p.N; a.shared_rows = srows; a.tile_base = base[1]; a.G = G;
    a.a = p.d_perm; a.lda = d; a.a_shared = p.dy;
    a.b0 = p.w2; a.b_stride = (int64_t)d * F; a.ldb = F; a.bs0 = p.ws2;
    a.Nout = F; a.Nout_shared = p.F_shared; a.Kdim = d;
    a.c = U; a.c2 = V; a.c3 = H; a.c_shared = Us; a.c2_shared = Vs; a.c3_shared = Hs; a.ldc = F;
    if (saved_uv) {
      a.cin = p.u_in;
      a.cin2 = p.v_in;
      a.cin_shared = (const char*)p.u_in + (size_t)rows * F * el;
      a.cin2_shared = (const char*)p.v_in + (size_t)rows * F * el;
    }
    const int64_t mt = row_tiles_bound(all_rows, G, bm2, F, bm2);
    if (TR)
      e = swiglu ? run_bwd_tr<false, true, false, false, BEPI_SWIGLU_BWD>(a, mt, s)
                 : run_bwd_tr<false, true, false, false, BEPI_GELU_BWD>(a, mt, s);
    else
      e = swiglu ? run_bwd<128, false, true, false, false, BEPI_SWIGLU_BWD>(a, mt, bf16, s)
                 : run_bwd<128, false, true, false, false, BEPI_GELU_BWD>(a, mt, bf16, s);
    if (e != hipSuccess) return e;
    if ((e = mark(1)) != hipSuccess) return e;
  }
  // ---- 3. dW2[g] = d_perm_g^T h_g  ([d, F])
  {
    BwdArgs a = {};
    a.offset = p.offset; a.n_routed = p.N; a.shared_rows = srows; a.G = G;
    a.a = p.d_perm; a.lda = d; a.a_shared = p.dy;
    a.b0 = H; a.ldb = F; a.bs0 = Hs;
    a.Mout = d; a.Nout = F; a.Nout_shared = F;
    a.c = p.dw2; a.c_shared = p.dws2; a.ldc = F; a.c_gstride = (int64_t)d * F;
    const int64_t tiles = (int64_t)G * ((d + wbm - 1) / wbm) * ((F + wbm - 1) / wbm);
    e = wtr ? run_bwd_tr<true, false, false, false, BEPI_STORE>(a, tiles, s)
            : run_bwd<128, true, false, false, false, BEPI_STORE>(a, tiles, bf16, s);
    if (e != hipSuccess) return e;
    if ((e = mark(2)) != hipSuccess) return e;
  }
  // ---- 4. dx_perm = du W1 (+ dv W3)  (W1, W3 [F, d] read transposed)
  {
    BwdArgs a = {};
    a.offset = p.offset; a.n_routed = p.N; a.shared_rows = srows; a.tile_base = base[2]; a.G = G;
    a.a = U; a.a2 = V; a.lda = F; a.a_shared = Us; a.a2_shared = Vs;
    a.b0 = p.w1; a.b1 = p.w3; a.b_stride = (int64_t)F * d; a.ldb = d;
    a.bs0 = p.ws1; a.bs1 = p.ws3;
    a.Nout = d; a.Nout_shared = d; a.Kdim = F;
    a.c = p.dx_perm; a.c_shared = p.dx_shared; a.ldc = d;
    a.c2 = p.dx_perm2; a.c2_shared = p.dx_shared2;
    a.c2_plane = (int64_t)rows * d * el;
    a.c2_plane_shared = (int64_t)srows * d * el;
    const int64_t mt = row_tiles_bound(all_rows, G, bm4, d, bm4);
    const int parts = p.dx_perm2 ? ffn_backward_dx_parts(p.T, p.N, p.K, F, d, p.act, bf16) : 1;
    if (TR && parts == 4)  // K cut in parts that are separate tiles
      e = run_bwd_tr<false, true, false, true, BEPI_STORE, 4>(a, 4 * mt, s);
    else if (TR && parts == 2)
      e = run_bwd_tr<false, true, false, true, BEPI_STORE, 2>(a, 2 * mt, s);
    else if (TR)
      e = swiglu ? run_bwd_tr<false, true, false, true, BEPI_STORE>(a, mt, s)
                 : run_bwd_tr<false, true, false, false, BEPI_STORE>(a, mt, s);
    else
      e = swiglu ? run_bwd<128, false, true, false, true, BEPI_STORE>(a, mt, bf16, s)
                 : run_bwd<128, false, true, false, false, BEPI_STORE>(a, mt, bf16, s);
    if (e != hipSuccess) return e;
    if ((e = mark(3)) != hipSuccess) return e;
  }
  // ---- 5. dW1[g] = du_g^T x_g, dW3[g] = dv_g^T x_g  ([F, d])
  for (int pass = 0; pass < (swiglu ? 2 : 1); ++pass) {
    BwdArgs a = {};
    a.offset = p.offset; a.n_routed = p.N; a.shared_rows = srows; a.G = G;
    a.a = pass ? V : U; a.lda = F; a.a_shared = pass ? Vs : Us;
    a.b0 = Xp; a.ldb = d; a.bs0 = p.x;
    a.Mout = F; a.Nout = d; a.Nout_shared = d;
    a.c = pass ? p.dw3 : p.dw1; a.c_shared = pass ? p.dws3 : p.dws1; a.ldc = d;
    a.c_gstride = (int64_t)F * d;
    const int64_t tiles = (int64_t)G * ((F + wbm - 1) / wbm) * ((d + wbm - 1) / wbm);
    e = wtr ? run_bwd_tr<true, false, false, false, BEPI_STORE>(a, tiles, s)
            : run_bwd<128, true, false, false, false, BEPI_STORE>(a, tiles, bf16, s);
    if (e != hipSuccess) return e;
  }
  if ((e = mark(4)) != hipSuccess) return e;
  // ---- 6. GELU biases: db1 = column sums of du, db2 = column sums of d_perm
  if (!swiglu && p.db1) {
    dim3 grid((unsigned)((F + 255) / 256), (unsigned)p.N);
    if (bf16) group_colsum_kernel<true><<<grid, 256, 0, s>>>(U, p.offset, F, p.db1);
    else group_colsum_kernel<false><<<grid, 256, 0, s>>>(U, p.offset, F, p.db1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (!swiglu && p.db2) {
    dim3 grid((unsigned)((d + 255) / 256), (unsigned)p.N);
    if (bf16) group_colsum_kernel<true><<<grid, 256, 0, s>>>(p.d_perm, p.offset, d, p.db2);
    else group_colsum_kernel<false><<<grid, 256, 0, s>>>(p.d_perm, p.offset, d, p.db2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
