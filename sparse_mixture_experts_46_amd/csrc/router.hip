// Router: logits = x W_r^T (+ b_r), top-K selection, gates and the
// per-block partial sums of the load-balance and z-loss statistics.
//
// Pages (by title and section):
//   mzlw.cn "MoE 混合专家模型稀疏激活的架构原理与负载均衡挑战": 2.1 (router as
//     a light linear map of the token to one score per expert, top-K then
//     softmax), 2.2 (L_aux = alpha N sum f_i p_i), section 三 (MoERouter:
//     weight [N, d], logits = x W^T, topk on logits, softmax of the top-K
//     logits, counts of the flattened indices divided by T*K).
//   learnagent.wiki "混合专家模型（Mixture of Experts, MoE）": 结构 2
//     (G(x) = Softmax(W_r x)), 结构 4 (per-expert bias that only steers the
//     choice), 运行示例 (softmax, top-K on probabilities, divide by their sum).
//   wmrh.cn explainer ("MoE 的核心思想"): 公式表达重点 (renormalised gates),
//     Router Z-Loss (penalty on the squares of the router logits).
#include <type_traits>

#include "host_device.h"
#include "lds_dma.h"
#include "moe_common.h"
#include "moe_internal.h"
#include "rng.h"

namespace moe {

// ------------------------------------------------------------ logits GEMM --
// fp32 activations: fp32 MFMA (v_mfma_f32_32x32x2_f32) tile of 64 tokens x
// 64 experts, four waves in a 2x2 grid, K staged through LDS in chunks of
// 32.  Few token or expert tiles (small N, or decode-sized T) split K over
// gridDim.z: split z writes its partial dot products to part[z]; a reduce
// kernel sums the splits in order z = 0, 1, ... and adds the bias, so the
// result is deterministic.
namespace {

constexpr int RT_M = 64, RT_N = 64, RT_K = 32, RT_PAD = 1;

__global__ __launch_bounds__(256) void router_logits_kernel(
    const float* __restrict__ x, const float* __restrict__ w_r,
    const float* __restrict__ b_r, float* __restrict__ part, int64_t T, int d, int N) {
  __shared__ float xs[2][RT_M][RT_K + RT_PAD];
  __shared__ float ws[2][RT_N][RT_K + RT_PAD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.x * RT_M;
  const int e0 = blockIdx.y * RT_N;

  // staging assignment: x and W tiles 64 x 32 fp32, two 4-element chunks
  // per thread each
  float4 xr[2], wr[2];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int q = tid + i * 256, r = q >> 3, c = (q & 7) * 4;
      int64_t t = t0 + r; if (t >= T) t = T - 1;
      xr[i] = *(const float4*)(x + t * d + k0 + c);
      int e = e0 + r;
      if (e < N) wr[i] = *(const float4*)(w_r + (int64_t)e * d + k0 + c);
      else wr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int q = tid + i * 256, r = q >> 3, c = (q & 7) * 4;
      xs[buf][r][c + 0] = xr[i].x; xs[buf][r][c + 1] = xr[i].y;
      xs[buf][r][c + 2] = xr[i].z; xs[buf][r][c + 3] = xr[i].w;
      ws[buf][r][c + 0] = wr[i].x; ws[buf][r][c + 1] = wr[i].y;
      ws[buf][r][c + 2] = wr[i].z; ws[buf][r][c + 3] = wr[i].w;
    }
  };

  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;

  const int nks = d / RT_K;  // K steps in total; this split owns [k_lo, k_hi)
  const int k_lo = (int)(((int64_t)blockIdx.z * nks) / gridDim.z);
  const int k_hi = (int)(((int64_t)(blockIdx.z + 1) * nks) / gridDim.z);
  const int nk = k_hi - k_lo;
  load_tile(k_lo * RT_K);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile((k_lo + kt + 1) * RT_K);
    const int ar = wm * 32 + (lane & 31), br = wn * 32 + (lane & 31), kk = lane >> 5;
#pragma unroll
    for (int s = 0; s < RT_K / 2; ++s) {
      float a = xs[buf][ar][2 * s + kk];
      float b = ws[buf][br][2 * s + kk];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }
  // D layout: column = lane % 32, row = 8*(v/4) + 4*(lane/32) + v%4
  const int col = e0 + wn * 32 + (lane & 31);
  float* out = part + (int64_t)blockIdx.z * T * N;
  if (col < N) {
    // one split: this is the final logit, bias included
    const float bias = (gridDim.z == 1 && b_r) ? b_r[col] : 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int row = wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      int64_t t = t0 + row;
      if (t < T) out[t * N + col] = acc[v] + bias;
    }
  }
}

// bf16 activations: each fp32 router weight is split exactly into three
// bf16 parts, w = hi + mid + lo (hi the round-to-nearest bf16 of w, mid of
// w - hi, lo of what is left: 3 x 8 significand bits hold all 24).  Every
// product of a bf16 x with a part is exact in fp32 and the MFMA accumulates
// in fp32, so v_mfma_f32_32x32x16_bf16 gives fp32-accurate logits at bf16
// matrix-core rate.  The split is done while the weight tile is staged, so
// the fp32 weight is read once per tile and nothing is precomputed.
// Tile: 64*FM tokens x 64 experts, four waves in a 2x2 grid (wave tile
// 32*FM x 32).  K is staged RBK = 64 wide (d is a multiple of 64); the next
// slice is loaded into registers while the MFMAs of the current one run
// from LDS, and about 46 KB of LDS per workgroup lets three share a CU.  K
// splits over gridDim.z as in the fp32 kernel.
constexpr int RB_N = 64;

__device__ __forceinline__ void split3_bf16(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16(w);
  const float r1 = w - bf16_to_f32(hi);  // exact
  mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);  // exact
  lo = f32_to_bf16(r2);
}

__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) {
  return (uint32_t)a | ((uint32_t)b << 16);
}

template <int FM, int RBK>
__global__ __launch_bounds__(256) void router_logits_bf16x3_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w_r,
    const float* __restrict__ b_r, float* __restrict__ part, int64_t T, int d, int N) {
  constexpr int BM = 64 * FM;
  constexpr int LD = RBK + 8;                 // LDS row, bf16 elements (16-byte aligned rows)
  constexpr int XC = RBK / 8;                 // 16-byte x chunks per row
  constexpr int XL = BM * XC / 256;           // x chunks per thread
  constexpr int WC = RBK / 4;                 // float4 w chunks per row
  constexpr int WL = RB_N * WC / 256;         // w chunks per thread
  static_assert(XL >= 1 && WL >= 1 && (BM * XC) % 256 == 0 && (RB_N * WC) % 256 == 0, "staging");
  __shared__ __attribute__((aligned(16))) uint16_t xs[BM][LD];
  __shared__ __attribute__((aligned(16))) uint16_t ws[3][RB_N][LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.x * BM;
  const int e0 = blockIdx.y * RB_N;

  // staging registers as named variables (an indexed array ended up in
  // scratch memory)
  static_assert(XL <= 4 && WL <= 4, "staging registers");
  uint4 xr0, xr1, xr2, xr3;
  float4 wr0, wr1, wr2, wr3;
#define MOE_RB_LDX(I, K0)                                                            \
  if (XL > I) {                                                                      \
    const int q = tid + I * 256, r = q / XC, c = (q % XC) * 8;                       \
    const int64_t t = t0 + r < T ? t0 + r : T - 1;                                   \
    xr##I = *(const uint4*)(x + t * d + (K0) + c);                                   \
  }
#define MOE_RB_LDW(I, K0)                                                            \
  if (WL > I) {                                                                      \
    const int q = tid + I * 256, r = q / WC, c = (q % WC) * 4;                       \
    const int e = e0 + r;                                                            \
    wr##I = e < N ? *(const float4*)(w_r + (int64_t)e * d + (K0) + c)                \
                  : make_float4(0.f, 0.f, 0.f, 0.f);                                 \
  }
#define MOE_RB_STX(I)                                                                \
  if (XL > I) {                                                                      \
    const int q = tid + I * 256, r = q / XC, c = (q % XC) * 8;                       \
    *(uint4*)&xs[r][c] = xr##I;                                                      \
  }
#define MOE_RB_STW(I)                                                                \
  if (WL > I) {                                                                      \
    const int q = tid + I * 256, r = q / WC, c = (q % WC) * 4;                       \
    uint16_t h0, h1, h2, h3, m0, m1, m2, m3, l0, l1, l2, l3;                         \
    split3_bf16(wr##I.x, h0, m0, l0);                                                \
    split3_bf16(wr##I.y, h1, m1, l1);                                                \
    split3_bf16(wr##I.z, h2, m2, l2);                                                \
    split3_bf16(wr##I.w, h3, m3, l3);                                                \
    *(uint2*)&ws[0][r][c] = make_uint2(pack2(h0, h1), pack2(h2, h3));                \
    *(uint2*)&ws[1][r][c] = make_uint2(pack2(m0, m1), pack2(m2, m3));                \
    *(uint2*)&ws[2][r][c] = make_uint2(pack2(l0, l1), pack2(l2, l3));                \
  }
#define MOE_RB_LOAD(K0)                                                              \
  do {                                                                               \
    MOE_RB_LDX(0, K0) MOE_RB_LDX(1, K0) MOE_RB_LDX(2, K0) MOE_RB_LDX(3, K0)          \
    MOE_RB_LDW(0, K0) MOE_RB_LDW(1, K0) MOE_RB_LDW(2, K0) MOE_RB_LDW(3, K0)          \
  } while (0)
#define MOE_RB_STORE()                                                               \
  do {                                                                               \
    MOE_RB_STX(0) MOE_RB_STX(1) MOE_RB_STX(2) MOE_RB_STX(3)                          \
    MOE_RB_STW(0) MOE_RB_STW(1) MOE_RB_STW(2) MOE_RB_STW(3)                          \
  } while (0)

  f32x16_t acc[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

  const int nks = d / RBK;
  const int k_lo = (int)(((int64_t)blockIdx.z * nks) / gridDim.z);
  const int k_hi = (int)(((int64_t)(blockIdx.z + 1) * nks) / gridDim.z);
  const int nk = k_hi - k_lo;
  const int kq = (lane >> 5) * 8;
  const int k_last = k_hi > k_lo ? k_hi - 1 : k_lo;
  MOE_RB_LOAD((k_lo < k_last ? k_lo : k_last) * RBK);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();  // the previous slice's fragments have been read
    MOE_RB_STORE();
    __syncthreads();
    // next slice in flight during the MFMAs (the last step re-loads its own
    // slice: the loads stay unconditional and the registers are not used)
    {
      const int kn = k_lo + kt + 1 < k_last ? k_lo + kt + 1 : k_last;
      MOE_RB_LOAD(kn * RBK);
    }
#pragma unroll
    for (int ks = 0; ks < RBK / 16; ++ks) {
      const int kk = ks * 16 + kq;
      bf16x8_t fb[3];
#pragma unroll
      for (int p = 0; p < 3; ++p)
        fb[p] = __builtin_bit_cast(bf16x8_t, *(const uint4*)&ws[p][wn * 32 + (lane & 31)][kk]);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const bf16x8_t fa =
            __builtin_bit_cast(bf16x8_t, *(const uint4*)&xs[wm * 32 * FM + i * 32 + (lane & 31)][kk]);
#pragma unroll
        for (int p = 0; p < 3; ++p)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb[p], acc[i], 0, 0, 0);
      }
    }
  }
#undef MOE_RB_LDX
#undef MOE_RB_LDW
#undef MOE_RB_STX
#undef MOE_RB_STW
#undef MOE_RB_LOAD
#undef MOE_RB_STORE
  // D layout: column (expert) = lane % 32, row (token) = 8*(v/4) + 4*(lane/32) + v%4
  const int col = e0 + wn * 32 + (lane & 31);
  float* out = part + (int64_t)blockIdx.z * T * N;
  if (col < N) {
    const float bias = (gridDim.z == 1 && b_r) ? b_r[col] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 32 * FM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int64_t t = t0 + row;
        if (t < T) out[t * N + col] = acc[i][v] + bias;
      }
  }
}

// ---------------------------------------------- router GEMM, LDS DMA ----
// The same exact three-part split, done once per call into planes
// [3][N][d] bf16 (hi, mid, lo), so the logits become a plain bf16 GEMM of x
// [T, d] against 3N weight rows that the ping-pong scheme of the expert
// GEMMs can stream:
//  * 256 tokens x 64 experts per workgroup; its B tile holds the 64 experts'
//    rows of each plane (192 rows).  8 waves, 64 tokens x 32 experts each:
//    two token fragments and one fragment per plane, one accumulator per
//    plane and token fragment; the planes are added in the epilogue.
//  * Global -> LDS with buffer_load ... lds in 64-wide K blocks (8 rows x
//    128 bytes per wave instruction), rings of 2 A and 3 B blocks (136 KB),
//    16-byte chunks swizzled by pp_swz; every 32-wide K sub-step a wave reads
//    its fragments (memory phase) and runs its 12 MFMAs (compute phase), the
//    second group of four waves one phase behind the first, so each SIMD
//    has one wave on the matrix pipe while the other reads LDS.
//  * blockIdx.z takes an even share of the K blocks; with several shares
//    each writes fp32 partials [z, T, N] (added in split order by the top-K
//    kernel or router_split_reduce_kernel), with one the logits plus bias.
//  * A tile of at most 128 tokens loads and multiplies only its first half.
constexpr int RG_BM = 256, RG_BE = 64;

__global__ __launch_bounds__(256) void router_split_planes_kernel(
    const float* __restrict__ w, int64_t n, uint16_t* __restrict__ planes) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n;
       i += (int64_t)gridDim.x * 1024) {
    const float4 v = *(const float4*)(w + i);
    uint16_t h0, h1, h2, h3, m0, m1, m2, m3, l0, l1, l2, l3;
    split3_bf16(v.x, h0, m0, l0);
    split3_bf16(v.y, h1, m1, l1);
    split3_bf16(v.z, h2, m2, l2);
    split3_bf16(v.w, h3, m3, l3);
    *(uint2*)(planes + i) = make_uint2(pack2(h0, h1), pack2(h2, h3));
    *(uint2*)(planes + n + i) = make_uint2(pack2(m0, m1), pack2(m2, m3));
    *(uint2*)(planes + 2 * n + i) = make_uint2(pack2(l0, l1), pack2(l2, l3));
  }
}

__global__ __launch_bounds__(512, 1) void router_logits_pp_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ planes,
    const float* __restrict__ b_r, float* __restrict__ out, int64_t T, int d, int N) {
  constexpr int BM = RG_BM, BE = RG_BE, BN = 3 * BE, WM = 4, WN = 2, NW = 8, DA = 2, DB = 3;
  constexpr int FM = BM / (WM * 32);                     // token fragments per wave
  constexpr int LA = BM / (NW * 8), LB = BN / (NW * 8);  // DMA instructions per wave per block
  constexpr int ASLOT = BM * 128, BSLOT = BN * 128;
  static_assert(BE % 8 == 0 && WN * 32 == BE, "a DMA instruction's 8 rows are in one plane");
  extern __shared__ uint4 smem[];
  char* abuf = (char*)smem;
  char* bbuf = abuf + DA * ASLOT;
  const uint4* abuf4 = (const uint4*)abuf;
  const uint4* bbuf4 = (const uint4*)bbuf;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wm = wave / WN, wn = wave % WN;
  const int dh = lane >> 5, drow = (lane & 31) >> 2, dch = lane & 3, khalf = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * BM;
  const int e0 = blockIdx.y * BE;
  const int nkb = d / 64;
  const int kb0 = (int)(((int64_t)blockIdx.z * nkb) / gridDim.z);
  const int nk = (int)(((int64_t)(blockIdx.z + 1) * nkb) / gridDim.z) - kb0;  // >= 1
  const int Mt = (int)(T - t0 < BM ? T - t0 : BM);

  int aidx[FM], asw[FM], bidx[3], bsw[3];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = i * (32 * WM) + wm * 32 + (lane & 31);
    aidx[i] = (r >> 3) * 64 + (r & 7) * 4;
    asw[i] = pp_swz(r);
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int r = q * BE + wn * 32 + (lane & 31);
    bidx[q] = (r >> 3) * 64 + (r & 7) * 4;
    bsw[q] = pp_swz(r);
  }
  uint32_t aoff[LA], boff[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = (i * NW + wave) * 8 + drow;
    const int lr = r < Mt ? r : Mt - 1;
    aoff[i] = (uint32_t)(((t0 + lr) * d + dh * 32 + (dch ^ pp_swz(r)) * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (i * NW + wave) * 8 + drow;
    const int e = e0 + r % BE < N ? e0 + r % BE : N - 1;
    boff[i] = (uint32_t)((((int64_t)(r / BE) * N + e) * d + dh * 32 + (dch ^ pp_swz(r)) * 8) * 2);
  }

  auto run = [&](auto half_c) {
    constexpr bool HALF = decltype(half_c)::value;
    constexpr int FMA = HALF ? FM / 2 : FM;
    constexpr int LAA = HALF ? LA / 2 : LA;
    auto issue_a = [&](int blk, int slot) {
      const uint32_t kb = (uint32_t)(kb0 + (blk < nk ? blk : nk - 1)) * 128u;
      char* st = abuf + slot * ASLOT;
#pragma unroll
      for (int i = 0; i < LAA; ++i) buf_dma16(x, aoff[i] + kb, st + (i * NW + wave) * 1024);
    };
    auto issue_b = [&](int blk, int slot) {
      const uint32_t kb = (uint32_t)(kb0 + (blk < nk ? blk : nk - 1)) * 128u;
      char* st = bbuf + slot * BSLOT;
#pragma unroll
      for (int i = 0; i < LB; ++i) buf_dma16(planes, boff[i] + kb, st + (i * NW + wave) * 1024);
    };
    f32x16_t acc[3][FMA];
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < FMA; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][i][v] = 0.f;
    bf16x8_t fa[2][FMA], fb[2][3];
    auto read_fragments = [&](int sa, int sb, int h) {
      const uint4* sA = abuf4 + sa * (ASLOT / 16) + h * 32;
      const uint4* sB = bbuf4 + sb * (BSLOT / 16) + h * 32;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ch = ks * 2 + khalf;
#pragma unroll
        for (int i = 0; i < FMA; ++i) fa[ks][i] = __builtin_bit_cast(bf16x8_t, sA[aidx[i] + (ch ^ asw[i])]);
#pragma unroll
        for (int q = 0; q < 3; ++q) fb[ks][q] = __builtin_bit_cast(bf16x8_t, sB[bidx[q] + (ch ^ bsw[q])]);
      }
    };
    auto finish_m_then_compute = [&]() {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
          for (int i = 0; i < FMA; ++i)
            acc[q][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][q], fa[ks][i], acc[q][i], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };

    issue_b(0, 0);
    issue_a(0, 0);
    issue_b(1, 1);
    wait_vmcnt<LB>();
    __syncthreads();
    if (grp == 1) __builtin_amdgcn_s_barrier();  // the second group runs one phase behind
    int sa = 0, sb = 0;
    for (int j = 0; j < nk; ++j) {
      const int sa1 = sa + 1 == DA ? 0 : sa + 1;
      const int sb1 = sb + 1 == DB ? 0 : sb + 1;
      const int sb2 = sb1 + 1 == DB ? 0 : sb1 + 1;
      read_fragments(sa, sb, 0);
      __builtin_amdgcn_sched_barrier(0);
      issue_a(j + 1, sa1);
      finish_m_then_compute();
      read_fragments(sa, sb, 1);
      __builtin_amdgcn_sched_barrier(0);
      issue_b(j + 2, sb2);
      wait_vmcnt<LB>();  // this wave's shares of A(j+1) and B(j+1) landed
      finish_m_then_compute();
      sa = sa1;
      sb = sb1;
    }
    if (grp == 0) __builtin_amdgcn_s_barrier();
    wait_vmcnt<0>();

    // 4 consecutive experts per lane and register quad
    const bool direct = gridDim.z == 1;
    float* o = out + (direct ? 0 : (int64_t)blockIdx.z * T * N);
#pragma unroll
    for (int i = 0; i < FMA; ++i) {
      const int lr = i * (32 * WM) + wm * 32 + (lane & 31);
      if (lr >= Mt) continue;
      float* orow = o + (t0 + lr) * N;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int e = e0 + wn * 32 + 8 * qd + 4 * khalf;
        float r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int v = 4 * qd + u;
          r[u] = acc[0][i][v] + acc[1][i][v] + acc[2][i][v];
          if (direct && b_r && e + u < N) r[u] += b_r[e + u];
        }
        if ((N & 3) == 0 && e + 3 < N) {
          *(float4*)(orow + e) = make_float4(r[0], r[1], r[2], r[3]);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (e + u < N) orow[e + u] = r[u];
        }
      }
    }
  };
  if (Mt <= BM / 2) run(std::true_type{});
  else run(std::false_type{});
}


// part[0][i] + part[1][i] + ... + part[nsplit - 1][i] (planes n apart), added
// in split order.  With ZB > 1 the partials are loaded ZB at a time before
// they are added, so a thread has ZB loads in flight instead of one after
// another (the small batches, whose many splits made this latency-bound);
// with few splits (the top-K kernel's large batches) the plain loop is
// cheaper.
template <int ZB>
__device__ __forceinline__ float sum_splits(const float* __restrict__ part, int nsplit, int64_t n,
                                            int64_t i) {
  float acc = part[i];
  if (ZB == 1) {
    for (int z = 1; z < nsplit; ++z) acc += part[(int64_t)z * n + i];
    return acc;
  }
  for (int z = 1; z < nsplit; z += ZB) {
    float v[ZB];
#pragma unroll
    for (int u = 0; u < ZB; ++u) v[u] = z + u < nsplit ? part[(int64_t)(z + u) * n + i] : 0.f;
#pragma unroll
    for (int u = 0; u < ZB; ++u)
      if (z + u < nsplit) acc += v[u];
  }
  return acc;
}

// logits[t, e] = sum_{z = 0, 1, ...} part[z, t, e] + b_r[e] (fixed order): the
// batches whose top-K kernel does not add the splits itself.
__global__ __launch_bounds__(256) void router_split_reduce_kernel(
    const float* __restrict__ part, int nsplit, const float* __restrict__ b_r,
    float* __restrict__ logits, int64_t T, int N) {
  const int64_t n = T * (int64_t)N;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    logits[i] = sum_splits<16>(part, nsplit, n, i) + (b_r ? b_r[i % N] : 0.f);
}

// --------------------------------------------------------------- top-K ----
// One wave per token.  Lane l holds experts l, l+64, ... (up to 16 each).
// Selection key s = logit + b_sel, turned into an unsigned key that orders
// like the float (NaN below -inf); ties go to the lower expert index by
// packing (key, ~index) into 64 bits and taking the maximum.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: lowest
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave reductions through DPP (no LDS round trip): within each row of 16
// lanes, quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror and row_mirror
// leave every lane with its row's result; row_bcast15 (into rows 1 and 3)
// and row_bcast31 (into rows 2 and 3) then carry rows 0-2 into row 3, and
// lane 63 is read into every lane.  The order of combination is fixed, so
// a sum is deterministic.  Lanes a broadcast step leaves out combine the
// identity.
template <int CTRL, int RMASK>
__device__ __forceinline__ uint32_t dpp_src(uint32_t v, uint32_t ident) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, RMASK, 0xF, false);
}
#define MOE_DPP_REDUCE(V, IDENT, OP)                                   \
  do {                                                                 \
    V = OP(V, (dpp_src<0xB1, 0xF>(V, IDENT)));                          \
    V = OP(V, (dpp_src<0x4E, 0xF>(V, IDENT)));                          \
    V = OP(V, (dpp_src<0x141, 0xF>(V, IDENT)));                         \
    V = OP(V, (dpp_src<0x140, 0xF>(V, IDENT)));                         \
    V = OP(V, (dpp_src<0x142, 0xA>(V, IDENT)));                         \
    V = OP(V, (dpp_src<0x143, 0xC>(V, IDENT)));                         \
    V = (uint32_t)__builtin_amdgcn_readlane((int)V, 63);               \
  } while (0)

__device__ __forceinline__ uint32_t umax_op(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t fmax_op(uint32_t a, uint32_t b) {
  return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
}
__device__ __forceinline__ uint32_t fadd_op(uint32_t a, uint32_t b) {
  return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
}
__device__ __forceinline__ uint32_t wave_umax_dpp(uint32_t v) {
  MOE_DPP_REDUCE(v, 0u, umax_op);
  return v;
}
__device__ __forceinline__ float wave_max_dpp(float x) {
  uint32_t v = __float_as_uint(x);
  MOE_DPP_REDUCE(v, 0xff800000u, fmax_op);  // identity -inf
  return __uint_as_float(v);
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
  uint32_t v = __float_as_uint(x);
  MOE_DPP_REDUCE(v, 0u, fadd_op);
  return __uint_as_float(v);
}
#undef MOE_DPP_REDUCE

// One token's softmax statistics, top-K selection and gates, computed by
// one wave: lane l holds the logits of experts l, l + 64, ... in l[].  Adds
// the token's probabilities to pacc, its sum of squared logits to zsum and
// its squared log-sum-exp to lsum and the entropy of its routing
// distribution to hsum; writes K ids and gates; counts each chosen expert in
// scnt (LDS, integer atomics).
template <int NJ>
__device__ __forceinline__ void topk_one_token(const float (&l)[NJ], const float (&bsel)[NJ],
                                               int lane, int N, int K, int gate_mode,
                                               float (&pacc)[NJ], float& zsum, float& lsum,
                                               float& hsum, int32_t* __restrict__ idx_t,
                                               float* __restrict__ gate_t, int32_t* scnt) {
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NJ; ++j) m = fmaxf(m, l[j]);
  m = wave_max_dpp(m);
  float ssum = 0.f, sq = 0.f, gap = 0.f;
  float ex[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    int e = lane + 64 * j;
    ex[j] = (e < N) ? expf(l[j] - m) : 0.f;
    ssum += ex[j];
    sq += (e < N) ? l[j] * l[j] : 0.f;
    gap += (ex[j] > 0.f) ? ex[j] * (m - l[j]) : 0.f;
  }
  ssum = wave_sum_dpp(ssum);
  sq = wave_sum_dpp(sq);
  gap = wave_sum_dpp(gap);
  const float inv = 1.0f / ssum;
#pragma unroll
  for (int j = 0; j < NJ; ++j) pacc[j] += ex[j] * inv;
  const float lse = m + logf(ssum);
  zsum += sq;
  lsum += lse * lse;
  // entropy -sum P log P = log(ssum) + sum P (m - l): two non-negative terms
  hsum += logf(ssum) + gap * inv;

  // K rounds of arg-max over the not-yet-taken experts
  uint32_t taken = 0;
  float my_l = 0.f;  // lane k keeps the logit of its chosen expert
  int my_e = 0;
  float lmax_sel = -INFINITY;
  for (int r = 0; r < K; ++r) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int e = lane + 64 * j;
      if (e < N && !((taken >> j) & 1u)) {
        unsigned long long key =
            ((unsigned long long)order_key(l[j] + bsel[j]) << 32) |
            (unsigned long long)(0xffffffffu - (uint32_t)e);
        best = key > best ? key : best;
      }
    }
    // the 64-bit maximum as two 32-bit ones: the largest key, then the
    // largest ~index among the lanes holding it (= the lowest index)
    const uint32_t khi = (uint32_t)(best >> 32);
    const uint32_t kmax = wave_umax_dpp(khi);
    const uint32_t ilo = wave_umax_dpp(khi == kmax ? (uint32_t)(best & 0xffffffffull) : 0u);
    const int ew = __builtin_amdgcn_readfirstlane((int)(0xffffffffu - ilo));
    const int jw = ew >> 6;
    float cand = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) cand = (j == jw) ? l[j] : cand;
    const float lw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cand), ew & 63));
    if (lane == (ew & 63)) taken |= 1u << jw;
    if (lane == r) { my_l = lw; my_e = ew; }
    lmax_sel = fmaxf(lmax_sel, lw);
    if (lane == 0) atomicAdd(&scnt[ew], 1);  // integer: order-independent
  }
  // gates
  float g;
  if (gate_mode == 2) {  // softmax over all N, not renormalised
    g = expf(my_l - m) * inv;
  } else {  // renormalised over the chosen K (both forms are equal)
    float ek = (lane < K) ? expf(my_l - lmax_sel) : 0.f;
    float den = wave_sum_dpp(ek);
    g = ek / den;
  }
  if (lane < K) {
    idx_t[lane] = my_e;
    gate_t[lane] = g;
  }
}

// With nsplit > 1 the logits are first formed from the K-split partials
// part [nsplit, T, N] (added in split order, then b_r) and written to
// logits; with one split they are read from logits.
template <int NJ>
__global__ __launch_bounds__(256) void router_topk_kernel(
    float* __restrict__ logits, const float* __restrict__ part, int nsplit,
    const float* __restrict__ b_r, RouterNoise noise,
    const float* __restrict__ b_sel, int32_t* __restrict__ idx, float* __restrict__ gate,
    float* __restrict__ part_p, int32_t* __restrict__ part_cnt,
    float* __restrict__ part_z, int64_t T, int N, int K, int gate_mode,
    int tpb) {
  extern __shared__ unsigned char smem_raw[];
  float* sp = (float*)smem_raw;                  // [4][N] per-wave prob sums
  int32_t* scnt = (int32_t*)(sp + 4 * N);        // [N] block counts
  float* sz = (float*)(scnt + N);                // [4][3]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < N; e += 256) scnt[e] = 0;
  __syncthreads();

  float pacc[NJ];
  float bsel[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    pacc[j] = 0.f;
    int e = lane + 64 * j;
    bsel[j] = (b_sel && e < N) ? b_sel[e] : 0.f;
  }
  float zsum = 0.f, lsum = 0.f, hsum = 0.f;

  const int64_t tb0 = (int64_t)blockIdx.x * tpb;
  const int per_wave = tpb / 4;
  for (int i = 0; i < per_wave; ++i) {
    const int64_t t = tb0 + (int64_t)wave * per_wave + i;
    if (t >= T) break;
    float l[NJ];
    const int64_t n = T * (int64_t)N;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int e = lane + 64 * j;
      if (e < N) {
        const int64_t i = t * N + e;
        if (nsplit > 1) {
          // many splits (few expert tiles, e.g. 64 experts: 8 splits): eight
          // partials in flight at a time; two: the plain loop, which measured
          // faster there
          l[j] = (nsplit > 2 ? sum_splits<8>(part, nsplit, n, i) : sum_splits<1>(part, nsplit, n, i)) +
                 (b_r ? b_r[e] : 0.f);
          logits[i] = l[j];
        } else {
          l[j] = logits[i];
        }
        if (noise_on(noise)) l[j] += noise.std * noise_draw(noise, i);
      } else {
        l[j] = -INFINITY;
      }
    }
    topk_one_token<NJ>(l, bsel, lane, N, K, gate_mode, pacc, zsum, lsum, hsum, idx + t * K,
                       gate + t * K, scnt);
  }
  // fixed-order reduction of the block's partial sums
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    int e = lane + 64 * j;
    if (e < N) sp[wave * N + e] = pacc[j];
  }
  if (lane == 0) { sz[wave * 3] = zsum; sz[wave * 3 + 1] = lsum; sz[wave * 3 + 2] = hsum; }
  __syncthreads();
  for (int e = tid; e < N; e += 256) {
    float s = sp[e];
    s += sp[N + e];
    s += sp[2 * N + e];
    s += sp[3 * N + e];
    part_p[(int64_t)blockIdx.x * N + e] = s;
    part_cnt[(int64_t)blockIdx.x * N + e] = scnt[e];
  }
  if (tid < 3) part_z[blockIdx.x * 3 + tid] = ((sz[tid] + sz[3 + tid]) + sz[6 + tid]) + sz[9 + tid];
}

// --------------------------------------------------------------- stats ----
// One auxiliary-loss-free step of the selection bias: up by bias_rate if the
// expert's count is below the mean load T*K/N, down if above, unchanged at
// it (compared exactly, as count*N against T*K).  b_sel may be null (0).
__device__ __forceinline__ float bias_step(const float* b_sel, int e, int64_t count, int64_t T,
                                           int K, int N, float bias_rate) {
  const int64_t diff = T * (int64_t)K - count * (int64_t)N;
  const float b = b_sel ? b_sel[e] : 0.f;
  return diff > 0 ? b + bias_rate : (diff < 0 ? b - bias_rate : b);
}

// Per-expert statistics.  Block b owns experts [64 b, 64 b + 64).  Thread t
// sums, for expert 64 b + t % 64, the block partials j = c, c + 16, ...
// (c = t / 64) in increasing j; the first 64 threads add the 16 chunk sums
// in order and write count, f and p; thread 0 adds the block's f_e * p_e in
// expert order into part_fp[b].  Every sum runs in a fixed order.
// Loss terms: aux = alpha * N * aux_sum (aux_sum: the part_fp values added in
// block order); z and z_lse from the per-token-block partials (strided sums,
// then a fixed tree).  Called by every thread of a block of 1024.
__device__ __forceinline__ void stats_final_body(float aux_sum, const float* __restrict__ part_z,
                                                 int64_t nblk, int64_t T, int N, float alpha,
                                                 float* __restrict__ loss,
                                                 float* __restrict__ entropy) {
  __shared__ float rz[1024], rl[1024], rh[1024];
  const int tid = threadIdx.x;
  float z = 0.f, zl = 0.f, h = 0.f;
  for (int64_t b = tid; b < nblk; b += 1024) {
    z += part_z[3 * b];
    zl += part_z[3 * b + 1];
    h += part_z[3 * b + 2];
  }
  rz[tid] = z;
  rl[tid] = zl;
  rh[tid] = h;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (tid < o) {
      rz[tid] += rz[tid + o];
      rl[tid] += rl[tid + o];
      rh[tid] += rh[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const float invT = 1.0f / (float)T;
    if (loss) {
      loss[0] = alpha * (float)N * aux_sum;
      loss[1] = rz[0] * invT;
      loss[2] = rl[0] * invT;
    }
    if (entropy) entropy[0] = rh[0] * invT;
  }
}

__global__ __launch_bounds__(1024) void router_stats_expert_kernel(
    const float* __restrict__ part_p, const int32_t* __restrict__ part_cnt, int64_t nblk,
    int64_t T, int N, int K, int32_t* __restrict__ count, float* __restrict__ f,
    float* __restrict__ p, float* __restrict__ part_fp, const float* b_sel, float* b_out,
    float bias_rate, const float* __restrict__ part_z, float alpha, float* __restrict__ loss,
    float* __restrict__ entropy) {
  __shared__ float sp[1024];
  __shared__ int64_t sc[1024];
  __shared__ float red[64];
  const int tid = threadIdx.x, el = tid & 63, c = tid >> 6;
  const int e = blockIdx.x * 64 + el;
  float s = 0.f;
  int64_t cnt = 0;
  if (e < N) {
    // eight partials loaded before they are added (in the same order): one
    // dependent load per partial made this latency-bound
    int64_t j = c;
    for (; j + 16 * 7 < nblk; j += 16 * 8) {
      float v[8];
      int32_t q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v[u] = part_p[(j + 16 * u) * N + e];
        q[u] = part_cnt[(j + 16 * u) * N + e];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s += v[u];
        cnt += q[u];
      }
    }
    for (; j < nblk; j += 16) {
      s += part_p[j * N + e];
      cnt += part_cnt[j * N + e];
    }
  }
  sp[tid] = s;
  sc[tid] = cnt;
  __syncthreads();
  if (tid < 64) {
    float st = 0.f;
    int64_t ct = 0;
    for (int q = 0; q < 16; ++q) {
      st += sp[q * 64 + tid];
      ct += sc[q * 64 + tid];
    }
    float fp = 0.f;
    if (e < N) {
      const float pe = st * (1.0f / (float)T);
      const float fe = (float)ct * (1.0f / ((float)T * (float)K));
      if (count) count[e] = (int32_t)ct;
      if (f) f[e] = fe;
      if (p) p[e] = pe;
      if (b_out) b_out[e] = bias_step(b_sel, e, ct, T, K, N, bias_rate);
      fp = fe * pe;
    }
    red[tid] = fp;
  }
  __syncthreads();
  __shared__ float fp_sum;
  if (tid == 0) {
    float acc = 0.f;
    for (int i = 0; i < 64; ++i) acc += red[i];
    part_fp[blockIdx.x] = acc;
    fp_sum = acc;
  }
  if (gridDim.x == 1 && (loss || entropy)) {
    // one block holds every expert: the loss terms here, without a launch
    __syncthreads();
    stats_final_body(0.f + fp_sum, part_z, nblk, T, N, alpha, loss, entropy);
  }
}

// The loss terms of more than 64 experts (several expert blocks).
__global__ __launch_bounds__(1024) void router_stats_final_kernel(
    const float* __restrict__ part_fp, int nfp, const float* __restrict__ part_z, int64_t nblk,
    int64_t T, int N, float alpha, float* __restrict__ loss, float* __restrict__ entropy) {
  float aux = 0.f;
  for (int i = 0; i < nfp; ++i) aux += part_fp[i];
  stats_final_body(aux, part_z, nblk, T, N, alpha, loss, entropy);
}


// ------------------------------------------------- few experts, fused ----
// N <= 16 with bf16 x, more than 64 tokens: the logits, softmax, top-K,
// gates and the block's partial statistics in one kernel.  The logit GEMM is then 2 T d N flops,
// too few to fill matrix-core tiles, so it runs as fp32 FMAs (each product
// of a bf16 x and an fp32 weight is exact inside the fma; the sums are
// fp32), with x read once.
//  * A block takes tpb tokens in groups of G = 64 / NE (NE = 8 or 16, >= N).
//    Its NW waves split d: wave w, lane l take the 8 columns from
//    8 (l + 64 (w + NW i)), i = 0, 1, ..., and keep one partial per (token,
//    expert) of the group, 64 per lane, each summed in column order.
//  * A butterfly over the lanes (strides 32, 16, ..., 1; at stride s a lane
//    keeps the upper half of its values when its bit s is set, else the
//    lower half, and adds the partner's copy of that half) leaves lane L
//    with the wave's partial for token L / NE, expert L % NE.  The logit is
//    the wave partials added in wave order, then + b_r.
//  * Then one wave per token as in the top-K kernel (topk_one_token), and
//    the block's partial sums in the same layout, for router_stats.
// (A one-block form for T <= 64, statistics included, measured no faster
// than the split logits kernel and the small-batch kernel there: 18.6 us
// against 19.4 on the Mixtral-shaped decode; latency-bound on one CU.)
template <int NE, int NW>
__global__ __launch_bounds__(64 * NW, 2) void router_fused_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w_r, const float* __restrict__ b_r,
    RouterNoise noise, const float* __restrict__ b_sel, float* __restrict__ logits,
    int32_t* __restrict__ idx, float* __restrict__ gate, float* __restrict__ part_p,
    int32_t* __restrict__ part_cnt, float* __restrict__ part_z, int64_t T, int d, int N, int K,
    int gate_mode, int tpb) {
  static_assert(NE == 8 || NE == 16, "8 or 16 expert slots");
  constexpr int G = 64 / NE;
  __shared__ float red[NW][64];
  __shared__ float sp[NW][16];
  __shared__ int32_t scnt[16];
  __shared__ float sz[NW][3];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < 16) scnt[tid] = 0;
  __syncthreads();

  float pacc[1] = {0.f}, bsel[1];
  bsel[0] = (b_sel && lane < N) ? b_sel[lane] : 0.f;
  float zsum = 0.f, lsum = 0.f, hsum = 0.f;
  const int64_t tb0 = (int64_t)blockIdx.x * tpb;
  const int64_t tend = tb0 + tpb < T ? tb0 + tpb : T;
  for (int64_t t0 = tb0; t0 < tend; t0 += G) {
    float acc[64];
#pragma unroll
    for (int v = 0; v < 64; ++v) acc[v] = 0.f;
    for (int k = 8 * (lane + 64 * wave); k < d; k += 8 * 64 * NW) {
      // every load of the pass issued before the first fma, with the token
      // and expert indices clamped in range instead of tested, so that one
      // memory latency covers them all; the slots past tend or N then hold
      // duplicates that are never read
      uint4 xr[G];  // 8 bf16 of each token of the group
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t tt = t0 + g < tend ? t0 + g : tend - 1;
        xr[g] = *(const uint4*)(x + tt * d + k);
      }
      float4 wa[NE], wb[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int ee = e < N ? e : N - 1;
        wa[e] = *(const float4*)(w_r + (int64_t)ee * d + k);
        wb[e] = *(const float4*)(w_r + (int64_t)ee * d + k + 4);
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = acc[g * NE + e];
          a = fmaf(__uint_as_float(xr[g].x << 16), wa[e].x, a);
          a = fmaf(__uint_as_float(xr[g].x & 0xffff0000u), wa[e].y, a);
          a = fmaf(__uint_as_float(xr[g].y << 16), wa[e].z, a);
          a = fmaf(__uint_as_float(xr[g].y & 0xffff0000u), wa[e].w, a);
          a = fmaf(__uint_as_float(xr[g].z << 16), wb[e].x, a);
          a = fmaf(__uint_as_float(xr[g].z & 0xffff0000u), wb[e].y, a);
          a = fmaf(__uint_as_float(xr[g].w << 16), wb[e].z, a);
          a = fmaf(__uint_as_float(xr[g].w & 0xffff0000u), wb[e].w, a);
          acc[g * NE + e] = a;
        }
      }
    }
    // butterfly: 64 values per lane -> one (token, expert) partial per lane
#pragma unroll
    for (int st = 0; st < 6; ++st) {
      const int s = 32 >> st;  // stride, and half the values still held
      const bool up = (lane & s) != 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i < s) {
          const float send = up ? acc[i] : acc[i + s];
          const float keep = up ? acc[i + s] : acc[i];
          acc[i] = keep + __shfl_xor(send, s);
        }
      }
    }
    red[wave][lane] = acc[0];
    __syncthreads();
    for (int g = wave; g < G; g += NW) {
      const int64_t t = t0 + g;
      if (t >= tend) break;
      float l[1];
      if (lane < N) {
        float v = red[0][g * NE + lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[w][g * NE + lane];
        v += b_r ? b_r[lane] : 0.f;
        logits[t * N + lane] = v;
        if (noise_on(noise)) v += noise.std * noise_draw(noise, t * N + lane);
        l[0] = v;
      } else {
        l[0] = -INFINITY;
      }
      topk_one_token<1>(l, bsel, lane, N, K, gate_mode, pacc, zsum, lsum, hsum, idx + t * K,
                        gate + t * K, scnt);
    }
    __syncthreads();  // red is read before the next group writes it
  }
  if (lane < N) sp[wave][lane] = pacc[0];
  if (lane == 0) { sz[wave][0] = zsum; sz[wave][1] = lsum; sz[wave][2] = hsum; }
  __syncthreads();
  if (tid < N) {
    float v = sp[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += sp[w][tid];
    part_p[(int64_t)blockIdx.x * N + tid] = v;
    part_cnt[(int64_t)blockIdx.x * N + tid] = scnt[tid];
  }
  if (tid < 3) {
    float v = sz[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += sz[w][tid];
    part_z[blockIdx.x * 3 + tid] = v;
  }
}

// ------------------------------------------------------- small batches ----
// Everything after the logit GEMM in one workgroup of 16 waves, for small T:
// the sum of the logit splits (in split order, as router_split_reduce_kernel),
// top-K and gates (topk_one_token), and the statistics.  Wave w takes tokens
// w, w + 16, ...; the per-expert probability sums and the z terms are then
// added over the waves in wave order, f_e * p_e over experts in expert
// order.  Saves four launches on decode-sized batches.
template <int NJ>
__global__ __launch_bounds__(1024) void router_small_kernel(
    const float* __restrict__ part, int nsplit, const float* __restrict__ b_r,
    RouterNoise noise, const float* b_sel,
    float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ gate, int64_t T,
    int N, int K, int gate_mode, float alpha, int32_t* __restrict__ count, float* __restrict__ f,
    float* __restrict__ p, float* __restrict__ loss, float* __restrict__ entropy, float* b_out,
    float bias_rate) {
  extern __shared__ unsigned char smem_raw[];
  float* sp = (float*)smem_raw;                  // [16][N] per-wave prob sums
  int32_t* scnt = (int32_t*)(sp + 16 * N);       // [N] counts
  float* sfp = (float*)(scnt + N);               // [N] f_e * p_e
  float* sz = sfp + N;                           // [16][3]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < N; e += 1024) scnt[e] = 0;
  __syncthreads();

  float pacc[NJ], bsel[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    pacc[j] = 0.f;
    const int e = lane + 64 * j;
    bsel[j] = (b_sel && e < N) ? b_sel[e] : 0.f;
  }
  float zsum = 0.f, lsum = 0.f, hsum = 0.f;
  const int64_t n = T * (int64_t)N;
  for (int64_t t = wave; t < T; t += 16) {
    float l[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (e < N) {
        const int64_t i = t * N + e;
        if (nsplit > 1) {
          l[j] = sum_splits<16>(part, nsplit, n, i) + (b_r ? b_r[e] : 0.f);
          logits[i] = l[j];
        } else {
          l[j] = logits[i];
        }
        if (noise_on(noise)) l[j] += noise.std * noise_draw(noise, i);
      } else {
        l[j] = -INFINITY;
      }
    }
    topk_one_token<NJ>(l, bsel, lane, N, K, gate_mode, pacc, zsum, lsum, hsum, idx + t * K,
                       gate + t * K, scnt);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    if (e < N) sp[wave * N + e] = pacc[j];
  }
  if (lane == 0) { sz[wave * 3] = zsum; sz[wave * 3 + 1] = lsum; sz[wave * 3 + 2] = hsum; }
  // every wave has read b_sel (bsel[] above) before this barrier, so b_out
  // may alias it
  __syncthreads();
  for (int e = tid; e < N; e += 1024) {
    float st = 0.f;
    for (int w = 0; w < 16; ++w) st += sp[w * N + e];
    const int32_t ct = scnt[e];
    const float pe = st * (1.0f / (float)T);
    const float fe = (float)ct * (1.0f / ((float)T * (float)K));
    if (count) count[e] = ct;
    if (f) f[e] = fe;
    if (p) p[e] = pe;
    if (b_out) b_out[e] = bias_step(b_sel, e, ct, T, K, N, bias_rate);
    sfp[e] = fe * pe;
  }
  __syncthreads();
  if (tid == 0) {
    float aux = 0.f;
    for (int e = 0; e < N; ++e) aux += sfp[e];
    float z = 0.f, zl = 0.f, h = 0.f;
    for (int w = 0; w < 16; ++w) {
      z += sz[3 * w];
      zl += sz[3 * w + 1];
      h += sz[3 * w + 2];
    }
    const float invT = 1.0f / (float)T;
    if (loss) {
      loss[0] = alpha * (float)N * aux;
      loss[1] = z * invT;
      loss[2] = zl * invT;
    }
    if (entropy) entropy[0] = h * invT;
  }
}
}  // namespace

int router_tokens_per_block(int64_t T) {
  // one wave per token; blocks of 4 waves.  Enough blocks to cover the CUs
  // for small T (>= 4 tokens per block), 64 tokens per block for large T and
  // more when T is huge, so at most 4096 blocks.
  int64_t tpb = 4;
  while (tpb < 64 && (T + tpb - 1) / tpb > 512) tpb *= 2;
  while ((T + tpb - 1) / tpb > 4096) tpb *= 2;
  return (int)tpb;
}

int64_t router_num_blocks(int64_t T) {
  int tpb = router_tokens_per_block(T);
  return (T + tpb - 1) / tpb;
}

int router_tile_m(int64_t T, bool x_bf16) {
  return (x_bf16 && T >= 1024) ? 128 : 64;
}

bool router_fused_path(int64_t T, int N, bool x_bf16) {
  return x_bf16 && N <= 16 && T > kRouterSmallT;
}

bool router_gemm_path(int64_t T, int d, int N, bool x_bf16) {
  // From 1024 tokens on: below that, writing and re-reading the planes costs
  // more than the register-staged kernel's fp32 weight reads.  32-bit byte
  // offsets into x and into the planes.
  return x_bf16 && !router_fused_path(T, N, x_bf16) && T >= 1024 && d % 64 == 0 &&
         (int64_t)2 * T * d < (int64_t(1) << 32) && (int64_t)6 * N * d < (int64_t(1) << 32);
}

size_t router_planes_bytes(int64_t T, int d, int N, bool x_bf16) {
  return router_gemm_path(T, d, N, x_bf16) ? (size_t)6 * N * d : 0;
}

int router_num_splits(int64_t T, int d, int N, bool x_bf16) {
  if (router_fused_path(T, N, x_bf16)) return 1;
  if (router_gemm_path(T, d, N, x_bf16)) {
    // >= 256 workgroups (one per CU), each at least one 64-wide K block
    const int64_t tiles = ((T + RG_BM - 1) / RG_BM) * ((N + RG_BE - 1) / RG_BE);
    int64_t s = (256 + tiles - 1) / tiles;
    const int64_t max_s = d / 64 < 64 ? d / 64 : 64;
    return (int)(s < 1 ? 1 : (s > max_s ? max_s : s));
  }
  // aim for >= 512 workgroups, with at least 128 K elements per split
  const int tm = router_tile_m(T, x_bf16);
  const int64_t tiles = ((T + tm - 1) / tm) * ((N + RT_N - 1) / RT_N);
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t max_s = d / 128 > 0 ? d / 128 : 1;
  if (s > max_s) s = max_s;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return (int)s;
}

bool router_topk_adds_splits(int64_t T, int nsplit) { return nsplit > 1 && T >= 1024; }

hipError_t launch_router_logits(const void* x, bool x_bf16, const float* w_r, const float* b_r,
                                uint16_t* planes, float* part, float* logits, int64_t T, int d,
                                int N, hipStream_t stream, bool reduce_splits) {
  static_assert(RB_N == RT_N, "both logit kernels tile experts alike");
  const int ns = router_num_splits(T, d, N, x_bf16);
  if (router_gemm_path(T, d, N, x_bf16)) {
    if (!planes) return hipErrorInvalidValue;
    const int64_t n = (int64_t)N * d;
    int64_t sb = (n / 4 + 255) / 256;
    if (sb > 2048) sb = 2048;
    router_split_planes_kernel<<<(unsigned)sb, 256, 0, stream>>>(w_r, n, planes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int smem = 2 * RG_BM * 128 + 3 * (3 * RG_BE) * 128;
    static std::atomic<uint64_t> lds_set{0};
    e = set_dynamic_lds_once((const void*)router_logits_pp_kernel, smem, lds_set);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)((T + RG_BM - 1) / RG_BM), (unsigned)((N + RG_BE - 1) / RG_BE),
              (unsigned)ns);
    router_logits_pp_kernel<<<grid, 512, smem, stream>>>((const uint16_t*)x, planes, b_r,
                                                         ns == 1 ? logits : part, T, d, N);
  } else {
    const int tm = router_tile_m(T, x_bf16);
    dim3 grid((unsigned)((T + tm - 1) / tm), (unsigned)((N + RT_N - 1) / RT_N), (unsigned)ns);
    float* out = ns == 1 ? logits : part;
    const uint16_t* xb = (const uint16_t*)x;
    if (x_bf16 && tm == 128)
      router_logits_bf16x3_kernel<2, 64><<<grid, 256, 0, stream>>>(xb, w_r, b_r, out, T, d, N);
    else if (x_bf16)
      router_logits_bf16x3_kernel<1, 64><<<grid, 256, 0, stream>>>(xb, w_r, b_r, out, T, d, N);
    else
      router_logits_kernel<<<grid, 256, 0, stream>>>((const float*)x, w_r, b_r, out, T, d, N);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1 || !reduce_splits) return e;
  int64_t blocks = (T * (int64_t)N + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  router_split_reduce_kernel<<<(unsigned)blocks, 256, 0, stream>>>(part, ns, b_r, logits, T, N);
  return hipGetLastError();
}

hipError_t launch_router_topk(float* logits, const float* part, int nsplit, const float* b_r,
                              const RouterNoise& noise, const float* b_sel, int32_t* idx,
                              float* gate, float* part_p, int32_t* part_cnt, float* part_z,
                              int64_t T, int N, int K, int gate_mode, hipStream_t stream) {
  const int tpb = router_tokens_per_block(T);
  const unsigned nblk = (unsigned)((T + tpb - 1) / tpb);
  const size_t smem = (size_t)4 * N * sizeof(float) + (size_t)N * sizeof(int32_t) + 12 * sizeof(float);
  const int nj = (N + 63) / 64;
#define MOE_TOPK_CASE(NJV)                                                              \
  case NJV:                                                                             \
    router_topk_kernel<NJV><<<nblk, 256, smem, stream>>>(logits, part, nsplit, b_r, noise, b_sel, \
        idx, gate, part_p, part_cnt, part_z, T, N, K, gate_mode, tpb);                 \
    break;
  switch (nj) {
    MOE_TOPK_CASE(1) MOE_TOPK_CASE(2) MOE_TOPK_CASE(3) MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(5) MOE_TOPK_CASE(6) MOE_TOPK_CASE(7) MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(9) MOE_TOPK_CASE(10) MOE_TOPK_CASE(11) MOE_TOPK_CASE(12)
    MOE_TOPK_CASE(13) MOE_TOPK_CASE(14) MOE_TOPK_CASE(15) MOE_TOPK_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

hipError_t launch_router_stats(const float* part_p, const int32_t* part_cnt,
                               const float* part_z, float* part_fp, int64_t nblk, int64_t T,
                               int N, int K, float alpha, int32_t* count,
                               float* f, float* p, float* loss, float* entropy,
                               const float* b_sel, float* b_sel_out, float bias_rate,
                               hipStream_t stream) {
  const int nfp = (N + 63) / 64;
  router_stats_expert_kernel<<<nfp, 1024, 0, stream>>>(part_p, part_cnt, nblk, T, N, K, count,
                                                       f, p, part_fp, b_sel, b_sel_out,
                                                       bias_rate, part_z, alpha, loss, entropy);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (!loss && !entropy) || nfp == 1) return e;
  router_stats_final_kernel<<<1, 1024, 0, stream>>>(part_fp, nfp, part_z, nblk, T, N, alpha, loss,
                                                    entropy);
  return hipGetLastError();
}

hipError_t launch_router_fused(const void* x, const float* w_r, const float* b_r,
                               const RouterNoise& noise, const float* b_sel, float* logits,
                               int32_t* idx, float* gate, float* part_p, int32_t* part_cnt,
                               float* part_z, int64_t T, int d, int N, int K, int gate_mode,
                               hipStream_t stream) {
  const int tpb = router_tokens_per_block(T);
  const unsigned nblk = (unsigned)((T + tpb - 1) / tpb);
  auto kern = N <= 8 ? router_fused_kernel<8, 4> : router_fused_kernel<16, 4>;
  kern<<<nblk, 256, 0, stream>>>((const uint16_t*)x, w_r, b_r, noise, b_sel, logits, idx, gate,
                                 part_p, part_cnt, part_z, T, d, N, K, gate_mode, tpb);
  return hipGetLastError();
}

bool router_small_path(int64_t T, int N) { return T <= kRouterSmallT && N <= 256; }

hipError_t launch_router_small(const float* part, int nsplit, const float* b_r,
                               const RouterNoise& noise, const float* b_sel, float* logits, int32_t* idx,
                               float* gate, int64_t T, int N, int K, int gate_mode, float alpha,
                               int32_t* count, float* f, float* p, float* loss, float* entropy,
                               float* b_sel_out, float bias_rate, hipStream_t stream) {
  const size_t smem = (size_t)18 * N * sizeof(float) + 48 * sizeof(float);
  const int nj = (N + 63) / 64;
#define MOE_SMALL_CASE(NJV)                                                                    \
  case NJV:                                                                                    \
    router_small_kernel<NJV><<<1, 1024, smem, stream>>>(part, nsplit, b_r, noise,             \
        b_sel, logits, idx, gate, T, N, K, gate_mode, alpha, count, f, p, loss, entropy,       \
        b_sel_out, bias_rate);                                                                \
    break;
  switch (nj) {
    MOE_SMALL_CASE(1) MOE_SMALL_CASE(2) MOE_SMALL_CASE(3) MOE_SMALL_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef MOE_SMALL_CASE
  return hipGetLastError();
}

}  // namespace moe
