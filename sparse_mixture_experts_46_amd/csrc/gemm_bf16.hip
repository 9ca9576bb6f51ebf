// Expert FFNs as grouped GEMMs on the gfx950 matrix cores (bf16 in, fp32
// accumulate).
//
// Pages (by title and section):
//   mzlw.cn "MoE 混合专家模型稀疏激活的架构原理与负载均衡挑战", section 三:
//     Expert.forward = down( silu(gate(x)) * up(x) ); the MoELayer runs one
//     expert at a time over its gathered rows and notes that production code
//     should use grouped matrix multiplication instead.
//   learnagent.wiki "混合专家模型（Mixture of Experts, MoE）", 运行示例: the GELU
//     expert Linear(h, 2h) -> GELU -> Linear(2h, h) with biases.
//   mstx.cn "MoE 如何替代 FFN？…", section 5: a shared expert that every
//     token passes through (DeepSeek-MoE); it runs here as one extra group.
//
// A group g is one expert: rows [offset[g], offset[g+1]) of the
// expert-contiguous row space, weights W_g of shape [Nout, Kdim] with K
// contiguous, so every GEMM is C = A B^T with both operands K-contiguous.
// Group N (when present) is the shared expert over all T tokens.
//
// Two kernels:
//   * tile kernel (prefill): a BM x BN workgroup tile, K staged through LDS
//     in slices of 64 with an XOR swizzle of the 16-byte chunks, double
//     buffered, v_mfma_f32_32x32x16_bf16.  For SwiGLU the B tile holds BN/2
//     gate rows and the same BN/2 up rows, so silu(gate) * up is formed in
//     registers in the epilogue.  Persistent: the grid is one workgroup per
//     CU and tiles are handed out in a fixed round-robin, with consecutive
//     tiles (same expert, neighbouring columns) kept on one XCD so they
//     share its L2.
//   * skinny kernel (decode, few rows per expert): one wave per 16 x 16
//     output block, v_mfma_f32_16x16x32_bf16, operands loaded straight from
//     global memory 64 contiguous bytes per lane; the work is streaming the
//     weights once.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

enum { EPI_SILU_MUL = 0, EPI_GELU = 1, EPI_BIAS = 2 };

struct GemmArgs {
  const uint16_t* a;        // routed A rows (x_perm / h), or x when a_rows
  const int32_t* a_rows;    // nullable gather map: row r -> a[a_rows[r] / a_div]
  int a_div;
  int64_t lda;
  const int32_t* offset;    // [n_routed + 1] row offsets of the routed groups
  int n_routed;
  int64_t shared_rows;      // rows of the shared group (0 = none)
  const uint16_t* a_shared; // A of the shared group
  const uint16_t* b0;       // routed weights (gate / single), [n_routed, Nout, Kdim]
  const uint16_t* b1;       // routed up weights (SwiGLU)
  int64_t b_stride;         // Nout * Kdim
  const uint16_t* bs0;      // shared weights
  const uint16_t* bs1;
  int Nout, Nout_shared, Kdim;
  const uint16_t* bias;     // routed bias [n_routed, Nout] (nullable)
  uint16_t* c;              // routed output [rows, Nout]
  uint16_t* c_shared;       // shared output [shared_rows, Nout_shared]
  const int32_t* tile_base; // [G + 1]
  int G;
};

// ------------------------------------------------------------ tile setup --
// tile_base[g] = sum_{g' < g} ceil(M_g'/BM) * ceil(Nout_g'/BNo), for two
// tilings at once (first and second GEMM).  One block of 1024 threads.
__global__ __launch_bounds__(1024) void tile_setup_kernel(
    const int32_t* __restrict__ offset, int n_routed, int64_t shared_rows,
    int bm1, int bno1, int nout1, int nout1_s, int bm2, int bno2, int nout2,
    int nout2_s, int32_t* __restrict__ base1, int32_t* __restrict__ base2) {
  __shared__ int32_t s1[2048], s2[2048];
  const int G = n_routed + (shared_rows > 0 ? 1 : 0);
  for (int g = threadIdx.x; g < 2048; g += 1024) {
    int32_t t1 = 0, t2 = 0;
    if (g < G) {
      int64_t M = g < n_routed ? (int64_t)(offset[g + 1] - offset[g]) : shared_rows;
      int n1 = g < n_routed ? nout1 : nout1_s, n2 = g < n_routed ? nout2 : nout2_s;
      t1 = (int32_t)(((M + bm1 - 1) / bm1) * ((n1 + bno1 - 1) / bno1));
      t2 = (int32_t)(((M + bm2 - 1) / bm2) * ((n2 + bno2 - 1) / bno2));
    }
    s1[g] = t1; s2[g] = t2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // G <= 1025: a short serial scan is enough
    int32_t r1 = 0, r2 = 0;
    for (int g = 0; g < G; ++g) {
      base1[g] = r1; base2[g] = r2;
      r1 += s1[g]; r2 += s2[g];
    }
    base1[G] = r1; base2[G] = r2;
  }
}

template <int EPI>
__device__ __forceinline__ float epi1(float acc, float bias) {
  if (EPI == EPI_GELU) return gelu_tanh_f(acc + bias);
  return acc + bias;
}

// Resolve tile -> (group, first row, rows, output columns, A/B/C pointers).
struct TileInfo {
  int g, M, Nout, mt, nt;
  bool shared;
  int64_t row0;
};

__device__ __forceinline__ TileInfo resolve_tile(const GemmArgs& p, int tile, int BM, int BNo) {
  TileInfo ti;
  ti.g = find_group(p.tile_base, p.G, tile);
  const int local = tile - p.tile_base[ti.g];
  ti.shared = (ti.g == p.n_routed);
  ti.row0 = ti.shared ? 0 : p.offset[ti.g];
  ti.M = ti.shared ? (int)p.shared_rows : (int)(p.offset[ti.g + 1] - ti.row0);
  ti.Nout = ti.shared ? p.Nout_shared : p.Nout;
  const int mtiles = (ti.M + BM - 1) / BM;
  ti.mt = local % mtiles;
  ti.nt = local / mtiles;
  (void)BNo;
  return ti;
}

// ================================================================ tile ====
// Direct global -> LDS loads (global_load_lds_dwordx4): one wave instruction
// fills 8 rows x 128 bytes of the stage; lane l writes LDS slot l of that
// 1 KB block, i.e. row l/8, physical chunk l%8, and therefore fetches the
// logical chunk (l%8) ^ (row & 7) of its row (the XOR swizzle that keeps
// the fragment reads free of bank conflicts).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__device__ __forceinline__ void lds_dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)l, 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int BM, int BN, int WM, int WN, bool DUAL, int EPI>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_tile_kernel(GemmArgs p) {
  constexpr int NW = WM * WN;
  constexpr int BK = 64;               // bf16 per staged row slice (128 B)
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int BNo = DUAL ? BN / 2 : BN;   // output columns per tile
  constexpr int LA = BM / (NW * 8), LB = BN / (NW * 8);  // DMA instructions per wave
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * 128;    // bytes per stage
  static_assert(BM % (NW * 8) == 0 && BN % (NW * 8) == 0, "tile/wave mismatch");
  static_assert(!DUAL || (FN % 2 == 0), "dual tile needs an even fragment count");
  extern __shared__ uint4 smem[];      // [2][ROWS][8] uint4
  char* sbase = (char*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int total = p.tile_base[p.G];
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int first = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int lrow = lane >> 3, pch = lane & 7;

  // rows of LDS this lane reads for its fragments
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * TM + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int r;
    if (DUAL) {
      constexpr int FH = FN / 2;
      r = (j < FH) ? wn * (TN / 2) + j * 32 : BN / 2 + wn * (TN / 2) + (j - FH) * 32;
    } else {
      r = wn * TN + j * 32;
    }
    brow[j] = BM + r + (lane & 31);
  }
  const int khalf = lane >> 5;

  for (int tile = first; tile < total; tile += nb) {
    const TileInfo ti = resolve_tile(p, tile, BM, BNo);
    const int64_t Kd = p.Kdim;
    // ---- this lane's DMA sources: uniform base + per-lane byte offset
    const char* abase = (const char*)(ti.shared ? p.a_shared : p.a);
    uint32_t aoff[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = i * NW * 8 + wave * 8 + lrow;
      int lr = ti.mt * BM + r;
      if (lr >= ti.M) lr = ti.M - 1;
      int64_t ar;
      if (ti.shared) ar = lr;
      else {
        const int64_t gr = ti.row0 + lr;
        ar = p.a_rows ? (int64_t)(p.a_rows[gr] / p.a_div) : gr;
      }
      aoff[i] = (uint32_t)((ar * p.lda + ((pch ^ (r & 7)) * 8)) * 2);
    }
    const char* bbase0 = (const char*)(ti.shared ? p.bs0 : p.b0 + (int64_t)ti.g * p.b_stride);
    const char* bbase1 = DUAL ? (const char*)(ti.shared ? p.bs1 : p.b1 + (int64_t)ti.g * p.b_stride)
                              : bbase0;
    uint32_t boff[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = i * NW * 8 + wave * 8 + lrow;
      int n = ti.nt * BNo + ((DUAL && r >= BN / 2) ? r - BN / 2 : r);
      if (n >= ti.Nout) n = ti.Nout - 1;
      boff[i] = (uint32_t)(((int64_t)n * Kd + ((pch ^ (r & 7)) * 8)) * 2);
    }

#define MOE_TILE_ISSUE(K0, BUF)                                                         \
    do {                                                                                \
      char* st_ = sbase + (BUF) * STAGE;                                                \
      const uint32_t kb_ = (uint32_t)(K0) * 2;                                          \
      _Pragma("unroll") for (int i = 0; i < LA; ++i)                                    \
        lds_dma16(abase + aoff[i] + kb_, st_ + (i * NW * 8 + wave * 8) * 128);          \
      _Pragma("unroll") for (int i = 0; i < LB; ++i) {                                  \
        const int r_ = i * NW * 8 + wave * 8;                                           \
        const char* bb_ = (DUAL && r_ >= BN / 2) ? bbase1 : bbase0;                     \
        lds_dma16(bb_ + boff[i] + kb_, st_ + (BM + r_) * 128);                          \
      }                                                                                 \
    } while (0)

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = (int)(Kd / BK);
    MOE_TILE_ISSUE(0, 0);
    wait_vmem();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) MOE_TILE_ISSUE((kt + 1) * BK, buf ^ 1);
      const uint4* s = smem + buf * ROWS * 8;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int ch = ks * 2 + khalf;
        bf16x8_t fa[FM], fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[i] = __builtin_bit_cast(bf16x8_t, s[arow[i] * 8 + (ch ^ (arow[i] & 7))]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[j] = __builtin_bit_cast(bf16x8_t, s[brow[j] * 8 + (ch ^ (brow[j] & 7))]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      wait_vmem();
      __syncthreads();
    }
#undef MOE_TILE_ISSUE

    // ---- epilogue.  D layout: col = lane % 32, row = 8*(v/4) + 4*(lane/32) + v%4
    uint16_t* cbase = ti.shared ? p.c_shared : p.c;
    const int64_t ldc = ti.Nout;
    constexpr int FO = DUAL ? FN / 2 : FN;
#pragma unroll
    for (int j = 0; j < FO; ++j) {
      const int col = ti.nt * BNo + (DUAL ? wn * (TN / 2) : wn * TN) + j * 32 + (lane & 31);
      if (col >= ti.Nout) continue;
      float bias = 0.f;
      if (EPI != EPI_SILU_MUL && p.bias && !ti.shared)
        bias = bf16_to_f32(p.bias[(int64_t)ti.g * p.Nout + col]);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = ti.mt * BM + wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (lr < ti.M) {
            float o;
            if (DUAL) o = silu_f(acc[i][j][v]) * acc[i][j + FN / 2][v];
            else o = epi1<EPI>(acc[i][j][v], bias);
            cbase[(ti.row0 + lr) * ldc + col] = f32_to_bf16(o);
          }
        }
      }
    }
  }
}

// ============================================================= skinny ====
// One wave computes a 16-row x 16-column output block.  Over a 128-wide K
// chunk, lane l (row l%16, quarter q = l/16) holds K elements
// [q*32, q*32+32) of its row in four 8-element slots; step j of the four
// MFMAs consumes slot j of A and of B, so both operands see the same K
// permutation and the product is unchanged.
template <bool DUAL, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave_g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const int total = p.tile_base[p.G];
  const int row = lane & 15, q = lane >> 4;
  for (int tile = wave_g; tile < total; tile += nwaves) {
    const TileInfo ti = resolve_tile(p, tile, 16, 16);
    const int64_t Kd = p.Kdim;
    int lr = ti.mt * 16 + row;
    if (lr >= ti.M) lr = ti.M - 1;
    const uint16_t* pa;
    if (ti.shared) {
      pa = p.a_shared + (int64_t)lr * p.lda;
    } else {
      const int64_t gr = ti.row0 + lr;
      const int64_t ar = p.a_rows ? (int64_t)(p.a_rows[gr] / p.a_div) : gr;
      pa = p.a + ar * p.lda;
    }
    int n = ti.nt * 16 + row;
    if (n >= ti.Nout) n = ti.Nout - 1;
    const uint16_t* pb0 = (ti.shared ? p.bs0 : p.b0 + (int64_t)ti.g * p.b_stride) + (int64_t)n * Kd;
    const uint16_t* pb1 = DUAL ? (ti.shared ? p.bs1 : p.b1 + (int64_t)ti.g * p.b_stride) + (int64_t)n * Kd
                               : nullptr;
    pa += q * 32; pb0 += q * 32;
    if (DUAL) pb1 += q * 32;

    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const int nk = (int)(Kd / 128);
    int kc = 0;
    for (; kc + 1 < nk; kc += 2) {
      uint4 a[8], b[8], c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int off = (j >> 2) * 128 + (j & 3) * 8;
        a[j] = *(const uint4*)(pa + kc * 128 + off);
        b[j] = *(const uint4*)(pb0 + kc * 128 + off);
        if (DUAL) c[j] = *(const uint4*)(pb1 + kc * 128 + off);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8_t fa = __builtin_bit_cast(bf16x8_t, a[j]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8_t, b[j]), acc0, 0, 0, 0);
        if (DUAL)
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8_t, c[j]), acc1, 0, 0, 0);
      }
    }
    for (; kc < nk; ++kc) {
      uint4 a[4], b[4], c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = *(const uint4*)(pa + kc * 128 + j * 8);
        b[j] = *(const uint4*)(pb0 + kc * 128 + j * 8);
        if (DUAL) c[j] = *(const uint4*)(pb1 + kc * 128 + j * 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t fa = __builtin_bit_cast(bf16x8_t, a[j]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8_t, b[j]), acc0, 0, 0, 0);
        if (DUAL)
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8_t, c[j]), acc1, 0, 0, 0);
      }
    }
    if (Kd % 128) {  // a final 64-wide chunk: lane quarter q holds [q*16, q*16+16)
      const int64_t k0 = (int64_t)nk * 128 - q * 32 + q * 16;
      const uint16_t* qa = pa + k0;
      const uint16_t* qb = pb0 + k0;
      const uint16_t* qc = DUAL ? pb1 + k0 : nullptr;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8_t fa = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qa + j * 8));
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            fa, __builtin_bit_cast(bf16x8_t, *(const uint4*)(qb + j * 8)), acc0, 0, 0, 0);
        if (DUAL)
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              fa, __builtin_bit_cast(bf16x8_t, *(const uint4*)(qc + j * 8)), acc1, 0, 0, 0);
      }
    }
    // D layout (16x16): col = lane % 16, row = 4*(lane/16) + v
    const int col = ti.nt * 16 + (lane & 15);
    if (col < ti.Nout) {
      uint16_t* cbase = ti.shared ? p.c_shared : p.c;
      float bias = 0.f;
      if (EPI != EPI_SILU_MUL && p.bias && !ti.shared)
        bias = bf16_to_f32(p.bias[(int64_t)ti.g * p.Nout + col]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = ti.mt * 16 + 4 * q + v;
        if (r < ti.M) {
          float o = DUAL ? silu_f(acc0[v]) * acc1[v] : epi1<EPI>(acc0[v], bias);
          cbase[(ti.row0 + r) * (int64_t)ti.Nout + col] = f32_to_bf16(o);
        }
      }
    }
  }
}

// ============================================================== host =====
namespace {

int g_num_cus = 0;

int num_cus() {
  if (g_num_cus <= 0) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
      g_num_cus = prop.multiProcessorCount;
    if (g_num_cus <= 0) g_num_cus = 256;
  }
  return g_num_cus;
}

struct TileCfg {
  int bm, bn, wm, wn;
};

template <int BM, int BN, int WM, int WN, bool DUAL, int EPI>
hipError_t run_tile(const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  auto kern = gemm_tile_kernel<BM, BN, WM, WN, DUAL, EPI>;
  const size_t smem = (size_t)2 * (BM + BN) * 128;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int64_t grid = num_cus();
  if (max_tiles < grid) grid = ((max_tiles + 7) / 8) * 8;
  if (grid < 8) grid = 8;
  kern<<<(unsigned)grid, WM * WN * 64, smem, s>>>(a);
  return hipGetLastError();
}

template <bool DUAL, int EPI>
hipError_t run_skinny(const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  int64_t grid = (max_tiles + 3) / 4;
  const int64_t cap = (int64_t)num_cus() * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  gemm_skinny_kernel<DUAL, EPI><<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// Tile shapes by the expected rows per expert.
enum Kind { K_SKINNY = 0, K_SMALL = 1, K_MID = 2, K_BIG = 3 };

Kind pick_kind(double rows_per_expert) {
  if (rows_per_expert <= 24.0) return K_SKINNY;
  if (rows_per_expert <= 96.0) return K_SMALL;
  if (rows_per_expert <= 640.0) return K_MID;
  return K_BIG;
}

// (BM, BN) per kind; BNo = BN/2 for the dual (SwiGLU gate/up) GEMM.
void kind_dims(Kind k, bool dual, int* bm, int* bno) {
  switch (k) {
    case K_SKINNY: *bm = 16; *bno = 16; return;
    case K_SMALL:  *bm = 64; *bno = dual ? 128 : 256; return;
    case K_MID:    *bm = 128; *bno = dual ? 128 : 256; return;
    default:       *bm = 256; *bno = dual ? 128 : 256; return;
  }
}

template <bool DUAL, int EPI>
hipError_t run_kind(Kind k, const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  switch (k) {
    case K_SKINNY: return run_skinny<DUAL, EPI>(a, max_tiles, s);
    case K_SMALL:  return run_tile<64, 256, 1, 4, DUAL, EPI>(a, max_tiles, s);
    case K_MID:    return run_tile<128, 256, 2, 2, DUAL, EPI>(a, max_tiles, s);
    default:       return run_tile<256, 256, 2, 2, DUAL, EPI>(a, max_tiles, s);
  }
}

int64_t max_tiles_for(int64_t rows, int G, int bm, int64_t cols, int bno) {
  // sum over groups of ceil(M_g/bm) <= rows/bm + G
  return (rows / bm + G) * ((cols + bno - 1) / bno);
}

}  // namespace

hipError_t launch_ffn_f32(const FfnProblem& p, hipStream_t stream);

size_t ffn_workspace_bytes(int64_t T, int d, int N, int K, int F, int F_shared, bool bf16) {
  (void)d; (void)N;
  const size_t el = bf16 ? 2 : 4;
  const int Fm = F > F_shared ? F : F_shared;
  size_t h = ((size_t)T * K + (F_shared > 0 ? (size_t)T : 0)) * (size_t)Fm * el;
  return (h + 255) / 256 * 256;
}

hipError_t launch_expert_ffn(const FfnProblem& p, hipStream_t stream, hipEvent_t ev_pre,
                             hipEvent_t ev_mid) {
  if (!p.bf16) {
    hipError_t e = ev_pre ? hipEventRecord(ev_pre, stream) : hipSuccess;
    if (e == hipSuccess) e = launch_ffn_f32(p, stream);
    if (e == hipSuccess && ev_mid) e = hipEventRecord(ev_mid, stream);
    return e;
  }
  const bool swiglu = (p.act == 0);
  const int64_t rows = p.T * p.K;
  const int64_t srows = p.F_shared > 0 ? p.T : 0;
  const int G = p.N + (srows > 0 ? 1 : 0);
  const double rpe = (double)rows / (double)p.N;
  Kind k1 = pick_kind(rpe), k2 = k1;
  int bm1, bno1, bm2, bno2;
  kind_dims(k1, swiglu, &bm1, &bno1);
  kind_dims(k2, false, &bm2, &bno2);
  int32_t* base1 = p.tile_base;
  int32_t* base2 = p.tile_base + (p.N + 2);
  tile_setup_kernel<<<1, 1024, 0, stream>>>(p.offset, p.N, srows, bm1, bno1, p.F, p.F_shared,
                                            bm2, bno2, p.d, p.d, base1, base2);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  const int Fm = p.F > p.F_shared ? p.F : p.F_shared;
  uint16_t* h = (uint16_t*)p.h;
  uint16_t* h_shared = h + (size_t)rows * Fm;

  // ---- GEMM 1: h = act(A W1^T [+ b1]) [* (A W3^T)]
  GemmArgs g1 = {};
  g1.a = (const uint16_t*)p.a;
  g1.a_rows = p.a_rows;
  g1.a_div = p.K;
  g1.lda = p.d;
  g1.offset = p.offset;
  g1.n_routed = p.N;
  g1.shared_rows = srows;
  g1.a_shared = (const uint16_t*)p.x_shared;
  g1.b0 = (const uint16_t*)p.w1;
  g1.b1 = (const uint16_t*)p.w3;
  g1.b_stride = (int64_t)p.F * p.d;
  g1.bs0 = (const uint16_t*)p.ws1;
  g1.bs1 = (const uint16_t*)p.ws3;
  g1.Nout = p.F;
  g1.Nout_shared = p.F_shared;
  g1.Kdim = p.d;
  g1.bias = (const uint16_t*)p.b1;
  g1.c = h;
  g1.c_shared = h_shared;
  g1.tile_base = base1;
  g1.G = G;
  const int64_t mt1 = max_tiles_for(rows + srows, G, bm1, Fm, bno1);
  if (ev_pre) {
    err = hipEventRecord(ev_pre, stream);
    if (err != hipSuccess) return err;
  }
  err = swiglu ? run_kind<true, EPI_SILU_MUL>(k1, g1, mt1, stream)
               : run_kind<false, EPI_GELU>(k1, g1, mt1, stream);
  if (err != hipSuccess) return err;
  if (ev_mid) {
    err = hipEventRecord(ev_mid, stream);
    if (err != hipSuccess) return err;
  }

  // ---- GEMM 2: y = h W2^T [+ b2]
  GemmArgs g2 = {};
  g2.a = h;
  g2.a_rows = nullptr;
  g2.a_div = 1;
  g2.lda = Fm;
  g2.offset = p.offset;
  g2.n_routed = p.N;
  g2.shared_rows = srows;
  g2.a_shared = h_shared;
  g2.b0 = (const uint16_t*)p.w2;
  g2.b1 = nullptr;
  g2.b_stride = (int64_t)p.d * p.F;
  g2.bs0 = (const uint16_t*)p.ws2;
  g2.bs1 = nullptr;
  g2.Nout = p.d;
  g2.Nout_shared = p.d;
  g2.Kdim = p.F;
  g2.bias = (const uint16_t*)p.b2;
  g2.c = (uint16_t*)p.y_perm;
  g2.c_shared = (uint16_t*)p.y_shared;
  g2.tile_base = base2;
  g2.G = G;
  // (F_shared is either 0 or F: checked on the host)
  const int64_t mt2 = max_tiles_for(rows + srows, G, bm2, p.d, bno2);
  err = run_kind<false, EPI_BIAS>(k2, g2, mt2, stream);
  return err;
}

}  // namespace moe
