// Router noise: a caller's [T, N] tensor of standard-normal draws, or draws
// made in the kernels from a counter-based generator.
//
// mzlw.cn "MoE 混合专家模型稀疏激活的架构原理与负载均衡挑战", section 三
// (MoERouter.forward): at training time noise_std times a standard normal
// draw is added to every logit.  The generator is Philox-4x32 with 10 rounds
// (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
// 3", SC 2011) and the Box-Muller transform (Box and Muller, Ann. Math.
// Statist. 29, 1958).  Normal number i of the stream (seed, offset):
//   block b = i / 4, counter (b lo, b hi, offset lo, offset hi), key (seed lo,
//   seed hi); outputs (x0, x1, x2, x3); pair (x0, x1) gives normals 4b, 4b+1
//   and (x2, x3) gives 4b+2, 4b+3 as (r cos a, r sin a) with
//   u1 = (x_even + 1) 2^-32, u2 = x_odd 2^-32, r = sqrt(-2 ln u1), a = 2 pi u2,
//   in double precision, rounded once to float.
// The noise of token t, expert e is normal number t * N + e.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ bool noise_on(const RouterNoise& n) { return n.tensor || n.philox; }

// Philox-4x32-10 block: each round multiplies words 0 and 2 by the two round
// constants, and the new words are (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
// hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key advances by the Weyl constants
// between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Normal number i of the stream (seed, offset).
__device__ __forceinline__ float philox_normal(uint64_t seed, uint64_t offset, uint64_t i) {
  const uint64_t b = i >> 2;
  const uint4 x = philox4x32_10(
      make_uint4((uint32_t)b, (uint32_t)(b >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)),
      (uint32_t)seed, (uint32_t)(seed >> 32));
  const int w = (int)(i & 3);
  const uint32_t xe = w < 2 ? x.x : x.z;
  const uint32_t xo = w < 2 ? x.y : x.w;
  const double u1 = ((double)xe + 1.0) * 0x1p-32;  // (0, 1]: the logarithm is finite
  const double u2 = (double)xo * 0x1p-32;          // [0, 1)
  const double r = sqrt(-2.0 * log(u1));
  const double a = 6.283185307179586476925286766559 * u2;  // 2 pi (nearest double) * u2
  return (float)((w & 1) ? r * sin(a) : r * cos(a));
}

// The draw for flat index i = t * N + e.
__device__ __forceinline__ float noise_draw(const RouterNoise& n, int64_t i) {
  return n.philox ? philox_normal(n.seed, n.offset, (uint64_t)i) : n.tensor[i];
}

}  // namespace moe
