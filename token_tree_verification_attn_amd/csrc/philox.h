// philox.h -- the counter-based generator the stochastic verifier draws its
// uniforms from: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11, "Parallel
// random numbers: as easy as 1, 2, 3").  A 256-bit counter and a 128-bit key
// give four 64-bit words after ten rounds; a round multiplies counter words 0
// and 2 by the paper's two 64-bit multipliers, keeps both halves of each
// 128-bit product and permutes, and the key is bumped between rounds by the
// paper's two Weyl increments.  Only output word 0 is used here, so the last
// round's other words are left to dead-code elimination.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttv {

__device__ __forceinline__ uint64_t philox4x64_10_word0(uint64_t c0, uint64_t c1, uint64_t c2,
                                                        uint64_t c3, uint64_t k0, uint64_t k1) {
  constexpr uint64_t kMulA = 0xD2E7470EE14C6C93ull, kMulB = 0xCA5A826395121157ull;
  constexpr uint64_t kWeylA = 0x9E3779B97F4A7C15ull, kWeylB = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t hA = __umul64hi(kMulA, c0), lA = kMulA * c0;
    const uint64_t hB = __umul64hi(kMulB, c2), lB = kMulB * c2;
    c0 = hB ^ c1 ^ k0;
    c1 = lB;
    c2 = hA ^ c3 ^ k1;
    c3 = lA;
    k0 += kWeylA;
    k1 += kWeylB;
  }
  return c0;
}

// The stochastic verifier's draws: key (seed, 0), counter (j, u, b, step) for
// the ratio test of the j-th child (ascending node index) of node u in
// request b, j = 2^63 for the final draw at u; the uniform is the 24 high bits
// of word 0 (as an integer R, or as the float R * 2^-24, exact).
constexpr uint64_t kBonusOrdinal = 0x8000000000000000ull;

__device__ __forceinline__ uint32_t mss_draw24(uint64_t seed, uint64_t step, uint64_t j, int u,
                                               int b) {
  return (uint32_t)(philox4x64_10_word0(j, (uint64_t)u, (uint64_t)b, step, seed, 0ull) >> 40);
}

}  // namespace ttv
