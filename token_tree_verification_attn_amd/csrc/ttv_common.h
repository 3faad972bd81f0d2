// ttv_common.h -- device-side helpers shared by the kernels of libttv.
//
// Sources cited (page title, then section):
//   [SI]  "SpecInfer: Accelerating Generative Large Language Model Serving with
//         Tree-based Speculative Inference and Verification" (paperlayer.ai
//         summary of arXiv 2305.09781v4).
//   [SSD] "Accelerating LLM Inference with Staged Speculative Decoding"
//         (paperlayer.ai summary of arXiv 2308.04623v1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttv.h"

namespace ttv {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kMaxNodes = TTV_MAX_NODES;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ------------------------------------------------------ wave primitives ----
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl(static_cast<uint32_t>(v), src);
  uint32_t hi = __shfl(static_cast<uint32_t>(v >> 32), src);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// -------------------------------------------- register-only wave sums ----
// Sums over the 64 lanes that stay in the VALU (a __shfl_xor step is an LDS
// round trip, ds_bpermute): two quad permutations and two row rotations
// (DPP) sum each 16-lane row, then v_permlane16_swap and v_permlane32_swap
// add the other rows.  Every lane gets the total; all 64 lanes must be
// active.  For doubles each DPP move carries both halves, so the sum is
// exact where the terms are (integer-valued doubles below 2^53).
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;  // row_ror:4
constexpr int kDppRowRor8 = 0x128;  // row_ror:8

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ int wave_allsum_i32(int v) {
  v += (int)dpp_u32<kDppQuadXor1>((uint32_t)v);
  v += (int)dpp_u32<kDppQuadXor2>((uint32_t)v);
  v += (int)dpp_u32<kDppRowRor4>((uint32_t)v);
  v += (int)dpp_u32<kDppRowRor8>((uint32_t)v);
  auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = (int)(r[0] + r[1]);
  r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int)(r[0] + r[1]);
}
// the two 64-bit words a permlane swap hands a lane (its own and its
// partner's; the low and the high halves come in the same order)
template <bool S32>
__device__ __forceinline__ void swap_pair_u64(uint64_t u, uint64_t& a, uint64_t& b) {
  const uint32_t l = (uint32_t)u, h = (uint32_t)(u >> 32);
  const auto lo = S32 ? __builtin_amdgcn_permlane32_swap(l, l, false, false)
                      : __builtin_amdgcn_permlane16_swap(l, l, false, false);
  const auto hi = S32 ? __builtin_amdgcn_permlane32_swap(h, h, false, false)
                      : __builtin_amdgcn_permlane16_swap(h, h, false, false);
  a = ((uint64_t)hi[0] << 32) | lo[0];
  b = ((uint64_t)hi[1] << 32) | lo[1];
}
__device__ __forceinline__ double wave_allsum_f64(double v) {
  v += dpp_f64<kDppQuadXor1>(v);
  v += dpp_f64<kDppQuadXor2>(v);
  v += dpp_f64<kDppRowRor4>(v);
  v += dpp_f64<kDppRowRor8>(v);
  uint64_t a, b;
  swap_pair_u64<false>((uint64_t)__double_as_longlong(v), a, b);
  v = __longlong_as_double((long long)a) + __longlong_as_double((long long)b);
  swap_pair_u64<true>((uint64_t)__double_as_longlong(v), a, b);
  return __longlong_as_double((long long)a) + __longlong_as_double((long long)b);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(x >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)x);
}
__device__ __forceinline__ uint64_t wave_allsum_u64(uint64_t v) {
  v += dpp_u64<kDppQuadXor1>(v);
  v += dpp_u64<kDppQuadXor2>(v);
  v += dpp_u64<kDppRowRor4>(v);
  v += dpp_u64<kDppRowRor8>(v);
  uint64_t a, b;
  swap_pair_u64<false>(v, a, b);
  swap_pair_u64<true>(a + b, a, b);
  return a + b;
}
__device__ __forceinline__ float wave_allsum_f32(float v) {
  v += __uint_as_float(dpp_u32<kDppQuadXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppQuadXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppRowRor4>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppRowRor8>(__float_as_uint(v)));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int wave_allmax_i32(int v) {
  v = max(v, (int)dpp_u32<kDppQuadXor1>((uint32_t)v));
  v = max(v, (int)dpp_u32<kDppQuadXor2>((uint32_t)v));
  v = max(v, (int)dpp_u32<kDppRowRor4>((uint32_t)v));
  v = max(v, (int)dpp_u32<kDppRowRor8>((uint32_t)v));
  auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = max((int)r[0], (int)r[1]);
  r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float wave_allmax_f32(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppQuadXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppQuadXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppRowRor4>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppRowRor8>(__float_as_uint(v))));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The (value, index) pair ranking first over the wave -- the larger value,
// the lower index on equal values -- in every lane, register-only as the
// sums above (the ranking is a total order, so any pairing order gives the
// same winner).
__device__ __forceinline__ void argmax_take(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp_step(float& v, int& i) {
  argmax_take(v, i, __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v))), (int)dpp_u32<CTRL>((uint32_t)i));
}
__device__ __forceinline__ void wave_allargmax(float& v, int& i) {
  argmax_dpp_step<kDppQuadXor1>(v, i);
  argmax_dpp_step<kDppQuadXor2>(v, i);
  argmax_dpp_step<kDppRowRor4>(v, i);
  argmax_dpp_step<kDppRowRor8>(v, i);
  auto rv = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  auto ri = __builtin_amdgcn_permlane16_swap((uint32_t)i, (uint32_t)i, false, false);
  v = __uint_as_float(rv[0]);
  i = (int)ri[0];
  argmax_take(v, i, __uint_as_float(rv[1]), (int)ri[1]);
  rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  ri = __builtin_amdgcn_permlane32_swap((uint32_t)i, (uint32_t)i, false, false);
  v = __uint_as_float(rv[0]);
  i = (int)ri[0];
  argmax_take(v, i, __uint_as_float(rv[1]), (int)ri[1]);
}

// --------------------------------------------------------- tree topology --
// Ancestor bitsets of one request's token tree, built by ONE wavefront.
// [SI] §4 "Tree Attention": node i stands for the sequence root -> i, so the
// mask row of node i is the set of nodes on that path ("topology-aware causal
// mask", §4 "Tree-Based Parallel Decoding").
//
// Lane l holds nodes l and l+64.  Pointer doubling: a node keeps the set A of
// path nodes it has gathered and a jump pointer J to the nearest path node not
// yet in A (initially A = {i}, J = parent(i)).  Each round every node with
// J >= 0 reads (A_J, J_J) of node J through a wave shuffle (ds_bpermute) and
// sets A |= A_J, J = J_J, so the covered path length doubles; a ballot ends
// the loop once every J is -1 (ceil(log2(depth+1)) rounds, at most 7).
// Validity (parents[0] == -1, 0 <= parents[i] < i) is checked with a ballot
// first; an invalid tree writes nothing and returns false.
//
// wave_tree_bits works in registers only: from the parents p0 = parents[l],
// p1 = parents[l + 64] (-1 past N) it returns in lane l the bitsets of nodes
// l (a0lo; its high word is 0) and l + 64 (a1lo, a1hi), or false for an
// invalid tree.  wave_build_tree loads the parents itself and stores the
// result in LDS: on return (valid tree) s_anc[2*i + w] holds word w of node
// i's bitset and s_depth[i] its depth, for i < N.  All 64 lanes must call
// either; the caller synchronises before other waves read the LDS arrays.
__device__ inline bool wave_tree_bits(int p0, int p1, int N, uint64_t& a0lo, uint64_t& a1lo,
                                      uint64_t& a1hi) {
  const int lane = lane_id();
  const int i0 = lane, i1 = lane + 64;
  const bool bad0 = i0 < N && (i0 == 0 ? p0 != -1 : (p0 < 0 || p0 >= i0));
  const bool bad1 = i1 < N && (p1 < 0 || p1 >= i1);
  a0lo = 0ull;
  a1lo = 0ull;
  a1hi = 0ull;
  if (__ballot(bad0 || bad1) != 0ull) return false;

  // A for node i0 (words lo/hi) and node i1; node i0 < 64 lives in word 0.
  a0lo = i0 < N ? (1ull << i0) : 0ull;
  a1hi = i1 < N ? (1ull << (i1 - 64)) : 0ull;
  int j0 = p0, j1 = p1;
  const bool two = N > 64;
  while (__ballot(j0 >= 0 || j1 >= 0) != 0ull) {
    // gather (A_J, J_J) for J = j0 and J = j1 from lane J & 63, slot J >> 6.
    // j0 < i0 < 64 always lies in slot 0, whose high word is 0.
    const int s0 = j0 & 63, s1 = j1 & 63;
    const uint64_t r0a = shfl_u64(a0lo, s0);
    const int r0j = __shfl(j0, s0);
    if (two) {
      // node j1 lies in slot 0 (j1 < 64) or slot 1 of lane s1
      const uint64_t r1a = shfl_u64(a0lo, s1);
      const int r1j = __shfl(j0, s1);
      const uint64_t q1a = shfl_u64(a1lo, s1);
      const uint64_t q1b = shfl_u64(a1hi, s1);
      const int q1j = __shfl(j1, s1);
      if (j1 >= 0) {
        if (j1 < 64) {
          a1lo |= r1a;
          j1 = r1j;
        } else {
          a1lo |= q1a;
          a1hi |= q1b;
          j1 = q1j;
        }
      }
    }
    if (j0 >= 0) {
      a0lo |= r0a;
      j0 = r0j;
    }
  }
  return true;
}

__device__ inline bool wave_build_tree(const int32_t* __restrict__ par, int N,
                                       uint64_t* s_anc, int32_t* s_depth) {
  const int lane = lane_id();
  const int i0 = lane, i1 = lane + 64;
  const int p0 = i0 < N ? par[i0] : -1;
  const int p1 = i1 < N ? par[i1] : -1;
  uint64_t a0lo, a1lo, a1hi;
  if (!wave_tree_bits(p0, p1, N, a0lo, a1lo, a1hi)) return false;
  const uint64_t a0hi = 0ull;
  if (i0 < N) {
    s_anc[2 * i0] = a0lo;
    s_anc[2 * i0 + 1] = a0hi;
    s_depth[i0] = __popcll(a0lo) + __popcll(a0hi) - 1;
  }
  if (i1 < N) {
    s_anc[2 * i1] = a1lo;
    s_anc[2 * i1 + 1] = a1hi;
    s_depth[i1] = __popcll(a1lo) + __popcll(a1hi) - 1;
  }
  return true;
}

// Nodes of request b in a batch of trees of different sizes: n_nodes[b]
// when given (rows hold N entries; entries at or past n_nodes[b] are padding
// and never used), else N.  A count outside [1, N] rejects the request; the
// kernels then work on the count clamped to [1, N] so that every access stays
// inside the rows.
__device__ __forceinline__ int nodes_raw(const int32_t* n_nodes, int b, int N) {
  return n_nodes ? n_nodes[b] : N;
}
__device__ __forceinline__ bool nodes_ok(int n, int N) { return n >= 1 && n <= N; }
__device__ __forceinline__ int nodes_used(int n, int N) { return min(max(n, 1), N); }

// Tree validity only (one wave): parents[0] == -1 and 0 <= parents[i] < i.
__device__ inline bool wave_tree_valid(const int32_t* __restrict__ par, int N) {
  bool bad = false;
  for (int i = lane_id(); i < N; i += kWave) {
    const int p = par[i];
    bad |= (i == 0) ? (p != -1) : (p < 0 || p >= i);
  }
  return __ballot(bad) == 0ull;
}

}  // namespace ttv
