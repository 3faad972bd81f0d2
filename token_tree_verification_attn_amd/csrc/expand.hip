// expand.hip -- one level of expansion-based token-tree construction ([SI]
// §3 "Expansion-based token tree construction": the top-k tokens of a
// speculative model at a node become that node's children).
//
// One 256-thread workgroup per (request b, frontier entry f).  Each thread
// keeps the KM best (probability, token) pairs of its share of the row in
// registers while streaming the row once (16-byte loads, 8 in flight per
// thread); it visits its tokens in increasing order, so an equal probability
// never displaces a lower token id.  The 256 lists go through LDS to wave 0,
// whose lanes each merge four of them; the k best of the 64 lane lists come
// out of k rounds of a wave arg-max (higher probability first, then the
// lower token id).  Every workgroup of a request reads the request's whole
// frontier (at most 128 entries) to find the request's validity and its own
// rank among the entries >= 0, so no workgroup waits for another.
#include <limits.h>

#include "launch.h"
#include "ttv_common.h"

namespace ttv {

namespace {

constexpr int kExpandThreads = 256;

// (v, i) ranks before (bv, bi): higher probability, then the lower token id
__device__ __forceinline__ bool ranks_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Insert (v, i) into the sorted list (best first) if it ranks before its last
// entry; fixed trip counts keep the list in registers.
template <int KM>
__device__ __forceinline__ void list_insert(float (&lv)[KM], int (&li)[KM], float v, int i) {
  if (!ranks_before(v, i, lv[KM - 1], li[KM - 1])) return;
  bool placed = false;
#pragma unroll
  for (int j = KM - 1; j >= 0; --j) {
    if (!placed) {
      if (j > 0 && ranks_before(v, i, lv[j - 1], li[j - 1])) {
        lv[j] = lv[j - 1];
        li[j] = li[j - 1];
      } else {
        lv[j] = v;
        li[j] = i;
        placed = true;
      }
    }
  }
}

}  // namespace

template <int KM, bool VEC>
__global__ __launch_bounds__(kExpandThreads) void tree_expand_kernel(
    int F, int V, int k, const float* __restrict__ probs, const int32_t* __restrict__ frontier,
    const int32_t* __restrict__ n_in, int Ncap, int32_t* __restrict__ parents,
    int32_t* __restrict__ tokens, int32_t* __restrict__ src_row, int32_t* __restrict__ n_out,
    int32_t* __restrict__ dev_status) {
  __shared__ float s_v[KM * kExpandThreads];
  __shared__ int s_i[KM * kExpandThreads];
  const int f = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // ---- the request's frontier: validity, entry count, this entry's rank
  const int nin = n_in[b];
  const int32_t* fb = frontier + (size_t)b * F;
  int count = 0, rank = 0;
  bool bad = false;
  for (int j0 = 0; j0 < F; j0 += 64) {
    const int j = j0 + lane;
    const int fr = j < F ? fb[j] : -1;
    bad |= fr < -1 || fr >= nin;
    const uint64_t m = __ballot(fr >= 0);
    count += __popcll(m);
    if (f >= j0) rank += __popcll(f - j0 >= 64 ? m : (m & ((1ull << (f - j0)) - 1ull)));
  }
  bad = __ballot(bad) != 0ull;
  const int st = bad ? TTV_E_TREE
                     : (nin < 1 || (long)nin + (long)count * k > Ncap ? TTV_E_SHAPE : TTV_OK);
  if (f == 0 && threadIdx.x == 0) {
    n_out[b] = st == TTV_OK ? nin + count * k : nin;
    if (dev_status) dev_status[b] = st;
  }
  const int fr = fb[f];
  if (st != TTV_OK || fr < 0) return;  // the same for the whole workgroup

  // ---- each thread's best KM of its share, tokens in increasing order
  float lv[KM];
  int li[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    lv[j] = -INFINITY;
    li[j] = INT_MAX;
  }
  const float* row = probs + ((size_t)b * F + f) * V;
  if (VEC) {
    const f32x4* r4 = reinterpret_cast<const f32x4*>(row);
    const int n4 = V / 4;
    for (int q0 = threadIdx.x; q0 < n4; q0 += 8 * kExpandThreads) {
      f32x4 q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int x = q0 + u * kExpandThreads;
        q[u] = x < n4 ? __builtin_nontemporal_load(r4 + x) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int x = q0 + u * kExpandThreads;
        if (x < n4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) list_insert(lv, li, q[u][e], 4 * x + e);
        }
      }
    }
  } else {
    for (int v = threadIdx.x; v < V; v += kExpandThreads) list_insert(lv, li, row[v], v);
  }

  // ---- merge: wave 0 lane l takes the lists of threads l, l+64, l+128, l+192
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    s_v[j * kExpandThreads + threadIdx.x] = lv[j];
    s_i[j * kExpandThreads + threadIdx.x] = li[j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kExpandThreads / 64; ++w)
#pragma unroll
    for (int j = 0; j < KM; ++j)
      list_insert(lv, li, s_v[j * kExpandThreads + w * 64 + lane], s_i[j * kExpandThreads + w * 64 + lane]);

  // ---- k rounds of a wave arg-max over the lists' heads; token ids are
  // distinct, so exactly one lane pops its head each round
  const size_t base = (size_t)b * Ncap + nin + (size_t)rank * k;
  for (int j = 0; j < k; ++j) {
    float bv = lv[0];
    int bi = li[0];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (li[0] == bi) {
#pragma unroll
      for (int t = 0; t + 1 < KM; ++t) {
        lv[t] = lv[t + 1];
        li[t] = li[t + 1];
      }
      lv[KM - 1] = -INFINITY;
      li[KM - 1] = INT_MAX;
    }
    if (lane == 0) {
      parents[base + j] = fr;
      tokens[base + j] = bi;
      if (src_row) src_row[base + j] = f;
    }
  }
}

template <int KM>
static hipError_t launch_expand_km(int B, int F, int V, int k, const float* probs,
                                   const int32_t* frontier, const int32_t* n_in, int Ncap,
                                   int32_t* parents, int32_t* tokens, int32_t* src_row,
                                   int32_t* n_out, int32_t* dev_status, bool vec, hipStream_t s) {
  const dim3 grid(F, B);
  if (vec)
    hipLaunchKernelGGL((tree_expand_kernel<KM, true>), grid, dim3(kExpandThreads), 0, s, F, V, k,
                       probs, frontier, n_in, Ncap, parents, tokens, src_row, n_out, dev_status);
  else
    hipLaunchKernelGGL((tree_expand_kernel<KM, false>), grid, dim3(kExpandThreads), 0, s, F, V, k,
                       probs, frontier, n_in, Ncap, parents, tokens, src_row, n_out, dev_status);
  return hipGetLastError();
}

hipError_t launch_tree_expand(int B, int F, int V, int k, const float* probs,
                              const int32_t* frontier, const int32_t* n_in, int Ncap,
                              int32_t* parents, int32_t* tokens, int32_t* src_row,
                              int32_t* n_out, int32_t* dev_status, bool vec, hipStream_t s) {
  if (k <= 4)
    return launch_expand_km<4>(B, F, V, k, probs, frontier, n_in, Ncap, parents, tokens, src_row,
                               n_out, dev_status, vec, s);
  if (k <= 8)
    return launch_expand_km<8>(B, F, V, k, probs, frontier, n_in, Ncap, parents, tokens, src_row,
                               n_out, dev_status, vec, s);
  return launch_expand_km<16>(B, F, V, k, probs, frontier, n_in, Ncap, parents, tokens, src_row,
                              n_out, dev_status, vec, s);
}

}  // namespace ttv
