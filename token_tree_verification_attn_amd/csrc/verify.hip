// verify.hip -- ttv_tree_verify kernels.
//
// [SI] §4 "Token Tree Verification": every candidate sequence of the tree is
// verified in parallel against the LLM's output at each node; §4 "Token
// Verification": greedy matching, or multi-step speculative sampling that
// tests the children of the current node in turn against a residual
// distribution and keeps the LLM's output distribution.
#include <limits.h>

#include "launch.h"
#include "philox.h"
#include "softmax_exact.h"
#include "ttv_common.h"

namespace ttv {

// Inclusive prefix sum over the 64 lanes in lane order, all in the VALU (all
// lanes active): within each 16-lane row lane i adds the row's lanes i-1,
// i-2..i-3, i-4..i-7, i-8..i-15 (row_shr by 1, 2, 4 and 8; a lane shifted in
// from outside the row reads 0); then row_bcast:15 adds the last lane of rows
// 0 and 2 to every lane of rows 1 and 3, and row_bcast:31 the last lane of
// row 1 to rows 2 and 3 (rows a move does not write keep 0).  Exact for
// integer-valued doubles below 2^53.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64_rows(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWS, 0xF, true);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double readlane_f64(double x, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_inclusive_sum_f64(double v) {
  v += dpp_f64_rows<kDppRowShr1, 0xF>(v);
  v += dpp_f64_rows<kDppRowShr2, 0xF>(v);
  v += dpp_f64_rows<kDppRowShr4, 0xF>(v);
  v += dpp_f64_rows<kDppRowShr8, 0xF>(v);
  v += dpp_f64_rows<kDppRowBcast15, 0xA>(v);
  v += dpp_f64_rows<kDppRowBcast31, 0xC>(v);
  return v;
}

// ====================================================================== //
// Greedy                                                                   //
// ====================================================================== //
// (value, index) max with the lowest index winning ties -- the same result
// as a left-to-right scan that replaces only on a strictly greater value.
__device__ __forceinline__ void amax_merge(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// Kernel A: per (node row, vocabulary slice) argmax, streaming the logits
// once with 16-byte loads.  grid = (B*N, splits).
template <bool VEC>
__global__ __launch_bounds__(256) void argmax_partial_kernel(const float* __restrict__ llm, int V,
                                                             int slice, int splits, int N,
                                                             const int32_t* __restrict__ n_nodes,
                                                             float* __restrict__ ws_val,
                                                             int* __restrict__ ws_idx) {
  __shared__ float s_v[4];
  __shared__ int s_i[4];
  const int row = blockIdx.x, sp = blockIdx.y;
  // rows of padding nodes (past the request's node count) are never used
  if (n_nodes && row % N >= nodes_used(n_nodes[row / N], N)) return;
  const int v0 = sp * slice, v1 = min(V, v0 + slice);
  const float* x = llm + (size_t)row * V;
  float bv = -INFINITY;
  int bi = INT_MAX;
  if (VEC) {
    // 8 independent 16-byte loads in flight per thread, merged in index order
    const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
    const int f1 = v1 / 4;
    for (int f0 = v0 / 4 + threadIdx.x; f0 < f1; f0 += 8 * 256) {
      f32x4 q[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int f = f0 + k * 256;
        q[k] = f < f1 ? __builtin_nontemporal_load(x4 + f) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int f = f0 + k * 256;
        if (f < f1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) amax_merge(bv, bi, q[k][e], 4 * f + e);
        }
      }
    }
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += 256) amax_merge(bv, bi, x[v], v);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax_merge(bv, bi, __shfl_xor(bv, m), __shfl_xor(bi, m));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_v[wave] = bv;
    s_i[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) amax_merge(bv, bi, s_v[w], s_i[w]);
    ws_val[(size_t)row * splits + sp] = bv;
    ws_idx[(size_t)row * splits + sp] = bi;
  }
}

// Kernel B: one wavefront per request; lane l holds nodes l and l + 64.
// Everything it reads (parents, tokens, the nodes' argmax partials) is
// requested at once; the rest works on registers: ancestor bitsets by
// shuffle pointer doubling, amax of a node's parent by a shuffle from the
// lane that holds it.  e_i = (token of i == amax of its parent),
// E = ballot(e_i or i == 0), and node i is accepted iff its whole root path
// lies in E, i.e. (anc[i] & ~E) == 0.  The path ends at the deepest accepted
// node (lowest index on ties), found with a wave max; LDS only orders the
// path's nodes by depth.
constexpr int kMaxSplits = 4;  // greedy_plan never makes more
constexpr int kVerifyCommitThreads = 1024;

// The scan of request b by one wavefront (lanes 0..63 of the caller).  Fills
// s_path[0..n-1] with the path's nodes by depth; writes path / out_tokens /
// path_len / dev_status when `write`.  Returns n (0 for a
// malformed tree, -1 for a node count outside [1, N]).  LDS is only written and read by this wavefront, whose LDS
// operations complete in order.
__device__ int greedy_scan_wave(int b, int N, int splits, const int32_t* __restrict__ parents,
                                const int32_t* __restrict__ tokens,
                                const int32_t* __restrict__ n_nodes,
                                const float* __restrict__ ws_val, const int* __restrict__ ws_idx,
                                int32_t* __restrict__ path, int32_t* __restrict__ path_len,
                                int32_t* __restrict__ out_tokens, int32_t* __restrict__ dev_status,
                                bool write, int32_t* s_path) {
  const int lane = threadIdx.x & 63;
  const int i0 = lane, i1 = lane + 64;
  const int32_t* par = parents + (size_t)b * N;
  const int32_t* tok = tokens + (size_t)b * N;
  // every entry of the rows is requested at once with the node count; the
  // entries of padding nodes are dropped afterwards
  const int n_raw = nodes_raw(n_nodes, b, N);
  const bool l0 = i0 < N, l1 = i1 < N;
  int p0 = l0 ? par[i0] : -1, p1 = l1 ? par[i1] : -1;
  const int t0 = l0 ? tok[i0] : -1, t1 = l1 ? tok[i1] : -1;
  float bv0[kMaxSplits], bv1[kMaxSplits];
  int bi0[kMaxSplits], bi1[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    const size_t r0 = ((size_t)b * N + i0) * splits + sp, r1 = ((size_t)b * N + i1) * splits + sp;
    const bool u0 = l0 && sp < splits, u1 = l1 && sp < splits;
    bv0[sp] = u0 ? ws_val[r0] : -INFINITY;
    bi0[sp] = u0 ? ws_idx[r0] : INT_MAX;
    bv1[sp] = u1 ? ws_val[r1] : -INFINITY;
    bi1[sp] = u1 ? ws_idx[r1] : INT_MAX;
  }
  float m0 = -INFINITY, m1 = -INFINITY;
  int am0 = INT_MAX, am1 = INT_MAX;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    amax_merge(m0, am0, bv0[sp], bi0[sp]);
    amax_merge(m1, am1, bv1[sp], bi1[sp]);
  }
  const int nU = nodes_used(n_raw, N);
  const bool n_ok = nodes_ok(n_raw, N);  // the same in every lane
  const bool v0 = i0 < nU, v1 = i1 < nU;
  p0 = v0 ? p0 : -1;
  p1 = v1 ? p1 : -1;
  uint64_t a0lo, a1lo, a1hi;
  if (!n_ok || !wave_tree_bits(p0, p1, nU, a0lo, a1lo, a1hi)) {
    if (write) {
      for (int k = lane; k < N; k += kWave) {
        path[(size_t)b * N + k] = -1;
        out_tokens[(size_t)b * N + k] = -1;
      }
      if (lane == 0) {
        path_len[b] = 0;
        if (dev_status) dev_status[b] = n_ok ? TTV_E_TREE : TTV_E_SHAPE;
      }
    }
    return n_ok ? 0 : -1;
  }
  // node x lives in lane x & 63, slot x >> 6: both slots are shuffled by
  // every lane, then each picks its own
  auto node_int = [&](int x0, int x1, int x) {
    const int a = __shfl(x0, x & 63), c = __shfl(x1, x & 63);
    return x < 64 ? a : c;
  };
  const int q0 = max(p0, 0), q1 = max(p1, 0);
  const int amp0 = node_int(am0, am1, q0), amp1 = node_int(am0, am1, q1);
  const bool e0 = v0 && (i0 == 0 || t0 == amp0);
  const bool e1 = v1 && t1 == amp1;
  const uint64_t E0 = __ballot(e0), E1 = __ballot(e1);
  const int d0 = __popcll(a0lo) - 1, d1 = __popcll(a1lo) + __popcll(a1hi) - 1;
  int key = -1;  // (depth, -index) of the deepest accepted node
  if (v0 && (a0lo & ~E0) == 0ull) key = max(key, (d0 << 8) | (255 - i0));
  if (v1 && (a1lo & ~E0) == 0ull && (a1hi & ~E1) == 0ull) key = max(key, (d1 << 8) | (255 - i1));
  key = wave_allmax_i32(key);  // the root is always accepted: key >= 0
  const int end = 255 - (key & 255), dend = key >> 8;
  const uint64_t x_lo0 = shfl_u64(a0lo, end & 63), x_lo1 = shfl_u64(a1lo, end & 63);
  const uint64_t x_hi1 = shfl_u64(a1hi, end & 63);
  const uint64_t pe0 = end < 64 ? x_lo0 : x_lo1, pe1 = end < 64 ? 0ull : x_hi1;
  if (v0 && ((pe0 >> i0) & 1ull)) s_path[d0] = i0;
  if (v1 && ((pe1 >> (i1 - 64)) & 1ull)) s_path[d1] = i1;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  if (write) {
    const int am_end = node_int(am0, am1, end);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k = lane + r * kWave;
      const int nxt = (k < N && k < dend) ? s_path[k + 1] : 0;
      const int tk = node_int(t0, t1, nxt);
      if (k < N) {
        path[(size_t)b * N + k] = k <= dend ? s_path[k] : -1;
        out_tokens[(size_t)b * N + k] = k < dend ? tk : (k == dend ? am_end : -1);
      }
    }
    if (lane == 0) {
      path_len[b] = dend + 1;
      if (dev_status) dev_status[b] = TTV_OK;
    }
  }
  return dend + 1;
}

// Kernel B: one wavefront per request; lane l holds nodes l and l + 64.
// Everything it reads (parents, tokens, the nodes' argmax partials) is
// requested at once; the rest works on registers: ancestor bitsets by
// shuffle pointer doubling, amax of a node's parent by a shuffle from the
// lane that holds it.  e_i = (token of i == amax of its parent),
// E = ballot(e_i or i == 0), and node i is accepted iff its whole root path
// lies in E, i.e. (anc[i] & ~E) == 0.  The path ends at the deepest accepted
// node (lowest index on ties), found with a wave max; LDS only orders the
// path's nodes by depth.
__global__ __launch_bounds__(64) void greedy_scan_kernel(int N, int splits,
                                                         const int32_t* __restrict__ parents,
                                                         const int32_t* __restrict__ tokens,
                                                         const int32_t* __restrict__ n_nodes,
                                                         const float* __restrict__ ws_val,
                                                         const int* __restrict__ ws_idx,
                                                         int32_t* __restrict__ path,
                                                         int32_t* __restrict__ path_len,
                                                         int32_t* __restrict__ out_tokens,
                                                         int32_t* __restrict__ dev_status) {
  __shared__ int32_t s_path[kMaxNodes];
  greedy_scan_wave(blockIdx.x, N, splits, parents, tokens, n_nodes, ws_val, ws_idx, path,
                   path_len, out_tokens, dev_status, true, s_path);
}

// Kernel B and the KV commit in one launch.  Wave 0 scans request b's tree
// into LDS (the request's first workgroup also writes the verifier's
// outputs); after one barrier the workgroup copies the path's rows of its kv
// heads, node s_path[j] to cache row L + j, in 16-byte vectors.  The commit
// so needs neither a launch of its own nor a read of the path back from
// memory.  Reading every tree row while the scan runs, to keep only the
// path's, measured slower: the path is short and its rows are few.
// Distinct length arrays: one 256-thread workgroup per (request, kv head).
// Shared ones: one 1024-thread workgroup per request copies every head; only
// thread 0 reads cache_len_in[b] (the others take it from LDS after the
// barrier), and its write of cache_len_out[b] depends on that read, so the
// read precedes the write without any ordering between waves (no other
// workgroup touches entry b).
// Statuses: the verifier's if it rejects the tree, else the commit's.
__global__ __launch_bounds__(kVerifyCommitThreads) void greedy_scan_commit_kernel(
    int N, int splits, const int32_t* __restrict__ parents, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ n_nodes, const float* __restrict__ ws_val,
    const int* __restrict__ ws_idx, int32_t* __restrict__ path,
    int32_t* __restrict__ path_len, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ dev_status, int row_vecs, int Hkv, int Lcap, int Lmax,
    const u32x4* __restrict__ k_tree, const u32x4* __restrict__ v_tree,
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache, const int32_t* cache_len_in,
    int32_t* cache_len_out, int32_t* __restrict__ committed_src) {
  __shared__ int32_t s_path[kMaxNodes];
  __shared__ int s_n, s_len;
  const int b = blockIdx.x, tid = threadIdx.x;
  const bool per_head = gridDim.y > 1;
  const int h0 = per_head ? (int)blockIdx.y : 0, nh = per_head ? 1 : Hkv;
  const bool first = blockIdx.y == 0;  // writes the request's verifier outputs and lengths
  if (tid < kWave) {
    const int Lr = tid == 0 ? cache_len_in[b] : 0;  // requested with the scan's loads
    const int n = greedy_scan_wave(b, N, splits, parents, tokens, n_nodes, ws_val, ws_idx, path,
                                   path_len, out_tokens, nullptr, first, s_path);
    if (tid == 0) {
      s_n = n;
      s_len = Lr;
    }
  }
  __syncthreads();
  const int n = s_n;  // 0: malformed tree, -1: bad node count
  const int L = s_len;
  const bool shape_ok = L >= 0 && L <= Lmax && (long)L + n <= Lcap;
  const bool ok = n > 0 && shape_ok;
  if (ok) {
    const int per = n * row_vecs, total = nh * per;
    for (int t = tid; t < total; t += blockDim.x) {
      const int hh = t / per;
      const int r = t - hh * per;
      const int j = r / row_vecs, e = r - (r / row_vecs) * row_vecs;
      const size_t bh = (size_t)b * Hkv + h0 + hh;
      const size_t src = (bh * N + s_path[j]) * row_vecs + e;
      const size_t dst = (bh * Lcap + (size_t)(L + j)) * row_vecs + e;
      const u32x4 kx = k_tree[src], vx = v_tree[src];
      k_cache[dst] = kx;
      v_cache[dst] = vx;
    }
  }
  if (first) {
    if (committed_src)
      for (int j = tid; j < N; j += blockDim.x)
        committed_src[(size_t)b * N + j] = (ok && j < n) ? s_path[j] : -1;
    if (tid == 0) {
      cache_len_out[b] = ok ? L + n : L;
      if (dev_status)
        dev_status[b] = n == 0 ? TTV_E_TREE : (n > 0 && shape_ok ? TTV_OK : TTV_E_SHAPE);
    }
  }
}

hipError_t launch_verify_greedy_commit(int B, int N, int V, const int32_t* parents,
                                       const int32_t* tokens, const int32_t* n_nodes,
                                       const float* llm, int32_t* path,
                                       int32_t* path_len, int32_t* out_tokens,
                                       int32_t* dev_status, void* ws, const GreedyPlan& p,
                                       int elt, int Hkv, int D, int Lcap, int Lmax,
                                       const void* k_tree, const void* v_tree, void* k_cache,
                                       void* v_cache, const int32_t* cache_len_in,
                                       int32_t* cache_len_out, int32_t* committed_src,
                                       hipStream_t s) {
  float* ws_val = static_cast<float*>(ws);
  int* ws_idx = reinterpret_cast<int*>(ws_val + (size_t)B * N * p.splits);
  const bool vec = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(llm) & 15) == 0);
  const dim3 grid(B * N, p.splits);
  if (vec)
    hipLaunchKernelGGL(argmax_partial_kernel<true>, grid, dim3(256), 0, s, llm, V, p.slice,
                       p.splits, N, n_nodes, ws_val, ws_idx);
  else
    hipLaunchKernelGGL(argmax_partial_kernel<false>, grid, dim3(256), 0, s, llm, V, p.slice,
                       p.splits, N, n_nodes, ws_val, ws_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool per_head = cache_len_out != cache_len_in && Hkv > 1 && Hkv <= 65535;
  const dim3 grid2(B, per_head ? Hkv : 1), block2(per_head ? 256 : kVerifyCommitThreads);
  hipLaunchKernelGGL(greedy_scan_commit_kernel, grid2, block2, 0, s, N, p.splits, parents, tokens,
                     n_nodes, ws_val, ws_idx, path, path_len, out_tokens, dev_status, D * elt / 16, Hkv,
                     Lcap, Lmax, static_cast<const u32x4*>(k_tree),
                     static_cast<const u32x4*>(v_tree), static_cast<u32x4*>(k_cache),
                     static_cast<u32x4*>(v_cache), cache_len_in, cache_len_out, committed_src);
  return hipGetLastError();
}

// Vocabulary splits per logits row: enough workgroups to cover the chip
// about four times (~1024: 512 rows x 32000 split in two run 6% faster than
// unsplit), at most 4 so the scan merges few partials (64 rows split in 7
// ran slower than in 4), none below 4096 entries.
GreedyPlan greedy_plan(int B, int N, int V) {
  GreedyPlan p;
  const long rows = (long)B * N;
  long s = (1024 + rows - 1) / rows;
  const long cap = V / 4096 > 1 ? V / 4096 : 1;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  int slice = (int)((V + s - 1) / s);
  slice = (slice + 3) / 4 * 4;
  p.slice = slice;
  p.splits = (V + slice - 1) / slice;
  p.ws_bytes = (size_t)rows * p.splits * 8;
  return p;
}

hipError_t launch_verify_greedy(int B, int N, int V, const int32_t* parents,
                                const int32_t* tokens, const int32_t* n_nodes, const float* llm,
                                int32_t* path, int32_t* path_len, int32_t* out_tokens,
                                int32_t* dev_status, void* ws, const GreedyPlan& p,
                                hipStream_t s) {
  float* ws_val = static_cast<float*>(ws);
  int* ws_idx = reinterpret_cast<int*>(ws_val + (size_t)B * N * p.splits);
  const bool vec = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(llm) & 15) == 0);
  const dim3 grid(B * N, p.splits);
  if (vec)
    hipLaunchKernelGGL(argmax_partial_kernel<true>, grid, dim3(256), 0, s, llm, V, p.slice,
                       p.splits, N, n_nodes, ws_val, ws_idx);
  else
    hipLaunchKernelGGL(argmax_partial_kernel<false>, grid, dim3(256), 0, s, llm, V, p.slice,
                       p.splits, N, n_nodes, ws_val, ws_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_scan_kernel, dim3(B), dim3(kWave), 0, s, N, p.splits, parents, tokens,
                     n_nodes, ws_val, ws_idx, path, path_len, out_tokens, dev_status);
  return hipGetLastError();
}

// ====================================================================== //
// Stochastic: multi-step speculative sampling, one workgroup per request    //
// ====================================================================== //
constexpr int kMssThreads = 1024;

// LDS index of vocabulary entry v: four pad words after every 128 entries
// (16-byte groups stay aligned, and consecutive lanes reading consecutive
// 16-byte groups or words stay conflict-free).
__device__ __forceinline__ int widx(int v) { return v + 4 * (v >> 7); }

// floor(x * 2^40) -- the fixed-point mass of a probability -- as a double,
// for x in [0, 1]: the scaling by 2^40 and the floor are exact in fp32 (a
// power-of-two scale of a float, no overflow; a result of 2^23 or more is
// already an integer), the widening is exact, and so is any sum of such
// terms below 2^53 in any order.
__device__ __forceinline__ double fx40d(float x) { return (double)floorf(x * 0x1p40f); }

// The same sums with one f64 FMA per entry.  A double in [2^52, 2^53) has
// unit spacing, so with double-precision rounding toward -infinity
// (MODE.FP_ROUND[3:2] = 2) an accumulator biased by 2^52 takes acc + x*2^40
// to exactly acc + floor(x*2^40), for x in [0, 1] while the unbiased total
// stays below 2^52.  The mode is set and restored around an accumulation,
// and the FMAs are inline assembly, so that the compiler neither moves them
// out of that window nor folds them (it assumes round-to-nearest for the
// arithmetic it sees); the widening to double is exact in either mode.
constexpr double kFxBias = 0x1p52;
__device__ __forceinline__ void f64_round_down() {
  asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 2, 2), 2\n\ts_nop 1");
}
__device__ __forceinline__ void f64_round_nearest() {
  asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 2, 2), 0\n\ts_nop 1");
}
__device__ __forceinline__ void fx40_acc(double& acc, float x) {
  const double d = (double)x;
  asm volatile("v_fma_f64 %0, %1, %2, %0" : "+v"(acc) : "v"(d), "s"(0x1p40));
}

// max(d, +0) for finite d in one integer max of the bits: a positive float
// is a positive integer, a negative one (or -0) a negative integer, which
// becomes 0, i.e. +0.
__device__ __forceinline__ float clamp_pos(float d) { return __int_as_float(max(__float_as_int(d), 0)); }

__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}


// Sum over the block of integer-valued doubles (exact below 2^53).
__device__ __forceinline__ double block_sum_f64(double v, double* s_redd) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  v = wave_allsum_f64(v);
  __syncthreads();  // s_redd free from its previous use
  if (lane == 0) s_redd[wave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kMssThreads / 64; ++w) t += s_redd[w];
  return t;
}

// The same with one barrier, for reductions that alternate between two slot
// arrays (a late reader of the previous reduction's slots is never
// overwritten: the next write to them follows a barrier it has passed); lane
// w of every wave reads wave w's sum, and a wave sum adds them (exact, so in
// any order).
__device__ __forceinline__ double block_sum_f64_alt(double v, double* slots) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  v = wave_allsum_f64(v);
  if (lane == 0) slots[wave] = v;
  __syncthreads();
  return wave_allsum_f64(lane < kMssThreads / 64 ? slots[lane] : 0.0);
}


// Row passes.  Every wavefront owns a contiguous range of the vocabulary,
// wave w the entries [w*WS, (w+1)*WS), so the per-wave sums of a pass's
// block reduction are the masses of those ranges (the final draw uses them).
// Inside its range a wave's lanes interleave: with 16-byte-aligned rows
// (VEC) lane l takes the 16-byte chunks at w*WS + 4*(64*k + l), k < CH
// (WS = 256*CH), so each wave instruction moves 1 KB of consecutive entries;
// a row moves whole, every chunk requested at once (one memory round trip
// per pass).  Otherwise lane l takes the words w*WS + 64*k + l (WS = 64*CH),
// streamed 8 loads at a time.
constexpr int kMssWaves = kMssThreads / 64;
constexpr int kMssRowChunks = (kMssMaxVocab + 4 * kMssThreads - 1) / (4 * kMssThreads);  // 16-byte chunks per lane
constexpr int kMssSpan = 256 * kMssRowChunks;                 // WS of the single-buffered walks
constexpr int kMssWordChunks = kMssSpan / 64;                 // words per lane, unaligned rows
static_assert(kMssWaves * kMssSpan >= kMssMaxVocab, "the waves' ranges cover the vocabulary");
// first entry of lane-chunk k of thread t, 16-byte chunks, wave span 256*CH
template <int CH>
__device__ __forceinline__ int mss_chunk_v(int t, int k) {
  return 256 * CH * (t >> 6) + 4 * (64 * k + (t & 63));
}
// its LDS slot: widx(mss_chunk_v) = mss_slot0 + 66*4*k (each 256 entries of
// a wave's range take 264 LDS words)
template <int CH>
__device__ __forceinline__ int mss_slot0(int t) {
  return 264 * CH * (t >> 6) + 4 * (t & 63) + 4 * ((t & 63) >> 5);
}

// s_w[widx(v)] = row[v]
template <bool VEC>
__device__ __forceinline__ void mss_row_to_lds(const float* __restrict__ row, int V, float* s_w) {
  const int t = threadIdx.x;
  if (VEC) {
    f32x4 r[kMssRowChunks];
#pragma unroll
    for (int j = 0; j < kMssRowChunks; ++j) {
      const int v = mss_chunk_v<kMssRowChunks>(t, j);
      r[j] = v < V ? *reinterpret_cast<const f32x4*>(row + v) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x4* wp = reinterpret_cast<f32x4*>(s_w + mss_slot0<kMssRowChunks>(t));
#pragma unroll
    for (int j = 0; j < kMssRowChunks; ++j)
      if (mss_chunk_v<kMssRowChunks>(t, j) < V) wp[66 * j] = r[j];
  } else {
    const int v00 = kMssSpan * (t >> 6) + (t & 63);
#pragma unroll 1  // rolled: unrolled, every address and bound would be hoisted into registers
    for (int k0 = 0; k0 < kMssWordChunks; k0 += 8) {
      float x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int v = v00 + 64 * (k0 + k);
        x[k] = k0 + k < kMssWordChunks && v < V ? row[v] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int v = v00 + 64 * (k0 + k);
        if (k0 + k < kMssWordChunks && v < V) s_w[widx(v)] = x[k];
      }
    }
  }
}

// w = max(w - s*q, +0) in place; returns this thread's sum of fx40d(w)
template <bool VEC>
__device__ __forceinline__ double mss_residual(const float* __restrict__ q, int V, float s, float* s_w) {
  const int t = threadIdx.x;
  double part = 0.0;
  if (VEC) {
    f32x4 r[kMssRowChunks];
#pragma unroll
    for (int j = 0; j < kMssRowChunks; ++j) {
      const int v = mss_chunk_v<kMssRowChunks>(t, j);
      r[j] = v < V ? *reinterpret_cast<const f32x4*>(q + v) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x4* wp = reinterpret_cast<f32x4*>(s_w + mss_slot0<kMssRowChunks>(t));
#pragma unroll
    for (int j = 0; j < kMssRowChunks; ++j)
      if (mss_chunk_v<kMssRowChunks>(t, j) < V) {
        f32x4 w = wp[66 * j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d = fmaf(-s, r[j][e], w[e]);
          w[e] = clamp_pos(d);
          part += fx40d(w[e]);
        }
        wp[66 * j] = w;
      }
  } else {
    const int v00 = kMssSpan * (t >> 6) + (t & 63);
#pragma unroll 1  // rolled: unrolled, every address and bound would be hoisted into registers
    for (int k0 = 0; k0 < kMssWordChunks; k0 += 8) {
      float qv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int v = v00 + 64 * (k0 + k);
        qv[k] = k0 + k < kMssWordChunks && v < V ? q[v] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int v = v00 + 64 * (k0 + k);
        if (k0 + k < kMssWordChunks && v < V) {
          const float d = fmaf(-s, qv[k], s_w[widx(v)]);
          const float w = clamp_pos(d);
          s_w[widx(v)] = w;
          part += fx40d(w);
        }
      }
    }
  }
  return part;
}

// Rows given as logits: entry v of the row becomes its probability, computed
// from the row's statistics exactly as the probabilities kernel does.
template <bool LG>
__device__ __forceinline__ f32x4 mss_entry4(f32x4 x, int v, const RowStats& st, float c) {
  if constexpr (LG) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = row_prob(st, c, x[e], v + e);
  }
  return x;
}

// Residual in global memory, for vocabularies beyond the LDS (16-byte rows,
// V % 4 == 0, V <= kMssGmMaxVocab; rows of probabilities, or of logits made
// probabilities with their row's statistics): request b's residual is w[v],
// v < V, in the caller's workspace.  The waves keep contiguous ranges, wave w the
// entries [w*S, (w+1)*S) with S = 256*CH and CH = ceil(V / (4*kMssThreads))
// 16-byte chunks per lane (lane l: w*S + 4*(64*k + l)), so the per-wave sums
// of a pass are again the masses of the ranges; a pass goes through
// kMssGmBatch chunks at a time (loads of a batch issued together).
constexpr int kMssGmBatch = 8;
static_assert(kMssGmMaxVocab <= 4 * kMssThreads * 64,
              "the final draw's lanes take one group each of a lane run (at most 64)");
__device__ __forceinline__ int mss_gm_chunks(int V) {
  return (V + 4 * kMssThreads - 1) / (4 * kMssThreads);
}
// w = row; returns this thread's sum of fx40d of the entries copied
template <bool LG>
__device__ __forceinline__ double mss_gm_row_to_w(const float* __restrict__ row, int V, float* w,
                                                  int CH, const RowStats& st, float c) {
  const int t = threadIdx.x, base = 256 * CH * (t >> 6) + 4 * (t & 63);
  double part = 0.0;
#pragma unroll 1
  for (int k0 = 0; k0 < CH; k0 += kMssGmBatch) {
    f32x4 r[kMssGmBatch];
#pragma unroll
    for (int j = 0; j < kMssGmBatch; ++j) {
      const int v = base + 256 * (k0 + j);
      r[j] = k0 + j < CH && v < V ? *reinterpret_cast<const f32x4*>(row + v) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kMssGmBatch; ++j) {
      const int v = base + 256 * (k0 + j);
      if (k0 + j < CH && v < V) {
        const f32x4 p = mss_entry4<LG>(r[j], v, st, c);
        *reinterpret_cast<f32x4*>(w + v) = p;
#pragma unroll
        for (int e = 0; e < 4; ++e) part += fx40d(p[e]);
      }
    }
  }
  return part;
}
// w = max(w - s*q, +0); returns this thread's sum of fx40d(w)
template <bool LG>
__device__ __forceinline__ double mss_gm_residual(const float* __restrict__ q, int V, float s,
                                                  float* w, int CH, const RowStats& st, float c) {
  const int t = threadIdx.x, base = 256 * CH * (t >> 6) + 4 * (t & 63);
  double part = 0.0;
#pragma unroll 1
  for (int k0 = 0; k0 < CH; k0 += kMssGmBatch) {
    f32x4 r[kMssGmBatch], x[kMssGmBatch];
#pragma unroll
    for (int j = 0; j < kMssGmBatch; ++j) {
      const int v = base + 256 * (k0 + j);
      const bool in = k0 + j < CH && v < V;
      r[j] = in ? *reinterpret_cast<const f32x4*>(q + v) : f32x4{0.f, 0.f, 0.f, 0.f};
      x[j] = in ? *reinterpret_cast<const f32x4*>(w + v) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kMssGmBatch; ++j) {
      const int v = base + 256 * (k0 + j);
      if (k0 + j < CH && v < V) {
        f32x4 y = x[j];
        const f32x4 qv = mss_entry4<LG>(r[j], v, st, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[e] = clamp_pos(fmaf(-s, qv[e], y[e]));
          part += fx40d(y[e]);
        }
        *reinterpret_cast<f32x4*>(w + v) = y;
      }
    }
  }
  return part;
}

// Prefetching row passes (16-byte rows, V <= 4 * kMssThreads * kMssPfChunks):
// rows are requested into registers and consumed later, so the next child's
// row is in flight while the current one is used.  Wave span
// 256 * kMssPfChunks.
constexpr int kMssPfChunks = 8;
constexpr int kMssPfMaxVocab = 4 * kMssThreads * kMssPfChunks;
static_assert(kMssLogitsMaxVocab == kMssPfMaxVocab, "logits rows take the prefetching walk");

// Buffer loads: one resource per row and wave (base = the wave's first
// entry, range = the row's bytes from there), chunk j at byte 1024*j + 16*lane
// of it.  Entries past the row read as zero without a branch or a clamped
// address (loads under a branch would also make the compiler wait for all
// outstanding loads at their first use, draining the prefetch), and a chunk
// costs no scalar arithmetic.  The row pointer must be uniform: a resource
// lives in scalar registers.
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer access (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mss_row_rsrc(const float* __restrict__ row, int V) {
  const int first = 256 * kMssPfChunks * __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bytes = V > first ? 4 * (V - first) : 0;
  const float* base = V > first ? row + first : row;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, bytes, kBufferWord3);
}

__device__ __forceinline__ f32x4 mss_rsrc_chunk(__amdgpu_buffer_rsrc_t rs, int j) {
  return __builtin_bit_cast(
      f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (int)(threadIdx.x & 63), 1024 * j, 0));
}

__device__ __forceinline__ void mss_issue_row(const float* __restrict__ row, int V,
                                              f32x4 (&r)[kMssPfChunks]) {
  const __amdgpu_buffer_rsrc_t rs = mss_row_rsrc(row, V);
#pragma unroll
  for (int j = 0; j < kMssPfChunks; ++j) r[j] = mss_rsrc_chunk(rs, j);
}

// Two rows, their chunks requested in turn.
__device__ __forceinline__ void mss_issue_rows2(const float* __restrict__ a, const float* __restrict__ b,
                                                int V, f32x4 (&ra)[kMssPfChunks], f32x4 (&rb)[kMssPfChunks]) {
  const __amdgpu_buffer_rsrc_t sa = mss_row_rsrc(a, V), sb = mss_row_rsrc(b, V);
#pragma unroll
  for (int j = 0; j < kMssPfChunks; ++j) {
    ra[j] = mss_rsrc_chunk(sa, j);
    rb[j] = mss_rsrc_chunk(sb, j);
  }
}

// s_w[widx(v)] = r (probabilities, or logits made probabilities with `st`);
// returns this thread's sum of fx40d of them (computed only where used)
template <bool LG>
__device__ __forceinline__ double mss_regs_to_lds(const f32x4 (&r)[kMssPfChunks], int V, float* s_w,
                                                  const RowStats& st, float c) {
  const int t = threadIdx.x;
  f32x4* wp = reinterpret_cast<f32x4*>(s_w + mss_slot0<kMssPfChunks>(t));
  if constexpr (!LG) {
    // probabilities: every chunk of the span is written (the row's loads
    // read zeros past V, and the LDS holds the whole span), so w = 0 there
    // and no chunk needs a branch
    double part[2] = {0.0, 0.0};
#pragma unroll
    for (int j = 0; j < kMssPfChunks; ++j) {
      wp[66 * j] = r[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) part[e >> 1] += fx40d(r[j][e]);
    }
    return part[0] + part[1];
  }
  double part = 0.0;
#pragma unroll
  for (int j = 0; j < kMssPfChunks; ++j) {
    const int v = mss_chunk_v<kMssPfChunks>(t, j);
    if (v < V) {
      const f32x4 p = mss_entry4<LG>(r[j], v, st, c);
      wp[66 * j] = p;
#pragma unroll
      for (int e = 0; e < 4; ++e) part += fx40d(p[e]);
    }
  }
  return part;
}

// The residual of the prefetching walk lives in registers: thread t
// holds w of its chunks (entries mss_chunk_v<kMssPfChunks>(t, j)) in wr[j],
// and the speculator's rows stream through one register buffer qr, chunk j
// of the next row requested as soon as chunk j of the current one is used
// (one row in flight during a pass, no LDS traffic); the final draw from
// that residual reads the registers too.

// wr = the row loaded into it, as probabilities (LG: logits made
// probabilities with `st`, 0 past V; rows of probabilities read 0 there)
template <bool LG>
__device__ __forceinline__ void mss_row_regs(f32x4 (&wr)[kMssPfChunks], int V, const RowStats& st, float c) {
  if constexpr (LG) {
#pragma unroll
    for (int j = 0; j < kMssPfChunks; ++j) {
      const int v = mss_chunk_v<kMssPfChunks>(threadIdx.x, j);
      wr[j] = v < V ? mss_entry4<LG>(wr[j], v, st, c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// w = max(w - s*q, +0) with q in qr, whose chunk j then receives chunk j of
// `next` (nV of its entries; nV = 0 reads zeros without touching memory);
// returns this thread's sum of fx40d(w)
template <bool LG>
__device__ __forceinline__ double mss_residual_roll(f32x4 (&wr)[kMssPfChunks], f32x4 (&qr)[kMssPfChunks],
                                                    const float* __restrict__ next, int nV, int V,
                                                    float s, const RowStats& st, float c) {
  const __amdgpu_buffer_rsrc_t rs = mss_row_rsrc(next, nV);
  double part[4] = {kFxBias, kFxBias, kFxBias, kFxBias};
  f64_round_down();
#pragma unroll
  for (int j = 0; j < kMssPfChunks; ++j) {
    f32x4 q = qr[j];
    if constexpr (LG) {
      const int v = mss_chunk_v<kMssPfChunks>(threadIdx.x, j);
      q = v < V ? mss_entry4<LG>(q, v, st, c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // max(w - s*q, +0) as the FMA's clamp to [0, 1] (w <= 1 already; the
    // clamp gives +0 or -0 for a negative result, which every later use --
    // the masses, the tests, the draw -- takes as 0)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wr[j][e] = __builtin_amdgcn_fmed3f(fmaf(-s, q[e], wr[j][e]), 0.f, 1.f);
      fx40_acc(part[e], wr[j][e]);
    }
    // chunk j of q is used up; the request for its successor is ordered
    // after that use (the empty asm ties its resource to the last w), so the
    // new chunk can take the old one's registers: a copy at the end of the
    // pass would wait for every request in flight
    __amdgpu_buffer_rsrc_t rj = rs;
    asm volatile("" : "+s"(rj) : "v"(wr[j][3]));
    qr[j] = mss_rsrc_chunk(rj, j);
    // and no work of a later chunk is scheduled ahead of this one (it would
    // wait for that chunk's request, issued late in the previous pass)
    __builtin_amdgcn_sched_barrier(0);
  }
  f64_round_nearest();
  return ((part[0] - kFxBias) + (part[1] - kFxBias)) + ((part[2] - kFxBias) + (part[3] - kFxBias));
}

// w[x] from the registers of the thread that holds it (x = 2048*wave +
// 256*j + 4*lane + e), stored to *dst by that thread
__device__ __forceinline__ void mss_regs_entry(const f32x4 (&wr)[kMssPfChunks], int x, float* dst) {
  static_assert(256 * kMssPfChunks == 2048, "wave span");
  if ((int)threadIdx.x == ((x >> 11) << 6) + ((x & 255) >> 2)) {
    const int jx = (x >> 8) & (kMssPfChunks - 1), ex = x & 3;
    float val = 0.f;
#pragma unroll
    for (int j = 0; j < kMssPfChunks; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j == jx && e == ex) val = wr[j][e];
    *dst = val;
  }
}

// The final draw from a residual held in registers in the prefetching
// walk's layout (thread t: entries 2048*wave + 256*j + 4*lane + e, zero past
// V), with the masses of the waves' ranges in s_tot (total > 0): the wave
// whose range holds the target is found as in the LDS draw; inside it the
// masses of its eight 256-entry chunks, in order, locate the chunk, and a
// lane scan over the chunk's 4-entry groups the entry, which the crossing
// lane writes to *pick.  The same masses in the same order as the LDS draw.
__device__ __forceinline__ void mss_draw_regs(const f32x4 (&w)[kMssPfChunks], const double* s_tot,
                                              uint32_t R, int* pick) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double cw = wave_inclusive_sum_f64(lane < kMssWaves ? s_tot[lane] : 0.0);
  const uint64_t S = (uint64_t)readlane_f64(cw, kMssWaves - 1);
  const double T = (double)((uint64_t)R * (S >> 24) + (((uint64_t)R * (S & 0xffffffull)) >> 24));
  const uint64_t past = __ballot(lane < kMssWaves && cw > T);
  const int ws = past ? __ffsll((unsigned long long)past) - 1 : kMssWaves - 1;
  if (wave != ws) return;
  auto group = [](const f32x4& g4) {
    return (fx40d(g4[0]) + fx40d(g4[1])) + (fx40d(g4[2]) + fx40d(g4[3]));
  };
  double before = ws > 0 ? readlane_f64(cw, ws - 1) : 0.0;
  int jx = kMssPfChunks - 1;
  bool found = false;
#pragma unroll
  for (int j = 0; j < kMssPfChunks; ++j) {
    const double c = wave_allsum_f64(group(w[j]));
    if (!found) {
      if (before + c > T) {
        jx = j;
        found = true;
      } else {
        before += c;
      }
    }
  }
  f32x4 wx = w[0];
#pragma unroll
  for (int j = 1; j < kMssPfChunks; ++j)
    if (j == jx) wx = w[j];
  const double gx = group(wx);
  const double incl = wave_inclusive_sum_f64(gx);
  const double lo = before + (incl - gx);
  if (lo <= T && T < before + incl) {
    const int v0 = 2048 * ws + 256 * jx + 4 * lane;
    double cum = lo;
    int p = v0 + 3;
    bool hit = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cum += fx40d(wx[e]);
      if (!hit && cum > T) {
        p = v0 + e;
        hit = true;
      }
    }
    *pick = p;
  }
}

// LG: llm and ssm hold logits; st_llm / st_ssm [B*N] their rows' statistics
// (ttv_tree_verify_logits), c = (float)(log2(e) / T).
// GM: the residual lives in global memory (gm_w [B][V], see above), for
// vocabularies beyond the LDS; single-buffered 16-byte rows only.
template <bool VEC, bool PF, bool LG, bool GM>
__global__ __launch_bounds__(kMssThreads) void mss_kernel(
    int N, int V, const int32_t* __restrict__ parents, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ n_nodes, const float* __restrict__ llm,
    const float* __restrict__ ssm, MssDraws dr, LogitRows lr,
    int32_t* __restrict__ path, int32_t* __restrict__ path_len,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ dev_status, float* __restrict__ gm_w,
    CommitArgs cm) {
  static_assert(!GM || (VEC && !PF), "the global residual takes single-buffered 16-byte rows");
  extern __shared__ __attribute__((aligned(16))) float s_w[];  // residual w, widx() layout
  __shared__ int32_t s_par[kMaxNodes];
  __shared__ int32_t s_tok[kMaxNodes];
  __shared__ int32_t s_path[kMaxNodes];
  __shared__ float s_rq[kMaxNodes];  // r_c * q_c[token c]: the left side of c's test at s = 1
  __shared__ float s_wx[2];  // w[token] of the next child tested (alternating slots)
  __shared__ uint32_t s_bonus[kMaxNodes];  // the final draw's 24-bit integer if the walk ends at u
  __shared__ unsigned long long s_kids[kMaxNodes][2];
  __shared__ uint64_t s_first_ok[2];
  __shared__ double s_red3[3][kMssThreads / 64];  // [0]: two-barrier sums, [1], [2]: alternating
  double* const s_redd = s_red3[0];
  __shared__ int s_status, s_pick, s_len, s_nodes;
  __shared__ float s_av[GM ? kMssWaves : 1];  // the all-zero fallback of the global residual
  __shared__ int s_ai[GM ? kMssWaves : 1];

  const int b = blockIdx.x, t = threadIdx.x, wave = t >> 6;
  const size_t rowN = (size_t)b * N;
  // the residual: this request's slice of gm_w, or LDS
  float* const wg = GM ? gm_w + (size_t)b * V : nullptr;
  const int gmCH = GM ? mss_gm_chunks(V) : 0;
  auto wref = [&](int v) -> float& {
    if constexpr (GM) return wg[v];
    else return s_w[widx(v)];
  };
  // uniforms: drawn here from Philox (seed, step), or given by the caller
  const bool seeded = dr.u_accept == nullptr;
  // statistics of row u of llm / row c of ssm when they hold logits (read
  // when a row is turned into probabilities; wave-uniform scalar loads)
  auto p_stats = [&](int u) { return LG ? lr.st_llm[rowN + u] : RowStats{}; };
  auto q_stats = [&](int c) { return LG ? lr.st_ssm[rowN + c] : RowStats{}; };
  // with the commit: thread 0 alone reads the prefix length (the others take
  // it from LDS after the set-up's barrier); its write of the new one, which
  // may alias it, depends on that read, and only this workgroup touches
  // entry b
  const bool commit = cm.k_tree != nullptr;
  // ---- the set-up, with one barrier.  Wave 0 alone (lane l holds nodes l
  // and l + 64, so its LDS accesses need no barrier) reads the tree, checks
  // it, builds the children bitsets and makes the first-attempt test of
  // every non-root node (r*q[x] against p[x] of its parent, mass 1; only
  // first children use it), the gathers going out first.  Wave 1 draws the
  // final-draw integer of every node (the walk may end anywhere).  With the
  // prefetching walk, the root's row and that of node 1 (the root's first
  // child in every tree of two or more nodes) are requested by every wave --
  // at once by the others, after their work by waves 0 and 1 -- so that they
  // stream in during the set-up; the walk starts from them when node 1's
  // test fails.  (With N = 1 there is no row of node 1: the root's q row is
  // read instead, and not used.)
  f32x4 wr[kMssPfChunks], qr[kMssPfChunks];
  const float* const p0row = llm + rowN * V;
  const float* const q1row = ssm + (rowN + (N >= 2 ? 1 : 0)) * V;
  if constexpr (PF) {
    if (wave >= 2) mss_issue_rows2(p0row, q1row, V, wr, qr);
  }
  if (wave == 0) {
    const int lane = t;
    const int n_raw0 = nodes_raw(n_nodes, b, N);
    const int nU0 = nodes_used(n_raw0, N);
    int par[2], tok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = lane + 64 * h;
      par[h] = i < N ? parents[rowN + i] : -1;
      tok[h] = i < N ? tokens[rowN + i] : 0;
      if (i < N) {
        s_par[i] = par[h];
        s_tok[i] = tok[h];
        s_kids[i][0] = 0ull;
        s_kids[i][1] = 0ull;
      }
    }
    if (lane == 0) {
      s_len = commit ? cm.cache_len_in[b] : 0;
      s_nodes = n_raw0;
      s_path[0] = 0;
    }
    bool bad_tree = false, bad_tok = false;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = lane + 64 * h;
      if (i < nU0) {
        bad_tree |= (i == 0) ? (par[h] != -1) : (par[h] < 0 || par[h] >= i);
        bad_tok |= i > 0 && (tok[h] < 0 || tok[h] >= V);
      }
    }
    const int st0 = (__ballot(bad_tree) ? 1 : 0) | ((__ballot(bad_tok) || !nodes_ok(n_raw0, N)) ? 2 : 0);
    if (lane == 0) s_status = st0;
    if (st0 == 0) {
      float qx[2] = {0.f, 0.f}, px[2] = {0.f, 0.f}, ua[2] = {0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = lane + 64 * h;
        if (i >= 1 && i < nU0) {
          atomicOr(&s_kids[par[h]][i >> 6], 1ull << (i & 63));
          qx[h] = ssm[(rowN + i) * V + tok[h]];
          px[h] = llm[(rowN + par[h]) * V + tok[h]];
          if constexpr (LG) {
            qx[h] = row_prob(lr.st_ssm[rowN + i], lr.c, qx[h], tok[h]);
            px[h] = row_prob(lr.st_llm[rowN + par[h]], lr.c, px[h], tok[h]);
          }
          if (!seeded) ua[h] = dr.u_accept[rowN + i];
        }
      }
      // the bitsets are complete: this wave's LDS operations run in order
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      bool first_ok[2] = {false, false};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = lane + 64 * h;
        if (i >= 1 && i < nU0) {
          float r = ua[h];
          if (seeded) {  // i is the j-th child of its parent, j = its lower siblings
            const uint64_t lo = s_kids[par[h]][0], hi = s_kids[par[h]][1];
            const int j = i < 64 ? __popcll(lo & ((1ull << i) - 1ull))
                                 : __popcll(lo) + __popcll(hi & ((1ull << (i - 64)) - 1ull));
            r = (float)mss_draw24(dr.seed, dr.step, (uint64_t)j, par[h], b) * 0x1p-24f;
          }
          const float rq = r * qx[h];
          s_rq[i] = rq;
          first_ok[h] = rq * 1.0f < px[h];
        }
      }
      const uint64_t ok0 = __ballot(first_ok[0]), ok1 = __ballot(first_ok[1]);
      if (lane == 0) {
        s_first_ok[0] = ok0;
        s_first_ok[1] = ok1;
      }
    }
  } else if (wave == 1) {
    static_assert(kMaxNodes <= 128, "two nodes per lane");
    const float ub = seeded ? 0.f : dr.u_bonus[b];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = (t - 64) + 64 * h;
      if (i < N)
        s_bonus[i] = seeded ? mss_draw24(dr.seed, dr.step, kBonusOrdinal, i, b)
                            : (uint32_t)(ub * 16777216.0f);  // exact: scaling by 2^24
    }
  }
  if constexpr (PF) {
    if (wave < 2) mss_issue_rows2(p0row, q1row, V, wr, qr);
  }
  __syncthreads();
  const int L = s_len;
  // the request's nodes (entries past them are padding, never used)
  const int n_raw = s_nodes;
  const int nU = nodes_used(n_raw, N);
  const bool pre = PF && nU >= 2;
  const int st = s_status;
  if (st != 0) {
    for (int k = t; k < N; k += kMssThreads) {
      path[rowN + k] = -1;
      out_tokens[rowN + k] = -1;
    }
    if (commit && cm.committed_src)
      for (int k = t; k < N; k += kMssThreads) cm.committed_src[rowN + k] = -1;
    if (t == 0) {
      path_len[b] = 0;
      // a bad node count or token is TTV_E_SHAPE, a malformed tree TTV_E_TREE
      if (dev_status)
        dev_status[b] = !nodes_ok(n_raw, N) ? TTV_E_SHAPE : (st & 1) ? TTV_E_TREE : TTV_E_SHAPE;
      if (commit) cm.cache_len_out[b] = L;
    }
    return;
  }

  // s_w = p_u.  The first barrier lets every thread finish reading the old
  // residual (the test that led here reads it), the second publishes p_u.
  // (GM: with the masses of the waves' ranges in s_redd, left by the
  // reduction whose barriers publish w)
  auto load_p_row = [&](int u) {
    __syncthreads();
    if constexpr (GM) {
      block_sum_f64(mss_gm_row_to_w<LG>(llm + (rowN + u) * V, V, wg, gmCH, p_stats(u), lr.c), s_redd);
    } else {
      mss_row_to_lds<VEC>(llm + (rowN + u) * V, V, s_w);
      __syncthreads();
    }
  };

  // ---- the walk: control flow is uniform, decisions are recomputed by every
  // thread from the same LDS values.  Every row is requested whole: one
  // memory round trip per pass.  s_path[d] gets the node at depth d as the
  // walk descends (it never backtracks; each entry is written before one of
  // the walk's barriers).  `totals`: s_redd holds the masses of the waves'
  // ranges of what s_w holds for the final draw (the last residual pass, or
  // the copy of p_u the draw comes from, left them there).
  int u = 0, depth = 0, wx_slot = 0, red_alt = 0;
  bool totals = false;
  const double* s_tot = s_redd;  // the slots holding the masses of the waves' ranges (totals)
  auto descend = [&](int c) {
    u = c;
    ++depth;
    if (t == 0) s_path[depth] = c;
  };

  // ---- the commit's first rows (one 16-byte vector of K and of V per
  // thread), requested once the walk has ended: before the final draw in
  // LDS, so their round trip overlaps it (the draw from registers at the end
  // of the walk returns at once in every wave but the one that holds the
  // target, which requests them after it)
  const int rv = cm.row_vecs;
  int cper = 0, ncopy = 0;
  bool cok = false;  // the commit fits the cache
  const u32x4* ktr = static_cast<const u32x4*>(cm.k_tree);
  const u32x4* vtr = static_cast<const u32x4*>(cm.v_tree);
  u32x4* kca = static_cast<u32x4*>(cm.k_cache);
  u32x4* vca = static_cast<u32x4*>(cm.v_cache);
  auto copy_src = [&](int x, size_t& dst) {
    const int h = x / cper, r = x - h * cper;
    const int j = r / rv, e = r - j * rv;
    const size_t bh = (size_t)b * cm.Hkv + h;
    dst = (bh * cm.Lcap + (size_t)(L + j)) * rv + e;
    return (bh * N + s_path[j]) * rv + e;
  };
  u32x4 kx0 = {0u, 0u, 0u, 0u}, vx0 = {0u, 0u, 0u, 0u};
  size_t dst0 = 0;
  auto issue_commit = [&](int len_) {
    cok = commit && L >= 0 && L <= cm.Lmax && (long)L + len_ <= cm.Lcap;
    cper = len_ * rv;
    ncopy = cok ? cm.Hkv * cper : 0;
    if (t < ncopy) {
      const size_t src = copy_src(t, dst0);
      kx0 = ktr[src];
      vx0 = vtr[src];
    }
  };
  // the walk that ends in the residual of the prefetching tests draws the
  // bonus from its registers (s_pick)
  bool drawn = false;
  // PF: the residual tests at node u once its first child c0 has failed its
  // test, with p_u in wr and q of c0 in qr (requested by the caller; k0/k1
  // the other children).  The residual stays in registers, and while child
  // c's residual pass runs, the next child's row streams into qr chunk by
  // chunk (after the last child, requests of an empty range, which return
  // zeros without a memory access, so that no request is under a branch).  w[x] of the child tested next goes through
  // LDS from the thread that holds it, published by the pass's reduction;
  // its slots alternate, so no barrier is needed before the next pass writes
  // one.  Returns the accepted child, or -1 when the walk ends at u: every
  // child rejected, with the bonus drawn from the registers (s_pick), or the
  // residual emptied, with p_u in s_w and its waves' masses in s_redd.
  auto pf_node = [&](int u, uint64_t k0, uint64_t k1, int c0, f32x4 (&wr)[kMssPfChunks],
                     f32x4 (&qr)[kMssPfChunks]) -> int {
    mss_row_regs<LG>(wr, V, p_stats(u), lr.c);
    float s = 1.0f;
    int ccur = c0;
    for (;;) {
      int cn = -1;
      if (k0) {
        cn = __ffsll((unsigned long long)k0) - 1;
        k0 &= k0 - 1;
      } else if (k1) {
        cn = 64 + __ffsll((unsigned long long)k1) - 1;
        k1 &= k1 - 1;
      }
      const int crow = ccur;  // the child whose q row is in qr
      ccur = cn;
      const double part = mss_residual_roll<LG>(wr, qr, ssm + (rowN + (cn >= 0 ? cn : crow)) * V,
                                                cn >= 0 ? V : 0, V, s, q_stats(crow), lr.c);
      if (cn >= 0) mss_regs_entry(wr, s_tok[cn], &s_wx[wx_slot]);
      // its barriers publish s_wx (the walk over logits, short of registers,
      // keeps the two-barrier form)
      double S;
      if constexpr (LG) {
        S = block_sum_f64(part, s_redd);
      } else {
        double* const sl = s_red3[1 + red_alt];
        red_alt ^= 1;
        S = block_sum_f64_alt(part, sl);
        s_tot = sl;
      }
      s = (float)(S * 0x1p-40);
      if (s == 0.0f) {  // empty residual: stop testing, sample from p_u
        mss_issue_row(llm + (rowN + u) * V, V, qr);
        __syncthreads();
        block_sum_f64(mss_regs_to_lds<LG>(qr, V, s_w, p_stats(u), lr.c), s_redd);
        s_tot = s_redd;
        return -1;
      }
      if (cn < 0) {  // every child rejected: the bonus from the residual in wr
        mss_draw_regs(wr, s_tot, s_bonus[u], &s_pick);
        drawn = true;
        return -1;
      }
      const bool accept = s_rq[cn] * s < s_wx[wx_slot];
      wx_slot ^= 1;
      if (accept) return cn;
    }
  };
  bool ended = false;
  if constexpr (PF) {
    // the root, with the rows requested during the set-up, if its first
    // child (node 1) failed its test
    if (pre && !(s_first_ok[0] & 2ull)) {
      const int nx = pf_node(0, uniform_u64(s_kids[0][0]) & ~2ull, uniform_u64(s_kids[0][1]), 1, wr, qr);
      totals = true;
      if (nx < 0) ended = true;
      else descend(nx);
    }
  }
  while (!ended) {
    // the same in every lane: scalar registers (children, nodes and row
    // addresses derived from them stay scalar)
    uint64_t k0 = uniform_u64(s_kids[u][0]), k1 = uniform_u64(s_kids[u][1]);
    if ((k0 | k1) == 0ull) {  // leaf: the bonus comes from p_u
      if constexpr (PF) {
        f32x4 ra[kMssPfChunks];
        mss_issue_row(llm + (rowN + u) * V, V, ra);
        __syncthreads();
        // the masses of the waves' ranges come with the copy; the
        // reduction's barriers publish s_w
        block_sum_f64(mss_regs_to_lds<LG>(ra, V, s_w, p_stats(u), lr.c), s_redd);
        s_tot = s_redd;
        totals = true;
      } else {
        load_p_row(u);
        totals = GM;
      }
      break;
    }
    const int c0 = k0 ? __ffsll((unsigned long long)k0) - 1 : 64 + __ffsll((unsigned long long)k1) - 1;
    const bool ok0 = (c0 < 64 ? (s_first_ok[0] >> c0) : (s_first_ok[1] >> (c0 - 64))) & 1ull;
    if (ok0) {
      descend(c0);
      continue;
    }
    // first child rejected: sequential residual tests at u
    if constexpr (PF) {
      // p_u and q of the first child, requested together
      f32x4 ra[kMssPfChunks], rb[kMssPfChunks];
      mss_issue_row(llm + (rowN + u) * V, V, ra);
      mss_issue_row(ssm + (rowN + c0) * V, V, rb);
      if (k0) k0 &= k0 - 1;
      else k1 &= k1 - 1;
      const int nx = pf_node(u, k0, k1, c0, ra, rb);
      totals = true;
      if (nx < 0) break;  // bonus from the residual in s_w (or p_u)
      descend(nx);
      continue;
    }
    load_p_row(u);
    float s = 1.0f;
    int next = -1;
    bool first = true, emptied = false;
    while (k0 | k1) {
      // lowest remaining child (written out: a helper taking both words by
      // reference made the compiler keep them in private memory)
      int c;
      if (k0) {
        c = __ffsll((unsigned long long)k0) - 1;
        k0 &= k0 - 1;
      } else {
        c = 64 + __ffsll((unsigned long long)k1) - 1;
        k1 &= k1 - 1;
      }
      if (!first) {  // c's test against w, mass s
        const bool accept = s_rq[c] * s < wref(s_tok[c]);
        __syncthreads();  // every thread has read w[x] before it is updated below
        if (accept) {
          next = c;
          break;
        }
      }
      first = false;
      // rejected: w = max(w - s*q_c, +0), s = its mass in 2^-40 units
      double part;
      if constexpr (GM) part = mss_gm_residual<LG>(ssm + (rowN + c) * V, V, s, wg, gmCH, q_stats(c), lr.c);
      else part = mss_residual<VEC>(ssm + (rowN + c) * V, V, s, s_w);
      const double S = block_sum_f64(part, s_redd);  // its barriers publish s_w
      s = (float)(S * 0x1p-40);
      if (s == 0.0f) {  // empty residual: stop testing, sample from p_u
        load_p_row(u);
        emptied = true;
        break;
      }
    }
    if (next < 0) {  // bonus from the residual in s_w (or p_u)
      totals = GM || !emptied;
      break;
    }
    descend(next);
  }
  const int len = depth + 1;
  issue_commit(len);

  // ---- bonus: inverse CDF over the exact integer prefix sums of fx40d(w).
  // The masses of the waves' ranges (left by the walk, else summed here,
  // each wave over its own range in the row passes' order)
  // locate the wave whose range holds the target; that wave alone finds the
  // entry: lane l takes P consecutive entries of the range (P a multiple of
  // 4: each 4-entry group is 16 aligned bytes of s_w), an exclusive scan over
  // the lanes gives each run's start, and the lane whose run crosses the
  // target walks its groups.  Masses are exact integers carried in doubles.
  if (drawn) {  // drawn from the registers at the end of the walk
  } else if constexpr (GM) {
    // the same search over the wave ranges in global memory (span 256*CH,
    // lane runs of 4*CH entries); the masses of the ranges are in s_redd
    // (every exit of the walk leaves them there)
    const int span = 256 * gmCH, P = 4 * gmCH;
    double Sd = 0.0;
#pragma unroll
    for (int w = 0; w < kMssWaves; ++w) Sd += s_tot[w];
    if (Sd > 0.0) {
      const uint64_t S = (uint64_t)Sd, R = s_bonus[u];
      const double T = (double)(R * (S >> 24) + ((R * (S & 0xffffffull)) >> 24));  // floor(R*S/2^24)
      double before = 0.0;
      int ws = kMssWaves - 1;
      bool found = false;
#pragma unroll
      for (int w = 0; w < kMssWaves; ++w) {
        const double g = s_tot[w];
        if (!found && before + g > T) {
          ws = w;
          found = true;
        } else if (!found) {
          before += g;
        }
      }
      if (wave == ws) {
        const int lane = t & 63;
        const int v_lo = min(V, ws * span + lane * P), v_hi = min(V, v_lo + P);
        double mine = 0.0;
#pragma unroll 4
        for (int i = 0; i < gmCH; ++i) {
          const int v = v_lo + 4 * i;
          if (v < v_hi) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(wg + v);
#pragma unroll
            for (int e = 0; e < 4; ++e) mine += v + e < v_hi ? fx40d(w4[e]) : 0.0;
          }
        }
        const double incl = wave_inclusive_sum_f64(mine);
        const double lo = before + (incl - mine);
        const uint64_t crossing = __ballot(lo <= T && T < before + incl);
        if (crossing != 0ull) {
          // the lanes take the groups of the crossing lane's run, one each
          // (a run has CH <= 64 groups), and scan them
          const int Lc = __ffsll((unsigned long long)crossing) - 1;
          const double loL = __shfl(lo, Lc);
          const int vloL = __shfl(v_lo, Lc), vhiL = __shfl(v_hi, Lc);
          const int v = vloL + 4 * lane;
          f32x4 w4 = {0.f, 0.f, 0.f, 0.f};
          double g = 0.0;
          if (lane < gmCH && v < vhiL) {
            w4 = *reinterpret_cast<const f32x4*>(wg + v);
#pragma unroll
            for (int e = 0; e < 4; ++e) g += v + e < vhiL ? fx40d(w4[e]) : 0.0;
          }
          const double gin = wave_inclusive_sum_f64(g);
          double cum = loL + (gin - g);
          if (cum <= T && T < loL + gin) {
            int pick = vhiL - 1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (v + e < vhiL) {
                cum += fx40d(w4[e]);
                if (cum > T) {
                  pick = v + e;
                  break;
                }
              }
            }
            s_pick = pick;
          }
        }
      }
    } else {  // nothing representable left: the largest entry (lowest index on ties)
      float bv = -INFINITY;
      int bi = INT_MAX;
      for (int v = t; v < V; v += kMssThreads)
        if (wg[v] > bv) {
          bv = wg[v];
          bi = v;
        }
      wave_allargmax(bv, bi);
      if ((t & 63) == 0) {
        s_av[wave] = bv;
        s_ai[wave] = bi;
      }
      __syncthreads();
      if (t == 0) {
        float v0 = s_av[0];
        int i0 = s_ai[0];
        for (int w = 1; w < kMssWaves; ++w) argmax_take(v0, i0, s_av[w], s_ai[w]);
        s_pick = i0;
      }
    }
  } else {
    constexpr int kSpan = PF ? 256 * kMssPfChunks : kMssSpan;
    if (!totals) {
      double part = 0.0;
  #pragma unroll
      for (int k = 0; k < kSpan / 256; ++k) {
        const int v = kSpan * wave + 4 * (64 * k + (t & 63));
        if (v < V) {
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(s_w + widx(v));
  #pragma unroll
          for (int e = 0; e < 4; ++e) part += v + e < V ? fx40d(w4[e]) : 0.0;
        }
      }
      block_sum_f64(part, s_redd);  // s_redd[w] = mass of wave w's range
      s_tot = s_redd;
    }
    // masses below 2^53: exact in doubles, compared as doubles.  Lane w of
    // every wave takes wave w's mass; their prefix sums give the total, the
    // first wave whose cumulative mass exceeds the target (a ballot) and the
    // mass before it.
    const int lw = t & 63;
    const double cw = wave_inclusive_sum_f64(lw < kMssWaves ? s_tot[lw] : 0.0);
    const double Sd = readlane_f64(cw, kMssWaves - 1);
    if (Sd > 0.0) {
      const uint64_t S = (uint64_t)Sd, R = s_bonus[u];
      const double T = (double)(R * (S >> 24) + ((R * (S & 0xffffffull)) >> 24));  // floor(R*S/2^24)
      const uint64_t past = __ballot(lw < kMssWaves && cw > T);  // T < S: wave kMssWaves-1 is set
      const int ws = past ? __ffsll((unsigned long long)past) - 1 : kMssWaves - 1;
      const double before = ws > 0 ? readlane_f64(cw, ws - 1) : 0.0;
      if (wave == ws) {
        constexpr int P = kSpan / 64, kG = P / 4;
        const int lane = t & 63;
        const int v_lo = min(V, ws * kSpan + lane * P), v_hi = min(V, v_lo + P);
        double mine = 0.0, gsum[kG];  // gsum[i]: mass of the group at v_lo + 4i
  #pragma unroll
        for (int i = 0; i < kG; ++i) {
          const int v = v_lo + 4 * i;
          double g = 0.0;
          if (v < v_hi) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(s_w + widx(v));
  #pragma unroll
            for (int e = 0; e < 4; ++e) g += v + e < v_hi ? fx40d(w4[e]) : 0.0;
          }
          gsum[i] = g;
          mine += g;
        }
        const double incl = wave_inclusive_sum_f64(mine);
        const double lo = before + (incl - mine), hi = before + incl;
        if (lo <= T && T < hi) {
          // the group that crosses T from the register sums, then its entries
          // (unrolled with constant indices: gsum stays in registers; a group
          // with no entries has mass 0 and never crosses)
          double cum = lo;
          int gi = kG - 1;
          bool gfound = false;
  #pragma unroll
          for (int i = 0; i < kG; ++i) {
            if (!gfound && cum + gsum[i] > T) {
              gi = i;
              gfound = true;
            } else if (!gfound) {
              cum += gsum[i];
            }
          }
          const int v = v_lo + 4 * gi;
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(s_w + widx(v));
          int pick = v_hi - 1;
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (v + e < v_hi) {
              cum += fx40d(w4[e]);
              if (cum > T) {
                pick = v + e;
                break;
              }
            }
          }
          s_pick = pick;
        }
      }
    } else if (t == 0) {  // nothing representable left: the largest entry
      int bi = 0;
      for (int v = 1; v < V; ++v)
        if (s_w[widx(v)] > s_w[widx(bi)]) bi = v;
      s_pick = bi;
    }
  }
  __syncthreads();
  const int bonus = s_pick;

  // ---- path root -> u and the emitted tokens
  for (int k = t; k < N; k += kMssThreads) {
    path[rowN + k] = k < len ? s_path[k] : -1;
    out_tokens[rowN + k] = k + 1 < len ? s_tok[s_path[k + 1]] : (k + 1 == len ? bonus : -1);
  }
  // ---- the commit: row L + j of every kv head takes tree node s_path[j]
  if (commit) {
    if (t < ncopy) {
      kca[dst0] = kx0;
      vca[dst0] = vx0;
    }
    for (int x = t + kMssThreads; x < ncopy; x += kMssThreads) {
      size_t dst;
      const size_t src = copy_src(x, dst);
      const u32x4 kx = ktr[src], vx = vtr[src];
      kca[dst] = kx;
      vca[dst] = vx;
    }
    if (cm.committed_src)
      for (int k = t; k < N; k += kMssThreads) cm.committed_src[rowN + k] = (cok && k < len) ? s_path[k] : -1;
    if (t == 0) cm.cache_len_out[b] = cok ? L + len : L;
  }
  if (t == 0) {
    path_len[b] = len;
    if (dev_status) dev_status[b] = (!commit || cok) ? TTV_OK : TTV_E_SHAPE;
  }
}

hipError_t launch_verify_mss(int B, int N, int V, const int32_t* parents,
                             const int32_t* tokens, const int32_t* n_nodes, const float* llm,
                             const float* ssm, const MssDraws& dr, const LogitRows& lr,
                             int32_t* path, int32_t* path_len, int32_t* out_tokens,
                             int32_t* dev_status, float* gm_w, const CommitArgs& cm,
                             hipStream_t s) {
  const bool lg = lr.st_llm != nullptr;
  // the residual in global memory (host checks: V % 4 == 0, 16-byte rows,
  // gm_w): vocabularies beyond the LDS, and logits rows beyond the
  // prefetching walk's registers
  if (V > kMssMaxVocab || (lg && V > kMssPfMaxVocab)) {
    auto kern = lg ? mss_kernel<true, false, true, true> : mss_kernel<true, false, false, true>;
    hipLaunchKernelGGL(kern, dim3(B), dim3(kMssThreads), 0, s, N, V, parents, tokens, n_nodes,
                       llm, ssm, dr, lr, path, path_len, out_tokens, dev_status, gm_w, cm);
    return hipGetLastError();
  }
  const bool vec = V % 4 == 0 && (reinterpret_cast<uintptr_t>(llm) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(ssm) & 15) == 0;
  // widx(V - 1) + 1, 16-byte padded; the prefetching walk over
  // probabilities keeps its whole span (kMssPfMaxVocab entries) in LDS
  const int Vl = (vec && !lg && V <= kMssPfMaxVocab) ? kMssPfMaxVocab : V;
  const size_t lds = (size_t)(Vl + 4 * (Vl >> 7) + 4) * sizeof(float);
  auto kern = lg ? mss_kernel<true, true, true, false>
                 : (!vec ? mss_kernel<false, false, false, false>
                         : (V <= kMssPfMaxVocab ? mss_kernel<true, true, false, false>
                                                : mss_kernel<true, false, false, false>));
  constexpr int kMaxLds = (kMssMaxVocab + 4 * (kMssMaxVocab >> 7) + 4) * (int)sizeof(float);
  hipError_t e = lds_limit_once(reinterpret_cast<const void*>(kern), kMaxLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(B), dim3(kMssThreads), lds, s, N, V, parents, tokens, n_nodes, llm,
                     ssm, dr, lr, path, path_len, out_tokens, dev_status, nullptr, cm);
  return hipGetLastError();
}

}  // namespace ttv
