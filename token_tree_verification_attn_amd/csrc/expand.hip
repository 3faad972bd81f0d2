// expand.hip -- one level of expansion-based token-tree construction ([SI]
// §3 "Expansion-based token tree construction": the top-k tokens of a
// speculative model at a node become that node's children).
//
// One 512-thread workgroup per (request b, frontier entry f), in three steps:
//   1. read the row once for each thread's maximum; T, a lower bound of the
//      row's k-th largest probability, is the k-th largest of the 8 wave
//      maxima (k <= 8) or of the 512 thread maxima.  A row of up to 32768 entries is requested whole at the
//      start (16 16-byte loads per thread, right after the frontier's, so
//      the frontier check does not wait for them) and stays in registers;
//      a longer one is streamed (8 loads in flight per thread);
//   2. gather the entries >= T into an LDS buffer (usually only a little
//      more than k of them), from the registers (a ballot per entry, in the
//      waves that hold any) or by reading the row again (then from L2);
//   3. wave 0 takes the k best of the buffer by k rounds of a wave arg-max,
//      each over the entries that rank after the previous winner (higher
//      probability first, then the lower token id), so the order is exact
//      and no entry needs marking.
// A row with so many entries equal to T that they overflow the buffer (rows
// of equal probabilities) takes the same k rounds over the whole row
// instead, each a block-wide arg-max.  Every workgroup of a request reads the
// request's whole frontier (at most 128 entries) to find the request's
// validity and its own rank among the entries >= 0, so no workgroup waits
// for another.
#include <limits.h>

#include "launch.h"
#include "ttv_common.h"

namespace ttv {

namespace {

constexpr int kExpandThreads = 512;
constexpr int kExpandWaves = kExpandThreads / 64;
constexpr int kExpandCandidates = 2048;  // LDS buffer of step 2
constexpr int kExpandRegQuads = 16;      // 16-byte loads per thread of a row kept in registers

// (v, i) ranks before (bv, bi): higher probability, then the lower token id
__device__ __forceinline__ bool ranks_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_argmax(float& bv, int& bi) { wave_allargmax(bv, bi); }

}  // namespace

template <bool VEC>
__global__ __launch_bounds__(kExpandThreads) void tree_expand_kernel(
    int F, int V, int k, const float* __restrict__ probs, const int32_t* __restrict__ frontier,
    const int32_t* __restrict__ n_in, int Ncap, int32_t* __restrict__ parents,
    int32_t* __restrict__ tokens, int32_t* __restrict__ src_row, int32_t* __restrict__ n_out,
    int32_t* __restrict__ dev_status) {
  __shared__ float s_max[kExpandThreads];
  __shared__ float s_cv[kExpandCandidates];
  __shared__ int s_ci[kExpandCandidates];
  __shared__ float s_wv[kExpandWaves];
  __shared__ float s_wm[kExpandWaves];
  __shared__ int s_wi[kExpandWaves];
  __shared__ int s_cnt;
  __shared__ float s_thr;
  const int f = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- the frontier (requested first), then the whole row when it fits
  const int nin = n_in[b];
  const int32_t* fb = frontier + (size_t)b * F;
  const int fr = fb[f];
  int fj[TTV_MAX_NODES / 64];
#pragma unroll
  for (int u = 0; u < TTV_MAX_NODES / 64; ++u) fj[u] = u * 64 + lane < F ? fb[u * 64 + lane] : -1;
  const float* row = probs + ((size_t)b * F + f) * V;
  const f32x4* r4 = reinterpret_cast<const f32x4*>(row);
  const int n4 = V / 4;
  const bool in_regs = VEC && n4 <= kExpandRegQuads * kExpandThreads;
  f32x4 rq[kExpandRegQuads];
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kExpandRegQuads; ++u) {
      const int x = tid + u * kExpandThreads;
      rq[u] = x < n4 ? r4[x] : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
  }

  // visit(v, i) for every entry of this thread's share of the row, from
  // memory (the row is read again if it was read before)
  auto stream = [&](auto visit) {
    if (VEC) {
      for (int q0 = tid; q0 < n4; q0 += 8 * kExpandThreads) {
        f32x4 q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int x = q0 + u * kExpandThreads;
          q[u] = x < n4 ? r4[x] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int x = q0 + u * kExpandThreads;
          if (x < n4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) visit(q[u][e], 4 * x + e);
          }
        }
      }
    } else {
      for (int v = tid; v < V; v += kExpandThreads) visit(row[v], v);
    }
  };

  // the row's entries of this thread: from the registers when it fits
  auto visit_row = [&](auto visit) {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kExpandRegQuads; ++u) {
        const int x = tid + u * kExpandThreads;
        if (x < n4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) visit(rq[u][e], 4 * x + e);
        }
      }
    } else {
      stream(visit);
    }
  };

  // ---- 1. per-thread maxima and their k-th largest, T
  float tmax = -INFINITY;
  visit_row([&](float v, int) { tmax = fmaxf(tmax, v); });

  // ---- the request's validity, entry count and this entry's rank
  int count = 0, rank = 0;
  bool bad = false;
#pragma unroll
  for (int u = 0; u < TTV_MAX_NODES / 64; ++u) {
    const int j0 = u * 64;
    const int e = fj[u];
    bad |= e < -1 || e >= nin;
    const uint64_t m = __ballot(e >= 0);
    count += __popcll(m);
    if (f >= j0) rank += __popcll(f - j0 >= 64 ? m : (m & ((1ull << (f - j0)) - 1ull)));
  }
  bad = __ballot(bad) != 0ull;
  const int st = bad ? TTV_E_TREE
                     : (nin < 1 || (long)nin + (long)count * k > Ncap ? TTV_E_SHAPE : TTV_OK);
  if (f == 0 && tid == 0) {
    n_out[b] = st == TTV_OK ? nin + count * k : nin;
    if (dev_status) dev_status[b] = st;
  }
  // An entry with nothing to expand still runs through (the same for the
  // whole workgroup) and only skips its writes: an early return here would
  // let the compiler move the row's loads behind the frontier check.
  const bool active = st == TTV_OK && fr >= 0;

  // ---- T.  k <= 8: the k-th largest of the 8 wave maxima (k distinct
  // entries of the row are >= it, so the row's k best are too), found by
  // every thread after one barrier.  Larger k: the k-th largest of the 512
  // thread maxima, found by wave 0 (k rounds, each removing one copy of the
  // largest) and handed over through LDS.
  const float wmax = wave_allmax_f32(tmax);
  if (lane == 0) s_wm[wave] = wmax;
  s_max[tid] = tmax;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  float thr = -INFINITY;
  if (k <= kExpandWaves) {
    float a[kExpandWaves];
#pragma unroll
    for (int w = 0; w < kExpandWaves; ++w) a[w] = s_wm[w];
    for (int r = 0; r < k; ++r) {
      float m = a[0];
#pragma unroll
      for (int w = 1; w < kExpandWaves; ++w) m = fmaxf(m, a[w]);
      bool done = false;
#pragma unroll
      for (int w = 0; w < kExpandWaves; ++w)
        if (!done && a[w] == m) {
          a[w] = -INFINITY;
          done = true;
        }
      thr = m;
    }
  } else {
    if (wave == 0) {
      constexpr int PER = kExpandThreads / 64;
      float a[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) a[j] = s_max[j * 64 + lane];
      float t = -INFINITY;
      for (int r = 0; r < k; ++r) {
        float lm = a[0];
#pragma unroll
        for (int j = 1; j < PER; ++j) lm = fmaxf(lm, a[j]);
        const float wm = wave_allmax_f32(lm);
        const uint64_t has = __ballot(lm == wm);
        if (lane == __ffsll((unsigned long long)has) - 1) {
          bool done = false;
#pragma unroll
          for (int j = 0; j < PER; ++j)
            if (!done && a[j] == wm) {
              a[j] = -INFINITY;
              done = true;
            }
        }
        t = wm;
      }
      if (lane == 0) s_thr = t;
    }
    __syncthreads();
    thr = s_thr;
  }

  // ---- 2. the entries >= T.  From the registers, a wave whose threads'
  // maxima are all below T has none; the others test their entries with a
  // ballot each, and the wave takes the slots of an entry's hits with one
  // LDS atomic (entries >= T are few: usually a little more than k).
  if (in_regs) {
    if (__ballot(tmax >= thr) != 0ull) {
      const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
      for (int u = 0; u < kExpandRegQuads; ++u) {
        const int x = tid + u * kExpandThreads;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool hit = x < n4 && rq[u][e] >= thr;
          const uint64_t m = __ballot(hit);
          if (m != 0ull) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&s_cnt, __popcll(m));
            base = __builtin_amdgcn_readfirstlane(base);
            const int slot = base + __popcll(m & below);
            if (hit && slot < kExpandCandidates) {
              s_cv[slot] = rq[u][e];
              s_ci[slot] = 4 * x + e;
            }
          }
        }
      }
    }
  } else {
    stream([&](float v, int i) {
      if (v >= thr) {
        const int slot = atomicAdd(&s_cnt, 1);
        if (slot < kExpandCandidates) {
          s_cv[slot] = v;
          s_ci[slot] = i;
        }
      }
    });
  }
  __syncthreads();
  const int cnt = s_cnt;

  // ---- 3. k rounds, each the best entry ranking after the previous winner
  const size_t base = (size_t)b * Ncap + nin + (size_t)rank * k;
  float pv = INFINITY;
  int pi = -1;
  if (cnt <= kExpandCandidates) {
    if (wave != 0) return;
    // the first 64 candidates stay in registers across the rounds
    const float cv0 = lane < cnt ? s_cv[lane] : -INFINITY;
    const int ci0 = lane < cnt ? s_ci[lane] : INT_MAX;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = INT_MAX;
      if (lane < cnt && ranks_before(pv, pi, cv0, ci0)) {
        bv = cv0;
        bi = ci0;
      }
      for (int c = lane + 64; c < cnt; c += 64) {
        const float v = s_cv[c];
        const int i = s_ci[c];
        if (ranks_before(pv, pi, v, i) && ranks_before(v, i, bv, bi)) {
          bv = v;
          bi = i;
        }
      }
      wave_argmax(bv, bi);
      if (lane == 0 && active) {
        parents[base + j] = fr;
        tokens[base + j] = bi;
        if (src_row) src_row[base + j] = f;
      }
      pv = bv;
      pi = bi;
    }
    return;
  }
  for (int j = 0; j < k; ++j) {  // too many ties for the buffer: the whole row
    float bv = -INFINITY;
    int bi = INT_MAX;
    stream([&](float v, int i) {
      if (ranks_before(pv, pi, v, i) && ranks_before(v, i, bv, bi)) {
        bv = v;
        bi = i;
      }
    });
    wave_argmax(bv, bi);
    if (lane == 0) {
      s_wv[wave] = bv;
      s_wi[wave] = bi;
    }
    __syncthreads();
    bv = s_wv[0];
    bi = s_wi[0];
#pragma unroll
    for (int w = 1; w < kExpandWaves; ++w)
      if (ranks_before(s_wv[w], s_wi[w], bv, bi)) {
        bv = s_wv[w];
        bi = s_wi[w];
      }
    __syncthreads();  // every thread has read s_wv before the next round writes it
    if (tid == 0 && active) {
      parents[base + j] = fr;
      tokens[base + j] = bi;
      if (src_row) src_row[base + j] = f;
    }
    pv = bv;
    pi = bi;
  }
}

hipError_t launch_tree_expand(int B, int F, int V, int k, const float* probs,
                              const int32_t* frontier, const int32_t* n_in, int Ncap,
                              int32_t* parents, int32_t* tokens, int32_t* src_row,
                              int32_t* n_out, int32_t* dev_status, bool vec, hipStream_t s) {
  const dim3 grid(F, B);
  if (vec)
    hipLaunchKernelGGL(tree_expand_kernel<true>, grid, dim3(kExpandThreads), 0, s, F, V, k, probs,
                       frontier, n_in, Ncap, parents, tokens, src_row, n_out, dev_status);
  else
    hipLaunchKernelGGL(tree_expand_kernel<false>, grid, dim3(kExpandThreads), 0, s, F, V, k, probs,
                       frontier, n_in, Ncap, parents, tokens, src_row, n_out, dev_status);
  return hipGetLastError();
}

}  // namespace ttv
