// probs.hip -- next-token probabilities from logits at a temperature,
// optionally over the top-k logits only ([SI] §4 "Token Verification": the
// stochastic verifier takes the LLM's and the speculators' distributions;
// [SSD] §4 samples with top-k, k = 50, at T = 1).
//
// One 1024-thread workgroup per row.  A row of up to 32768 logits is requested
// whole (8 16-byte loads per thread) and kept in registers; a longer one is
// streamed, once per pass.  With top-k, the k-th entry of the row in the
// order (higher logit, then lower token id) is found much as in tree
// expansion: the smallest over the 16 waves of each wave's ceil(k/16)-th
// largest per-thread maximum bounds it from below, the entries at or above
// that bound are gathered in LDS, and the one that exactly k-1
// gathered entries rank before is it (each thread counts for its own
// candidates; a row whose ties overflow the buffer takes k rounds of a
// block arg-max over the whole row instead); an entry is kept iff it ranks at
// or before it.  Then m = the row maximum (always
// kept), s = the sum over kept entries of 2^((z - m) * log2(e) / T), and
// probs = 2^((z - m) * log2(e) / T) / s for kept entries, 0 for the others.
// The row is read once from HBM and written once.
#include <limits.h>

#include "launch.h"
#include "ttv_common.h"

namespace ttv {

namespace {

constexpr int kProbThreads = 1024;  // 512 measured 3.5% slower with top-50
constexpr int kProbWaves = kProbThreads / 64;
constexpr int kProbRegQuads = 8;
constexpr int kProbCandidates = 2048;

__device__ __forceinline__ bool p_ranks_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void p_wave_argmax(float& bv, int& bi) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m);
    const int oi = __shfl_xor(bi, m);
    if (p_ranks_before(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
}

}  // namespace

template <bool VEC>
__global__ __launch_bounds__(kProbThreads) void probs_kernel(int V, float c, int topk,
                                                             const float* __restrict__ logits,
                                                             float* __restrict__ probs) {
  __shared__ float s_red[kProbWaves];
  __shared__ float s_cv[kProbCandidates];
  __shared__ int s_ci[kProbCandidates];
  __shared__ float s_wv[kProbWaves];
  __shared__ int s_wi[kProbWaves];
  __shared__ int s_cnt;
  __shared__ float s_thr;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* row = logits + (size_t)blockIdx.x * V;
  float* out = probs + (size_t)blockIdx.x * V;
  const f32x4* r4 = reinterpret_cast<const f32x4*>(row);
  f32x4* o4 = reinterpret_cast<f32x4*>(out);
  const int n4 = V / 4;
  const bool in_regs = VEC && n4 <= kProbRegQuads * kProbThreads;
  f32x4 rq[kProbRegQuads];
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kProbRegQuads; ++u) {
      const int x = tid + u * kProbThreads;
      rq[u] = x < n4 ? r4[x] : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
  }
  // visit(z, i) for this thread's entries (registers, or the row in memory)
  auto visit_row = [&](auto visit) {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kProbRegQuads; ++u) {
        const int x = tid + u * kProbThreads;
        if (x < n4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) visit(rq[u][e], 4 * x + e);
        }
      }
    } else if (VEC) {
      for (int x = tid; x < n4; x += kProbThreads) {
        const f32x4 q = r4[x];
#pragma unroll
        for (int e = 0; e < 4; ++e) visit(q[e], 4 * x + e);
      }
    } else {
      for (int v = tid; v < V; v += kProbThreads) visit(row[v], v);
    }
  };
  auto block_max = [&](float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    if (lane == 0) s_red[wave] = x;
    __syncthreads();
    float r = s_red[0];
#pragma unroll
    for (int w = 1; w < kProbWaves; ++w) r = fmaxf(r, s_red[w]);
    __syncthreads();
    return r;
  };
  auto block_sum = [&](float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    if (lane == 0) s_red[wave] = x;
    __syncthreads();
    float r = s_red[0];
#pragma unroll
    for (int w = 1; w < kProbWaves; ++w) r += s_red[w];
    __syncthreads();
    return r;
  };

  // ---- the row maximum, from the per-thread maxima
  float tmax = -INFINITY;
  visit_row([&](float z, int) { tmax = fmaxf(tmax, z); });
  const float m = block_max(tmax);

  // ---- top-k: the k-th entry (kv, ki); every entry is kept without top-k
  float kv = -INFINITY;
  int ki = INT_MAX;
  if (topk > 0 && topk < V) {
    // a lower bound of the k-th entry: every wave takes the ceil(k/16)-th
    // largest of its 64 per-thread maxima, and the smallest of those has at
    // least 16*ceil(k/16) >= k entries of the row at or above it
    if (tid == 0) s_cnt = 0;
    {
      const int kw = (topk + kProbWaves - 1) / kProbWaves;
      float a = tmax, wm = -INFINITY;
      for (int r = 0; r < kw; ++r) {  // remove one copy of the wave's largest per round
        wm = a;
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) wm = fmaxf(wm, __shfl_xor(wm, s));
        const uint64_t has = __ballot(a == wm);
        if (lane == __ffsll((unsigned long long)has) - 1) a = -INFINITY;
      }
      if (lane == 0) s_red[wave] = wm;
      __syncthreads();
      if (tid == 0) {
        float t = s_red[0];
#pragma unroll
        for (int w = 1; w < kProbWaves; ++w) t = fminf(t, s_red[w]);
        s_thr = t;
      }
      __syncthreads();
    }
    const float thr = s_thr;
    visit_row([&](float z, int i) {
      if (z >= thr) {
        const int slot = atomicAdd(&s_cnt, 1);
        if (slot < kProbCandidates) {
          s_cv[slot] = z;
          s_ci[slot] = i;
        }
      }
    });
    __syncthreads();
    const int cnt = s_cnt;
    if (cnt <= kProbCandidates) {
      // the gathered pairs are distinct (distinct ids), so their ranks are
      // 0..cnt-1 and exactly one candidate has rank topk-1 (cnt >= topk)
      for (int q = tid; q < cnt; q += kProbThreads) {
        const float z = s_cv[q];
        const int i = s_ci[q];
        int rank = 0;
        for (int u = 0; u < cnt; ++u) rank += p_ranks_before(s_cv[u], s_ci[u], z, i) ? 1 : 0;
        if (rank == topk - 1) {
          s_wv[0] = z;
          s_wi[0] = i;
        }
      }
      __syncthreads();
      kv = s_wv[0];
      ki = s_wi[0];
    } else {
      // too many ties for the buffer: topk rounds over the whole row, each
      // the best entry ranking after the previous winner
      float pv = INFINITY;
      int pi = -1;
      for (int j = 0; j < topk; ++j) {
        float bv = -INFINITY;
        int bi = INT_MAX;
        visit_row([&](float z, int i) {
          if (p_ranks_before(pv, pi, z, i) && p_ranks_before(z, i, bv, bi)) {
            bv = z;
            bi = i;
          }
        });
        p_wave_argmax(bv, bi);
        if (lane == 0) {
          s_wv[wave] = bv;
          s_wi[wave] = bi;
        }
        __syncthreads();
        bv = s_wv[0];
        bi = s_wi[0];
#pragma unroll
        for (int w = 1; w < kProbWaves; ++w)
          if (p_ranks_before(s_wv[w], s_wi[w], bv, bi)) {
            bv = s_wv[w];
            bi = s_wi[w];
          }
        __syncthreads();
        pv = bv;
        pi = bi;
      }
      kv = pv;
      ki = pi;
    }
  }
  auto kept = [&](float z, int i) { return z > kv || (z == kv && i <= ki); };

  // ---- normaliser and probabilities
  float part = 0.f;
  visit_row([&](float z, int i) {
    if (kept(z, i)) part += __builtin_amdgcn_exp2f((z - m) * c);
  });
  const float inv = 1.f / block_sum(part);
  auto prob = [&](float z, int i) { return kept(z, i) ? __builtin_amdgcn_exp2f((z - m) * c) * inv : 0.f; };
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kProbRegQuads; ++u) {
      const int x = tid + u * kProbThreads;
      if (x < n4)
        o4[x] = f32x4{prob(rq[u][0], 4 * x), prob(rq[u][1], 4 * x + 1), prob(rq[u][2], 4 * x + 2),
                      prob(rq[u][3], 4 * x + 3)};
    }
  } else if (VEC) {
    for (int x = tid; x < n4; x += kProbThreads) {
      const f32x4 q = r4[x];
      o4[x] = f32x4{prob(q[0], 4 * x), prob(q[1], 4 * x + 1), prob(q[2], 4 * x + 2), prob(q[3], 4 * x + 3)};
    }
  } else {
    for (int v = tid; v < V; v += kProbThreads) out[v] = prob(row[v], v);
  }
}

hipError_t launch_probs(int R, int V, float T, int topk, const float* logits, float* probs,
                        bool vec, hipStream_t s) {
  const float c = 1.4426950408889634f / T;  // log2(e) / T
  if (vec)
    hipLaunchKernelGGL(probs_kernel<true>, dim3(R), dim3(kProbThreads), 0, s, V, c, topk, logits, probs);
  else
    hipLaunchKernelGGL(probs_kernel<false>, dim3(R), dim3(kProbThreads), 0, s, V, c, topk, logits, probs);
  return hipGetLastError();
}

}  // namespace ttv
