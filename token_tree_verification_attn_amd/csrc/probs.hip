// probs.hip -- next-token probabilities from logits at a temperature, over
// the top-k logits and/or the top-p share of the mass ([SI] §4 "Token
// Verification": the stochastic verifier takes the LLM's and the
// speculators' distributions; §7 "Multi-sample decoding": top-k or top-p
// sampling; [SSD] §4 samples with top-k, k = 50, at T = 1).  The arithmetic
// is fixed to the bit (softmax_exact.h).
//
// One workgroup per row (1024 threads, or 512 with top-k/top-p), two per CU.
// A row of up to 32768 logits is requested whole (8 or 16 16-byte loads per
// thread) and kept in registers (without selection its 2^t values replace
// it; with selection they are formed again where a pass needs them); a
// longer one is streamed, once per pass.
//  * top-k: the k-th entry in the order (higher logit, then lower token id)
//    is found as in tree expansion: the smallest over the W waves of each
//    wave's ceil(k/W)-th largest per-thread maximum bounds it from below,
//    the entries at or above that bound are gathered in LDS, and the one that
//    exactly k-1 gathered entries rank before is it (a row whose ties
//    overflow the buffer takes k rounds of a block arg-max instead).
//  * top-p: with S the exact mass kept by top-k and P = floor(top_p * 2^24),
//    the last kept token is the one where the running mass in that order
//    first reaches ceil(P * S / 2^24).  It is found by histograms of the
//    masses over 2048 equal bins of the logit range (LDS 64-bit atomics;
//    exact integer sums, so any order gives the same bins): the bin where the
//    running mass crosses becomes the next range until it holds at most
//    1024 tokens, which are gathered and ranked in LDS; a range of equal
//    logits (equal masses) is settled by counting token ids.
// Then S' = the kept mass, p = 2^t * (float)(2^40 / S') for kept tokens, 0
// for the others.  The row is read once from HBM and written once; with
// `stats` the kernel writes the row's (max, normaliser, last kept token)
// instead, for a consumer that computes probabilities from the logits itself.
#include <limits.h>

#include "launch.h"
#include "softmax_exact.h"
#include "ttv_common.h"

namespace ttv {

namespace {

// Threads per row: 1024 without selection (8 16-byte loads each); with
// top-k/top-p, 512 (16 loads each) holding the row's logits in 128 VGPRs per
// lane, so that two workgroups share a CU and one's loads and stores overlap
// the other's passes.  (Keeping the exponentials in registers too took 256
// VGPRs and one workgroup per CU: top-50 116 vs 87 us, top-p 0.9 167 vs 129
// us on 1024 x 32000 logits; at 1024 threads it spilled to scratch.)
template <bool SEL>
struct ProbShape {
  static constexpr int kThreads = SEL ? 512 : 1024;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kRegQuads = 32768 / 4 / kThreads;  // rows up to 32768 stay in registers
};
constexpr int kProbMaxWaves = 16;
constexpr int kProbCandidates = 2048;
constexpr int kPBins = 2048;        // top-p histogram bins
constexpr int kPGather = 1024;      // top-p: tokens ranked in LDS at once

__device__ __forceinline__ bool p_ranks_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void p_wave_argmax(float& bv, int& bi) { wave_allargmax(bv, bi); }

// An unsigned key of a logit that orders like the logit (-0 taken as +0, so
// that equal logits have equal keys).
__device__ __forceinline__ uint32_t p_order_key(float z) {
  const uint32_t u = __float_as_uint(z + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}


}  // namespace

// SEL: top-k and/or top-p.  Either way two workgroups share a CU, so one's
// loads are in flight while the other computes.
template <bool VEC, bool SEL>
__global__ __launch_bounds__(ProbShape<SEL>::kThreads) __attribute__((amdgpu_waves_per_eu(SEL ? 4 : 8)))
void probs_kernel(int V, float c, int topk,
                                                             uint32_t top_p24,
                                                             const float* __restrict__ logits,
                                                             float* __restrict__ probs,
                                                             RowStats* __restrict__ stats) {
  constexpr int kProbThreads = ProbShape<SEL>::kThreads;
  constexpr int kProbWaves = ProbShape<SEL>::kWaves;
  constexpr int kProbRegQuads = ProbShape<SEL>::kRegQuads;
  __shared__ float s_red[kProbMaxWaves];
  __shared__ uint64_t s_red64[kProbMaxWaves];
  __shared__ float s_cv[kProbCandidates];
  __shared__ int s_ci[kProbCandidates];
  __shared__ uint64_t s_hist[kPBins];
  __shared__ float s_wv[kProbMaxWaves];
  __shared__ int s_wi[kProbMaxWaves];
  __shared__ int s_cnt, s_bin;
  __shared__ float s_thr, s_zt;
  __shared__ int s_it;
  __shared__ uint64_t s_above, s_need, s_kept;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* row = logits + (size_t)blockIdx.x * V;
  const f32x4* r4 = reinterpret_cast<const f32x4*>(row);
  const int n4 = V / 4;
  const bool in_regs = VEC && n4 <= kProbRegQuads * kProbThreads;
  // the row's logits; without selection their exponentials overwrite them
  // (the logits are not needed again)
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
    x = wave_allmax_f32(x);
    if (lane == 0) s_red[wave] = x;
    __syncthreads();
    float r = s_red[0];
#pragma unroll
    for (int w = 1; w < kProbWaves; ++w) r = fmaxf(r, s_red[w]);
    __syncthreads();
    return r;
  };
  auto block_min = [&](float x) { return -block_max(-x); };
  auto block_sum_u64 = [&](uint64_t x) {
    x = wave_allsum_u64(x);
    if (lane == 0) s_red64[wave] = x;
    __syncthreads();
    uint64_t r = 0;
#pragma unroll
    for (int w = 0; w < kProbWaves; ++w) r += s_red64[w];
    __syncthreads();
    return r;
  };

  // ---- the row maximum, from the per-thread maxima (and the per-thread
  // minima, which top-p without top-k starts its range from)
  float tmax = -INFINITY, tmin = INFINITY;
  visit_row([&](float z, int) {
    tmax = fmaxf(tmax, z);
    tmin = fminf(tmin, z);
  });
  const float m = block_max(tmax);
  const bool use_topk = SEL && topk > 0 && topk < V;
  const bool use_topp = SEL && top_p24 > 0u && top_p24 < (1u << 24);
  // without selection: 2^t of every entry, in place of its logit
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kProbRegQuads; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) if constexpr (!SEL) rq[u][e] = exp2_taylor((rq[u][e] - m) * c);
  }
  // Per-entry values that a loop over passes would otherwise hoist out of
  // it (order keys, exponentials, 64-bit masses: registers per entry, which
  // spilled)
  // are kept inside by declaring the row's registers rewritten (no code).
  auto pin_row = [&]() {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kProbRegQuads; ++u) asm volatile("" : "+v"(rq[u]));
    }
  };
  // visit(z, 2^t, i) for this thread's entries (with selection 2^t is
  // formed here, from the logit and the row maximum)
  auto visit_ze = [&](auto visit) {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kProbRegQuads; ++u) {
        const int x = tid + u * kProbThreads;
        if (x < n4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (SEL) visit(rq[u][e], exp2_taylor((rq[u][e] - m) * c), 4 * x + e);
            else visit(rq[u][e], rq[u][e], 4 * x + e);
          }
        }
      }
    } else {
      visit_row([&](float z, int i) { visit(z, exp2_taylor((z - m) * c), i); });
    }
  };

  // the kept mass S', when a selection step has it (else summed at the end)
  bool have_kept = false;
  uint64_t kept_mass = 0;

  // ---- top-k: the k-th entry (kv, ki); every entry is kept without top-k
  float kv = -INFINITY;
  int ki = INT_MAX;
  if (use_topk) {
    // a lower bound of the k-th entry: every wave takes the ceil(k/W)-th
    // largest of its 64 per-thread maxima (W waves), and the smallest of
    // those has at least W*ceil(k/W) >= k entries of the row at or above it
    if (tid == 0) s_cnt = 0;
    {
      const int kw = (topk + kProbWaves - 1) / kProbWaves;
      float a = tmax, wm = -INFINITY;
      for (int r = 0; r < kw; ++r) {  // remove one copy of the wave's largest per round
        wm = wave_allmax_f32(a);
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
    // (without top-p the kept mass is summed from the candidates' masses;
    // top-p finds its own)
    const bool sum_kept = !use_topp;
    if (sum_kept) {
      visit_ze([&](float z, float e, int i) {
        if (z >= thr) {
          const int slot = atomicAdd(&s_cnt, 1);
          if (slot < kProbCandidates) {
            s_cv[slot] = z;
            s_ci[slot] = i;
            s_hist[slot] = (uint64_t)mass40(e);
          }
        }
      });
    } else {
      visit_row([&](float z, int i) {
        if (z >= thr) {
          const int slot = atomicAdd(&s_cnt, 1);
          if (slot < kProbCandidates) {
            s_cv[slot] = z;
            s_ci[slot] = i;
          }
        }
      });
    }
    __syncthreads();
    const int cnt = s_cnt;
    if (cnt <= kProbCandidates) {
      // the gathered pairs are distinct (distinct ids), so their ranks are
      // 0..cnt-1 and exactly one candidate has rank topk-1 (cnt >= topk)
      // (wave w ranks candidates w, w + W, ...; its lanes compare one with
      // every 64th of the others, and a register-only wave sum counts)
      // The kept tokens are exactly the candidates of rank < topk: their
      // masses, summed per wave and then over the waves, are the kept mass.
      uint64_t kmass = 0;
      for (int q = wave; q < cnt; q += kProbWaves) {
        const float z = s_cv[q];
        const int i = s_ci[q];
        int rank = 0;
        for (int u = lane; u < cnt; u += 64) rank += p_ranks_before(s_cv[u], s_ci[u], z, i) ? 1 : 0;
        rank = wave_allsum_i32(rank);
        if (rank == topk - 1 && lane == 0) {
          s_wv[0] = z;
          s_wi[0] = i;
        }
        if (sum_kept && rank < topk) kmass += s_hist[q];
      }
      if (lane == 0) s_red64[wave] = kmass;
      __syncthreads();
      if (sum_kept) {
        kept_mass = 0;
#pragma unroll
        for (int w = 0; w < kProbWaves; ++w) kept_mass += s_red64[w];
        have_kept = true;
      }
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
    __syncthreads();  // s_wv / s_cnt are reused below
  }
  auto kept_k = [&](float z, int i) { return z > kv || (z == kv && i <= ki); };
  float zthr = kv;
  int ithr = ki;

  // ---- top-p: the token where the running mass reaches ceil(P*S/2^24),
  // S the kept mass (taken from the first histogram, which holds every kept
  // token); the running mass there is the kept mass S' the probabilities
  // are normalised by
  const float row_min = use_topp && !use_topk ? block_min(tmin) : 0.f;
  if (use_topp) {
    // the candidate range of logits (all kept_k tokens in it): from the
    // smallest kept logit (the k-th with top-k) to the maximum
    float lo = use_topk ? kv : row_min, hi = m;
    uint64_t above = 0;  // the mass of the tokens ranking before the range
    uint64_t need = 0;   // ceil(P * S / 2^24), known after the first histogram
    for (int it = 0; it < 64; ++it) {
      pin_row();
      if (it > 0 && lo == hi) {
        // every candidate has the logit lo, hence the same mass mu: the
        // crossing is the c-th lowest token id among them, c = ceil((need -
        // above) / mu); binary search on the id
        const uint64_t mu = (uint64_t)mass40(exp2_taylor((lo - m) * c));
        const uint64_t cneed = mu > 0 ? (need - above + mu - 1) / mu : 1;
        int a = 0, b = V - 1;  // the smallest id x with count(id <= x) >= cneed
        while (a < b) {
          const int mid = a + (b - a) / 2;
          double n = 0.0;
          visit_row([&](float z, int i) { n += (z == lo && kept_k(z, i) && i <= mid) ? 1.0 : 0.0; });
          const uint64_t cnt = block_sum_u64((uint64_t)n);
          if (cnt >= cneed) b = mid;
          else a = mid + 1;
        }
        zthr = lo;
        ithr = a;
        kept_mass = above + cneed * mu;  // the range's first cneed tokens, mass mu each
        have_kept = true;
        break;
      }
      // histogram of the candidates' masses over 2048 bins, higher logits
      // first: bins of equal width in logit value (or, for a range too
      // narrow for that in fp32, in the logits' order keys); any monotone
      // map keeps each bin a range of logits
      const float scv = (float)kPBins / (hi - lo);
      const bool linear = (hi - lo) >= 1e-30f && scv <= 3.0e38f;
      const uint32_t khi = p_order_key(hi);
      const float sck = (float)kPBins / ((float)(khi - p_order_key(lo)) + 1.0f);
      auto bin_of = [&](float z) {
        const float x = linear ? (hi - z) * scv : (float)(khi - p_order_key(z)) * sck;
        return min(kPBins - 1, (int)x);
      };
      if (tid == 0) s_cnt = 0;  // the gather's counter (last read before a barrier)
      for (int b = tid; b < kPBins; b += kProbThreads) s_hist[b] = 0ull;
      __syncthreads();
      visit_ze([&](float z, float e, int i) {
        if (z >= lo && z <= hi && kept_k(z, i))
          atomicAdd(reinterpret_cast<unsigned long long*>(&s_hist[bin_of(z)]),
                    (unsigned long long)mass40(e));
      });
      __syncthreads();
      if (wave == 0) {  // lane l scans bins 32l .. 32l+31
        uint64_t loc = 0;
        for (int k = 0; k < kPBins / 64; ++k) loc += s_hist[lane * (kPBins / 64) + k];
        uint64_t incl = loc;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const uint64_t o = ((uint64_t)(uint32_t)__shfl_up((int)(incl >> 32), d) << 32) |
                             (uint32_t)__shfl_up((int)(uint32_t)incl, d);
          if (lane >= d) incl += o;
        }
        const uint64_t excl = incl - loc;
        if (it == 0) {  // every kept token is in this histogram: S is its total
          const uint64_t S = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(incl >> 32), 63) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)incl, 63);
          // need = ceil(P * S / 2^24) with S = hi*2^24 + lo split (no overflow)
          need = (uint64_t)top_p24 * (S >> 24) +
                 (((uint64_t)top_p24 * (S & 0xffffffull) + 0xffffffull) >> 24);
          if (lane == 0) s_need = need;
        }
        const uint64_t first = __ballot(above + incl >= need);
        const int L = first ? __ffsll((unsigned long long)first) - 1 : 63;
        if (lane == L) {
          uint64_t run = above + excl;
          int b = lane * (kPBins / 64);
          for (int k = 0; k < kPBins / 64; ++k) {
            const uint64_t h = s_hist[lane * (kPBins / 64) + k];
            if (run + h >= need || k == kPBins / 64 - 1) {
              b = lane * (kPBins / 64) + k;
              break;
            }
            run += h;
          }
          s_bin = b;
          s_above = run;
        }
      }
      __syncthreads();
      const int bsel = s_bin;
      above = s_above;
      need = s_need;
      // gather the crossing bin's tokens into LDS (at most kPGather of them;
      // the counter counts them all) and rank them there: the crossing token
      // is the one whose running mass (above + the tokens ranking before it,
      // itself included) first reaches need
      visit_ze([&](float z, float e, int i) {
        if (z >= lo && z <= hi && kept_k(z, i) && bin_of(z) == bsel) {
          const int slot = atomicAdd(&s_cnt, 1);
          if (slot < kPGather) {
            s_cv[slot] = z;
            s_ci[slot] = i;
            s_hist[slot] = (uint64_t)mass40(e);
          }
        }
      });
      __syncthreads();
      const int nc = s_cnt;
      if (nc <= kPGather) {
        for (int q = tid; q < nc; q += kProbThreads) {
          const float z = s_cv[q];
          const int i = s_ci[q];
          uint64_t before = 0;
          for (int u = 0; u < nc; ++u)
            if (p_ranks_before(s_cv[u], s_ci[u], z, i)) before += s_hist[u];
          if (above + before < need && above + before + s_hist[q] >= need) {
            s_zt = z;
            s_it = i;
            s_kept = above + before + s_hist[q];
          }
        }
        __syncthreads();
        zthr = s_zt;
        ithr = s_it;
        kept_mass = s_kept;
        have_kept = true;
        break;
      }
      // too many: the next range is the crossing bin (its members are
      // exactly the kept tokens with logits in [nlo, nhi])
      float bmin = INFINITY, bmax = -INFINITY;
      visit_row([&](float z, int i) {
        if (z >= lo && z <= hi && kept_k(z, i) && bin_of(z) == bsel) {
          bmin = fminf(bmin, z);
          bmax = fmaxf(bmax, z);
        }
      });
      const float nlo = block_min(bmin), nhi = block_max(bmax);
      lo = nlo;
      hi = nhi;
    }
  }

  // ---- normaliser and probabilities (or the row's statistics)
  auto kept = [&](float z, int i) { return !SEL || z > zthr || (z == zthr && i <= ithr); };
  uint64_t S = kept_mass;
  if (!have_kept) {
    double part = 0.0;  // at most 64 masses below 2^40 each per thread: exact
    visit_ze([&](float z, float e, int i) {
      if (kept(z, i)) part += mass40(e);
    });
    S = block_sum_u64((uint64_t)part);
  }
  const float inv = (float)(1099511627776.0 / (double)S);
  if (stats) {
    if (tid == 0) stats[blockIdx.x] = RowStats{m, inv, zthr, ithr};
    return;
  }
  float* out = probs + (size_t)blockIdx.x * V;
  f32x4* o4 = reinterpret_cast<f32x4*>(out);
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kProbRegQuads; ++u) {
      const int x = tid + u * kProbThreads;
      if (x < n4) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (SEL) o[e] = kept(rq[u][e], 4 * x + e) ? exp2_taylor((rq[u][e] - m) * c) * inv : 0.f;
          else o[e] = rq[u][e] * inv;
        }
        o4[x] = o;
      }
    }
  } else {
    const RowStats rs{m, inv, zthr, ithr};
    if (VEC) {
      for (int x = tid; x < n4; x += kProbThreads) {
        const f32x4 q = r4[x];
        o4[x] = f32x4{row_prob(rs, c, q[0], 4 * x), row_prob(rs, c, q[1], 4 * x + 1),
                      row_prob(rs, c, q[2], 4 * x + 2), row_prob(rs, c, q[3], 4 * x + 3)};
      }
    } else {
      for (int v = tid; v < V; v += kProbThreads) out[v] = row_prob(rs, c, row[v], v);
    }
  }
}

float probs_scale(float T) { return (float)(kLog2Ed / (double)T); }

uint32_t probs_top_p24(float top_p) {
  return top_p > 0.f && top_p < 1.f ? (uint32_t)(top_p * 16777216.0f) : 0u;
}

hipError_t launch_probs(int R, int V, float T, int topk, float top_p, const float* logits,
                        float* probs, RowStats* stats, bool vec, hipStream_t s) {
  const float c = probs_scale(T);
  const uint32_t p24 = probs_top_p24(top_p);
  const bool sel = (topk > 0 && topk < V) || p24 != 0u;
  auto kern = vec ? (sel ? probs_kernel<true, true> : probs_kernel<true, false>)
                  : (sel ? probs_kernel<false, true> : probs_kernel<false, false>);
  const int threads = sel ? ProbShape<true>::kThreads : ProbShape<false>::kThreads;
  hipLaunchKernelGGL(kern, dim3(R), dim3(threads), 0, s, V, c, topk, p24, logits, probs, stats);
  return hipGetLastError();
}

}  // namespace ttv
