// attn_plan.h -- the balanced split of tree attention, computed on the device
// from the actual prefix lengths (internal; included by the kernels that need
// it).
//
// Every (request b, kv head, row block) owns n_b = ceil(N_b/64) + ceil(L_b/64)
// key tiles (N_b the nodes of its tree): the prefix tiles, then the in-tree
// tiles.  The launched
// workgroups are shared out so that the longest chunk is as short as it can
// be: with s tiles per chunk a unit takes C_b = min(chunks, ceil(n_b / s))
// chunks, and s is the smallest value (at least kBalancedMinTiles) for which
// all chunks fit in the launch.  Work items are numbered request by request,
// then kv head, chunk and row block (row blocks fastest, so that the row
// blocks streaming one chunk are neighbours and share an XCD's L2).  Chunk c
// of a unit covers its tiles [c*n_b/C_b, (c+1)*n_b/C_b).
#pragma once

#include <limits.h>

#include "launch.h"
#include "ttv_common.h"

namespace ttv {

struct PlanItem {
  int b, h, rb, c;  // request, kv head, row block, chunk
  int C;            // chunks of this request's units
  int t0, t1;       // the chunk's tiles
  int nT;           // in-tree tiles of a unit (the last nT of its tiles)
  int L;            // the request's prefix length, clamped to [0, Lmax]
};

__device__ __forceinline__ int plan_wave_sum(int v) { return wave_allsum_i32(v); }

// Work item `item` of the balanced split, computed by one wavefront (every
// wave of a workgroup computes the same values); false when the item is not
// used.  Requires B <= kBalancedMaxB.
__device__ inline bool attn_plan_item(const AttnArgs& a, int item, PlanItem& it) {
  const int lane = threadIdx.x & 63;
  const int U = a.Hkv * a.row_blocks;  // units per request
  int L = 0, n = 0, nT = 0;
  if (lane < a.B) {
    L = min(max(a.cache_len[lane], 0), a.Lmax);
    nT = (nodes_used(nodes_raw(a.n_nodes, lane, a.N), a.N) + 63) / 64;
    n = nT + (L + 63) / 64;
  }
  const long T = (long)U * plan_wave_sum(n);
  const long G = a.items;
  const long fixed = (long)U * a.B;  // one chunk per unit
  auto fits = [&](int s) {
    const int C = lane < a.B ? min(a.chunks, (n + s - 1) / s) : 0;
    return (long)U * plan_wave_sum(C) <= G;
  };
  int s;
  if (G <= fixed) {
    s = INT_MAX / 2;  // one chunk per unit
  } else {
    // fits(hi) holds: sum ceil(n_b/hi) <= T/(U*hi) + B <= G/U
    int lo = (int)max((long)kBalancedMinTiles, (T + G - 1) / G);
    int hi = (int)max((long)lo, (T + (G - fixed) - 1) / (G - fixed));
    while (lo < hi) {
      const int mid = lo + (hi - lo) / 2;
      if (fits(mid)) hi = mid;
      else lo = mid + 1;
    }
    s = lo;
  }
  const int C = lane < a.B ? min(a.chunks, max(1, (n + s - 1) / s)) : 0;
  // inclusive prefix over requests of their work items
  int incl = U * C;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  const uint64_t past = __ballot(lane < a.B && incl > item);
  if (past == 0ull) return false;
  // every result is wave-uniform; readfirstlane tells the compiler so, which
  // keeps the tile bookkeeping that depends on it in scalar registers
  const int b = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)past) - 1);
  it.b = b;
  it.C = __builtin_amdgcn_readfirstlane(__shfl(C, b));
  it.L = __builtin_amdgcn_readfirstlane(__shfl(L, b));
  const int nb = __builtin_amdgcn_readfirstlane(__shfl(n, b));
  const int j = item - __builtin_amdgcn_readfirstlane(__shfl(incl, b) - U * it.C);
  it.rb = j % a.row_blocks;
  it.c = (j / a.row_blocks) % it.C;
  it.h = j / (a.row_blocks * it.C);
  it.t0 = (int)((long)it.c * nb / it.C);
  it.t1 = (int)((long)(it.c + 1) * nb / it.C);
  it.nT = __builtin_amdgcn_readfirstlane(__shfl(nT, b));
  return true;
}

}  // namespace ttv
