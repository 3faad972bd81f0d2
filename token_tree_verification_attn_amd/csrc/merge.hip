// merge.hip -- merge-based token-tree construction ([SI] §3 "Merge-based
// token tree construction": the outputs of several speculative models are
// combined into one tree that contains each of their token sequences).
//
// One workgroup per request.  Its threads copy the request's S <= 64
// sequences into LDS (one coalesced pass), then wave 0 builds the tree depth
// by depth with lane s holding sequence s.  Two sequences share their node at
// depth d iff they share it at depth d-1 and have the same token at position
// d-1, so a lane's node is new exactly when no lower lane whose sequence
// reaches depth d has the same (node at d-1, token) key; the lanes' keys are
// compared by reading each lower lane's key with readlane (S steps, uniform).
// New nodes take consecutive ids in lane order (ballot and popcount), the
// other lanes take their leader's id by a shuffle.  When 1 + sum(len) could
// exceed the capacity, a first pass only counts the nodes, so that a request
// that does not fit gets nothing written.
#include "launch.h"
#include "ttv_common.h"

namespace ttv {

namespace {
constexpr int kMergeThreads = 256;
}  // namespace

__global__ __launch_bounds__(kMergeThreads) void tree_merge_kernel(
    int S, int Ls, const int32_t* __restrict__ seqs, const int32_t* __restrict__ seq_len,
    const int32_t* __restrict__ root_tok, int Ncap, int32_t* __restrict__ parents,
    int32_t* __restrict__ tokens, int32_t* __restrict__ src, int32_t* __restrict__ n_out,
    int32_t* __restrict__ dev_status) {
  __shared__ int32_t s_tok[kMergeMaxSeqs * kMergeMaxLen];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int32_t* sq = seqs + (size_t)b * S * Ls;
  for (int i = tid; i < S * Ls; i += kMergeThreads) s_tok[i] = sq[i];
  const int len = lane < S ? seq_len[(size_t)b * S + lane] : 0;
  __syncthreads();
  if (tid >= 64) return;

  const bool bad = __ballot(lane < S && (len < 0 || len > Ls)) != 0ull;
  int maxlen = bad ? 0 : len, total = bad ? 0 : len;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    maxlen = max(maxlen, __shfl_xor(maxlen, m));
    total += __shfl_xor(total, m);
  }
  const size_t base = (size_t)b * Ncap;

  // one pass over the depths; returns the node count, writes the nodes if asked
  auto build = [&](bool write) {
    int node = 0, next = 1;
    for (int d = 1; d <= maxlen; ++d) {
      const bool act = lane < S && len >= d;
      const int t = act ? s_tok[lane * Ls + d - 1] : 0;
      const uint32_t klo = (uint32_t)t, khi = (uint32_t)node;
      const uint64_t actm = __ballot(act);
      int lead = lane;
      for (int j = 0; j < S; ++j) {  // lower lanes whose sequences reach depth d
        const uint32_t jlo = (uint32_t)__builtin_amdgcn_readlane((int)klo, j);
        const uint32_t jhi = (uint32_t)__builtin_amdgcn_readlane((int)khi, j);
        if (j < lead && ((actm >> j) & 1ull) && jlo == klo && jhi == khi) lead = j;
      }
      const bool is_lead = act && lead == lane;
      const uint64_t L = __ballot(is_lead);
      const int my_id = next + __popcll(L & ((1ull << lane) - 1ull));
      const int lead_id = __shfl(my_id, lead);
      if (write && is_lead) {
        parents[base + my_id] = node;
        tokens[base + my_id] = t;
        if (src) src[base + my_id] = lane * Ls + d - 1;
      }
      if (act) node = lead_id;
      next += __popcll(L);
    }
    return next;
  };
  bool ok = !bad;
  if (ok && 1 + total > Ncap) ok = build(false) <= Ncap;
  const int n = ok ? build(true) : 0;
  if (lane == 0) {
    if (ok) {
      parents[base] = -1;
      tokens[base] = root_tok[b];
      if (src) src[base] = -1;
    }
    n_out[b] = n;
    if (dev_status) dev_status[b] = ok ? TTV_OK : TTV_E_SHAPE;
  }
}

hipError_t launch_tree_merge(int B, int S, int Ls, const int32_t* seqs, const int32_t* seq_len,
                             const int32_t* root_tok, int Ncap, int32_t* parents, int32_t* tokens,
                             int32_t* src, int32_t* n_out, int32_t* dev_status, hipStream_t s) {
  hipLaunchKernelGGL(tree_merge_kernel, dim3(B), dim3(kMergeThreads), 0, s, S, Ls, seqs, seq_len,
                     root_tok, Ncap, parents, tokens, src, n_out, dev_status);
  return hipGetLastError();
}

}  // namespace ttv
