// topology.hip -- ttv_tree_topology: ancestor bitsets and depths of every
// request's token tree ([SI] §4 "Tree Attention", "Tree-Based Parallel
// Decoding": the topology-aware causal mask; [SSD] §3 "Implementation": the
// tree also fixes the positions).  One wavefront per request.
#include "launch.h"
#include "ttv_common.h"

namespace ttv {

__global__ __launch_bounds__(64) void topology_kernel(int N, const int32_t* __restrict__ parents,
                                                      const int32_t* __restrict__ n_nodes,
                                                      uint64_t* __restrict__ anc_out,
                                                      int32_t* __restrict__ depth_out,
                                                      int32_t* __restrict__ dev_status) {
  __shared__ uint64_t s_anc[2 * kMaxNodes];
  __shared__ int32_t s_depth[kMaxNodes];
  const int b = blockIdx.x;
  const int W = (N + 63) / 64;
  // the request's nodes: padding nodes past them get no bits and depth -1
  const int n_raw = nodes_raw(n_nodes, b, N);
  const int n = nodes_used(n_raw, N);
  const bool n_ok = nodes_ok(n_raw, N);
  const bool ok = n_ok && wave_build_tree(parents + (size_t)b * N, n, s_anc, s_depth);
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += kWave) {
    const bool real = ok && i < n;
    if (anc_out) {
      for (int w = 0; w < W; ++w) anc_out[((size_t)b * N + i) * W + w] = real ? s_anc[2 * i + w] : 0ull;
    }
    if (depth_out) depth_out[(size_t)b * N + i] = real ? s_depth[i] : -1;
  }
  if (dev_status && threadIdx.x == 0) dev_status[b] = !n_ok ? TTV_E_SHAPE : ok ? TTV_OK : TTV_E_TREE;
}

hipError_t launch_topology(int B, int N, const int32_t* parents, const int32_t* n_nodes,
                           uint64_t* anc_out, int32_t* depth_out, int32_t* dev_status,
                           hipStream_t s) {
  hipLaunchKernelGGL(topology_kernel, dim3(B), dim3(kWave), 0, s, N, parents, n_nodes, anc_out,
                     depth_out, dev_status);
  return hipGetLastError();
}

}  // namespace ttv
