// topology.hip -- ttv_tree_topology: ancestor bitsets and depths of every
// request's token tree ([SI] §4 "Tree Attention", "Tree-Based Parallel
// Decoding": the topology-aware causal mask; [SSD] §3 "Implementation": the
// tree also fixes the positions).  One wavefront per request.
#include "launch.h"
#include "ttv_common.h"

namespace ttv {

__global__ __launch_bounds__(64) void topology_kernel(int N, const int32_t* __restrict__ parents,
                                                      uint64_t* __restrict__ anc_out,
                                                      int32_t* __restrict__ depth_out,
                                                      int32_t* __restrict__ dev_status) {
  __shared__ uint64_t s_anc[2 * kMaxNodes];
  __shared__ int32_t s_depth[kMaxNodes];
  const int b = blockIdx.x;
  const int W = (N + 63) / 64;
  const bool ok = wave_build_tree(parents + (size_t)b * N, N, s_anc, s_depth);
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += kWave) {
    if (anc_out) {
      for (int w = 0; w < W; ++w) anc_out[((size_t)b * N + i) * W + w] = ok ? s_anc[2 * i + w] : 0ull;
    }
    if (depth_out) depth_out[(size_t)b * N + i] = ok ? s_depth[i] : -1;
  }
  if (dev_status && threadIdx.x == 0) dev_status[b] = ok ? TTV_OK : TTV_E_TREE;
}

hipError_t launch_topology(int B, int N, const int32_t* parents, uint64_t* anc_out,
                           int32_t* depth_out, int32_t* dev_status, hipStream_t s) {
  hipLaunchKernelGGL(topology_kernel, dim3(B), dim3(kWave), 0, s, N, parents, anc_out,
                     depth_out, dev_status);
  return hipGetLastError();
}

}  // namespace ttv
