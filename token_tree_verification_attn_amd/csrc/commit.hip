// commit.hip -- ttv_kv_commit: append the accepted path's KV rows to the
// contiguous cache ([SI] §4 "Tree-Based Parallel Decoding": verified and
// speculated tokens share one key-value cache; what stays is the accepted
// path).  Rows move in 16-byte vectors, kCommitIlp vectors of K and of V per
// thread in flight at once; the path is read straight from the verifier's
// device output, so no host round trip sits between the two calls.
// With distinct length arrays one workgroup of 256 threads per (request, kv
// head) copies that head's path_len rows: the heads' cache regions lie far
// apart, and spread over CUs their copies and address translations proceed
// in parallel (32 heads x 12 rows: 2.5 us against 3.6 us for one workgroup).
// When cache_len_out is cache_len_in, one workgroup of 1024 threads per
// request copies every head, so entry b is touched by one workgroup only;
// in it thread 0 alone reads cache_len_in[b] and writes cache_len_out[b] =
// L + n, which depends on that read.
#include "launch.h"
#include "ttv_common.h"

namespace ttv {

constexpr int kCommitThreads = 1024;    // one workgroup per request
constexpr int kCommitHeadThreads = 256;  // one workgroup per (request, kv head)
constexpr int kCommitIlp = 4;

__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(
    int row_bytes, int N, int Hkv, int Lcap, int Lmax, const u32x4* __restrict__ k_tree,
    const u32x4* __restrict__ v_tree, u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
    const int32_t* cache_len_in, int32_t* cache_len_out,
    const int32_t* __restrict__ path, const int32_t* __restrict__ path_len,
    int32_t* __restrict__ committed_src, int32_t* __restrict__ dev_status) {
  __shared__ int32_t s_path[kMaxNodes];
  __shared__ int s_bad_node, s_len;
  const int b = blockIdx.x;
  // gridDim.y = Hkv: this workgroup copies head blockIdx.y only; else all.
  // cache_len_out may alias cache_len_in only in the second case: then only
  // this workgroup touches entry b; thread 0 alone reads it (the others take
  // it from LDS) and its write of the new length depends on that read.
  const bool per_head = gridDim.y > 1;
  const int h0 = per_head ? (int)blockIdx.y : 0, nh = per_head ? 1 : Hkv;
  const bool first = blockIdx.y == 0;  // writes the request's lengths and sources
  // lengths and the whole path row are requested together (one round trip)
  const int n = path_len[b];
  const int pj = threadIdx.x < N ? path[(size_t)b * N + threadIdx.x] : -1;
  if (threadIdx.x == 0) {
    s_bad_node = 0;
    s_len = cache_len_in[b];
  }
  __syncthreads();
  const int L = s_len;
  const bool shape_ok = L >= 0 && L <= Lmax && n >= 0 && n <= N && L + n <= Lcap;
  if (threadIdx.x < N) {
    s_path[threadIdx.x] = pj;
    if (shape_ok && threadIdx.x < n && (pj < 0 || pj >= N)) s_bad_node = 1;  // same value from every writer
  }
  __syncthreads();
  const bool ok = shape_ok && s_bad_node == 0;
  if (ok) {
    const int vec = row_bytes / 16;  // 16-byte vectors per row
    const int per_head = n * vec;
    const int total = nh * per_head;
    const int nt = blockDim.x;
    for (int t0 = threadIdx.x; t0 < total; t0 += kCommitIlp * nt) {
      // all loads of this round first, then the stores
      size_t dst[kCommitIlp];
      u32x4 kv[kCommitIlp], vv[kCommitIlp];
#pragma unroll
      for (int u = 0; u < kCommitIlp; ++u) {
        const int t = t0 + u * nt;
        if (t < total) {
          const int h = h0 + t / per_head;
          const int r = t - (h - h0) * per_head;
          const int j = r / vec;
          const int e = r - j * vec;
          const size_t src = (((size_t)b * Hkv + h) * N + s_path[j]) * vec + e;
          dst[u] = (((size_t)b * Hkv + h) * Lcap + (L + j)) * vec + e;
          kv[u] = k_tree[src];
          vv[u] = v_tree[src];
        }
      }
#pragma unroll
      for (int u = 0; u < kCommitIlp; ++u) {
        if (t0 + u * nt < total) {
          k_cache[dst[u]] = kv[u];
          v_cache[dst[u]] = vv[u];
        }
      }
    }
  }
  if (committed_src && first) {
    for (int j = threadIdx.x; j < N; j += blockDim.x)
      committed_src[(size_t)b * N + j] = (ok && j < n) ? s_path[j] : -1;
  }
  __syncthreads();
  if (threadIdx.x == 0 && first) {
    cache_len_out[b] = ok ? L + n : L;
    if (dev_status) dev_status[b] = ok ? TTV_OK : TTV_E_SHAPE;
  }
}

hipError_t launch_kv_commit(int elt, int B, int N, int Hkv, int D, int Lcap,
                            const void* k_tree, const void* v_tree, void* k_cache,
                            void* v_cache, const int32_t* cache_len_in,
                            int32_t* cache_len_out, int Lmax, const int32_t* path,
                            const int32_t* path_len, int32_t* committed_src,
                            int32_t* dev_status, hipStream_t s) {
  const bool per_head = cache_len_out != cache_len_in && Hkv > 1 && Hkv <= 65535;
  const dim3 grid(B, per_head ? Hkv : 1), block(per_head ? kCommitHeadThreads : kCommitThreads);
  hipLaunchKernelGGL(kv_commit_kernel, grid, block, 0, s, D * elt, N, Hkv, Lcap, Lmax,
                     static_cast<const u32x4*>(k_tree), static_cast<const u32x4*>(v_tree),
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), cache_len_in,
                     cache_len_out, path, path_len, committed_src, dev_status);
  return hipGetLastError();
}

// ttv_kv_commit_inplace: the tree's K/V live in the cache after the prefix
// (node i at row L + i); row L + j takes the old row L + path[j].  Sources
// and destinations overlap, so each (request, kv head) first reads its n
// source rows of K and V into LDS, then -- after a barrier -- writes them
// (path entries grow along the path, so only this staging order matters
// when the rows move in parallel).  As above: one workgroup per (request,
// kv head), or one per request over all heads when cache_len_out is
// cache_len_in.
__global__ __launch_bounds__(kCommitHeadThreads) void kv_commit_inplace_kernel(
    int row_bytes, int N, int Hkv, int Lcap, int Lmax, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, const int32_t* cache_len_in, int32_t* cache_len_out,
    const int32_t* __restrict__ path, const int32_t* __restrict__ path_len,
    int32_t* __restrict__ committed_src, int32_t* __restrict__ dev_status) {
  extern __shared__ u32x4 s_rows[];  // [K | V][N rows][vec]
  __shared__ int32_t s_path[kMaxNodes];
  __shared__ int s_bad_node, s_len;
  const int b = blockIdx.x;
  const bool per_head = gridDim.y > 1;
  const int h0 = per_head ? (int)blockIdx.y : 0, nh = per_head ? 1 : Hkv;
  const bool first = blockIdx.y == 0;
  // thread 0 alone reads the prefix length (its write of the new one, which
  // may alias it, depends on that read); the others take it from LDS
  const int n = path_len[b];
  if (threadIdx.x == 0) {
    s_bad_node = 0;
    s_len = cache_len_in[b];
  }
  __syncthreads();
  const int L = s_len;
  const bool shape_ok = L >= 0 && L <= Lmax && n >= 0 && n <= N && (long)L + N <= Lcap;
  for (int j = threadIdx.x; j < N; j += blockDim.x) {
    const int pj = path[(size_t)b * N + j];
    s_path[j] = pj;
    if (shape_ok && j < n && (pj < 0 || pj >= N)) s_bad_node = 1;  // same value from every writer
  }
  __syncthreads();
  const bool ok = shape_ok && s_bad_node == 0;
  if (ok) {
    const int vec = row_bytes / 16;
    const int total = n * vec;
    for (int h = h0; h < h0 + nh; ++h) {
      const size_t base = ((size_t)b * Hkv + h) * Lcap + L;  // row L of this head
      for (int t = threadIdx.x; t < total; t += blockDim.x) {
        const int j = t / vec, e = t - (t / vec) * vec;
        const size_t src = (base + s_path[j]) * vec + e;
        s_rows[t] = k_cache[src];
        s_rows[N * vec + t] = v_cache[src];
      }
      __syncthreads();  // every source row is read before any is written
      for (int t = threadIdx.x; t < total; t += blockDim.x) {
        const int j = t / vec, e = t - (t / vec) * vec;
        const size_t dst = (base + j) * vec + e;
        k_cache[dst] = s_rows[t];
        v_cache[dst] = s_rows[N * vec + t];
      }
      __syncthreads();  // before the next head's rows overwrite the staging area
    }
  }
  if (committed_src && first) {
    for (int j = threadIdx.x; j < N; j += blockDim.x)
      committed_src[(size_t)b * N + j] = (ok && j < n) ? s_path[j] : -1;
  }
  __syncthreads();
  if (threadIdx.x == 0 && first) {
    cache_len_out[b] = ok ? L + n : L;
    if (dev_status) dev_status[b] = ok ? TTV_OK : TTV_E_SHAPE;
  }
}

hipError_t launch_kv_commit_inplace(int elt, int B, int N, int Hkv, int D, int Lcap, void* k_cache,
                                    void* v_cache, const int32_t* cache_len_in,
                                    int32_t* cache_len_out, int Lmax, const int32_t* path,
                                    const int32_t* path_len, int32_t* committed_src,
                                    int32_t* dev_status, hipStream_t s) {
  const bool per_head = cache_len_out != cache_len_in && Hkv > 1 && Hkv <= 65535;
  const size_t lds = (size_t)2 * N * D * elt;  // K and V rows of one head: at most 128 KB
  const dim3 grid(B, per_head ? Hkv : 1);
  // the most any launch takes: 128 rows of 128 fp32 values, K and V
  hipError_t e = lds_limit_once(reinterpret_cast<const void*>(kv_commit_inplace_kernel),
                                2 * TTV_MAX_NODES * 128 * 4);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_commit_inplace_kernel, grid, dim3(kCommitHeadThreads), lds, s, D * elt, N,
                     Hkv, Lcap, Lmax, static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache),
                     cache_len_in, cache_len_out, path, path_len, committed_src, dev_status);
  return hipGetLastError();
}

}  // namespace ttv
