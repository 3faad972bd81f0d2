// attn.hip -- ttv_tree_attn kernels.
//
// Tree attention ([SI] §4 "Tree Attention", "Tree-Based Parallel Decoding"):
// every tree node's query attends, in one launch, to its request's prefix KV
// and to the tree-KV rows of the nodes on its root path (the topology-aware
// causal mask).  As in [SSD] §3 "Implementation", the keys split into a cache
// part (rows 0..L_b-1 of k/v_cache, unmasked) and an in-tree part (k/v_tree,
// masked by the ancestor bitset); both feed one online softmax.
//
// This file holds the FMA path (fp32, or bf16 with fewer than 16 query rows
// per kv head) and the split-KV combine; the matrix-core path is in
// attn_mfma.hip.  Work decomposition (one workgroup = 4 wavefronts):
//   blockIdx.z = b * Hkv + h          request and kv head
//   blockIdx.y = row block            query rows r = i * G + g (node i, head
//                                     g of the GQA group) packed together, so
//                                     every KV tile staged in LDS serves all
//                                     N*G rows of the group
//   blockIdx.x = KV chunk             prefix keys [c*chunk, (c+1)*chunk); chunk 0
//                                     also takes the tree keys
// With one chunk the workgroup writes the normalised output directly;
// otherwise it writes fp32 partials (unnormalised output, running max, sum)
// and attn_combine_kernel merges them by log-sum-exp.
//
// Scores are kept in log2 units (q.k * scale * log2 e) so the exponentials
// are single v_exp_f32 instructions.
#include "launch.h"
#include "ttv_common.h"

namespace ttv {

constexpr float kLn2 = 0.693147180559945309f;
constexpr int kKeysPerTile = 64;

// Status of request b as every kernel of the call sees it (n_raw its node
// count as given).
__device__ __forceinline__ int request_status(bool tree_ok, int L, int Lmax, int n_raw, int N) {
  if (!nodes_ok(n_raw, N)) return TTV_E_SHAPE;
  if (!tree_ok) return TTV_E_TREE;
  if (L < 0 || L > Lmax) return TTV_E_SHAPE;
  return TTV_OK;
}

template <typename T>
__device__ __forceinline__ float load_elt(const T* p);
template <>
__device__ __forceinline__ float load_elt<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elt<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void store_elt(T* p, float v);
template <>
__device__ __forceinline__ void store_elt<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_elt<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

// =========================================================================
// FMA path: fp32 inputs, or bf16 with fewer than 16 query rows per kv head.
// Each wavefront owns up to 4 query rows; per 64-key tile a lane scores one
// key (dot product over D from LDS), the wave does the online-softmax update
// with register-only wave reductions (DPP and lane swaps), then each lane
// accumulates D/64 output columns, reading each key's probability from its
// lane with v_readlane.
// =========================================================================
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_fma_kernel(AttnArgs a) {
  constexpr int KT = kKeysPerTile;
  constexpr int RPW = 4;          // rows per wave
  constexpr int RPB = 4 * RPW;    // rows per block
  constexpr int DP = D + 1;       // padded LDS row (floats): conflict-free lane=key reads
  constexpr int E = D / 64;       // output columns per lane
  __shared__ float s_k[KT * DP];
  __shared__ float s_v[KT * DP];
  __shared__ float s_q[RPB * D];
  __shared__ uint64_t s_anc[2 * kMaxNodes];
  __shared__ int32_t s_depth[kMaxNodes];
  __shared__ int s_status;

  const int c = blockIdx.x, rb = blockIdx.y, bh = blockIdx.z;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = a.N, G = a.G, R = a.R;
  const int L = a.cache_len[b];
  const int n_raw = nodes_raw(a.n_nodes, b, N);
  const int nU = nodes_used(n_raw, N);
  const int Rn = nU * G;  // rows of real nodes; rows Rn..R-1 are padding
  if (wave == 0) {
    const bool tree_ok = wave_build_tree(a.parents + (size_t)b * N, nU, s_anc, s_depth);
    if (lane == 0) {
      s_status = request_status(tree_ok, L, a.Lmax, n_raw, N);
      if (a.dev_status && c == 0 && rb == 0 && h == 0) a.dev_status[b] = s_status;
    }
  }
  __syncthreads();
  const int status = s_status;

  const int k_begin = c * a.chunk_keys;
  const int k_end = min(L, k_begin + a.chunk_keys);
  const int row0 = rb * RPB;
  if (status != TTV_OK) {
    if (a.chunks == 1) {  // rejected request: zero output (a combine writes it otherwise)
      for (int t = threadIdx.x; t < RPB * D; t += blockDim.x) {
        const int r = row0 + t / D, d = t % D;
        if (r >= R) continue;
        const int i = r / G, hq = h * G + (r - i * G);
        store_elt<T>(static_cast<T*>(a.out) + (((size_t)b * N + i) * a.Hq + hq) * D + d, 0.f);
        if (d == 0 && a.lse) a.lse[((size_t)b * N + i) * a.Hq + hq] = 0.f;
      }
    }
    return;
  }
  const int nP = (k_begin < k_end) ? (k_end - k_begin + KT - 1) / KT : 0;
  const int nT = (c == 0) ? (nU + KT - 1) / KT : 0;
  if (nP + nT == 0) return;  // empty chunk: the combine skips it

  // queries of this block's rows, widened to fp32
  const T* q = static_cast<const T*>(a.q);
  for (int t = threadIdx.x; t < RPB * D; t += blockDim.x) {
    const int rr = t / D, d = t % D, r = row0 + rr;
    float v = 0.f;
    if (r < Rn) {
      const int i = r / G, hq = h * G + (r - i * G);
      v = load_elt<T>(q + (((size_t)b * N + i) * a.Hq + hq) * D + d);
    }
    s_q[rr * D + d] = v;
  }

  float m[RPW], l[RPW], acc[RPW][E];
  uint64_t anc_w[RPW][2];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    m[k] = -INFINITY;
    l[k] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[k][e] = 0.f;
    const int r = row0 + wave * RPW + k;
    const int i = r < Rn ? r / G : 0;
    anc_w[k][0] = r < Rn ? s_anc[2 * i] : 0ull;
    anc_w[k][1] = r < Rn ? s_anc[2 * i + 1] : 0ull;
  }

  const T* kc = static_cast<const T*>(a.k_cache) + ((size_t)bh * a.Lcap) * D;
  const T* vc = static_cast<const T*>(a.v_cache) + ((size_t)bh * a.Lcap) * D;
  // the tree's K/V: their own tensors, or the cache rows after the prefix
  // (node i at row Lc + i, Lc = L clamped to [0, Lmax]; rows < Lmax + N <= Lcap)
  const int Lc = min(max(L, 0), a.Lmax);
  const T* kt = a.tree_in_cache ? kc + (size_t)Lc * D : static_cast<const T*>(a.k_tree) + ((size_t)bh * N) * D;
  const T* vt = a.tree_in_cache ? vc + (size_t)Lc * D : static_cast<const T*>(a.v_tree) + ((size_t)bh * N) * D;

  for (int tile = 0; tile < nP + nT; ++tile) {
    const bool is_tree = tile >= nP;
    const int key0 = is_tree ? (tile - nP) * KT : k_begin + tile * KT;
    const int nvalid = is_tree ? min(KT, nU - key0) : min(KT, k_end - key0);
    const T* ks = is_tree ? kt : kc;
    const T* vs = is_tree ? vt : vc;
    __syncthreads();  // previous tile fully consumed
    for (int t = threadIdx.x; t < KT * D; t += blockDim.x) {
      const int j = t / D, d = t % D;
      float kv = 0.f, vv = 0.f;
      if (j < nvalid) {
        kv = load_elt<T>(ks + (size_t)(key0 + j) * D + d);
        vv = load_elt<T>(vs + (size_t)(key0 + j) * D + d);
      }
      s_k[j * DP + d] = kv;
      s_v[j * DP + d] = vv;
    }
    __syncthreads();
    bool key_ok = lane < nvalid;
    // the scores and the online-softmax update of the wave's rows (padding
    // rows get p = 0 and stay empty), then one pass over the tile's keys
    // that reads each V row once for all of them
    float p[RPW];
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const int rr = wave * RPW + k;
      p[k] = 0.f;
      if (row0 + rr >= Rn) continue;  // wave-uniform
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) dot = fmaf(s_q[rr * D + d], s_k[lane * DP + d], dot);
      bool ok = key_ok;
      if (is_tree) {
        const int j = key0 + lane;
        ok = ok && ((anc_w[k][j >> 6] >> (j & 63)) & 1ull);
      }
      const float t = ok ? dot * a.scale_log2 : -INFINITY;
      const float m_new = fmaxf(m[k], wave_allmax_f32(t));
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      p[k] = __builtin_amdgcn_exp2f(t - m_use);
      const float alpha = __builtin_amdgcn_exp2f(m[k] - m_use);
      l[k] = l[k] * alpha + wave_allsum_f32(p[k]);
      m[k] = m_new;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[k][e] *= alpha;
    }
#pragma unroll 8
    for (int j = 0; j < KT; ++j) {
      float vj[E];
#pragma unroll
      for (int e = 0; e < E; ++e) vj[e] = s_v[j * DP + lane + 64 * e];
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        // key j's probability from lane j (a register read, no LDS round trip)
        const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[k]), j));
#pragma unroll
        for (int e = 0; e < E; ++e) acc[k][e] = fmaf(pj, vj[e], acc[k][e]);
      }
    }
  }

#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int r = row0 + wave * RPW + k;
    if (r >= R) continue;
    const int i = r / G, hq = h * G + (r - i * G);
    if (a.chunks == 1) {
      const bool real = r < Rn;  // a padding node's row gets zeros
      const float inv = real ? 1.f / l[k] : 0.f;
      T* o = static_cast<T*>(a.out) + (((size_t)b * N + i) * a.Hq + hq) * D;
#pragma unroll
      for (int e = 0; e < E; ++e) store_elt<T>(o + lane + 64 * e, real ? acc[k][e] * inv : 0.f);
      if (lane == 0 && a.lse)
        a.lse[((size_t)b * N + i) * a.Hq + hq] = real ? (m[k] + __log2f(l[k])) * kLn2 : 0.f;
    } else {
      const size_t pr = ((size_t)bh * a.chunks + c) * R + r;
      if constexpr (sizeof(T) == 2) {
        // bf16 output: the chunk's normalised output in bf16 (a row that
        // sees no key of the chunk has l = 0 and weight 0: stored as 0)
        uint16_t* wsb = reinterpret_cast<uint16_t*>(a.ws_acc);
        const float inv = l[k] > 0.f ? 1.f / l[k] : 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) wsb[pr * D + lane + 64 * e] = f32_to_bf16(acc[k][e] * inv);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) a.ws_acc[pr * D + lane + 64 * e] = acc[k][e];
      }
      if (lane == 0) {
        a.ws_ml[pr * 2] = m[k];
        a.ws_ml[pr * 2 + 1] = l[k];
      }
    }
  }
}

// =========================================================================
// Split-KV combine: o = sum_c acc_c 2^(m_c - M) / sum_c l_c 2^(m_c - M),
// M = max_c m_c, over the chunks that hold keys of request b (chunk 0 always
// does: it owns the tree keys, and every node sees at least itself; with the
// balanced split every chunk of the request holds keys).  A lane takes 16
// bytes of a row's partial (LPR lanes per row, 64/LPR rows per wavefront);
// the partials of kCombineBatch chunks are requested together and merged
// with a running max, so a row costs about two memory round trips for the
// usual few chunks.  (bf16 partials are each chunk's normalised output,
// weighted by l_c 2^(m_c - M); fp32 partials are the unnormalised sums.)
// =========================================================================
constexpr int kCombineBatch = 4;
constexpr int kCombineWaves = 4;
template <typename T, int D>
struct CombineShape {
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane
  static constexpr int LPR = D / EPL;               // lanes per row
  static constexpr int RPW = 64 / LPR;              // rows per wavefront
  static constexpr int RPB = kCombineWaves * RPW;   // rows per workgroup
  static_assert(D % EPL == 0 && 64 % LPR == 0, "combine lanes");
};

template <typename T, int D>
__global__ __launch_bounds__(64 * kCombineWaves) void attn_combine_kernel(AttnArgs a) {
  using Sh = CombineShape<T, D>;
  constexpr int EPL = Sh::EPL;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.y;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int col = (lane % Sh::LPR) * EPL;
  const int r = (blockIdx.x * kCombineWaves + wave) * Sh::RPW + lane / Sh::LPR;
  const int N = a.N, G = a.G, R = a.R;
  const int L = a.cache_len[b];
  const int n_raw = nodes_raw(a.n_nodes, b, N);
  const int nU = nodes_used(n_raw, N);
  const bool tree_ok = wave_tree_valid(a.parents + (size_t)b * N, nU);  // every lane takes part
  if (r >= R) return;
  const int i = r / G, hq = h * G + (r - i * G);
  T* o = static_cast<T*>(a.out) + (((size_t)b * N + i) * a.Hq + hq) * D + col;
  float* lse = a.lse && col == 0 ? a.lse + ((size_t)b * N + i) * a.Hq + hq : nullptr;
  // a rejected request or a padding node's row: zeros
  if (request_status(tree_ok, L, a.Lmax, n_raw, N) != TTV_OK || i >= nU) {
    *reinterpret_cast<u32x4*>(o) = u32x4{0u, 0u, 0u, 0u};
    if (lse) *lse = 0.f;
    return;
  }
  int used = 1;
  if (a.balanced) {
    used = a.ws_nchunks[b];  // written by the request's first work item
    if (used == 1) return;   // that item wrote the output itself
  } else {
    while (used < a.chunks && used * a.chunk_keys < L) ++used;
  }
  const size_t base = (size_t)bh * a.chunks * R + r;
  const T* part = reinterpret_cast<const T*>(a.ws_acc);
  float M = -INFINITY, lsum = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int c0 = 0; c0 < used; c0 += kCombineBatch) {
    // chunks past the last re-read the last one (from cache) with weight 0
    float2 ml[kCombineBatch];
    u32x4 pv[kCombineBatch];
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const size_t pr = base + (size_t)min(c0 + k, used - 1) * R;
      ml[k] = *reinterpret_cast<const float2*>(a.ws_ml + pr * 2);
      pv[k] = *reinterpret_cast<const u32x4*>(part + pr * D + col);
    }
    // chunk 0 (in the first batch) has a finite max, so M is finite after it
    float mb = M;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k)
      if (c0 + k < used) mb = fmaxf(mb, ml[k].x);
    const float sc = __builtin_amdgcn_exp2f(M - mb);  // 0 for the first batch
    lsum *= sc;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= sc;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      if (c0 + k >= used) continue;
      const float w = __builtin_amdgcn_exp2f(ml[k].x - mb);
      if constexpr (sizeof(T) == 2) {
        const float lw = ml[k].y * w;
        lsum += lw;
#pragma unroll
        for (int e = 0; e < EPL; e += 2) {
          const uint32_t x = pv[k][e / 2];
          acc[e] = fmaf(bf16_to_f32((uint16_t)(x & 0xffffu)), lw, acc[e]);
          acc[e + 1] = fmaf(bf16_to_f32((uint16_t)(x >> 16)), lw, acc[e + 1]);
        }
      } else {
        lsum = fmaf(ml[k].y, w, lsum);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(__uint_as_float(pv[k][e]), w, acc[e]);
      }
    }
    M = mb;
  }
  const float inv = 1.f / lsum;
  u32x4 ov;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < EPL; e += 2) ov[e / 2] = pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) ov[e] = __float_as_uint(acc[e] * inv);
  }
  *reinterpret_cast<u32x4*>(o) = ov;
  if (lse) *lse = (M + __log2f(lsum)) * kLn2;
}

// ------------------------------------------------------------- launchers --
static dim3 attn_grid(const AttnArgs& a) {
  return dim3(a.chunks, (a.R + a.rows_per_block - 1) / a.rows_per_block, a.B * a.Hkv);
}

hipError_t launch_attn_fma(const AttnArgs& a, bool bf16, hipStream_t s) {
  const dim3 grid = attn_grid(a);
  if (bf16) {
    if (a.D == 64) hipLaunchKernelGGL((attn_fma_kernel<uint16_t, 64>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_fma_kernel<uint16_t, 128>), grid, dim3(256), 0, s, a);
  } else {
    if (a.D == 64) hipLaunchKernelGGL((attn_fma_kernel<float, 64>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_fma_kernel<float, 128>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
static void combine_launch(const AttnArgs& a, hipStream_t s) {
  constexpr int RPB = CombineShape<T, D>::RPB;
  const dim3 grid((a.R + RPB - 1) / RPB, a.B * a.Hkv);
  hipLaunchKernelGGL((attn_combine_kernel<T, D>), grid, dim3(64 * kCombineWaves), 0, s, a);
}

hipError_t launch_attn_combine(const AttnArgs& a, bool bf16, hipStream_t s) {
  if (bf16) {
    if (a.D == 64) combine_launch<uint16_t, 64>(a, s);
    else combine_launch<uint16_t, 128>(a, s);
  } else {
    if (a.D == 64) combine_launch<float, 64>(a, s);
    else combine_launch<float, 128>(a, s);
  }
  return hipGetLastError();
}

}  // namespace ttv
