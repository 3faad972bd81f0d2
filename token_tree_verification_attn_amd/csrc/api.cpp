// api.cpp -- the C ABI of libttv (declared in include/ttv.h): argument
// validation (before any HIP call), launch plans, launches.  No allocation,
// no global state.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <utility>
#include <vector>

#include "launch.h"
#include "softmax_exact.h"
#include "ttv.h"

using namespace ttv;

namespace {

constexpr int kMaxGridYZ = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Launch plan of ttv_tree_attn; returns TTV_OK or the status the call gives.
ttv_status attn_plan(ttv_dtype dt, int B, int N, int Hq, int Hkv, int D, int Lmax,
                     int rpb_hint, int chunk_hint, AttnPlan* p) {
  if (dt != TTV_F32 && dt != TTV_BF16) return TTV_E_DTYPE;
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || D < 1 || Lmax < 0) return TTV_E_SHAPE;
  if (N > TTV_MAX_NODES || (D != 64 && D != 128) || Hq % Hkv != 0) return TTV_E_UNSUPPORTED;
  if (rpb_hint < 0 || chunk_hint < 0 || chunk_hint % 64 != 0) return TTV_E_UNSUPPORTED;
  const int G = Hq / Hkv;
  const long R = (long)N * G;
  if (R > (1L << 24)) return TTV_E_UNSUPPORTED;
  p->rows = (int)R;
  p->mfma = dt == TTV_BF16 && R >= 16;
  const long pairs = (long)B * Hkv;
  if (pairs > kMaxGridYZ) return TTV_E_UNSUPPORTED;
  // Workgroups that fit on the chip at once: one matrix-core workgroup per CU
  // (up to 256 VGPRs per lane), two FMA workgroups; 256 CUs.
  long slots = 512;
  if (p->mfma) {
    if (rpb_hint) {
      if (rpb_hint != 64 && rpb_hint != 128 && rpb_hint != 256) return TTV_E_UNSUPPORTED;
      p->rows_per_block = rpb_hint;
    } else {
      // 128-row blocks (8 waves x 16 queries) up to 512 rows per kv head:
      // their softmax work per wave is the lightest, and a second row block
      // re-reads the head's KV from L2 rather than HBM.  Above that, every
      // extra row block costs one more pass of the KV through the CU copy
      // engines, and 256-row blocks win.  (Measured on MI355X: 256 rows x
      // 2048 keys per head, 128-row blocks unsplit run 13% faster than
      // 256-row blocks with a 2-way split; 1024 rows x 32768 keys, 256-row
      // blocks run 17% faster than 128-row ones.)
      p->rows_per_block = R <= 64 ? 64 : (R <= 512 ? 128 : 256);
    }
    slots = 256;
  } else {
    if (rpb_hint && rpb_hint != 16) return TTV_E_UNSUPPORTED;
    p->rows_per_block = 16;
  }
  p->row_blocks = ceil_div(R, p->rows_per_block);
  if (p->row_blocks > kMaxGridYZ) return TTV_E_UNSUPPORTED;
  const long units = pairs * p->row_blocks;
  int chunk;
  if (chunk_hint) {
    chunk = chunk_hint;
  } else {
    // split the prefix only as far as needed to occupy the free slots, in
    // chunks of at least 128 keys (partials cost ~rows/chunk of the KV in
    // bf16, twice that in fp32), and not at all up to 256 keys, where a split
    // saves at most a few tiles per workgroup (measured on MI355X: 32 heads x
    // 64 rows x 512 keys, 32 workgroups streaming 9 tiles each: 128-key
    // chunks 14.1 us, 64-key 15.4, 256-key 15.3, unsplit 15.7)
    const long want = (slots + units - 1) / units;
    long c = want > 1 && Lmax > 256 ? (Lmax + want - 1) / want : Lmax;
    c = (c + 63) / 64 * 64;
    if (c < 128) c = 128;
    chunk = (int)c;
  }
  p->chunk_keys = chunk;
  p->chunks = Lmax > 0 ? ceil_div(Lmax, chunk) : 1;
  if (p->chunks < 1) p->chunks = 1;
  p->items = 0;
  // Several requests and fewer work units than CUs: the prefix lengths may
  // differ, so the matrix-core path plans the split on the device from the
  // actual lengths (attn_plan.h) over `slots` workgroups, a unit taking at
  // most twice the even share of chunks (which bounds the workspace).  The
  // plan costs one more memory round trip before the first copy, so it is
  // only used where the split can change (measured on MI355X: 8 requests of
  // 1169..3643 keys run 4% faster; 256 units, each its own workgroup either
  // way, 12% slower).
  p->balanced = p->mfma && !chunk_hint && B > 1 && B <= kBalancedMaxB && units < slots;
  if (p->balanced) {
    const long tiles_max = (N + 63) / 64 + ((long)Lmax + 63) / 64;
    long cmax = (2 * slots + units - 1) / units;
    if (cmax > tiles_max) cmax = tiles_max;
    p->chunks = cmax > 1 ? (int)cmax : 1;
    p->chunk_keys = 0;
    p->items = (int)slots;
  }
  // partials: the output part (bf16 for bf16 outputs, fp32 sums otherwise)
  // and the (max, sum) pair of every (pair, chunk, row)
  const size_t part_elt = dt == TTV_BF16 ? 2 : 4;
  p->ws_bytes = p->chunks > 1 ? (size_t)pairs * p->chunks * R * ((size_t)D * part_elt + 8) : 0;
  if (p->balanced && p->chunks > 1) p->ws_bytes += (size_t)B * sizeof(int32_t);  // chunks per request
  return TTV_OK;
}

ttv_status launch_status(hipError_t e) { return e == hipSuccess ? TTV_OK : TTV_E_LAUNCH; }

}  // namespace

namespace ttv {

hipError_t lds_limit_once(const void* kern, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> done;  // (kernel, device) pairs already set
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& d : done)
    if (d.first == kern && d.second == dev) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.emplace_back(kern, dev);
  return e;
}

ttv_status attn_prepare(ttv_dtype dt, int B, int N, int Hq, int Hkv, int D, float scale,
                        const void* q, const void* k_cache, const void* v_cache, int Lcap,
                        const int32_t* cache_len, int Lmax, const void* k_tree,
                        const void* v_tree, const int32_t* parents, const void* out,
                        int rows_per_block, int chunk_keys, AttnPlan* p) {
  if (dt != TTV_F32 && dt != TTV_BF16) return TTV_E_DTYPE;
  if (!q || !k_cache || !v_cache || !cache_len || !parents || !out || (!k_tree != !v_tree))
    return TTV_E_NULL;
  const bool tree_in_cache = !k_tree;  // both NULL: node i at cache row L_b + i
  if (Lcap < 0 || Lmax > Lcap || !std::isfinite(scale) || !(scale > 0.f)) return TTV_E_SHAPE;
  if (tree_in_cache && (long)Lmax + N > Lcap) return TTV_E_SHAPE;
  const ttv_status st = attn_plan(dt, B, N, Hq, Hkv, D, Lmax, rows_per_block, chunk_keys, p);
  if (st != TTV_OK) return st;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (!tree_in_cache && (!aligned16(k_tree) || !aligned16(v_tree))) || !aligned16(out))
    return TTV_E_ALIGN;
  return TTV_OK;
}

// The launches of one validated ttv_tree_attn call: the topology (only when
// its outputs are asked for; the attention kernels rebuild it in registers
// and report the request's status), the attention kernel, the combine of
// split partials.  ws = the partials (p.ws_bytes bytes).
ttv_status launch_attn(const AttnPlan& p, ttv_dtype dt, int B, int N, int Hq, int Hkv, int D,
                       float scale, const void* q, const void* k_cache, const void* v_cache,
                       int Lcap, const int32_t* cache_len, int Lmax, const void* k_tree,
                       const void* v_tree, const int32_t* parents, const int32_t* n_nodes,
                       void* out, float* lse, uint64_t* anc_out, int32_t* depth_out,
                       int32_t* dev_status, void* ws, hipStream_t s) {
  if (anc_out || depth_out) {
    if (launch_topology(B, N, parents, n_nodes, anc_out, depth_out, nullptr, s) != hipSuccess)
      return TTV_E_LAUNCH;
  }
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.tree_in_cache = k_tree ? 0 : 1;
  a.cache_len = cache_len;
  a.parents = parents;
  a.n_nodes = n_nodes;
  a.out = out;
  a.lse = lse;
  a.dev_status = dev_status;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.D = D;
  a.Lcap = Lcap;
  a.Lmax = Lmax;
  a.R = p.rows;
  a.rows_per_block = p.rows_per_block;
  a.chunk_keys = p.chunk_keys;
  a.chunks = p.chunks;
  a.balanced = p.balanced ? 1 : 0;
  a.row_blocks = p.row_blocks;
  a.items = p.items;
  a.scale_log2 = scale * 1.44269504088896340736f;
  if (p.chunks > 1) {
    const size_t parts = (size_t)B * Hkv * p.chunks * p.rows;
    char* w = static_cast<char*>(ws);
    a.ws_acc = reinterpret_cast<float*>(w);
    a.ws_ml = reinterpret_cast<float*>(w + parts * D * (dt == TTV_BF16 ? 2 : 4));
    if (p.balanced) a.ws_nchunks = reinterpret_cast<int32_t*>(a.ws_ml + parts * 2);
  }
  const hipError_t e = p.mfma ? launch_attn_mfma(a, s) : launch_attn_fma(a, dt == TTV_BF16, s);
  if (e != hipSuccess) return TTV_E_LAUNCH;
  if (p.chunks > 1) return launch_status(launch_attn_combine(a, dt == TTV_BF16, s));
  return TTV_OK;
}

}  // namespace ttv

extern "C" {

const char* ttv_status_string(ttv_status s) {
  switch (s) {
    case TTV_OK: return "ok";
    case TTV_E_NULL: return "null pointer";
    case TTV_E_SHAPE: return "bad shape or size";
    case TTV_E_DTYPE: return "bad dtype or mode";
    case TTV_E_UNSUPPORTED: return "unsupported size or option";
    case TTV_E_WORKSPACE: return "workspace missing or too small";
    case TTV_E_LAUNCH: return "kernel launch failed";
    case TTV_E_TREE: return "malformed token tree";
    case TTV_E_ALIGN: return "pointer not 16-byte aligned";
    case TTV_E_SCRATCH: return "needs more than the no-allocation entry point's static scratch";
    default: return "unknown status";
  }
}

int32_t ttv_version(void) { return 200; }

ttv_status ttv_tree_topology(int32_t B, int32_t N, const int32_t* parents, uint64_t* anc_out,
                             int32_t* depth_out, int32_t* dev_status, void* stream) {
  if (!parents) return TTV_E_NULL;
  if (B < 1 || N < 1) return TTV_E_SHAPE;
  if (N > TTV_MAX_NODES) return TTV_E_UNSUPPORTED;
  return launch_status(launch_topology(B, N, parents, nullptr, anc_out, depth_out, dev_status,
                                       static_cast<hipStream_t>(stream)));
}

size_t ttv_tree_attn_tuned_workspace_size(ttv_dtype dt, int32_t B, int32_t N, int32_t Hq,
                                          int32_t Hkv, int32_t D, int32_t Lmax,
                                          int32_t rows_per_block, int32_t chunk_keys) {
  AttnPlan p;
  if (attn_plan(dt, B, N, Hq, Hkv, D, Lmax, rows_per_block, chunk_keys, &p) != TTV_OK)
    return (size_t)-1;
  return p.ws_bytes;
}

size_t ttv_tree_attn_workspace_size(ttv_dtype dt, int32_t B, int32_t N, int32_t Hq,
                                    int32_t Hkv, int32_t D, int32_t Lmax) {
  return ttv_tree_attn_tuned_workspace_size(dt, B, N, Hq, Hkv, D, Lmax, 0, 0);
}

}  // extern "C"

namespace {

// ttv_tree_attn with per-request node counts (nullptr: N each) and a launch
// shape (0, 0: automatic).
ttv_status tree_attn_call(ttv_dtype dt, int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                          float scale, const void* q, const void* k_cache, const void* v_cache,
                          int32_t Lcap, const int32_t* cache_len, int32_t Lmax,
                          const void* k_tree, const void* v_tree, const int32_t* parents,
                          const int32_t* n_nodes, void* out, float* lse, uint64_t* anc_out,
                          int32_t* depth_out, int32_t* dev_status, void* workspace,
                          size_t workspace_bytes, int32_t rows_per_block, int32_t chunk_keys,
                          void* stream) {
  AttnPlan p;
  const ttv_status st = attn_prepare(dt, B, N, Hq, Hkv, D, scale, q, k_cache, v_cache, Lcap,
                                     cache_len, Lmax, k_tree, v_tree, parents, out,
                                     rows_per_block, chunk_keys, &p);
  if (st != TTV_OK) return st;
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return TTV_E_WORKSPACE;
  if (p.ws_bytes > 0 && !aligned16(workspace)) return TTV_E_ALIGN;
  return launch_attn(p, dt, B, N, Hq, Hkv, D, scale, q, k_cache, v_cache, Lcap, cache_len, Lmax,
                     k_tree, v_tree, parents, n_nodes, out, lse, anc_out, depth_out, dev_status,
                     workspace, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

ttv_status ttv_tree_attn_tuned(ttv_dtype dt, int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                               int32_t D, float scale, const void* q, const void* k_cache,
                               const void* v_cache, int32_t Lcap, const int32_t* cache_len,
                               int32_t Lmax, const void* k_tree, const void* v_tree,
                               const int32_t* parents, void* out, float* lse,
                               uint64_t* anc_out, int32_t* depth_out, int32_t* dev_status,
                               void* workspace, size_t workspace_bytes, int32_t rows_per_block,
                               int32_t chunk_keys, void* stream) {
  return tree_attn_call(dt, B, N, Hq, Hkv, D, scale, q, k_cache, v_cache, Lcap, cache_len, Lmax,
                        k_tree, v_tree, parents, nullptr, out, lse, anc_out, depth_out,
                        dev_status, workspace, workspace_bytes, rows_per_block, chunk_keys,
                        stream);
}

ttv_status ttv_tree_attn(ttv_dtype dt, int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                         int32_t D, float scale, const void* q, const void* k_cache,
                         const void* v_cache, int32_t Lcap, const int32_t* cache_len,
                         int32_t Lmax, const void* k_tree, const void* v_tree,
                         const int32_t* parents, void* out, float* lse, uint64_t* anc_out,
                         int32_t* depth_out, int32_t* dev_status, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return tree_attn_call(dt, B, N, Hq, Hkv, D, scale, q, k_cache, v_cache, Lcap, cache_len, Lmax,
                        k_tree, v_tree, parents, nullptr, out, lse, anc_out, depth_out,
                        dev_status, workspace, workspace_bytes, 0, 0, stream);
}

ttv_status ttv_tree_attn_varlen(ttv_dtype dt, int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                int32_t D, float scale, const void* q, const void* k_cache,
                                const void* v_cache, int32_t Lcap, const int32_t* cache_len,
                                int32_t Lmax, const void* k_tree, const void* v_tree,
                                const int32_t* parents, const int32_t* n_nodes, void* out,
                                float* lse, uint64_t* anc_out, int32_t* depth_out,
                                int32_t* dev_status, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!n_nodes) return TTV_E_NULL;
  return tree_attn_call(dt, B, N, Hq, Hkv, D, scale, q, k_cache, v_cache, Lcap, cache_len, Lmax,
                        k_tree, v_tree, parents, n_nodes, out, lse, anc_out, depth_out,
                        dev_status, workspace, workspace_bytes, 0, 0, stream);
}

// Stochastic verification: no workspace while the residual fits the LDS; for
// larger vocabularies (V % 4 == 0) the residual, B*V floats.
static size_t mss_workspace_bytes(int32_t B, int32_t V) {
  if (V <= kMssMaxVocab) return 0;
  if (V > kMssGmMaxVocab || V % 4 != 0) return (size_t)-1;
  return (size_t)B * (size_t)V * sizeof(float);
}

// The stochastic launch with the host checks of its residual: a vocabulary
// beyond the LDS needs V % 4 == 0 and a 16-byte-aligned workspace of
// mss_workspace_bytes.
static ttv_status launch_mss_checked(int32_t B, int32_t N, int32_t V, const int32_t* parents,
                                     const int32_t* tokens, const int32_t* n_nodes,
                                     const float* llm, const float* ssm, const MssDraws& dr,
                                     int32_t* path, int32_t* path_len, int32_t* out_tokens,
                                     int32_t* dev_status, void* workspace,
                                     size_t workspace_bytes, const CommitArgs& cm,
                                     hipStream_t s) {
  const size_t need = mss_workspace_bytes(B, V);
  if (need == (size_t)-1) return TTV_E_UNSUPPORTED;
  if (!aligned16(llm) || !aligned16(ssm)) return TTV_E_ALIGN;
  float* gm_w = nullptr;
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return TTV_E_WORKSPACE;
    if (!aligned16(workspace)) return TTV_E_ALIGN;
    gm_w = static_cast<float*>(workspace);
  }
  return launch_status(launch_verify_mss(B, N, V, parents, tokens, n_nodes, llm, ssm, dr,
                                         LogitRows{}, path, path_len, out_tokens, dev_status,
                                         gm_w, cm, s));
}

size_t ttv_tree_verify_workspace_size(ttv_verify_mode mode, int32_t B, int32_t N, int32_t V) {
  if (mode != TTV_GREEDY && mode != TTV_STOCHASTIC) return (size_t)-1;
  if (B < 1 || N < 1 || V < 1 || N > TTV_MAX_NODES) return (size_t)-1;
  if (mode == TTV_STOCHASTIC) return mss_workspace_bytes(B, V);
  if ((long)B * N > 0x7fffffffL) return (size_t)-1;
  return greedy_plan(B, N, V).ws_bytes;
}

// ttv_tree_verify with per-request node counts (nullptr: N each).
static ttv_status tree_verify_call(ttv_verify_mode mode, int32_t B, int32_t N, int32_t V,
                                   const int32_t* parents, const int32_t* tokens,
                                   const int32_t* n_nodes, const float* llm, const float* ssm,
                                   uint64_t seed, uint64_t step, int32_t* path,
                                   int32_t* path_len, int32_t* out_tokens, int32_t* dev_status,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (mode != TTV_GREEDY && mode != TTV_STOCHASTIC) return TTV_E_DTYPE;
  if (!parents || !tokens || !llm || !path || !path_len || !out_tokens) return TTV_E_NULL;
  if (mode == TTV_STOCHASTIC && !ssm) return TTV_E_NULL;
  if (B < 1 || N < 1 || V < 1) return TTV_E_SHAPE;
  if (N > TTV_MAX_NODES) return TTV_E_UNSUPPORTED;
  if ((long)B * N > 0x7fffffffL) return TTV_E_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == TTV_STOCHASTIC)
    return launch_mss_checked(B, N, V, parents, tokens, n_nodes, llm, ssm,
                              MssDraws{nullptr, nullptr, seed, step}, path, path_len, out_tokens,
                              dev_status, workspace, workspace_bytes, CommitArgs{}, s);
  const GreedyPlan p = greedy_plan(B, N, V);
  if (p.splits > kMaxGridYZ) return TTV_E_UNSUPPORTED;
  if (!aligned16(llm)) return TTV_E_ALIGN;
  if (!workspace || workspace_bytes < p.ws_bytes) return TTV_E_WORKSPACE;
  if (!aligned16(workspace)) return TTV_E_ALIGN;
  return launch_status(launch_verify_greedy(B, N, V, parents, tokens, n_nodes, llm, path,
                                            path_len, out_tokens, dev_status, workspace, p, s));
}

ttv_status ttv_tree_verify(ttv_verify_mode mode, int32_t B, int32_t N, int32_t V,
                           const int32_t* parents, const int32_t* tokens, const float* llm,
                           const float* ssm, uint64_t seed, uint64_t step, int32_t* path,
                           int32_t* path_len, int32_t* out_tokens, int32_t* dev_status,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return tree_verify_call(mode, B, N, V, parents, tokens, nullptr, llm, ssm, seed, step, path,
                          path_len, out_tokens, dev_status, workspace, workspace_bytes, stream);
}

ttv_status ttv_tree_verify_varlen(ttv_verify_mode mode, int32_t B, int32_t N, int32_t V,
                                  const int32_t* parents, const int32_t* tokens,
                                  const int32_t* n_nodes, const float* llm, const float* ssm,
                                  uint64_t seed, uint64_t step, int32_t* path, int32_t* path_len,
                                  int32_t* out_tokens, int32_t* dev_status, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!n_nodes) return TTV_E_NULL;
  return tree_verify_call(mode, B, N, V, parents, tokens, n_nodes, llm, ssm, seed, step, path,
                          path_len, out_tokens, dev_status, workspace, workspace_bytes, stream);
}

ttv_status ttv_tree_verify_uniforms(int32_t B, int32_t N, int32_t V, const int32_t* parents,
                                    const int32_t* tokens, const float* llm, const float* ssm,
                                    const float* u_accept, const float* u_bonus, int32_t* path,
                                    int32_t* path_len, int32_t* out_tokens, int32_t* dev_status,
                                    void* stream) {
  if (!parents || !tokens || !llm || !ssm || !u_accept || !u_bonus || !path || !path_len ||
      !out_tokens)
    return TTV_E_NULL;
  if (B < 1 || N < 1 || V < 1) return TTV_E_SHAPE;
  if (N > TTV_MAX_NODES || V > kMssMaxVocab) return TTV_E_UNSUPPORTED;
  if ((long)B * N > 0x7fffffffL) return TTV_E_UNSUPPORTED;
  if (!aligned16(llm) || !aligned16(ssm)) return TTV_E_ALIGN;
  return launch_status(launch_verify_mss(B, N, V, parents, tokens, nullptr, llm, ssm,
                                         MssDraws{u_accept, u_bonus, 0, 0}, LogitRows{}, path, path_len,
                                         out_tokens, dev_status, nullptr, CommitArgs{},
                                         static_cast<hipStream_t>(stream)));
}

ttv_status ttv_kv_commit(ttv_dtype dt, int32_t B, int32_t N, int32_t Hkv, int32_t D,
                         int32_t Lcap, const void* k_tree, const void* v_tree, void* k_cache,
                         void* v_cache, const int32_t* cache_len_in, int32_t* cache_len_out,
                         int32_t Lmax, const int32_t* path, const int32_t* path_len,
                         int32_t* committed_src, int32_t* dev_status, void* stream) {
  if (dt != TTV_F32 && dt != TTV_BF16) return TTV_E_DTYPE;
  if (!k_tree || !v_tree || !k_cache || !v_cache || !cache_len_in || !cache_len_out || !path ||
      !path_len)
    return TTV_E_NULL;
  if (B < 1 || N < 1 || Hkv < 1 || D < 1 || Lmax < 0 || Lcap < 0) return TTV_E_SHAPE;
  if (N > TTV_MAX_NODES || (D != 64 && D != 128)) return TTV_E_UNSUPPORTED;
  if ((long)Lmax + N > Lcap) return TTV_E_SHAPE;
  if (!aligned16(k_tree) || !aligned16(v_tree) || !aligned16(k_cache) || !aligned16(v_cache))
    return TTV_E_ALIGN;
  const int elt = dt == TTV_BF16 ? 2 : 4;
  return launch_status(launch_kv_commit(elt, B, N, Hkv, D, Lcap, k_tree, v_tree, k_cache, v_cache,
                                        cache_len_in, cache_len_out, Lmax, path, path_len,
                                        committed_src, dev_status,
                                        static_cast<hipStream_t>(stream)));
}

// ttv_tree_verify_commit with per-request node counts (nullptr: N each).
static ttv_status tree_verify_commit_call(
    ttv_verify_mode mode, ttv_dtype dt, int32_t B, int32_t N, int32_t V, int32_t Hkv, int32_t D,
    int32_t Lcap, const int32_t* parents, const int32_t* tokens, const int32_t* n_nodes,
    const float* llm, const float* ssm, uint64_t seed, uint64_t step, const void* k_tree,
    const void* v_tree, void* k_cache, void* v_cache, const int32_t* cache_len_in,
    int32_t* cache_len_out, int32_t Lmax, int32_t* path, int32_t* path_len, int32_t* out_tokens,
    int32_t* committed_src, int32_t* dev_status, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (mode != TTV_GREEDY && mode != TTV_STOCHASTIC) return TTV_E_DTYPE;
  if (dt != TTV_F32 && dt != TTV_BF16) return TTV_E_DTYPE;
  if (!parents || !tokens || !llm || !k_tree || !v_tree || !k_cache || !v_cache ||
      !cache_len_in || !cache_len_out || !path || !path_len || !out_tokens)
    return TTV_E_NULL;
  if (mode == TTV_STOCHASTIC && !ssm) return TTV_E_NULL;
  if (B < 1 || N < 1 || V < 1 || Hkv < 1 || D < 1 || Lmax < 0 || Lcap < 0) return TTV_E_SHAPE;
  if (N > TTV_MAX_NODES || (D != 64 && D != 128)) return TTV_E_UNSUPPORTED;
  if ((long)B * N > 0x7fffffffL) return TTV_E_UNSUPPORTED;
  if ((long)Lmax + N > Lcap) return TTV_E_SHAPE;
  if (!aligned16(llm) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return TTV_E_ALIGN;
  const int elt = dt == TTV_BF16 ? 2 : 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == TTV_STOCHASTIC) {
    CommitArgs cm{D * elt / 16, Hkv, Lcap, Lmax, k_tree, v_tree, k_cache, v_cache,
                  cache_len_in, cache_len_out, committed_src};
    return launch_mss_checked(B, N, V, parents, tokens, n_nodes, llm, ssm,
                              MssDraws{nullptr, nullptr, seed, step}, path, path_len, out_tokens,
                              dev_status, workspace, workspace_bytes, cm, s);
  }
  const GreedyPlan p = greedy_plan(B, N, V);
  if (p.splits > kMaxGridYZ) return TTV_E_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.ws_bytes) return TTV_E_WORKSPACE;
  if (!aligned16(workspace)) return TTV_E_ALIGN;
  return launch_status(launch_verify_greedy_commit(
      B, N, V, parents, tokens, n_nodes, llm, path, path_len, out_tokens, dev_status, workspace, p,
      elt, Hkv, D, Lcap, Lmax, k_tree, v_tree, k_cache, v_cache, cache_len_in, cache_len_out,
      committed_src, s));
}

ttv_status ttv_tree_verify_commit(ttv_verify_mode mode, ttv_dtype dt, int32_t B, int32_t N,
                                  int32_t V, int32_t Hkv, int32_t D, int32_t Lcap,
                                  const int32_t* parents, const int32_t* tokens, const float* llm,
                                  const float* ssm, uint64_t seed, uint64_t step,
                                  const void* k_tree, const void* v_tree, void* k_cache,
                                  void* v_cache, const int32_t* cache_len_in,
                                  int32_t* cache_len_out, int32_t Lmax, int32_t* path,
                                  int32_t* path_len, int32_t* out_tokens, int32_t* committed_src,
                                  int32_t* dev_status, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return tree_verify_commit_call(mode, dt, B, N, V, Hkv, D, Lcap, parents, tokens, nullptr, llm,
                                 ssm, seed, step, k_tree, v_tree, k_cache, v_cache, cache_len_in,
                                 cache_len_out, Lmax, path, path_len, out_tokens, committed_src,
                                 dev_status, workspace, workspace_bytes, stream);
}

ttv_status ttv_tree_verify_commit_varlen(
    ttv_verify_mode mode, ttv_dtype dt, int32_t B, int32_t N, int32_t V, int32_t Hkv, int32_t D,
    int32_t Lcap, const int32_t* parents, const int32_t* tokens, const int32_t* n_nodes,
    const float* llm, const float* ssm, uint64_t seed, uint64_t step, const void* k_tree,
    const void* v_tree, void* k_cache, void* v_cache, const int32_t* cache_len_in,
    int32_t* cache_len_out, int32_t Lmax, int32_t* path, int32_t* path_len, int32_t* out_tokens,
    int32_t* committed_src, int32_t* dev_status, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (!n_nodes) return TTV_E_NULL;
  return tree_verify_commit_call(mode, dt, B, N, V, Hkv, D, Lcap, parents, tokens, n_nodes, llm,
                                 ssm, seed, step, k_tree, v_tree, k_cache, v_cache, cache_len_in,
                                 cache_len_out, Lmax, path, path_len, out_tokens, committed_src,
                                 dev_status, workspace, workspace_bytes, stream);
}

ttv_status ttv_tree_expand(int32_t B, int32_t F, int32_t V, int32_t k, const float* probs,
                           const int32_t* frontier, const int32_t* n_in, int32_t Ncap,
                           int32_t* parents, int32_t* tokens, int32_t* src_row, int32_t* n_out,
                           int32_t* dev_status, void* stream) {
  if (!probs || !frontier || !n_in || !parents || !tokens || !n_out) return TTV_E_NULL;
  if (B < 1 || F < 1 || V < 1 || Ncap < 1 || k < 1 || k > V) return TTV_E_SHAPE;
  if (k > kExpandMaxK || F > TTV_MAX_NODES || Ncap > TTV_MAX_NODES || B > kMaxGridYZ)
    return TTV_E_UNSUPPORTED;
  // 16-byte loads when every row starts on a 16-byte boundary
  const bool vec = V % 4 == 0 && aligned16(probs);
  return launch_status(launch_tree_expand(B, F, V, k, probs, frontier, n_in, Ncap, parents, tokens,
                                          src_row, n_out, dev_status, vec,
                                          static_cast<hipStream_t>(stream)));
}

ttv_status ttv_tree_merge(int32_t B, int32_t S, int32_t Ls, const int32_t* seqs,
                          const int32_t* seq_len, const int32_t* root_tok, int32_t Ncap,
                          int32_t* parents, int32_t* tokens, int32_t* src, int32_t* n_out,
                          int32_t* dev_status, void* stream) {
  if (!seqs || !seq_len || !root_tok || !parents || !tokens || !n_out) return TTV_E_NULL;
  if (B < 1 || S < 1 || Ls < 1 || Ncap < 1) return TTV_E_SHAPE;
  if (S > kMergeMaxSeqs || Ls > kMergeMaxLen || Ncap > TTV_MAX_NODES || B > 2147483647 / 64)
    return TTV_E_UNSUPPORTED;
  return launch_status(launch_tree_merge(B, S, Ls, seqs, seq_len, root_tok, Ncap, parents, tokens,
                                         src, n_out, dev_status,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Host checks of the logits processing arguments shared by the entry points.
ttv_status probs_args_ok(int32_t V, float temperature, int32_t topk, float top_p) {
  if (V < 1 || topk < 0 || !std::isfinite(temperature) || !(temperature > 0.f) ||
      !std::isfinite(probs_scale(temperature)) || !(top_p > 0.f && top_p <= 1.f))
    return TTV_E_SHAPE;
  if (topk > kProbsMaxTopk && topk < V) return TTV_E_UNSUPPORTED;
  return TTV_OK;
}

}  // namespace

extern "C" {

ttv_status ttv_probs_from_logits(int32_t R, int32_t V, float temperature, int32_t topk,
                                 float top_p, const float* logits, float* probs, void* stream) {
  if (!logits || !probs) return TTV_E_NULL;
  if (R < 1) return TTV_E_SHAPE;
  const ttv_status st = probs_args_ok(V, temperature, topk, top_p);
  if (st != TTV_OK) return st;
  const bool vec = V % 4 == 0 && aligned16(logits) && aligned16(probs);
  return launch_status(launch_probs(R, V, temperature, topk, top_p, logits, probs, nullptr, vec,
                                    static_cast<hipStream_t>(stream)));
}

// Row statistics of both tensors (2*B*N RowStats), then, for logits rows
// past the walk's registers, the residual (B*V floats); -1 for V the
// verifier does not take.
static size_t logits_workspace_bytes(int32_t B, int32_t N, int32_t V) {
  if (B < 1 || N < 1 || N > TTV_MAX_NODES || V < 1) return (size_t)-1;
  if (V % 4 != 0 || V > kMssGmMaxVocab) return (size_t)-1;
  const size_t stats = (size_t)2 * B * N * sizeof(RowStats);
  return V > kMssLogitsMaxVocab ? stats + (size_t)B * V * sizeof(float) : stats;
}

size_t ttv_tree_verify_logits_workspace_size(int32_t B, int32_t N, int32_t V) {
  return logits_workspace_bytes(B, N, V);
}

ttv_status ttv_tree_verify_logits(int32_t B, int32_t N, int32_t V, const int32_t* parents,
                                  const int32_t* tokens, const int32_t* n_nodes,
                                  const float* llm_logits, const float* ssm_logits,
                                  float temperature, int32_t topk, float top_p, uint64_t seed,
                                  uint64_t step, int32_t* path, int32_t* path_len,
                                  int32_t* out_tokens, int32_t* dev_status, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!parents || !tokens || !llm_logits || !ssm_logits || !path || !path_len || !out_tokens)
    return TTV_E_NULL;
  if (B < 1 || N < 1) return TTV_E_SHAPE;
  const ttv_status st = probs_args_ok(V, temperature, topk, top_p);
  if (st != TTV_OK) return st;
  if (N > TTV_MAX_NODES || (long)B * N > 0x7fffffffL) return TTV_E_UNSUPPORTED;
  const size_t need = logits_workspace_bytes(B, N, V);
  if (need == (size_t)-1) return TTV_E_UNSUPPORTED;
  if (!aligned16(llm_logits) || !aligned16(ssm_logits)) return TTV_E_ALIGN;
  if (!workspace || workspace_bytes < need) return TTV_E_WORKSPACE;
  if (!aligned16(workspace)) return TTV_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RowStats* st_llm = static_cast<RowStats*>(workspace);
  RowStats* st_ssm = st_llm + (size_t)B * N;
  // the residual, for rows past the walk's registers (16-byte aligned: the
  // statistics are 16-byte records)
  float* gm_w = V > kMssLogitsMaxVocab ? reinterpret_cast<float*>(st_ssm + (size_t)B * N) : nullptr;
  // each row's statistics, then the walk computes the probabilities it reads
  if (launch_probs(B * N, V, temperature, topk, top_p, llm_logits, nullptr, st_llm, true, s) !=
          hipSuccess ||
      launch_probs(B * N, V, temperature, topk, top_p, ssm_logits, nullptr, st_ssm, true, s) !=
          hipSuccess)
    return TTV_E_LAUNCH;
  return launch_status(launch_verify_mss(
      B, N, V, parents, tokens, n_nodes, llm_logits, ssm_logits,
      MssDraws{nullptr, nullptr, seed, step}, LogitRows{st_llm, st_ssm, probs_scale(temperature)},
      path, path_len, out_tokens, dev_status, gm_w, CommitArgs{}, s));
}

ttv_status ttv_kv_commit_inplace(ttv_dtype dt, int32_t B, int32_t N, int32_t Hkv, int32_t D,
                                 int32_t Lcap, void* k_cache, void* v_cache,
                                 const int32_t* cache_len_in, int32_t* cache_len_out,
                                 int32_t Lmax, const int32_t* path, const int32_t* path_len,
                                 int32_t* committed_src, int32_t* dev_status, void* stream) {
  if (dt != TTV_F32 && dt != TTV_BF16) return TTV_E_DTYPE;
  if (!k_cache || !v_cache || !cache_len_in || !cache_len_out || !path || !path_len)
    return TTV_E_NULL;
  if (B < 1 || N < 1 || Hkv < 1 || D < 1 || Lmax < 0 || Lcap < 0) return TTV_E_SHAPE;
  if (N > TTV_MAX_NODES || (D != 64 && D != 128)) return TTV_E_UNSUPPORTED;
  if ((long)Lmax + N > Lcap) return TTV_E_SHAPE;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return TTV_E_ALIGN;
  const int elt = dt == TTV_BF16 ? 2 : 4;
  return launch_status(launch_kv_commit_inplace(elt, B, N, Hkv, D, Lcap, k_cache, v_cache,
                                                cache_len_in, cache_len_out, Lmax, path,
                                                path_len, committed_src, dev_status,
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
