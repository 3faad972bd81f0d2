// launch.h -- host-side launch plans and launcher declarations (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ttv.h"

namespace ttv {

// Raises kernel `kern`'s dynamic-LDS limit to `bytes` (the most any launch of
// it requests) once per device and kernel, instead of on every launch.
hipError_t lds_limit_once(const void* kern, int bytes);

// ------------------------------------------------------------- attention --
// Launch plan of ttv_tree_attn, a pure function of the call's sizes (the
// size query and the call compute the same plan).
struct AttnPlan {
  bool mfma;           // matrix-core path (bf16 and >= 16 query rows per kv head)
  bool balanced;       // split planned on the device from the actual prefix lengths
  int rows;            // R = N * G query rows per (request, kv head)
  int rows_per_block;  // query rows handled by one workgroup
  int row_blocks;      // ceil(R / rows_per_block)
  int chunk_keys;      // fixed split: prefix keys per workgroup (multiple of 64)
  int chunks;          // fixed split: ceil(Lmax / chunk_keys); balanced: the most
                       // chunks one (request, kv head, row block) may get
  int items;           // balanced: workgroups launched
  size_t ws_bytes;     // split-KV partials (0 when chunks == 1)
};

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const void* k_tree;
  const void* v_tree;
  const int32_t* cache_len;
  const int32_t* parents;
  const int32_t* n_nodes;  // [B] nodes of each request's tree, or nullptr: N each
  void* out;
  float* lse;
  int32_t* dev_status;
  float* ws_acc;   // [B*Hkv][chunks][R][D] partial outputs: fp32 sums (fp32 output), or
                   // the normalised output in bf16 (bf16 output; 2 bytes per element)
  float* ws_ml;    // [B*Hkv][chunks][R][2]  running max (log2 units) and sum, right after
  int32_t* ws_nchunks;  // [B] balanced split: chunks request b got
  int B, N, Hq, Hkv, G, D, Lcap, Lmax, R;
  int rows_per_block, chunk_keys, chunks;
  int balanced, row_blocks, items;
  int tree_in_cache;  // k_tree/v_tree NULL: node i's K/V at cache row L_b + i
  float scale_log2;  // softmax scale * log2(e): scores are kept in log2 units
};

// Balanced split: at most this many requests (one per lane of a wavefront),
// and at least this many 64-key tiles per chunk.
constexpr int kBalancedMaxB = 64;
constexpr int kBalancedMinTiles = 2;

// Host validation of one ttv_tree_attn call (everything but the workspace)
// and its launch plan.
ttv_status attn_prepare(ttv_dtype dt, int B, int N, int Hq, int Hkv, int D, float scale,
                        const void* q, const void* k_cache, const void* v_cache, int Lcap,
                        const int32_t* cache_len, int Lmax, const void* k_tree,
                        const void* v_tree, const int32_t* parents, const void* out,
                        int rows_per_block, int chunk_keys, AttnPlan* p);
// The launches of a validated call; ws = p.ws_bytes of device scratch.
ttv_status launch_attn(const AttnPlan& p, ttv_dtype dt, int B, int N, int Hq, int Hkv, int D,
                       float scale, const void* q, const void* k_cache, const void* v_cache,
                       int Lcap, const int32_t* cache_len, int Lmax, const void* k_tree,
                       const void* v_tree, const int32_t* parents, const int32_t* n_nodes,
                       void* out, float* lse, uint64_t* anc_out, int32_t* depth_out,
                       int32_t* dev_status, void* ws, hipStream_t s);

hipError_t launch_attn_fma(const AttnArgs& a, bool bf16, hipStream_t s);
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_combine(const AttnArgs& a, bool bf16, hipStream_t s);

// -------------------------------------------------------------- topology --
hipError_t launch_topology(int B, int N, const int32_t* parents, const int32_t* n_nodes,
                           uint64_t* anc_out, int32_t* depth_out, int32_t* dev_status,
                           hipStream_t s);

// ---------------------------------------------------------- verification --
struct GreedyPlan {
  int splits;       // workgroups per logits row
  int slice;        // vocabulary entries per split (multiple of 4)
  size_t ws_bytes;  // (value, index) partial argmax per (row, split)
};
GreedyPlan greedy_plan(int B, int N, int V);

hipError_t launch_verify_greedy(int B, int N, int V, const int32_t* parents,
                                const int32_t* tokens, const int32_t* n_nodes, const float* llm,
                                int32_t* path, int32_t* path_len, int32_t* out_tokens,
                                int32_t* dev_status, void* ws, const GreedyPlan& p,
                                hipStream_t s);

// Greedy verification and the KV commit in one pass: argmax partials, then
// one launch that scans each tree and copies the path's rows.
hipError_t launch_verify_greedy_commit(int B, int N, int V, const int32_t* parents,
                                       const int32_t* tokens, const int32_t* n_nodes,
                                       const float* llm, int32_t* path,
                                       int32_t* path_len, int32_t* out_tokens,
                                       int32_t* dev_status, void* ws, const GreedyPlan& p,
                                       int elt, int Hkv, int D, int Lcap, int Lmax,
                                       const void* k_tree, const void* v_tree, void* k_cache,
                                       void* v_cache, const int32_t* cache_len_in,
                                       int32_t* cache_len_out, int32_t* committed_src,
                                       hipStream_t s);

// The KV commit of the accepted path, done by the verifier's own workgroup
// (k_tree == nullptr: no commit).  row_vecs = 16-byte vectors per K/V row.
struct CommitArgs {
  int row_vecs, Hkv, Lcap, Lmax;
  const void* k_tree;
  const void* v_tree;
  void* k_cache;
  void* v_cache;
  const int32_t* cache_len_in;
  int32_t* cache_len_out;
  int32_t* committed_src;
};

// Uniforms of the stochastic verifier: u_accept == nullptr draws them from
// Philox4x64-10 (seed, step); otherwise u_accept[B,N] and u_bonus[B] hold them.
struct MssDraws {
  const float* u_accept;
  const float* u_bonus;
  uint64_t seed, step;
};

// Rows of llm / ssm given as logits: their statistics (from launch_probs in
// statistics mode) and c = (float)(log2(e) / T); st_llm == nullptr means the
// rows are probabilities.
struct RowStats;
struct LogitRows {
  const RowStats* st_llm;
  const RowStats* st_ssm;
  float c;
};

// Largest vocabulary the stochastic verifier holds in LDS (rows given as
// logits: kMssLogitsMaxVocab, 16-byte rows).  Larger vocabularies (V % 4 ==
// 0, at most kMssGmMaxVocab) keep the residual in global memory: gm_w, B*V
// floats of workspace, 16-byte aligned.
constexpr int kMssMaxVocab = 36864;
constexpr int kMssLogitsMaxVocab = 32768;
constexpr int kMssGmMaxVocab = 1 << 18;
hipError_t launch_verify_mss(int B, int N, int V, const int32_t* parents,
                             const int32_t* tokens, const int32_t* n_nodes, const float* llm,
                             const float* ssm, const MssDraws& dr, const LogitRows& lr,
                             int32_t* path, int32_t* path_len, int32_t* out_tokens,
                             int32_t* dev_status, float* gm_w, const CommitArgs& cm,
                             hipStream_t s);

// ----------------------------------------------------------------- commit --
hipError_t launch_kv_commit(int elt, int B, int N, int Hkv, int D, int Lcap,
                            const void* k_tree, const void* v_tree, void* k_cache,
                            void* v_cache, const int32_t* cache_len_in,
                            int32_t* cache_len_out, int Lmax, const int32_t* path,
                            const int32_t* path_len, int32_t* committed_src,
                            int32_t* dev_status, hipStream_t s);

// ------------------------------------------------------ tree expansion --
// Largest top-k one expansion call takes.
constexpr int kExpandMaxK = 16;
hipError_t launch_tree_expand(int B, int F, int V, int k, const float* probs,
                              const int32_t* frontier, const int32_t* n_in, int Ncap,
                              int32_t* parents, int32_t* tokens, int32_t* src_row,
                              int32_t* n_out, int32_t* dev_status, bool vec, hipStream_t s);

// ------------------------------------------------------------ tree merge --
constexpr int kMergeMaxSeqs = 64;   // sequences per request: one per lane of a wavefront
constexpr int kMergeMaxLen = 128;   // tokens per sequence (the tree has at most 128 nodes)
hipError_t launch_tree_merge(int B, int S, int Ls, const int32_t* seqs, const int32_t* seq_len,
                             const int32_t* root_tok, int Ncap, int32_t* parents, int32_t* tokens,
                             int32_t* src, int32_t* n_out, int32_t* dev_status, hipStream_t s);

// --------------------------------------------------------- probabilities --
constexpr int kProbsMaxTopk = 512;  // the top-k bound takes ceil(k/16) <= 64 maxima per wave
// probabilities (probs != nullptr) or each row's statistics (stats)
hipError_t launch_probs(int R, int V, float T, int topk, float top_p, const float* logits,
                        float* probs, RowStats* stats, bool vec, hipStream_t s);
float probs_scale(float T);  // (float)(log2(e) / T)

hipError_t launch_kv_commit_inplace(int elt, int B, int N, int Hkv, int D, int Lcap, void* k_cache,
                                    void* v_cache, const int32_t* cache_len_in,
                                    int32_t* cache_len_out, int Lmax, const int32_t* path,
                                    const int32_t* path_len, int32_t* committed_src,
                                    int32_t* dev_status, hipStream_t s);

}  // namespace ttv
