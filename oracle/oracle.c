/*
 * oracle.c -- plain, slow CPU reference of the tree-based parallel decoding
 * step.  TEST INFRASTRUCTURE ONLY: the library under test never links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or constant with the GPU library.
 *
 * Every function follows a plain definition, in the order the definition
 * states it, with no blocking, fusion or reordering:
 *   [SI]  "SpecInfer: Accelerating Generative Large Language Model Serving with
 *         Tree-based Speculative Inference and Verification" (paperlayer.ai
 *         summary of arXiv 2305.09781v4).
 *   [SSD] "Accelerating LLM Inference with Staged Speculative Decoding"
 *         (paperlayer.ai summary of arXiv 2308.04623v1).
 * Attention is computed in fp64 from the exact input values.  The stochastic
 * verifier works in fp32 with the operation order its definition fixes,
 * because its accept/reject decisions and sampled tokens are integers that
 * must come out the same on every implementation.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -fPIC -shared -lm
 * (-ffp-contract=off: no multiply-add is fused unless written as fmaf).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_SHAPE 2
#define ORC_E_TREE 7

/* ------------------------------------------------------------------------ */
/* Tree topology.  [SI] §4 "Tree Attention": node i stands for the token     */
/* sequence on the path root -> i.  A tree is valid iff parents[0] == -1 and  */
/* 0 <= parents[i] < i.                                                       */
/* ------------------------------------------------------------------------ */
static int tree_is_valid(int N, const int32_t* par) {
  if (par[0] != -1) return 0;
  for (int i = 1; i < N; ++i)
    if (par[i] < 0 || par[i] >= i) return 0;
  return 1;
}

/* Nodes of request b: n_nodes[b] when given (a batch of trees of different
 * sizes stored in rows of N entries; entries at or past n_nodes[b] are
 * padding and never read), else N.  [SI] §5 "Scheduling": requests of a
 * continuous batch are verified together whatever their tree sizes. */
static int nodes_of(const int32_t* n_nodes, int b, int N) {
  return n_nodes ? n_nodes[b] : N;
}

/* depth[b,i] = edges from the root; anc[b,i,w] = bitset of the nodes on the
 * path root -> i (i included), found by walking the parent pointers.  Padding
 * nodes (i >= n) get depth -1 and no bits; n outside [1, N] is ORC_E_SHAPE. */
void orc_topology(int B, int N, const int32_t* parents, const int32_t* n_nodes,
                  int32_t* depth, uint64_t* anc, int32_t* status) {
  const int W = (N + 63) / 64;
  for (int b = 0; b < B; ++b) {
    const int32_t* par = parents + (size_t)b * N;
    int32_t* dep = depth + (size_t)b * N;
    uint64_t* an = anc + (size_t)b * N * W;
    const int n = nodes_of(n_nodes, b, N);
    memset(an, 0, sizeof(uint64_t) * (size_t)N * W);
    for (int i = 0; i < N; ++i) dep[i] = -1;
    if (n < 1 || n > N) {
      status[b] = ORC_E_SHAPE;
      continue;
    }
    if (!tree_is_valid(n, par)) {
      status[b] = ORC_E_TREE;
      continue;
    }
    for (int i = 0; i < n; ++i) {
      int d = -1;
      for (int j = i; j != -1; j = par[j]) {
        an[(size_t)i * W + j / 64] |= (uint64_t)1 << (j % 64);
        d += 1;
      }
      dep[i] = d;
    }
    status[b] = ORC_OK;
  }
}

/* ------------------------------------------------------------------------ */
/* Tree attention.  [SI] §4 "Tree Attention" / "Tree-Based Parallel          */
/* Decoding": the output of node i is causal attention of q_i over the        */
/* sequence node i represents = the request's prefix KV rows 0..L_b-1 then    */
/* the tree KV rows of the nodes on root -> i, in that order ([SSD] §3        */
/* "Implementation": cache part + in-batch part).  Query head hq reads kv     */
/* head hq / (Hq/Hkv).                                                        */
/*   s_j = scale * sum_d q[d] k_j[d]   (fp64)                                 */
/*   o   = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),  m = max_j s_j        */
/*   lse = m + ln sum_j exp(s_j - m)                                          */
/* Only the listed rows (b, i, hq) are computed, so a large problem can be     */
/* checked on a sample.  Inputs are float arrays holding the exact values      */
/* (bf16 widens to float exactly).  status[r]: 0, ORC_E_TREE, ORC_E_SHAPE;     */
/* a rejected row gets o = 0 and lse = 0.  With n_nodes, rows of padding       */
/* nodes (i >= n_nodes[b]) are 0 with the request's status.                    */
/* ------------------------------------------------------------------------ */
void orc_tree_attn_rows(int B, int N, int Hq, int Hkv, int D, double scale,
                        const float* q, const float* k_cache,
                        const float* v_cache, int Lcap,
                        const int32_t* cache_len, const float* k_tree,
                        const float* v_tree, const int32_t* parents,
                        const int32_t* n_nodes, int nrows, const int32_t* rows,
                        double* out, double* lse, int32_t* status) {
  const int G = Hq / Hkv;
  (void)B;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nrows; ++r) {
    const int b = rows[3 * r + 0], i = rows[3 * r + 1], hq = rows[3 * r + 2];
    const int h = hq / G;
    const int32_t* par = parents + (size_t)b * N;
    const int L = cache_len[b];
    double* o = out + (size_t)r * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    lse[r] = 0.0;
    const int n = nodes_of(n_nodes, b, N);
    if (n < 1 || n > N) { status[r] = ORC_E_SHAPE; continue; }
    if (!tree_is_valid(n, par)) { status[r] = ORC_E_TREE; continue; }
    if (L < 0 || L > Lcap || i < 0 || i >= N) { status[r] = ORC_E_SHAPE; continue; }
    if (i >= n) { status[r] = ORC_OK; continue; } /* a padding node: zero output */

    /* the key/value rows of the sequence node i represents */
    int* path = (int*)malloc(sizeof(int) * (size_t)N);
    int depth = 0;
    for (int j = i; j != -1; j = par[j]) path[depth++] = j; /* i .. root */
    const int nkeys = L + depth;
    const float** krow = (const float**)malloc(sizeof(float*) * (size_t)nkeys);
    const float** vrow = (const float**)malloc(sizeof(float*) * (size_t)nkeys);
    double* s = (double*)malloc(sizeof(double) * (size_t)nkeys);
    for (int t = 0; t < L; ++t) {
      size_t off = (((size_t)b * Hkv + h) * Lcap + t) * D;
      krow[t] = k_cache + off;
      vrow[t] = v_cache + off;
    }
    for (int t = 0; t < depth; ++t) {
      int node = path[depth - 1 - t]; /* root first */
      size_t off = (((size_t)b * Hkv + h) * N + node) * D;
      krow[L + t] = k_tree + off;
      vrow[L + t] = v_tree + off;
    }
    const float* qi = q + (((size_t)b * N + i) * Hq + hq) * D;

    /* pass 1: scores and their maximum */
    double m = -INFINITY;
    for (int t = 0; t < nkeys; ++t) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += (double)qi[d] * (double)krow[t][d];
      s[t] = scale * dot;
      if (s[t] > m) m = s[t];
    }
    /* pass 2: normaliser and weighted sum of values */
    double den = 0.0;
    for (int t = 0; t < nkeys; ++t) {
      double e = exp(s[t] - m);
      den += e;
      for (int d = 0; d < D; ++d) o[d] += e * (double)vrow[t][d];
    }
    for (int d = 0; d < D; ++d) o[d] /= den;
    lse[r] = m + log(den);
    status[r] = ORC_OK;
    free(path);
    free(krow);
    free(vrow);
    free(s);
  }
}

/* Writes path[b,k] (node at depth k, -1 after the end) for the path root->end
 * and returns its length (end's depth + 1). */
static int write_path(int N, const int32_t* par, int end, int32_t* path) {
  int len = 0;
  for (int j = end; j != -1; j = par[j]) ++len;
  for (int k = 0; k < N; ++k) path[k] = -1;
  int k = len - 1;
  for (int j = end; j != -1; j = par[j]) path[k--] = j;
  return len;
}

/* ------------------------------------------------------------------------ */
/* Greedy verification.  [SI] §4 "Token Tree Verification" and §6 (greedy    */
/* verification emits exactly incremental decoding's tokens):                 */
/*   amax[u] = argmax_v llm[b,u,v]  (fp32 compare, first index wins ties)     */
/*   accepted(0); accepted(c) iff accepted(parent c) and tokens[c] ==          */
/*                amax[parent c]                                               */
/*   end d = deepest accepted node (lowest index on ties)                     */
/*   path = root -> d; out_tokens = tokens of path[1..], then amax[d].        */
/* ------------------------------------------------------------------------ */
void orc_verify_greedy(int B, int N, int V, const int32_t* parents,
                       const int32_t* tokens, const int32_t* n_nodes,
                       const float* llm, int32_t* path, int32_t* path_len,
                       int32_t* out_tokens, int32_t* status) {
  int32_t* amax = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int32_t* dep = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  char* acc = (char*)malloc((size_t)N);
  for (int b = 0; b < B; ++b) {
    const int32_t* par = parents + (size_t)b * N;
    const int32_t* tok = tokens + (size_t)b * N;
    int32_t* pb = path + (size_t)b * N;
    int32_t* ob = out_tokens + (size_t)b * N;
    const int n = nodes_of(n_nodes, b, N);
    for (int k = 0; k < N; ++k) { pb[k] = -1; ob[k] = -1; }
    if (n < 1 || n > N) {
      path_len[b] = 0;
      status[b] = ORC_E_SHAPE;
      continue;
    }
    if (!tree_is_valid(n, par)) {
      path_len[b] = 0;
      status[b] = ORC_E_TREE;
      continue;
    }
    for (int u = 0; u < n; ++u) {
      const float* row = llm + ((size_t)b * N + u) * V;
      int best = 0;
      for (int v = 1; v < V; ++v)
        if (row[v] > row[best]) best = v;
      amax[u] = best;
    }
    acc[0] = 1;
    dep[0] = 0;
    for (int c = 1; c < n; ++c) {
      dep[c] = dep[par[c]] + 1;
      acc[c] = acc[par[c]] && tok[c] == amax[par[c]];
    }
    int end = 0;
    for (int c = 1; c < n; ++c)
      if (acc[c] && dep[c] > dep[end]) end = c;
    int len = write_path(N, par, end, pb);
    for (int k = 0; k + 1 < len; ++k) ob[k] = tok[pb[k + 1]];
    ob[len - 1] = amax[end];
    path_len[b] = len;
    status[b] = ORC_OK;
  }
  free(amax);
  free(dep);
  free(acc);
}

/* ------------------------------------------------------------------------ */
/* Counter-based random numbers: Philox4x64-10 as published by Salmon,        */
/* Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"       */
/* (SC'11).  A 256-bit counter c (four 64-bit words, word 0 least            */
/* significant) and a 128-bit key k give four 64-bit outputs after ten       */
/* rounds.  One round multiplies c0 and c2 by the paper's two 64-bit         */
/* multipliers, keeps the high and low halves of each 128-bit product, and    */
/* permutes:  c' = (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1,       */
/* lo(M0*c0)).  Between rounds the key is bumped by the paper's two Weyl      */
/* constants (the golden ratio and sqrt(3) - 1 in 64-bit fixed point).        */
/* ------------------------------------------------------------------------ */
static void mul64_hilo(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
  const unsigned __int128 p = (unsigned __int128)a * b;
  *hi = (uint64_t)(p >> 64);
  *lo = (uint64_t)p;
}

void orc_philox4x64_10(const uint64_t* ctr, const uint64_t* key, uint64_t* out) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint64_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { k0 += W0; k1 += W1; }
    uint64_t hi0, lo0, hi1, lo1;
    mul64_hilo(M0, c0, &hi0, &lo0);
    mul64_hilo(M1, c2, &hi1, &lo1);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 24 high bits of output word 0 for key (seed, 0) and counter
 * (j, u, b, step): the ratio test of the j-th child (ascending node index,
 * j = 0, 1, ..) of node u, or the final draw at u when j = 2^63. */
static uint64_t philox_bits24(uint64_t seed, uint64_t step, uint64_t j, int u, int b) {
  const uint64_t ctr[4] = {j, (uint64_t)u, (uint64_t)b, step};
  const uint64_t key[2] = {seed, 0};
  uint64_t out[4];
  orc_philox4x64_10(ctr, key, out);
  return out[0] >> 40;
}
#define ORC_BONUS_ORDINAL 0x8000000000000000ull

/* ------------------------------------------------------------------------ */
/* Stochastic verification: multi-step speculative sampling, [SI] §4 "Token   */
/* Verification" (verifies across branches and keeps the LLM's distribution). */
/* The page states the guarantee, not the arithmetic; the arithmetic below is  */
/* this library's fixed reading of it (residual w with mass s, children in     */
/* ascending node index, one uniform per tested child and one per request     */
/* for the final sample, exact integer sums in 2^-40 units).  The uniforms    */
/* are either given (u_accept[b,c] for the test of child c, u_bonus[b]) or    */
/* drawn from Philox4x64-10 with key (seed, 0): the test of the j-th child of */
/* u uses counter (j, u, b, step), the final draw at u counter (2^63, u, b,   */
/* step); r = (out0 >> 40) * 2^-24 and R = out0 >> 40.                       */
/* ------------------------------------------------------------------------ */
static uint64_t fx(float x) { return (uint64_t)((double)x * 1099511627776.0); }

static float mass(const float* w, int V) {
  uint64_t S = 0;
  for (int v = 0; v < V; ++v) S += fx(w[v]);
  return (float)((double)S * (1.0 / 1099511627776.0));
}

/* Inverse-CDF draw from the unnormalised w with the 24-bit integer R. */
static int sample_from(const float* w, int V, uint64_t R) {
  uint64_t S = 0;
  for (int v = 0; v < V; ++v) S += fx(w[v]);
  if (S == 0) {
    int best = 0;
    for (int v = 1; v < V; ++v)
      if (w[v] > w[best]) best = v;
    return best;
  }
  uint64_t hi = S >> 24, lo = S & 0xFFFFFFu;
  uint64_t T = R * hi + ((R * lo) >> 24); /* floor(R*S / 2^24), no overflow */
  uint64_t c = 0;
  for (int v = 0; v < V; ++v) {
    c += fx(w[v]);
    if (c > T) return v;
  }
  return V - 1; /* unreachable: T < S */
}

/* One request's walk; the uniforms come from u_accept/u_bonus when they are
 * given (seeded == 0), else from Philox (seed, step). */
static void mss_request(int b, int N, int n, int V, const int32_t* par, const int32_t* tok,
                        const float* llm, const float* ssm, const float* u_accept,
                        const float* u_bonus, int seeded, uint64_t seed, uint64_t step,
                        int32_t* pb, int32_t* ob, int32_t* path_len, int32_t* status) {
  for (int k = 0; k < N; ++k) { pb[k] = -1; ob[k] = -1; }
  if (n < 1 || n > N) {
    path_len[b] = 0;
    status[b] = ORC_E_SHAPE;
    return;
  }
  if (!tree_is_valid(n, par)) {
    path_len[b] = 0;
    status[b] = ORC_E_TREE;
    return;
  }
  int tokens_ok = 1; /* every drafted token must index the vocabulary */
  for (int c = 1; c < n; ++c)
    if (tok[c] < 0 || tok[c] >= V) tokens_ok = 0;
  if (!tokens_ok) {
    path_len[b] = 0;
    status[b] = ORC_E_SHAPE;
    return;
  }
  float* w = (float*)malloc(sizeof(float) * (size_t)V);
  int u = 0;
  for (;;) {
    const float* p_u = llm + ((size_t)b * N + u) * V;
    memcpy(w, p_u, sizeof(float) * (size_t)V);
    float s = 1.0f;
    int next = -1;
    uint64_t j = 0; /* attempt ordinal at u */
    for (int c = u + 1; c < n; ++c) { /* children of u, ascending index */
      if (par[c] != u) continue;
      const float* qc = ssm + ((size_t)b * N + c) * V;
      const int x = tok[c];
      const float r = seeded ? (float)philox_bits24(seed, step, j, u, b) * 0x1p-24f
                             : u_accept[(size_t)b * N + c];
      ++j;
      const float lhs = (r * qc[x]) * s;
      if (lhs < w[x]) { next = c; break; } /* accepted */
      /* rejected: w <- max(w - s*q, 0), s <- its mass */
      for (int v = 0; v < V; ++v) {
        float d = fmaf(-s, qc[v], w[v]);
        w[v] = d > 0.0f ? d : 0.0f;
      }
      s = mass(w, V);
      if (s == 0.0f) { /* empty residual: stop, sample from p_u */
        memcpy(w, p_u, sizeof(float) * (size_t)V);
        break;
      }
    }
    if (next < 0) break;
    u = next;
  }
  const uint64_t R = seeded ? philox_bits24(seed, step, ORC_BONUS_ORDINAL, u, b)
                            : (uint64_t)(u_bonus[b] * 16777216.0f); /* exact: scaling by 2^24 */
  const int bonus = sample_from(w, V, R);
  const int len = write_path(N, par, u, pb);
  for (int k = 0; k + 1 < len; ++k) ob[k] = tok[pb[k + 1]];
  ob[len - 1] = bonus;
  path_len[b] = len;
  status[b] = ORC_OK;
  free(w);
}

void orc_verify_mss(int B, int N, int V, const int32_t* parents,
                    const int32_t* tokens, const int32_t* n_nodes, const float* llm,
                    const float* ssm, const float* u_accept, const float* u_bonus,
                    int32_t* path, int32_t* path_len, int32_t* out_tokens,
                    int32_t* status) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < B; ++b)
    mss_request(b, N, nodes_of(n_nodes, b, N), V, parents + (size_t)b * N, tokens + (size_t)b * N, llm, ssm, u_accept,
                u_bonus, 0, 0, 0, path + (size_t)b * N, out_tokens + (size_t)b * N, path_len,
                status);
}

void orc_verify_mss_seeded(int B, int N, int V, const int32_t* parents,
                           const int32_t* tokens, const int32_t* n_nodes, const float* llm,
                           const float* ssm, uint64_t seed, uint64_t step, int32_t* path,
                           int32_t* path_len, int32_t* out_tokens, int32_t* status) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < B; ++b)
    mss_request(b, N, nodes_of(n_nodes, b, N), V, parents + (size_t)b * N, tokens + (size_t)b * N, llm, ssm, NULL, NULL,
                1, seed, step, path + (size_t)b * N, out_tokens + (size_t)b * N, path_len,
                status);
}

/* ------------------------------------------------------------------------ */
/* KV commit.  [SI] §4 "Tree-Based Parallel Decoding": verified and          */
/* speculated tokens share one KV cache; the accepted path's rows are kept.   */
/*   cache[b,h,L+j,:] = tree[b,h,path[b,j],:]  (j < path_len[b], every h)     */
/*   new_len[b] = L + path_len[b]; committed_src[b,j] = path[b,j] or -1.      */
/* Byte copies (elt = bytes per element).  A request whose L or path breaks   */
/* the bounds is left untouched (status ORC_E_SHAPE, new_len = L).            */
/* ------------------------------------------------------------------------ */
void orc_kv_commit(int B, int N, int Hkv, int D, int elt, int Lcap, int Lmax,
                   const void* k_tree, const void* v_tree, void* k_cache,
                   void* v_cache, const int32_t* cache_len_in,
                   int32_t* cache_len_out, const int32_t* path,
                   const int32_t* path_len, int32_t* committed_src,
                   int32_t* status) {
  const size_t row = (size_t)D * elt;
  for (int b = 0; b < B; ++b) {
    const int L = cache_len_in[b];
    const int n = path_len[b];
    const int32_t* pb = path + (size_t)b * N;
    int ok = L >= 0 && L <= Lmax && L <= Lcap && n >= 0 && n <= N &&
             L + n <= Lcap;
    for (int j = 0; ok && j < n; ++j)
      if (pb[j] < 0 || pb[j] >= N) ok = 0;
    for (int j = 0; j < N; ++j)
      committed_src[(size_t)b * N + j] = (ok && j < n) ? pb[j] : -1;
    if (!ok) {
      cache_len_out[b] = L;
      status[b] = ORC_E_SHAPE;
      continue;
    }
    for (int h = 0; h < Hkv; ++h)
      for (int j = 0; j < n; ++j) {
        size_t src = (((size_t)b * Hkv + h) * N + pb[j]) * row;
        size_t dst = (((size_t)b * Hkv + h) * Lcap + (L + j)) * row;
        memcpy((char*)k_cache + dst, (const char*)k_tree + src, row);
        memcpy((char*)v_cache + dst, (const char*)v_tree + src, row);
      }
    cache_len_out[b] = L + n;
    status[b] = ORC_OK;
  }
}

/* ------------------------------------------------------------------------ */
/* Expansion-based token-tree construction, one level.  [SI] §3 "Expansion- */
/* based token tree construction": a speculative model's top-k tokens at a   */
/* node become that node's children (the LLM's token is often among them).   */
/* For request b, the existing tree has n_in[b] nodes; every frontier node   */
/* fr = frontier[b,f] >= 0, taken in order of f, gets k children: the k      */
/* tokens of highest probability in its row probs[b,f,:], most probable      */
/* first, an equal probability going to the lower token id.  They are        */
/* appended as nodes n_in[b] + r*k + j (r = the rank of f among the frontier */
/* entries >= 0), with src_row = f, so parents < children holds.             */
/* A frontier entry outside [-1, n_in[b]) gives ORC_E_TREE, more than Ncap   */
/* nodes (or n_in[b] < 1) ORC_E_SHAPE; such a request keeps n_out = n_in and */
/* gets nothing written.  Selection by repeated scans for the best untaken   */
/* token (k passes over the row).                                            */
/* ------------------------------------------------------------------------ */
void orc_tree_expand(int B, int F, int V, int k, const float* probs, const int32_t* frontier,
                     const int32_t* n_in, int Ncap, int32_t* parents, int32_t* tokens,
                     int32_t* src_row, int32_t* n_out, int32_t* status) {
  unsigned char* taken = (unsigned char*)malloc((size_t)V);
  for (int b = 0; b < B; ++b) {
    const int32_t* fb = frontier + (size_t)b * F;
    const int nin = n_in[b];
    int count = 0, bad = 0;
    for (int f = 0; f < F; ++f) {
      if (fb[f] < -1 || fb[f] >= nin) bad = 1;
      if (fb[f] >= 0) ++count;
    }
    n_out[b] = nin;
    if (bad) {
      status[b] = ORC_E_TREE;
      continue;
    }
    if (nin < 1 || (long)nin + (long)count * k > Ncap) {
      status[b] = ORC_E_SHAPE;
      continue;
    }
    int pos = nin;
    for (int f = 0; f < F; ++f) {
      if (fb[f] < 0) continue;
      const float* row = probs + ((size_t)b * F + f) * V;
      memset(taken, 0, (size_t)V);
      for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int v = 0; v < V; ++v)
          if (!taken[v] && (best < 0 || row[v] > row[best])) best = v;  /* strict: lower id wins ties */
        taken[best] = 1;
        parents[(size_t)b * Ncap + pos] = fb[f];
        tokens[(size_t)b * Ncap + pos] = best;
        src_row[(size_t)b * Ncap + pos] = f;
        ++pos;
      }
    }
    n_out[b] = pos;
    status[b] = ORC_OK;
  }
  free(taken);
}

/* ------------------------------------------------------------------------ */
/* Merge-based token-tree construction.  [SI] §3 "Merge-based token tree     */
/* construction": the outputs of several speculative models are combined    */
/* into one tree that contains each of their token sequences.  For request b */
/* the S sequences seqs[b,s,0..len[b,s]-1] hang below the root (node 0,      */
/* token root_tok[b]); every distinct non-empty prefix becomes one node, a    */
/* shared prefix once.  Nodes are numbered depth by depth, and within a depth */
/* in order of the lowest sequence index whose prefix it is (its "leader");   */
/* src[b,node] = s*Ls + d for leader s and position d (-1 for the root).     */
/* A length outside [0, Ls] or more than Ncap nodes gives ORC_E_SHAPE (n_out */
/* = 0, nothing written).  Prefixes are compared token by token.             */
/* ------------------------------------------------------------------------ */
static int same_prefix(const int32_t* a, const int32_t* c, int d) {
  for (int t = 0; t < d; ++t)
    if (a[t] != c[t]) return 0;
  return 1;
}

void orc_tree_merge(int B, int S, int Ls, const int32_t* seqs, const int32_t* seq_len,
                    const int32_t* root_tok, int Ncap, int32_t* parents, int32_t* tokens,
                    int32_t* src, int32_t* n_out, int32_t* status) {
  int32_t* node_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)S * (Ls + 1));
  for (int b = 0; b < B; ++b) {
    const int32_t* sq = seqs + (size_t)b * S * Ls;
    const int32_t* ln = seq_len + (size_t)b * S;
    int bad = 0, maxlen = 0;
    for (int s = 0; s < S; ++s) {
      if (ln[s] < 0 || ln[s] > Ls) bad = 1;
      else if (ln[s] > maxlen) maxlen = ln[s];
    }
    /* count the nodes first: a request that does not fit gets nothing */
    int n = 1;
    if (!bad) {
      for (int d = 1; d <= maxlen; ++d)
        for (int s = 0; s < S; ++s) {
          if (ln[s] < d) continue;
          int leader = 1;
          for (int t = 0; t < s && leader; ++t)
            if (ln[t] >= d && same_prefix(sq + (size_t)t * Ls, sq + (size_t)s * Ls, d)) leader = 0;
          n += leader;
        }
    }
    if (bad || n > Ncap) {
      n_out[b] = 0;
      status[b] = ORC_E_SHAPE;
      continue;
    }
    int32_t* pb = parents + (size_t)b * Ncap;
    int32_t* tb = tokens + (size_t)b * Ncap;
    int32_t* rb = src + (size_t)b * Ncap;
    pb[0] = -1;
    tb[0] = root_tok[b];
    rb[0] = -1;
    for (int s = 0; s < S; ++s) node_of[(size_t)s * (Ls + 1)] = 0;
    int next = 1;
    for (int d = 1; d <= maxlen; ++d)
      for (int s = 0; s < S; ++s) {
        if (ln[s] < d) continue;
        int lead = s;
        for (int t = 0; t < s; ++t)
          if (ln[t] >= d && same_prefix(sq + (size_t)t * Ls, sq + (size_t)s * Ls, d)) {
            lead = t;
            break;
          }
        if (lead == s) {
          pb[next] = node_of[(size_t)s * (Ls + 1) + d - 1];
          tb[next] = sq[(size_t)s * Ls + d - 1];
          rb[next] = s * Ls + d - 1;
          node_of[(size_t)s * (Ls + 1) + d] = next++;
        } else {
          node_of[(size_t)s * (Ls + 1) + d] = node_of[(size_t)lead * (Ls + 1) + d];
        }
      }
    n_out[b] = next;
    status[b] = ORC_OK;
  }
  free(node_of);
}

/* ------------------------------------------------------------------------ */
/* Probabilities from logits.  [SI] §4 "Token Verification" takes the LLM's  */
/* and the speculators' next-token distributions for stochastic decoding     */
/* (§7 "Multi-sample decoding": top-k or top-p sampling); [SSD] §4 samples    */
/* with top-k (k = 50) at temperature T = 1.  Row r of logits z:             */
/*   order  tokens by logit, higher first, equal logits by lower token id;   */
/*   top-k  with 0 < topk < V, keep the first topk in that order;            */
/*   top-p  with 0 < top_p < 1, keep the shortest prefix (of what top-k      */
/*          kept, in the same order) holding at least the share top_p of its */
/*          probability mass;                                                */
/*   p_v    proportional to exp((z_v - m) / T) over the kept tokens, 0 off   */
/*          them, m = the largest logit.                                     */
/* The arithmetic is fixed exactly (the GPU computes the same bits): with    */
/* c = (float)(log2(e) / T) the exponent is t_v = (z_v - m) * c in fp32 and   */
/* e_v = 2^t_v by range reduction to the nearest integer n and the Taylor    */
/* polynomial of 2^f = exp(f ln 2), |f| <= 1/2, to degree 7 in Horner form    */
/* with fused multiply-adds (truncation error below 1e-8 relative), 0 when   */
/* n < -125; masses are M_v = floor(e_v * 2^40) as exact integers; top-p      */
/* keeps the prefix up to the token where the running mass first reaches     */
/* ceil(P * S / 2^24), P = floor(top_p * 2^24), S the kept mass before top-p; */
/* p_v = e_v * (float)(2^40 / S') in fp32, S' the kept mass.                   */
/* ------------------------------------------------------------------------ */
#define ORC_LOG2E 1.4426950408889634
#define ORC_LN2 0.6931471805599453

/* Taylor coefficients ln(2)^k / k!, each from the previous one by one       */
/* multiplication and one division in double, then rounded to float.         */
static void exp2_coefficients(float* cf) {
  double a = 1.0;
  cf[0] = 1.0f;
  for (int k = 1; k <= 7; ++k) {
    a = (a * ORC_LN2) / (double)k;
    cf[k] = (float)a;
  }
}

static float exp2_taylor(float t, const float* cf) {
  const float n = rintf(t); /* nearest integer, ties to even */
  if (n < -125.0f) return 0.0f;
  const float f = t - n; /* exact, |f| <= 1/2 */
  float p = cf[7];
  for (int k = 6; k >= 0; --k) p = fmaf(p, f, cf[k]);
  return ldexpf(p, (int)n);
}

static uint64_t mass40(float e) { return (uint64_t)((double)e * 1099511627776.0); }

/* exact 2^t of the probabilities' definition, for the pins */
void orc_exp2_taylor(int n, const float* t, float* out) {
  float cf[8];
  exp2_coefficients(cf);
  for (int i = 0; i < n; ++i) out[i] = exp2_taylor(t[i], cf);
}

static const float* g_sort_z; /* the row being ordered (qsort has no context) */
static int by_logit_then_id(const void* a, const void* b) {
  const int i = *(const int*)a, j = *(const int*)b;
  if (g_sort_z[i] > g_sort_z[j]) return -1;
  if (g_sort_z[i] < g_sort_z[j]) return 1;
  return i < j ? -1 : (i > j ? 1 : 0);
}

void orc_probs_from_logits(int R, int V, float T, int topk, float top_p, const float* logits,
                           float* probs) {
  float cf[8];
  exp2_coefficients(cf);
  const float c = (float)(ORC_LOG2E / (double)T);
  int* order = (int*)malloc(sizeof(int) * (size_t)V);
  float* e = (float*)malloc(sizeof(float) * (size_t)V);
  for (int r = 0; r < R; ++r) {
    const float* z = logits + (size_t)r * V;
    float* p = probs + (size_t)r * V;
    for (int v = 0; v < V; ++v) order[v] = v;
    g_sort_z = z;
    qsort(order, (size_t)V, sizeof(int), by_logit_then_id);
    const float m = z[order[0]];
    for (int v = 0; v < V; ++v) e[v] = exp2_taylor((z[v] - m) * c, cf);
    int kept = (topk > 0 && topk < V) ? topk : V; /* the first `kept` of the order */
    if (top_p > 0.0f && top_p < 1.0f) {
      uint64_t S = 0;
      for (int j = 0; j < kept; ++j) S += mass40(e[order[j]]);
      const uint64_t P = (uint64_t)(top_p * 16777216.0f); /* exact: scaling by 2^24 */
      const uint64_t need = (uint64_t)(((unsigned __int128)P * S + 16777215u) >> 24);
      uint64_t run = 0;
      int j = 0;
      while (j < kept) {
        run += mass40(e[order[j]]);
        ++j;
        if (run >= need) break;
      }
      kept = j;
    }
    uint64_t S = 0;
    for (int j = 0; j < kept; ++j) S += mass40(e[order[j]]);
    const float inv = (float)(1099511627776.0 / (double)S);
    for (int v = 0; v < V; ++v) p[v] = 0.0f;
    for (int j = 0; j < kept; ++j) p[order[j]] = e[order[j]] * inv;
  }
  free(order);
  free(e);
}

/* ------------------------------------------------------------------------ */
/* KV commit with the tree inside the cache.  [SI] §4 "Tree-Based Parallel  */
/* Decoding": verified and speculated tokens are stored together in one      */
/* key-value cache.  Here tree node i's K/V sit at cache row L + i (L =      */
/* cache_len_in[b]); committing keeps the accepted path: row L + j takes the */
/* old row L + path[b,j] for j < n = path_len[b] (the n source rows are all  */
/* taken before any is written), cache_len_out[b] = L + n, committed_src as  */
/* in orc_kv_commit.  A bad length or path entry (as there, with the tree    */
/* rows L .. L+N-1 inside the cache) gives ORC_E_SHAPE and nothing written.  */
/* ------------------------------------------------------------------------ */
void orc_kv_commit_inplace(int B, int N, int Hkv, int D, int elt, int Lcap, int Lmax,
                           void* k_cache, void* v_cache, const int32_t* cache_len_in,
                           int32_t* cache_len_out, const int32_t* path,
                           const int32_t* path_len, int32_t* committed_src, int32_t* status) {
  const size_t row = (size_t)D * elt;
  char* tk = (char*)malloc(row * (size_t)(N > 0 ? N : 1));
  char* tv = (char*)malloc(row * (size_t)(N > 0 ? N : 1));
  for (int b = 0; b < B; ++b) {
    const int L = cache_len_in[b];
    const int n = path_len[b];
    const int32_t* pb = path + (size_t)b * N;
    int ok = L >= 0 && L <= Lmax && n >= 0 && n <= N && (long)L + N <= Lcap;
    for (int j = 0; ok && j < n; ++j)
      if (pb[j] < 0 || pb[j] >= N) ok = 0;
    for (int j = 0; j < N; ++j)
      committed_src[(size_t)b * N + j] = (ok && j < n) ? pb[j] : -1;
    if (!ok) {
      cache_len_out[b] = L;
      status[b] = ORC_E_SHAPE;
      continue;
    }
    for (int h = 0; h < Hkv; ++h) {
      const size_t base = ((size_t)b * Hkv + h) * Lcap;
      for (int j = 0; j < n; ++j) {  /* take the sources ... */
        memcpy(tk + (size_t)j * row, (const char*)k_cache + (base + L + pb[j]) * row, row);
        memcpy(tv + (size_t)j * row, (const char*)v_cache + (base + L + pb[j]) * row, row);
      }
      for (int j = 0; j < n; ++j) {  /* ... then write them */
        memcpy((char*)k_cache + (base + L + j) * row, tk + (size_t)j * row, row);
        memcpy((char*)v_cache + (base + L + j) * row, tv + (size_t)j * row, row);
      }
    }
    cache_len_out[b] = n + L;
    status[b] = ORC_OK;
  }
  free(tk);
  free(tv);
}

/* Threads of the parallel loops above (the CPU baseline runs the oracle on all
 * host cores and on one). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }
