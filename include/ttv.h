/*
 * ttv.h -- C ABI of the token-tree verification library (tree-based parallel
 * decoding step of tree speculative inference) for AMD Instinct MI355X (gfx950).
 *
 * Sources cited below (page title, then the section on it):
 *   [SI]  "SpecInfer: Accelerating Generative Large Language Model Serving with
 *         Tree-based Speculative Inference and Verification" -- source-linked
 *         summary of arXiv 2305.09781v4 (paperlayer.ai).
 *   [SSD] "Accelerating LLM Inference with Staged Speculative Decoding" --
 *         source-linked summary of arXiv 2308.04623v1 (paperlayer.ai).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument except `stream` is a DEVICE pointer owned by the
 *    caller.  The library never allocates, frees or retains a pointer.
 *  - Calls are asynchronous on `stream` (NULL = the default stream); no call
 *    synchronises the host.  Failures inside a kernel surface at the caller's
 *    next synchronisation.
 *  - All arguments are validated on the host BEFORE any HIP call, so every
 *    error status below except TTV_E_LAUNCH can be produced on a machine
 *    without a GPU.  On an error status nothing has been enqueued.
 *  - Per-request problems that only the device can see (a malformed tree, a
 *    prefix length that breaks the host's promise) are reported in the nullable
 *    `dev_status[B]` array (TTV_OK or the error code per request); the outputs
 *    of such a request are defined per entry point.
 *  - Tensors are dense, row-major, with the shapes written next to them.
 *    Pointers to q, k_*, v_*, out (and llm, ssm) must be 16-byte aligned
 *    (TTV_E_ALIGN otherwise); allocator-returned device memory always is.
 *  - Node 0 of every tree is its root; a tree is valid iff parents[0] == -1 and
 *    0 <= parents[i] < i for i >= 1 (any topological numbering; depth-first is
 *    one valid numbering but is not assumed).
 *  - The library holds no global state besides the static scratch of
 *    ttv_tree_attn_noalloc and a record of the kernel attributes it has set
 *    per device; calls on different streams are independent as long as
 *    their output buffers do not overlap.
 */
#ifndef TTV_H
#define TTV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility: these declarations are its
 * only exported symbols. */
#pragma GCC visibility push(default)

typedef int32_t ttv_status;
enum {
  TTV_OK = 0,
  TTV_E_NULL = 1,        /* a required pointer is NULL                         */
  TTV_E_SHAPE = 2,       /* a size is out of range or inconsistent             */
  TTV_E_DTYPE = 3,       /* unknown dtype / mode enum value                    */
  TTV_E_UNSUPPORTED = 4, /* N > 128, D not in {64,128}, Hq % Hkv != 0, ...      */
  TTV_E_WORKSPACE = 5,   /* workspace NULL or smaller than *_workspace_size    */
  TTV_E_LAUNCH = 6,      /* a kernel launch failed (hipGetLastError)           */
  TTV_E_TREE = 7,        /* device: malformed parents[] of one request         */
  TTV_E_ALIGN = 8,       /* a tensor pointer is not 16-byte aligned            */
  TTV_E_SCRATCH = 9      /* needs more than the no-allocation entry point's
                            static scratch (TTV_NOALLOC_SCRATCH_BYTES)         */
};

typedef int32_t ttv_dtype;
enum { TTV_F32 = 0, TTV_BF16 = 1 };

typedef int32_t ttv_verify_mode;
enum { TTV_GREEDY = 0, TTV_STOCHASTIC = 1 };

#define TTV_MAX_NODES 128 /* N <= 128: one or two 64-bit ancestor words per node */

/* Human-readable name of a status code (static string, never NULL). */
const char* ttv_status_string(ttv_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t ttv_version(void);

/*
 * ttv_tree_topology -- the topology-aware causal mask of every request's token
 * tree [SI] §4 "Tree-Based Parallel Decoding" (topology-aware causal masking)
 * and "Tree Attention" (a node stands for the token sequence from the root to
 * it), plus the node depths that position encodings need ([SSD] §3
 * "Implementation": the tree controls positional embeddings and causal mask).
 *
 *   parents   int32 [B,N]      parent node of each node, parents[b,0] == -1
 *   anc_out   uint64 [B,N,W]   W = ceil(N/64); bit j%64 of word j/64 of
 *                              anc_out[b,i] is set iff node j lies on the path
 *                              root -> i (node i itself included).  Nullable.
 *   depth_out int32 [B,N]      number of edges from the root.  Nullable.
 *   dev_status int32 [B]       nullable; TTV_E_TREE for a malformed tree, whose
 *                              anc_out rows are then 0 and depth_out rows -1.
 * Errors: TTV_E_NULL (parents), TTV_E_SHAPE (B < 1 or N < 1),
 *         TTV_E_UNSUPPORTED (N > 128), TTV_E_LAUNCH.
 */
ttv_status ttv_tree_topology(int32_t B, int32_t N, const int32_t* parents,
                             uint64_t* anc_out, int32_t* depth_out,
                             int32_t* dev_status, void* stream);

/*
 * ttv_tree_attn -- tree attention for every node of every request in one
 * launch [SI] §4 "Tree Attention" and "Tree-Based Parallel Decoding": the
 * output of node i is ordinary causal attention of node i's query over the
 * sequence node i represents, i.e. the request's prefix KV (positions
 * 0..L_b-1) followed by the tree-KV rows of the nodes on the path root -> i.
 * The prefix part and the in-tree part are two parts of one softmax ([SSD] §3
 * "Implementation" partitions attention the same way).
 *
 *   dt          TTV_F32 or TTV_BF16: element type of q, k_*, v_*, out.
 *   B,N         requests, tree nodes per request (1 <= N <= 128).
 *   Hq,Hkv,D    query heads, key/value heads (Hq % Hkv == 0; query head hq
 *               reads kv head hq / (Hq/Hkv)), head dim D in {64,128}.
 *   scale       softmax scale applied to q.k, finite and > 0 (usually
 *               1/sqrt(D)); TTV_E_SHAPE otherwise.
 *   q           [B,N,Hq,D]  queries of the tree nodes (positions already
 *               encoded by the caller at L_b + depth).
 *   k_cache,v_cache [B,Hkv,Lcap,D]  prefix cache; rows 0..L_b-1 are read.
 *   cache_len   int32 [B] (device) L_b, the prefix length of request b.
 *   Lmax        host promise: max_b L_b (sizes the launch); requires
 *               0 <= Lmax <= Lcap.  A request with L_b < 0 or L_b > Lmax is
 *               reported as TTV_E_SHAPE in dev_status and gets zero output.
 *   k_tree,v_tree [B,Hkv,N,D]  keys/values of the tree nodes themselves;
 *               or both NULL: the tree's K/V are stored in the cache after
 *               the prefix ([SI] §4: verified and speculated tokens share one
 *               cache), node i at row L_b + i (row min(max(L_b,0),Lmax) + i
 *               for a rejected length), which requires Lmax + N <= Lcap
 *               (TTV_E_SHAPE otherwise).  One NULL alone is TTV_E_NULL.
 *   parents     int32 [B,N]  tree of each request (see conventions).
 *   out         [B,N,Hq,D]  attention output, type dt (bf16 rounded to
 *               nearest even from fp32).  A request with a malformed tree gets
 *               zeros and dev_status TTV_E_TREE.
 *   lse         float [B,N,Hq], nullable: natural-log sum-exp of the scaled
 *               scores (0 for a rejected request).
 *   anc_out     uint64 [B,N,W], nullable: the tree mask, as ttv_tree_topology
 *               writes it (ancestor bitset of every node, self included).
 *   depth_out   int32 [B,N], nullable: node depths, as ttv_tree_topology
 *               writes them (the positions are L_b + depth).  When either is
 *               given, the call adds one small launch that writes them.
 *   workspace   device scratch of >= ttv_tree_attn_workspace_size(...) bytes
 *               (may be NULL when that size is 0): fp32 partials of the
 *               split-KV launch (and, when the split is planned on the
 *               device, the chunk count of each request).  Its contents need
 *               no initialisation and are garbage afterwards; calls sharing
 *               one must not overlap.
 * The launch shape (query rows per workgroup, split of the prefix over
 * workgroups) is chosen from the sizes; ttv_tree_attn_tuned fixes it.
 * Errors: TTV_E_NULL, TTV_E_SHAPE, TTV_E_DTYPE, TTV_E_UNSUPPORTED,
 *         TTV_E_ALIGN, TTV_E_WORKSPACE, TTV_E_LAUNCH.
 */
ttv_status ttv_tree_attn(ttv_dtype dt, int32_t B, int32_t N, int32_t Hq,
                         int32_t Hkv, int32_t D, float scale, const void* q,
                         const void* k_cache, const void* v_cache, int32_t Lcap,
                         const int32_t* cache_len, int32_t Lmax,
                         const void* k_tree, const void* v_tree,
                         const int32_t* parents, void* out, float* lse,
                         uint64_t* anc_out, int32_t* depth_out,
                         int32_t* dev_status, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Bytes of workspace ttv_tree_attn needs for these sizes (0 if none);
 * returns (size_t)-1 for arguments ttv_tree_attn would reject. */
size_t ttv_tree_attn_workspace_size(ttv_dtype dt, int32_t B, int32_t N,
                                    int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t Lmax);

/*
 * ttv_tree_attn_tuned -- ttv_tree_attn with a fixed launch shape (the same
 * results up to rounding order).
 *   rows_per_block, chunk_keys  0 = automatic; otherwise query rows per
 *               workgroup (64, 128 or 256 on the matrix-core path, which
 *               serves bf16 with N*Hq/Hkv >= 16; 16 on the FMA path) and
 *               prefix keys per workgroup (a positive multiple of 64); other
 *               values give TTV_E_UNSUPPORTED.  The same values must be given
 *               to ttv_tree_attn_tuned_workspace_size.  With chunk_keys = 0,
 *               2..64 requests and fewer (request, kv head, row block) units
 *               than CUs, the split follows the actual prefix lengths read on
 *               the device (longer requests get more workgroups).
 */
ttv_status ttv_tree_attn_tuned(ttv_dtype dt, int32_t B, int32_t N, int32_t Hq,
                               int32_t Hkv, int32_t D, float scale,
                               const void* q, const void* k_cache,
                               const void* v_cache, int32_t Lcap,
                               const int32_t* cache_len, int32_t Lmax,
                               const void* k_tree, const void* v_tree,
                               const int32_t* parents, void* out, float* lse,
                               uint64_t* anc_out, int32_t* depth_out,
                               int32_t* dev_status, void* workspace,
                               size_t workspace_bytes, int32_t rows_per_block,
                               int32_t chunk_keys, void* stream);

size_t ttv_tree_attn_tuned_workspace_size(ttv_dtype dt, int32_t B, int32_t N,
                                          int32_t Hq, int32_t Hkv, int32_t D,
                                          int32_t Lmax, int32_t rows_per_block,
                                          int32_t chunk_keys);

/*
 * Batches of trees of different sizes ([SI] §5 "Scheduling": iteration-level
 * continuous batching verifies the requests of a batch together, whatever
 * the size of each one's token tree).  The _varlen entry points take, after
 * `parents`/`tokens`, a device array
 *   n_nodes   int32 [B]: request b's tree is nodes 0..n_nodes[b]-1; every
 *             [B,N,...] tensor keeps N entries per request and the entries
 *             of nodes >= n_nodes[b] are padding: never read for the result
 *             (they may hold anything, NaN included) and, for outputs,
 *             written as stated below.
 * and otherwise mean exactly what the entry point without the suffix means;
 * each request's results equal that entry point's on the request alone with
 * its rows cut to n_nodes[b] (the stochastic draws keep their counters
 * (j, u, b, step), b the request's index in the batch).  A count outside
 * [1, N] rejects the request with dev_status TTV_E_SHAPE (attention: zero
 * output; verification: path_len 0, nothing committed).  NULL n_nodes is
 * TTV_E_NULL.
 *
 * ttv_tree_attn_varlen: rows of padding nodes get zero output and lse 0;
 *   anc_out/depth_out give padding nodes 0 words and depth -1.  The launch
 *   still covers N nodes per request (the split of the prefix follows each
 *   request's node count).
 */
ttv_status ttv_tree_attn_varlen(ttv_dtype dt, int32_t B, int32_t N, int32_t Hq,
                                int32_t Hkv, int32_t D, float scale,
                                const void* q, const void* k_cache,
                                const void* v_cache, int32_t Lcap,
                                const int32_t* cache_len, int32_t Lmax,
                                const void* k_tree, const void* v_tree,
                                const int32_t* parents, const int32_t* n_nodes,
                                void* out, float* lse, uint64_t* anc_out,
                                int32_t* depth_out, int32_t* dev_status,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* Bytes of the device array ttv_tree_attn_noalloc keeps its partials in. */
#define TTV_NOALLOC_SCRATCH_BYTES (48u << 20)

/*
 * ttv_tree_attn_noalloc -- ttv_tree_attn_tuned without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, results and errors are those of ttv_tree_attn_tuned (0, 0 for
 * rows_per_block, chunk_keys: the automatic shape of ttv_tree_attn), and so
 * are the kernels.  The split-KV partials go to a static device array of
 * TTV_NOALLOC_SCRATCH_BYTES (48 MiB) that each GPU the library runs on holds
 * until the process ends; a call whose ttv_tree_attn_tuned_workspace_size
 * exceeds it returns TTV_E_SCRATCH before anything is enqueued.  (The
 * automatic shape needs at most about 35 MB of partials, e.g. 33 MiB for 4
 * requests x 8 kv heads x 1024 query rows x 32768 keys; small forced chunks
 * can need more.)  The
 * array's address on the current device is looked up on the first call made
 * on that device (a failure there gives TTV_E_LAUNCH).  Nothing is allocated
 * or freed.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other host threads) race and
 * must be serialised by the caller; the array needs no initialisation.
 */
ttv_status ttv_tree_attn_noalloc(ttv_dtype dt, int32_t B, int32_t N,
                                 int32_t Hq, int32_t Hkv, int32_t D,
                                 float scale, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 int32_t Lcap, const int32_t* cache_len,
                                 int32_t Lmax, const void* k_tree,
                                 const void* v_tree, const int32_t* parents,
                                 void* out, float* lse, uint64_t* anc_out,
                                 int32_t* depth_out, int32_t* dev_status,
                                 int32_t rows_per_block, int32_t chunk_keys,
                                 void* stream);

/*
 * ttv_tree_verify -- verify every request's token tree against the LLM's
 * outputs at each node and return the longest accepted root-to-node path
 * ([SI] §4 "Token Tree Verification", "Token Verification"; §6: greedy
 * verification reproduces incremental decoding's token sequences).
 *
 *   mode     TTV_GREEDY: llm holds logits; node c is accepted iff its parent
 *            is accepted and tokens[c] == argmax of llm[b,parent(c),:]
 *            (fp32 compare, lowest index wins ties; logits must be finite).
 *            The path ends at the deepest accepted node d (lowest index on
 *            ties) and the bonus token is argmax llm[b,d,:].
 *            TTV_STOCHASTIC: multi-step speculative sampling.  llm[b,u,:] is
 *            the LLM's next-token distribution after node u, ssm[b,c,:] is
 *            the distribution node c's token was drawn from (row 0 unused).
 *            Starting at the root with residual w = llm[b,u,:] and mass s = 1,
 *            the children c of u are tested in ascending node index, the
 *            j-th of them (j = 0, 1, ..) with the uniform r(j, u): accept iff
 *            (r*q[x])*s < w[x] (fp32, two multiplies, strict), x = tokens[c],
 *            q = ssm[b,c,:].  On acceptance move to c (w = llm[b,c,:],
 *            s = 1).  On rejection w[v] = max(fmaf(-s, q[v], w[v]), +0) for
 *            all v and s = (float)(sum_v fx(w[v]) * 2^-40), fx(x) =
 *            floor(x * 2^40) as uint64; s == 0 stops testing and resets
 *            w = llm[b,u,:].  When no child is accepted the bonus token is
 *            drawn from w by inverse CDF over the exact integer prefix sums
 *            of fx(w): with S = sum fx(w), R = R(u), T = floor(R*S/2^24), the
 *            bonus is the smallest t with sum_{v<=t} fx(w[v]) > T (argmax w
 *            if S == 0).  Probabilities must lie in [0,1].
 *            The uniforms are drawn from Philox4x64-10 (Salmon, Moraes, Dror,
 *            Shaw, SC'11) with key (seed, 0): with o = output word 0 for the
 *            counter (j, u, b, step) (four 64-bit words, word 0 least
 *            significant), r(j, u) = (o >> 40) * 2^-24; R(u) = o >> 40 for
 *            the counter (2^63, u, b, step).  The same (seed, step) gives the
 *            same results; a new step gives fresh draws.
 *   B,N,V    requests, nodes per request (<= 128), vocabulary (>= 1).
 *   parents  int32 [B,N]; tokens int32 [B,N] (tokens[b,0] = root's token,
 *            unused); llm float [B,N,V]; ssm float [B,N,V] (stochastic only,
 *            else NULL; in stochastic mode both hold probabilities, every
 *            entry in [0, 1]); seed, step: the draws' key and counter word 3
 *            (stochastic only, else ignored).
 *   path     int32 [B,N]: path[b,k] = node at depth k on the accepted path,
 *            -1 after the end.   path_len int32 [B]: accepted nodes + 1 (>= 1).
 *   out_tokens int32 [B,N]: tokens of path[1..], then the bonus token, -1
 *            after (path_len entries in all).
 *   A malformed tree gives path_len 0 and -1 everywhere, dev_status TTV_E_TREE;
 *   in stochastic mode a non-root token outside [0,V) does the same with
 *   TTV_E_SHAPE.  Stochastic mode keeps the walk's residual distribution on
 *   chip up to V = 36864; from there up to V = 262144 (V % 4 == 0, else
 *   TTV_E_UNSUPPORTED) it keeps it in the workspace, B*V floats.
 *   workspace >= ttv_tree_verify_workspace_size(...) bytes, 16-byte aligned
 *            (contents need no initialisation); greedy: argmax partials;
 *            stochastic: none up to V = 36864, else the residual.
 * Errors: TTV_E_NULL, TTV_E_SHAPE, TTV_E_DTYPE (mode), TTV_E_UNSUPPORTED,
 *         TTV_E_ALIGN, TTV_E_WORKSPACE, TTV_E_LAUNCH.
 */
ttv_status ttv_tree_verify(ttv_verify_mode mode, int32_t B, int32_t N,
                           int32_t V, const int32_t* parents,
                           const int32_t* tokens, const float* llm,
                           const float* ssm, uint64_t seed, uint64_t step,
                           int32_t* path, int32_t* path_len,
                           int32_t* out_tokens, int32_t* dev_status,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* Bytes of workspace ttv_tree_verify(_varlen) and ttv_tree_verify_commit(_varlen)
 * need; (size_t)-1 for sizes they do not take. */
size_t ttv_tree_verify_workspace_size(ttv_verify_mode mode, int32_t B,
                                      int32_t N, int32_t V);

/* ttv_tree_verify for a batch of trees of different sizes (n_nodes as for
 * ttv_tree_attn_varlen): paths and tokens only ever name nodes < n_nodes[b];
 * the logits rows of padding nodes are not read. */
ttv_status ttv_tree_verify_varlen(ttv_verify_mode mode, int32_t B, int32_t N,
                                  int32_t V, const int32_t* parents,
                                  const int32_t* tokens, const int32_t* n_nodes,
                                  const float* llm, const float* ssm,
                                  uint64_t seed, uint64_t step, int32_t* path,
                                  int32_t* path_len, int32_t* out_tokens,
                                  int32_t* dev_status, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * ttv_tree_verify_uniforms -- stochastic ttv_tree_verify with the uniforms
 * given by the caller instead of drawn from (seed, step): the test of child c
 * uses r = u_accept[b,c] (each child is tested at most once) and the final
 * draw R = floor(u_bonus[b] * 2^24).  u_accept float [B,N], u_bonus float [B],
 * values in [0,1).  Needs no workspace; everything else as ttv_tree_verify.
 * Errors: TTV_E_NULL, TTV_E_SHAPE, TTV_E_UNSUPPORTED, TTV_E_ALIGN,
 *         TTV_E_LAUNCH.
 */
ttv_status ttv_tree_verify_uniforms(int32_t B, int32_t N, int32_t V,
                                    const int32_t* parents,
                                    const int32_t* tokens, const float* llm,
                                    const float* ssm, const float* u_accept,
                                    const float* u_bonus, int32_t* path,
                                    int32_t* path_len, int32_t* out_tokens,
                                    int32_t* dev_status, void* stream);

/*
 * ttv_kv_commit -- write the accepted path's KV rows into the contiguous cache
 * ([SI] §4 "Tree-Based Parallel Decoding": verified and speculated tokens share
 * one key-value cache; only the accepted ones stay).  For request b with
 * L = cache_len_in[b] and n = path_len[b]:
 *   k_cache[b,h,L+j,:] = k_tree[b,h,path[b,j],:] (same for v), j < n, all h;
 *   cache_len_out[b] = L + n;  committed_src[b,j] = path[b,j] (j < n), -1 after.
 * Copies are bit-exact.  Rows >= L+n and other requests are untouched.
 *
 *   dt           element type (only its size matters).
 *   k_tree,v_tree [B,Hkv,N,D];  k_cache,v_cache [B,Hkv,Lcap,D].
 *   cache_len_in, cache_len_out int32 [B] (may be the same array).
 *   Lmax         host promise max_b L_b; requires Lmax + N <= Lcap.
 *   path, path_len  as written by ttv_tree_verify (device, no host copy).
 *   committed_src int32 [B,N], nullable.
 *   dev_status   nullable; TTV_E_SHAPE when L < 0, L > Lmax, n outside
 *                [0,N] or a path entry outside [0,N): nothing of that request
 *                is written except cache_len_out[b] = L (and -1 sources).
 * Errors: TTV_E_NULL, TTV_E_SHAPE, TTV_E_DTYPE, TTV_E_UNSUPPORTED,
 *         TTV_E_ALIGN, TTV_E_LAUNCH.
 */
ttv_status ttv_kv_commit(ttv_dtype dt, int32_t B, int32_t N, int32_t Hkv,
                         int32_t D, int32_t Lcap, const void* k_tree,
                         const void* v_tree, void* k_cache, void* v_cache,
                         const int32_t* cache_len_in, int32_t* cache_len_out,
                         int32_t Lmax, const int32_t* path,
                         const int32_t* path_len, int32_t* committed_src,
                         int32_t* dev_status, void* stream);

/*
 * ttv_tree_verify_commit -- ttv_tree_verify followed by ttv_kv_commit of its
 * path in one pass ([SI] §4 "Token Tree Verification", "Token Verification"
 * and "Tree-Based Parallel Decoding": verify the tree, keep the accepted
 * path's KV).  Every output (path, path_len, out_tokens, the k_cache/v_cache
 * rows, cache_len_out, committed_src) equals what ttv_tree_verify(mode, ...)
 * and then ttv_kv_commit on its path give; the arguments mean what they mean
 * there.  The path goes from the verifier to the row copy through on-chip
 * memory: greedy mode runs the argmax partials and then one launch that scans
 * and copies; stochastic mode copies from the walk's own workgroup.
 *
 *   dev_status  nullable: the verifier's status if it rejects the request
 *               (TTV_E_TREE, or TTV_E_SHAPE for a bad stochastic token: path_len
 *               0, nothing committed, cache_len_out[b] = L), else TTV_E_SHAPE
 *               when L < 0, L > Lmax or L + path_len > Lcap (nothing
 *               committed, cache_len_out[b] = L), else TTV_OK.
 *   workspace   >= ttv_tree_verify_workspace_size(mode, B, N, V) bytes.
 *   cache_len_in and cache_len_out may be the same array, as in ttv_kv_commit.
 * Errors: TTV_E_NULL, TTV_E_SHAPE, TTV_E_DTYPE (mode or dt), TTV_E_UNSUPPORTED,
 *         TTV_E_ALIGN, TTV_E_WORKSPACE, TTV_E_LAUNCH.
 */
ttv_status ttv_tree_verify_commit(ttv_verify_mode mode, ttv_dtype dt,
                                  int32_t B, int32_t N, int32_t V,
                                  int32_t Hkv, int32_t D, int32_t Lcap,
                                  const int32_t* parents,
                                  const int32_t* tokens, const float* llm,
                                  const float* ssm, uint64_t seed,
                                  uint64_t step, const void* k_tree,
                                  const void* v_tree, void* k_cache,
                                  void* v_cache, const int32_t* cache_len_in,
                                  int32_t* cache_len_out, int32_t Lmax,
                                  int32_t* path, int32_t* path_len,
                                  int32_t* out_tokens, int32_t* committed_src,
                                  int32_t* dev_status, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ttv_tree_verify_commit for a batch of trees of different sizes (n_nodes
 * as for ttv_tree_attn_varlen). */
ttv_status ttv_tree_verify_commit_varlen(
    ttv_verify_mode mode, ttv_dtype dt, int32_t B, int32_t N, int32_t V,
    int32_t Hkv, int32_t D, int32_t Lcap, const int32_t* parents,
    const int32_t* tokens, const int32_t* n_nodes, const float* llm,
    const float* ssm, uint64_t seed, uint64_t step, const void* k_tree,
    const void* v_tree, void* k_cache, void* v_cache,
    const int32_t* cache_len_in, int32_t* cache_len_out, int32_t Lmax,
    int32_t* path, int32_t* path_len, int32_t* out_tokens,
    int32_t* committed_src, int32_t* dev_status, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * ttv_tree_expand -- one level of expansion-based token-tree construction
 * ([SI] §3 "Expansion-based token tree construction": a speculative model's
 * top-k tokens at a node become that node's children).  For request b, whose
 * tree has n_in[b] nodes in parents[b,:n_in[b]] / tokens[b,:n_in[b]], every
 * frontier entry fr = frontier[b,f] >= 0, in order of f, gets k children: the
 * k tokens of highest probability in probs[b,f,:], most probable first, an
 * equal probability going to the lower token id.  With r = the rank of f
 * among the request's entries >= 0, child j is node n = n_in[b] + r*k + j:
 *   parents[b,n] = fr;  tokens[b,n] = token;  src_row[b,n] = f;
 *   n_out[b] = n_in[b] + (number of entries >= 0) * k.
 * Nodes are so numbered parents-first (expanding one depth per call in index
 * order gives breadth-first numbering), and src_row tells which row each new
 * token came from (the draft distribution a stochastic verifier needs).
 * Entries < n_in[b] of parents/tokens/src_row and entries past n_out[b] are
 * untouched.
 *
 *   probs        float32 [B,F,V] device, no NaN (other values compared as
 *                they are).
 *   frontier     int32 [B,F] device: node ids in [0, n_in[b]), -1 = none.
 *   n_in         int32 [B] device, nodes already in the tree (>= 1: the root).
 *   Ncap         row length of parents/tokens/src_row, 1..128.
 *   parents, tokens  int32 [B,Ncap] device, appended to in place.
 *   src_row      int32 [B,Ncap] device, nullable.
 *   n_out        int32 [B] device (may not alias n_in).
 *   dev_status   int32 [B] device, nullable: TTV_E_TREE for a frontier entry
 *                outside [-1, n_in[b]), TTV_E_SHAPE for n_in[b] < 1 or more
 *                than Ncap nodes; such a request gets n_out[b] = n_in[b] and
 *                nothing else written.
 *   1 <= k <= min(16, V); F <= 128.
 * Errors: TTV_E_NULL, TTV_E_SHAPE, TTV_E_UNSUPPORTED, TTV_E_LAUNCH.
 */
ttv_status ttv_tree_expand(int32_t B, int32_t F, int32_t V, int32_t k,
                           const float* probs, const int32_t* frontier,
                           const int32_t* n_in, int32_t Ncap, int32_t* parents,
                           int32_t* tokens, int32_t* src_row, int32_t* n_out,
                           int32_t* dev_status, void* stream);

/*
 * ttv_tree_merge -- merge-based token-tree construction ([SI] §3
 * "Merge-based token tree construction": the outputs of several speculative
 * models are combined into one tree that contains each of their token
 * sequences).  For request b, the S sequences seqs[b,s,0..seq_len[b,s]-1]
 * hang below the root (node 0, token root_tok[b]); every distinct non-empty
 * prefix becomes one node, so a prefix the sequences share appears once.
 * Nodes are numbered depth by depth, and within a depth in order of the
 * lowest sequence index whose prefix the node is (its leader s), which puts
 * parents first:
 *   parents[b,0] = -1, tokens[b,0] = root_tok[b], src[b,0] = -1;
 *   node n at depth d+1: parents[b,n] = its prefix's node at depth d,
 *   tokens[b,n] = seqs[b,s,d], src[b,n] = s*Ls + d (the speculator row the
 *   token came from, for a stochastic verifier);  n_out[b] = node count.
 * Entries past n_out[b] are untouched.
 *
 *   seqs         int32 [B,S,Ls] device (token ids, compared for equality).
 *   seq_len      int32 [B,S] device, each in [0, Ls].
 *   root_tok     int32 [B] device.
 *   Ncap         row length of parents/tokens/src, 1..128.
 *   parents, tokens  int32 [B,Ncap] device (output).
 *   src          int32 [B,Ncap] device, nullable.
 *   n_out        int32 [B] device.
 *   dev_status   int32 [B] device, nullable: TTV_E_SHAPE for a length
 *                outside [0, Ls] or more than Ncap nodes; such a request
 *                gets n_out[b] = 0 and nothing else written.
 *   S <= 64, Ls <= 128.
 * Errors: TTV_E_NULL, TTV_E_SHAPE, TTV_E_UNSUPPORTED, TTV_E_LAUNCH.
 */
ttv_status ttv_tree_merge(int32_t B, int32_t S, int32_t Ls, const int32_t* seqs,
                          const int32_t* seq_len, const int32_t* root_tok,
                          int32_t Ncap, int32_t* parents, int32_t* tokens,
                          int32_t* src, int32_t* n_out, int32_t* dev_status,
                          void* stream);

/*
 * ttv_probs_from_logits -- next-token probabilities from logits at a
 * temperature, over the top-k logits and/or the top-p share of the mass
 * ([SI] §4 "Token Verification": the stochastic verifier takes the LLM's and
 * the speculators' next-token distributions; §7 "Multi-sample decoding":
 * top-k or top-p sampling; [SSD] §4 samples with top-k, k = 50, at T = 1).
 * For each of the R rows of V logits z, in the order (higher logit, then
 * lower token id):
 *   top-k  with 0 < topk < V the first topk tokens are kept (else all);
 *   top-p  with top_p < 1, of those the shortest prefix whose mass reaches
 *          ceil(P * S / 2^24), P = floor(top_p * 2^24), S their mass;
 *   probs[r,v] = 2^t_v * (float)(2^40 / S') for kept v, 0 otherwise, with
 *          t_v = (z_v - m) * (float)(log2(e) / T) (m = the row maximum),
 *          S' the mass of the kept tokens.
 * The arithmetic is fixed to the bit: 2^t = 2^n * P(t - n), n = t rounded to
 * the nearest integer (ties to even), P the degree-7 Taylor polynomial of
 * 2^f = exp(f ln 2) in Horner form with fused multiply-adds (coefficients
 * ln(2)^k / k! formed in double, rounded to float), 0 for n < -125; the mass
 * of a token is floor(2^t * 2^40) as an exact integer.  Each row is read
 * once from HBM and written once.
 *
 *   R            rows (e.g. B*N for [B,N,V] logits).
 *   logits       float32 [R,V] device, finite.
 *   probs        float32 [R,V] device (may not alias logits).
 *   temperature  finite, > 0, with log2(e)/T finite in float (TTV_E_SHAPE
 *                otherwise).
 *   topk         0 (or >= V): every token; 1..512: the topk highest;
 *                larger values below V give TTV_E_UNSUPPORTED.
 *   top_p        in (0, 1]; 1 keeps every token top-k kept (TTV_E_SHAPE
 *                outside).
 * Errors: TTV_E_NULL, TTV_E_SHAPE, TTV_E_UNSUPPORTED, TTV_E_LAUNCH.
 */
ttv_status ttv_probs_from_logits(int32_t R, int32_t V, float temperature,
                                 int32_t topk, float top_p, const float* logits,
                                 float* probs, void* stream);

/*
 * ttv_tree_verify_logits -- stochastic ttv_tree_verify(_varlen) fed with
 * logits: llm_logits [B,N,V] and ssm_logits [B,N,V] (float32, finite) stand
 * for the distributions ttv_probs_from_logits(temperature, topk, top_p)
 * gives for them, bit for bit, without those probabilities being written:
 * one pass per tensor computes each row's maximum, normaliser and last kept
 * token into the workspace, and the walk computes every probability it
 * reads from the logits.  Results equal ttv_tree_verify_varlen(STOCHASTIC,
 * ..., seed, step) on those probabilities; n_nodes is nullable (every
 * request has N nodes).  Needs V % 4 == 0 and V <= 262144 (TTV_E_UNSUPPORTED
 * otherwise) and 16-byte aligned logits.
 *   workspace >= ttv_tree_verify_logits_workspace_size(B, N, V) bytes: 2*B*N
 *   row statistics of 16 bytes, then for V > 32768 the walk's residual
 *   distribution, B*V floats (the rows no longer fit its registers); no
 *   initialisation, 16-byte aligned.
 * Errors: TTV_E_NULL, TTV_E_SHAPE, TTV_E_UNSUPPORTED, TTV_E_ALIGN,
 *         TTV_E_WORKSPACE, TTV_E_LAUNCH.
 */
ttv_status ttv_tree_verify_logits(int32_t B, int32_t N, int32_t V,
                                  const int32_t* parents, const int32_t* tokens,
                                  const int32_t* n_nodes,
                                  const float* llm_logits,
                                  const float* ssm_logits, float temperature,
                                  int32_t topk, float top_p, uint64_t seed,
                                  uint64_t step, int32_t* path,
                                  int32_t* path_len, int32_t* out_tokens,
                                  int32_t* dev_status, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Bytes of workspace ttv_tree_verify_logits needs; (size_t)-1 for sizes it
 * does not take. */
size_t ttv_tree_verify_logits_workspace_size(int32_t B, int32_t N, int32_t V);

/*
 * ttv_kv_commit_inplace -- ttv_kv_commit for a tree stored inside the cache
 * ([SI] §4 "Tree-Based Parallel Decoding": verified and speculated tokens
 * share one key-value cache; only the accepted ones stay).  Tree node i's K/V
 * are at row L + i (L = cache_len_in[b], the layout ttv_tree_attn reads with
 * NULL tree pointers); for n = path_len[b]:
 *   k_cache[b,h,L+j,:] = old k_cache[b,h,L+path[b,j],:] (same for v), j < n,
 *   all h (every source row is read before any destination is written);
 *   cache_len_out[b] = L + n;  committed_src[b,j] = path[b,j] (j < n), -1 after.
 * Copies are bit-exact.  Rows L+n .. L+N-1 keep stale tree rows; rows outside
 * [L, L+N) and other requests are untouched.
 *
 *   dt           element type (only its size matters).
 *   k_cache,v_cache [B,Hkv,Lcap,D] device, updated in place.
 *   cache_len_in, cache_len_out int32 [B] (may be the same array).
 *   Lmax         host promise max_b L_b; requires Lmax + N <= Lcap.
 *   path, path_len  as written by ttv_tree_verify (device, no host copy).
 *   committed_src int32 [B,N], nullable.
 *   dev_status   nullable; TTV_E_SHAPE when L < 0, L > Lmax, n outside
 *                [0,N] or a path entry outside [0,N): nothing of that request
 *                is written except cache_len_out[b] = L (and -1 sources).
 * Errors: TTV_E_NULL, TTV_E_SHAPE, TTV_E_DTYPE, TTV_E_UNSUPPORTED,
 *         TTV_E_ALIGN, TTV_E_LAUNCH.
 */
ttv_status ttv_kv_commit_inplace(ttv_dtype dt, int32_t B, int32_t N, int32_t Hkv,
                                 int32_t D, int32_t Lcap, void* k_cache,
                                 void* v_cache, const int32_t* cache_len_in,
                                 int32_t* cache_len_out, int32_t Lmax,
                                 const int32_t* path, const int32_t* path_len,
                                 int32_t* committed_src, int32_t* dev_status,
                                 void* stream);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif
#endif /* TTV_H */
