/*
 * spec_verify.h -- C ABI of the gfx950 (AMD Instinct MI355X) draft-token
 * verification library, libspecverify.so.
 *
 * Three operations of speculative decoding's verification step, batched over
 * sequences and streamed over the full vocabulary, and the two steps on either
 * side of tree verification:
 *
 *   spec_verify_chain        modified rejection sampling of a chain of drafts
 *   spec_verify_tree_greedy  greedy acceptance of the longest matching tree path
 *   spec_verify_tree         stochastic (T > 0) tree verification against residuals
 *   ngram_propose            prompt n-gram lookup drafting (one-hot draft q)
 *   spec_ngram_verify        the lookup and the verification of its drafts in one call
 *   spec_tree_mask           2-D tree-attention mask and node depths of a draft tree
 *   spec_commit_path         copy the accepted path's cache entries into the KV cache
 *
 * Pages that define the operations (cited by title):
 *   [Production]  "Speculative Decoding in Production: From Draft Models to
 *                 EAGLE-3 Dynamic Trees for 3x-5x Lossless Acceleration"
 *                 (blog.llmgo.top)
 *   [Accelerating] "Accelerating Autoregressive LLM Inference 3x with Lossless
 *                 Speculative Decoding and EAGLE Heads" (x078.com)
 *   [Medusa]      "Speculative decoding: Medusa, EAGLE, vLLM"
 *                 (vikram-blog.pages.dev)
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer to caller-owned memory; the
 *     library never allocates, frees or retains it.  Arrays are dense,
 *     row-major, with the shapes given below.  Outputs must not alias inputs.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise.  Results are valid once the stream has
 *     completed the call.
 *   - Errors that the host can see (sizes, NULL pointers, dtype, workspace
 *     size, alignment of the workspace) return a status synchronously and
 *     launch nothing.  SPEC_ERR_HIP reports a failed launch.
 *   - Errors in device data (an out-of-range token, a non-positive
 *     temperature, a uniform outside (0, 1], a bad tree topology) cannot be
 *     seen without a synchronisation: they mark the affected sequence in its
 *     outputs instead (documented per call), and other sequences are unaffected.
 *   - Results are deterministic: no floating-point atomics feed any result.
 *   - A workspace is scratch for one call at a time: its contents need no
 *     initialisation and are meaningless after the call.  A kernel uses only
 *     values written earlier in the same call (values that workgroups hand to
 *     each other carry the call's generation number, so whatever the
 *     workspace held before is recognised and ignored).  Calls that overlap
 *     in time (different streams) need different workspaces.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spec_status {
  SPEC_OK = 0,
  SPEC_ERR_INVALID_ARG = 1, /* a size, pointer or parameter the host can check is wrong */
  SPEC_ERR_UNSUPPORTED = 2, /* beyond a documented limit (SPEC_MAX_*) */
  SPEC_ERR_WORKSPACE = 3,   /* workspace NULL, too small or not 256-byte aligned */
  SPEC_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} spec_status_t;

typedef enum spec_dtype {
  SPEC_F32 = 0,  /* IEEE float32 logits */
  SPEC_BF16 = 1  /* bfloat16 logits (upper 16 bits of a float32) */
} spec_dtype_t;

typedef void* spec_stream_t; /* hipStream_t */

#define SPEC_MAX_K 64            /* drafted positions per sequence (chain) */
#define SPEC_MAX_TREE_NODES 1024 /* nodes per tree, root included */
#define SPEC_MAX_NGRAM_N 16      /* longest n-gram the lookup matches */

/* Human-readable name of a status code (static storage). */
const char* spec_status_string(spec_status_t status);

/* Detail message of the last non-OK status returned on the calling thread. */
const char* spec_last_error(void);

/* Count output (out_num_accepted, out_accept_len) of a sequence whose device data is
 * invalid, and of one whose cross-workgroup hand-over wait gave up (see below). */
#define SPEC_FLAG_INVALID (-1)
#define SPEC_FLAG_TIMED_OUT (-2)

/* Hand-over waits.  spec_verify_chain (after a rejection against draft rows),
 * spec_verify_tree and spec_verify_tree_greedy (without out_argmax) split each
 * sequence over several workgroups that hand partial sums to each other inside one
 * kernel and wait for them.  spec_verify_chain's waiting workgroup only waits for
 * workgroups dispatched before it, which never wait, so its waits end whatever else
 * runs on the device.  spec_verify_chain and spec_ngram_verify run a small batch (chunks
 * of 4 vectors a lane, at most 1024 workgroups, and the whole grid resident on the
 * device at once) as a single launch whose workgroups keep their rows in registers and
 * each wait for every partial sum of their sequence: there every workgroup but the
 * sequence's last gives up after a short wait (about 2048 polls) and says so, and the
 * last one, which waits only for workgroups dispatched before it, then finishes the
 * sequence from memory; so those waits end as well, only later.  The tree walks'
 * workgroups of one sequence wait for each other: a launch holds at most half the
 * workgroups the device runs at once, so one or two such calls in flight together always
 * fit, but more (on other streams, or next to other kernels that wait on their own
 * workgroups) can keep a sequence's workgroups from all running at once.  Every wait is
 * bounded (SPEC_KNOB_POLL_LIMIT in spec_measure.h, at least a quarter of a second by
 * default): a sequence whose wait gives up gets count SPEC_FLAG_TIMED_OUT and -1 in its
 * other outputs, written by the one workgroup that writes the sequence's outputs, so a
 * flag never mixes with a result.  Issue the call again for such sequences. */

/* ---------------------------------------------------------------------------
 * Chain verification by modified rejection sampling.
 *
 * [Production] section I.1 "Verification via Modified Rejection Sampling":
 * for drafted token x_k, alpha_k = min(1, p_k(x_k) / q_k(x_k)) (step 1); with
 * r_k uniform, accept while r_k <= alpha_k and stop at the first rejection
 * (step 2); on a rejection at position n draw the replacement from
 * max(0, p_n - q_n) normalised (step 3).  The invariance theorem of the same
 * section is why this reproduces the target distribution.
 *
 * Readings where the page is silent: p_k = softmax(target_k / T_b) and
 * q_k = softmax(draft_k / T_b); when all k_b drafts are accepted a bonus token
 * is drawn from p_{k_b} (target row k_b); every draw from a weight vector w
 * uses inverse-CDF sampling in vocabulary order: the smallest index i whose
 * inclusive prefix sum reaches u * sum(w).
 *
 * target_logits [B, K+1, V] dtype.  Row k scores draft k; row k_b gives the bonus.
 * draft_logits  [B, K, V] dtype, or NULL: then q_k is one-hot at x_k (prompt
 *               lookup drafting), alpha_k = p_k(x_k), and the residual is p_n
 *               without x_n.  Draft rows are then never read.
 * draft_tokens  [B, K] int32 in [0, V) for k < k_b (entries k >= k_b are ignored).
 * draft_len     [B] int32 k_b in [0, K], or NULL meaning k_b = K for every b.
 *               Rows beyond k_b are never read.
 * temperature   [B] float32, finite and >= 0.  T_b = 0 selects greedy
 *               verification for sequence b (the invariance theorem of
 *               section I.1 covers greedy decoding; "Speculative decoding:
 *               Medusa, EAGLE, vLLM" runs its example at temperature 0): draft
 *               k is accepted iff it is the argmax of target row k (raw logits,
 *               smallest index on ties), the emitted row ends with the argmax
 *               of target row n, no draft row and no uniform is read, and
 *               out_probs[b] is 0.  Greedy and sampled sequences may share a
 *               batch.
 * u_accept      [B, K] float32 in (0, 1]: r_k of the accept test of draft k
 *               (ignored when T_b = 0).
 * u_final       [B] float32 in (0, 1]: the one uniform of the replacement or
 *               bonus draw (ignored when T_b = 0).
 * out_tokens    [B, K+1] int32: x_0..x_{n-1}, then the drawn token, then -1.
 * out_num_accepted [B] int32: n, the number of accepted drafts (0..k_b).
 * out_probs     [B, K, 3] float32 (p_k(x_k), q_k(x_k), alpha_k) for k < k_b,
 *               zeros for k >= k_b; or NULL.
 * out_packed    [B*(K+1)] int32 or NULL: the emitted tokens of all sequences
 *               back to back (sequence b's n_b+1 tokens at out_offsets[b]).
 * out_offsets   [B+1] int32 or NULL (both or neither of packed/offsets):
 *               exclusive prefix sums of the per-sequence token counts.
 * workspace     device scratch of at least spec_verify_chain_workspace_size()
 *               bytes, 256-byte aligned.
 *
 * Invalid device data for sequence b (token out of range, k_b outside [0, K],
 * T negative or not finite, a uniform outside (0, 1] when T > 0) sets out_num_accepted[b]
 * = -1, out_tokens[b, :] = -1, out_probs[b] = 0 and gives it no packed tokens.  A
 * sequence whose hand-over wait gave up (see "Hand-over waits") gets the same outputs
 * with out_num_accepted[b] = SPEC_FLAG_TIMED_OUT (-2).
 * Limits: 1 <= K <= SPEC_MAX_K, V >= 1, B >= 0, B*(K+1)*V < 2^47.
 * Logits may be -inf (probability 0); +inf and NaN are not supported; each
 * used row needs at least one finite logit.
 * ------------------------------------------------------------------------- */
size_t spec_verify_chain_workspace_size(int B, int K, int V, spec_dtype_t dtype);

spec_status_t spec_verify_chain(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                const int32_t* draft_tokens, const int32_t* draft_len,
                                const float* temperature, const float* u_accept, const float* u_final,
                                int B, int K, int V,
                                int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                int32_t* out_packed, int32_t* out_offsets,
                                void* workspace, size_t workspace_bytes, spec_stream_t stream);

/* ---------------------------------------------------------------------------
 * spec_verify_chain without a workspace, for callers that cannot allocate device
 * memory (code recorded into a HIP graph, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and errors as spec_verify_chain; the scratch
 * space is a 16 MiB array that the library holds on each device it runs on, for the
 * life of the process (enough for B = 1024, K = 8, V = 152064 bf16).  A shape that
 * needs more returns SPEC_ERR_UNSUPPORTED and launches nothing.  The call allocates
 * nothing (the array's device address is looked up on the device's first call).
 * Every call on one device shares that device's array, so calls that overlap in
 * time on one device (different streams, host threads) race: issue them one after
 * another, or use spec_verify_chain with a workspace per stream.
 * ------------------------------------------------------------------------- */
spec_status_t spec_verify_chain_noalloc(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                        const int32_t* draft_tokens, const int32_t* draft_len,
                                        const float* temperature, const float* u_accept, const float* u_final,
                                        int B, int K, int V,
                                        int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                        int32_t* out_packed, int32_t* out_offsets, spec_stream_t stream);

/* ---------------------------------------------------------------------------
 * Greedy tree verification.
 *
 * [Production] section III.2 "The Tree Attention Verification Mechanism": all
 * branches of the flattened draft tree are scored in one target pass, and a
 * matching branch is accepted even when a sibling is rejected.  [Medusa],
 * "System Topology & Data Flow" figure (branch [t1,t2,t3] accepted, sibling
 * [t1,t2',t4] rejected) and its temperature-0 usage example.
 *
 * Readings: node i (i >= 1) is accepted iff its parent is accepted and its token
 * equals the argmax of its parent's row (smallest vocabulary index on ties; raw
 * logits, so temperature plays no part); the accepted path ends at the deepest
 * accepted node, smallest node index on ties; the bonus token is the argmax of
 * that node's row.
 *
 * target_logits [B, N1, V] dtype: row i = next-token logits after node i; row 0 = root.
 * parent        [B, N1] int32: parent[b,0] = -1, 0 <= parent[b,i] < i.
 * node_token    [B, N1] int32 in [0, V) for i >= 1 (entry 0 is ignored).
 * max_depth     capacity of the path outputs; must be >= the accepted depth.
 * out_accept_len [B] int32: accepted draft nodes on the path (root excluded).
 * out_tokens    [B, max_depth+1] int32: path tokens root-first, then the bonus, then -1.
 * out_path_nodes [B, max_depth+1] int32: path node indices root-first, then -1.
 * out_argmax    [B, N1] int32 row argmaxes, or NULL.
 * workspace     >= spec_verify_tree_greedy_workspace_size() bytes, as for the chain.
 *
 * Invalid device data for sequence b (bad parent, token out of range, accepted
 * depth > max_depth) sets out_accept_len[b] = -1 and its path outputs to -1.  Without
 * out_argmax the rows are read by a walk that hands partial results between
 * workgroups: a sequence whose wait gave up gets out_accept_len[b] = -2 and -1 path
 * outputs (see "Hand-over waits").
 * Limits: 1 <= N1 <= SPEC_MAX_TREE_NODES, V >= 1, 0 <= max_depth < N1 + 1.
 * ------------------------------------------------------------------------- */
size_t spec_verify_tree_greedy_workspace_size(int B, int N1, int V, spec_dtype_t dtype);

spec_status_t spec_verify_tree_greedy(const void* target_logits, spec_dtype_t dtype,
                                      const int32_t* parent, const int32_t* node_token,
                                      int B, int N1, int V, int max_depth,
                                      int32_t* out_accept_len, int32_t* out_tokens, int32_t* out_path_nodes,
                                      int32_t* out_argmax,
                                      void* workspace, size_t workspace_bytes, spec_stream_t stream);

/* ---------------------------------------------------------------------------
 * Stochastic tree verification (temperature > 0).
 *
 * [Production] section I.1 (accept with min(1, p/q), else draw from the normalised
 * residual max(0, p - q)) and section III.2 (a rejected branch B1 leaves its sibling
 * B2 free to be accepted).  The pages give the rule for a single drafted token only;
 * reading, from the published multi-candidate form of it: the children of a node
 * were drawn independently from the draft distribution q at that node and are tried
 * in node order against a residual r (r = p at first; after a rejection
 * r <- max(0, r - q) normalised).  An accepted child continues the walk; when every
 * child of a node is rejected a token is drawn from the last residual; a leaf reached
 * by acceptance yields a bonus token from its own p.  A chain-shaped tree is exactly
 * spec_verify_chain.  Temperature 0 (greedy) is spec_verify_tree_greedy.
 *
 * target_logits [B, N1, V] dtype: row i = target logits after node i (row 0 = root).
 * draft_logits  [B, N1, V] dtype: row i = draft logits that node i's children were
 *               drawn from (rows of leaves are never read).
 * parent, node_token as for spec_verify_tree_greedy.
 * temperature   [B] float32, > 0.
 * u_accept      [B, N1] float32 in (0, 1]: the uniform of node i's accept test
 *               (entry 0 unused).
 * u_final       [B] float32 in (0, 1]: the uniform of the final draw.
 * out_accept_len, out_tokens, out_path_nodes as for spec_verify_tree_greedy (the
 *               last token is the residual draw or the bonus).
 * workspace     >= spec_verify_tree_workspace_size() bytes, 256-byte aligned.
 *
 * Only the rows on the walk are read.  Invalid device data for sequence b (bad
 * parent, token out of range, temperature not > 0 or not finite, a uniform outside
 * (0, 1], accepted depth > max_depth) sets out_accept_len[b] = -1 and its outputs to
 * -1; a sequence whose hand-over wait gave up gets out_accept_len[b] = -2 and -1
 * outputs (see "Hand-over waits").  Each used row needs a finite logit.
 * Limits: 1 <= N1 <= SPEC_MAX_TREE_NODES, 0 <= max_depth <= N1, V <= 524288 (bf16) or
 * 262144 (fp32): at most 64 vocabulary slices of 8192 bf16 or 4096 fp32 logits.
 * ------------------------------------------------------------------------- */
size_t spec_verify_tree_workspace_size(int B, int N1, int V, spec_dtype_t dtype);

spec_status_t spec_verify_tree(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                               const int32_t* parent, const int32_t* node_token, const float* temperature,
                               const float* u_accept, const float* u_final, int B, int N1, int V, int max_depth,
                               int32_t* out_accept_len, int32_t* out_tokens, int32_t* out_path_nodes,
                               void* workspace, size_t workspace_bytes, spec_stream_t stream);

/* ---------------------------------------------------------------------------
 * Prompt n-gram lookup drafting.
 *
 * [Accelerating]: a zero-VRAM prompt n-gram lookup as the draft mechanism,
 * proposing K candidates; its deployment snippet (section 1) caps n at 4.
 *
 * Reading: for n = n_max down to n_min, find the earliest j with
 * context[j : j+n] == context[L-n : L] and j + n <= L - 1 (overlap allowed);
 * the first n that matches wins and the draft is context[j+n : min(j+n+K, L)].
 * Verify the result with spec_verify_chain(draft_logits = NULL,
 * draft_len = out_draft_len).
 *
 * context      [B, L_max] int32 token ids (any values; only equality is used).
 * context_len  [B] int32 L in [1, L_max].
 * out_draft_tokens [B, K] int32: the draft, then -1.
 * out_draft_len [B] int32 in [0, K] (0 = no match).
 * out_match_n  [B] int32 matched n (0 = none), or NULL.
 *
 * Invalid device data (L outside [1, L_max]) gives draft_len 0, match_n -1.
 * Limits: 1 <= n_min <= n_max <= SPEC_MAX_NGRAM_N, 1 <= K <= SPEC_MAX_K, L_max >= 1.
 * No workspace is needed.
 * ------------------------------------------------------------------------- */
spec_status_t ngram_propose(const int32_t* context, const int32_t* context_len,
                            int B, int L_max, int n_min, int n_max, int K,
                            int32_t* out_draft_tokens, int32_t* out_draft_len, int32_t* out_match_n,
                            spec_stream_t stream);

/* ---------------------------------------------------------------------------
 * Prompt n-gram lookup drafting and its verification in one call.
 *
 * [Accelerating] (prompt lookup drafts K tokens with q one-hot) and [Production]
 * section I.1 (the verification): the same results as ngram_propose followed by
 * spec_verify_chain(draft_logits = NULL, draft_tokens = out_draft_tokens,
 * draft_len = out_draft_len) on the same inputs, bit for bit, in one call whose
 * first kernel runs the lookup and the row statistics of all K+1 target rows of
 * every sequence side by side (every target row is read, also past a sequence's
 * draft length, since the lengths are not known until the lookup ends).
 *
 * context, context_len, L_max, n_min, n_max, out_draft_tokens, out_draft_len,
 * out_match_n: as for ngram_propose (K drafted tokens at most).
 * target_logits, dtype, temperature, u_accept, u_final, B, K, V, out_tokens,
 * out_num_accepted, out_probs, out_packed, out_offsets, workspace: as for
 * spec_verify_chain with draft_logits = NULL; the workspace is
 * spec_verify_chain_workspace_size(B, K, V, dtype) bytes.
 *
 * A sequence whose context length is invalid proposes nothing (draft length 0,
 * match_n -1) and is verified like any other with no draft: a token drawn from
 * p_0.  A proposed token outside [0, V) flags the sequence as spec_verify_chain does.
 * Limits: those of both calls.
 * ------------------------------------------------------------------------- */
spec_status_t spec_ngram_verify(const int32_t* context, const int32_t* context_len, int L_max, int n_min, int n_max,
                                const void* target_logits, spec_dtype_t dtype, const float* temperature,
                                const float* u_accept, const float* u_final, int B, int K, int V,
                                int32_t* out_draft_tokens, int32_t* out_draft_len, int32_t* out_match_n,
                                int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                int32_t* out_packed, int32_t* out_offsets,
                                void* workspace, size_t workspace_bytes, spec_stream_t stream);

/* ---------------------------------------------------------------------------
 * Tree-attention mask.
 *
 * [Production] section III.2 "The Tree Attention Verification Mechanism": the
 * candidate tree is flattened into one sequence (node order) and verified in one
 * target pass under a 2-D mask, so that each branch is scored on its own path.
 *
 * Reading: out_mask[b, i, j] = 1 iff node j lies on the path from the root to node
 * i, node i included (so row 0 is the root alone, column 0 is all ones, and the
 * mask is lower triangular); out_depth[b, i] = edges from the root to node i.  The
 * flattened sequence is the node order itself: node_token needs no reordering.
 *
 * parent    [B, N1] int32: parent[b,0] = -1, 0 <= parent[b,i] < i.
 * out_mask  [B, N1, N1] uint8 (0 or 1), or NULL; any alignment.
 * out_depth [B, N1] int32, or NULL (not both NULL).
 *
 * Invalid device data (a parent array that breaks the order) gives tree b an
 * all-zero mask and depth -1 for every node.
 * Limits: 1 <= N1 <= SPEC_MAX_TREE_NODES.  No workspace is needed.
 * ------------------------------------------------------------------------- */
spec_status_t spec_tree_mask(const int32_t* parent, int B, int N1, uint8_t* out_mask, int32_t* out_depth,
                             spec_stream_t stream);

/* ---------------------------------------------------------------------------
 * Commit of the accepted path's cache entries.
 *
 * [Medusa], "System Topology & Data Flow" figure: after tree verification the
 * tokens of the accepted branch are committed to the KV cache.
 *
 * Reading: the pass that scored the flattened tree produced one cache entry per
 * node, the root (the token emitted by the previous step) included.  For sequence
 * b with n = accept_len[b] and c = cache_len[b], the root's entry goes to cache
 * position c and the entry of the k-th accepted node to position c + k
 * (k = 1..n); out_cache_len[b] = c + n + 1.  The token emitted after the path has
 * no entry yet.  Without path_nodes the accepted nodes are 1..n (a chain).
 *
 * An entry is `planes` pieces of entry_bytes each (e.g. one per layer and K/V):
 * kv_nodes  piece p of node i of sequence b at byte
 *           p * node_plane_stride + (b * N1 + i) * entry_bytes;
 *           holds (planes - 1) * node_plane_stride + B * N1 * entry_bytes bytes.
 * kv_cache  piece p of position t of sequence b at byte
 *           p * cache_plane_stride + (b * L_cap + t) * entry_bytes;
 *           holds (planes - 1) * cache_plane_stride + B * L_cap * entry_bytes bytes.
 *           Only the committed positions are written.
 * path_nodes [B, path_stride] int32: accepted nodes from the root side, root
 *           excluded (out_path_nodes of spec_verify_tree_greedy, path_stride =
 *           max_depth + 1), or NULL for a chain.
 * accept_len [B] int32 (out_accept_len of verification; -1 = flagged invalid).
 * cache_len [B] int32 committed length before the call.
 * out_cache_len [B] int32 length after the call, or NULL; must not alias cache_len.
 * kv_nodes and kv_cache must not overlap; both 16-byte aligned; entry_bytes and
 * (with planes > 1) the plane strides are multiples of 16, each stride at least
 * one plane.
 *
 * Invalid device data for sequence b (accept_len < 0, n > path_stride or, without
 * path_nodes, n > N1 - 1, a path node outside [0, N1), c < 0 or c + n + 1 > L_cap)
 * writes nothing for b and sets out_cache_len[b] = -1.
 * Limits: planes * entry_bytes / 16 < 2^31, 1 <= path_stride <= SPEC_MAX_TREE_NODES + 1.
 * No workspace is needed.
 * ------------------------------------------------------------------------- */
spec_status_t spec_commit_path(const void* kv_nodes, const int32_t* path_nodes, int path_stride,
                               const int32_t* accept_len, const int32_t* cache_len,
                               int B, int N1, int L_cap, int planes, size_t entry_bytes,
                               size_t node_plane_stride, size_t cache_plane_stride,
                               void* kv_cache, int32_t* out_cache_len, spec_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
