/*
 * treeverify.h -- C ABI of libtreeverify.so, the tree-verification step of
 * EAGLE-2/3 dynamic-tree speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * One verification step is five calls, in this order:
 *   tree_build          draft log-probs  -> draft_tokens, parents, tree_size
 *   (tree_build_meta    tree_build and tree_mask_positions in tree_build's launches)
 *   tree_mask_positions parents          -> packed ancestor mask, positions,
 *                                           retrieve_indices, child/sibling lists
 *   tree_attention      Q, K/V cache, mask -> O (every node over prefix + ancestors)
 *   (tree_attention_rope the same with the queries' rotary embedding fused in)
 *   tree_accept         target argmax per node -> accepted path, bonus token
 *   (tree_accept_sample the same from target distributions, by rejection sampling;
 *    tree_sampling_probs filters the target logits into those distributions;
 *    tree_accept_sample_draft samples with the drafter's distribution as well)
 *   kv_compact          accepted path    -> K/V rows moved to contiguous slots
 *   tree_accept_compact the last two in one launch
 * and the same attention and compaction over a paged K/V cache (a block table
 * per request): tree_attention_paged, kv_compact_paged, tree_accept_compact_paged;
 * and the dynamic build one draft layer at a time, for a draft loop that runs
 * the draft model on each layer's frontier: tree_build_layer (D + 1 times),
 * then tree_build_finish.
 *
 * Sources for what each call computes (cited by page title and section):
 *   [E2]  EAGLE v2 dynamic-tree decoding walkthrough -- section 2 initialize_tree
 *         (outputs draft_tokens, retrieve_indices, tree_mask, tree_position_ids),
 *         section 3 topK_generate, section 4 tree_decoding, section 5
 *         evaluate_posterior.
 *   [HB]  AI-infra handbook, "Advanced speculative decoding: tree drafts and
 *         EAGLE" -- tree_spec.py (forward_with_mask, tree_mask, depths,
 *         build_draft_tree, tree_speculative_generate), the KV note after it,
 *         and the exercise "trees when sampling".
 *   [TRT] "TensorRT-LLM source dissection (22): EAGLE-3 one-model drafter" --
 *         section "dynamic draft tree": the three ledgers (parent buffer, packed
 *         mask [bs, N, ceil(N/32)], position offsets), the tree-build kernel,
 *         greedy verification on the child/sibling lists, the non-greedy path
 *         (target logits filtered per request, target-only rejection sampling),
 *         KV relocation.
 *
 * Conventions (all calls):
 *   - Every pointer is a DEVICE pointer unless marked "host".  The caller owns
 *     and allocates every buffer; the library keeps no state and allocates no
 *     memory.  Scratch memory comes from the caller as a workspace sized by the
 *     matching *_workspace_bytes() query.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work on that stream and never synchronize.
 *   - Return value: TV_OK, or a negative TV_E* code.  Arguments are validated on
 *     the host before anything is enqueued; nothing is clamped or truncated
 *     silently.  Out-of-range data that only the device can see (tree sizes,
 *     parents, prefix lengths) is reported per request in `status[b]`.
 *   - Per-request status (int32, in/out along the pipeline): TV_ST_OK or a
 *     TV_ST_* code.  A request with non-zero status degrades to the root-only
 *     tree (mask = bit 0, position = prefix_len, accept_len = 0, bonus =
 *     target_predict[0], compaction a no-op), mirroring the default linear
 *     chain / tree_valid fallback of [TRT] ("per-request trees stored by slot").
 *   - Tree layout: node 0 is the root; tree_size counts the root; parents[0] =
 *     -1 and 0 <= parents[i] < i.  T_max is the padded node dimension of every
 *     per-node array (T_max <= 256; trees of up to 64 nodes take one wavefront per
 *     request, larger ones a 256-thread workgroup).  Padding entries are
 *     -1 for tokens / parents / node ids, 0 for masks and positions, -inf for
 *     scores.  dcap is the deepest node depth the caller provisions for
 *     (retrieve rows and accepted paths have dcap + 1 columns).
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define TV_OK 0
#define TV_EINVAL (-1)       /* null pointer, bad dimension or inconsistent sizes */
#define TV_EUNSUPPORTED (-2) /* a size this build does not implement (d, T_max, dtype, K) */
#define TV_EWORKSPACE (-3)   /* workspace missing or smaller than the query says */
#define TV_ELAUNCH (-4)      /* the HIP runtime rejected a kernel launch */

/* per-request status codes */
#define TV_ST_OK 0
#define TV_ST_PARENTS 1   /* parents[0] != -1, or parents[i] outside [0, i) */
#define TV_ST_DEPTH 2     /* a node deeper than dcap */
#define TV_ST_SIZE 3      /* tree_size outside [1, T_max] */
#define TV_ST_LOGPROB 4   /* NaN / positive log-prob read, or a kept node whose parent was dropped */

#define TV_MODE_DYNAMIC 0
#define TV_MODE_STATIC 1
#define TV_DTYPE_BF16 0
#define TV_DTYPE_FP32 1

/* ------------------------------------------------------------------------- *
 * tree_build -- [E2] section 3 (topK_generate), [TRT] _select_topk_draft_tokens,
 * [HB] build_draft_tree.
 *
 * mode TV_MODE_DYNAMIC (EAGLE-2): logprobs is float32 [B][rows_per_req][V] with
 *   rows_per_req = 1 + D*K.  Row 0 is the draft distribution after the root; row
 *   1 + (l-1)*K + j is the distribution after frontier slot j of expansion round
 *   l (l = 1..D).  Base layer: the K best tokens of row 0 (log-prob descending,
 *   token ascending) are candidates 0..K-1 with score = log-prob.  Round l: every
 *   frontier slot j expands into the K best tokens r of its row, candidate id
 *   K + (l-1)K^2 + jK + r, score = float32(log-prob + score of slot j); the K best
 *   of those K^2 (score descending, jK+r ascending) are the next frontier.  Final:
 *   the total_tokens best of all C = K + D*K^2 candidates (score descending, id
 *   ascending) become nodes 1..total_tokens in ascending id; node 0 is the root
 *   (draft_tokens[0] = root_token[b], score 0).  tree_size = total_tokens + 1.
 *   Requires 1 <= K <= 16, 0 <= D <= 64, 0 <= total_tokens <= C, C <= 3072,
 *   total_tokens + 1 <= T_max, K <= V.  `branching` is ignored.
 * mode TV_MODE_STATIC ([HB] build_draft_tree): branching (host, n_levels
 *   entries, each 1..16) gives the width of each level; every node of the
 *   current frontier, in order, appends the top-branching[l] tokens of its own
 *   row as children.  Row n of logprobs is the distribution after node n;
 *   rows_per_req must equal the number of expanded (non-last-level) nodes.
 *   Node score = float32(log-prob + parent score).  K, D, total_tokens ignored.
 * Outputs (each [B][T_max], padded): draft_tokens int32, parents int32,
 *   node_score float32 (nullable), tree_size int32 [B], status int32 [B]
 *   (TV_ST_OK or TV_ST_LOGPROB: any NaN or positive value in a row that is read
 *   gives the root-only tree).
 * Workspace: tree_build_workspace_bytes(mode, B, V, K, rows_per_req) bytes (any
 *   contents); calls that share a workspace must not overlap in time.
 * ------------------------------------------------------------------------- */
size_t tree_build_workspace_bytes(int mode, int B, int V, int K, int rows_per_req);
int tree_build(int mode, int B, int V, int K, int D, int total_tokens,
               const int* branching /* host */, int n_levels,
               const float* logprobs, int rows_per_req, const int* root_token,
               int T_max, int* draft_tokens, int* parents, int* tree_size,
               float* node_score /* nullable */, int* status,
               void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * tree_build_layer / tree_build_finish -- the dynamic build of tree_build, one
 * draft layer at a time ([E2] section 3, topK_generate: the draft model runs on
 * the frontier each round chooses, so a round's rows exist only after it).
 *
 * Call tree_build_layer for layer = 0, 1, ..., D in order on one state, then
 * tree_build_finish.  Layer 0 takes rows [B][1][V], the draft distribution
 * after the root; layer l >= 1 takes rows [B][K][V], row j the distribution
 * after frontier slot j of layer l - 1 (what the draft model gives for the
 * token frontier_tokens[b][j] returned by the previous call).  Each call writes
 * the new frontier: frontier_tokens [B][K] in rank order, and (nullable)
 * frontier_parents [B][K], the slot of the previous frontier each extends (-1
 * at layer 0).  tree_build_finish then writes what tree_build writes (and, when
 * prefix_len is not NULL, what tree_mask_positions writes, as tree_build_meta
 * does; with prefix_len NULL the metadata pointers are ignored).
 * Results equal tree_build on the same rows stacked as [B][1 + D K][V].
 * rows_are_logits = 1: the rows are raw draft logits instead of log-probs.  A
 *   row's K best tokens are then taken by logit (token ascending on ties), the
 *   order of the row's log-softmax before rounding, and scored by its log-prob
 *   float32(x - lse), lse = m + log(sum exp(x - m)) computed in float64; NaN or
 *   +-inf in a row is a bad value (TV_ST_LOGPROB at finish).
 * The frontier outputs of a layer with a bad value are unspecified.
 * state: tree_build_layer_workspace_bytes(B, V, K, D) bytes (any contents
 *   before layer 0); it carries the build from call to call, so the calls of one
 *   build must not overlap another build on the same state.
 * Requires the dynamic-mode conditions of tree_build; total_tokens and T_max
 *   are checked by tree_build_finish.
 * ------------------------------------------------------------------------- */
size_t tree_build_layer_workspace_bytes(int B, int V, int K, int D);
int tree_build_layer(int layer, int B, int V, int K, int D, const float* rows, int rows_are_logits,
                     void* state, size_t state_bytes, int* frontier_tokens,
                     int* frontier_parents /* nullable */, void* stream);
int tree_build_finish(int B, int V, int K, int D, int total_tokens, const int* root_token, int T_max,
                      const void* state, size_t state_bytes, int* draft_tokens, int* parents,
                      int* tree_size, float* node_score /* nullable */, int* status, int dcap,
                      const int* prefix_len /* nullable: no metadata */, uint32_t* tree_mask,
                      int* tree_position_ids, int* positions, int* retrieve_indices, int* leaf_count,
                      int* first_child /* nullable */, int* next_sibling /* nullable */, void* stream);

/* ------------------------------------------------------------------------- *
 * tree_mask_positions -- [TRT] tree-build kernel (parents -> packed ancestor
 * mask, position offsets, retrieve lists; outputs fully rewritten each step),
 * [HB] tree_mask / depths, [E2] section 3 third step (tree_mask,
 * retrieve_indices, tree_position_ids).
 *
 * In:  parents [B][T_max], tree_size [B], prefix_len [B], status_in [B]
 *      (nullable = all TV_ST_OK; a non-zero entry is kept and gives the
 *      root-only tree; may alias status_out).
 * Out: tree_mask uint32 [B][T_max][W], W = ceil(T_max/32): row i has bit j&31 of
 *        word j>>5 set iff node j is node i or one of its ancestors;
 *      tree_position_ids [B][T_max] = node depth (root 0);
 *      positions [B][T_max] = prefix_len[b] + depth (siblings share a position);
 *      retrieve_indices [B][T_max][dcap+1]: one row per leaf (a node without
 *        children), leaves in ascending id, column k = the node at depth k on
 *        the root-to-leaf path, -1 padded; rows >= leaf_count all -1;
 *      leaf_count [B];
 *      first_child / next_sibling [B][T_max] (nullable): children in ascending
 *        id, -1 where none;
 *      status_out [B]: status_in if non-zero, else TV_ST_SIZE, TV_ST_PARENTS,
 *        TV_ST_DEPTH (checked in that order) or TV_ST_OK.
 * Requires 1 <= T_max <= 256, 0 <= dcap < T_max.
 * ------------------------------------------------------------------------- */
int tree_mask_positions(int B, int T_max, int dcap, const int* parents,
                        const int* tree_size, const int* prefix_len,
                        uint32_t* tree_mask, int* tree_position_ids, int* positions,
                        int* retrieve_indices, int* leaf_count,
                        int* first_child /* nullable */, int* next_sibling /* nullable */,
                        const int* status_in /* nullable */, int* status_out, void* stream);

/* ------------------------------------------------------------------------- *
 * tree_build_meta -- tree_build followed by tree_mask_positions on its output,
 * in the launches of tree_build alone.  Arguments: those of tree_build, then
 * dcap, prefix_len and the outputs of tree_mask_positions (status is both the
 * build's status and the metadata's status_out).  Results equal tree_build then
 * tree_mask_positions(status_in = status_out = status) on the same inputs, and
 * the checks of both calls apply.  For a step that runs both calls back to
 * back: the build's last kernel, which holds the new tree on chip, writes the
 * metadata too, which saves one kernel boundary.
 * ------------------------------------------------------------------------- */
int tree_build_meta(int mode, int B, int V, int K, int D, int total_tokens,
                    const int* branching /* host */, int n_levels,
                    const float* logprobs, int rows_per_req, const int* root_token,
                    int T_max, int* draft_tokens, int* parents, int* tree_size,
                    float* node_score /* nullable */, int* status,
                    void* workspace, size_t ws_bytes, int dcap, const int* prefix_len,
                    uint32_t* tree_mask, int* tree_position_ids, int* positions,
                    int* retrieve_indices, int* leaf_count,
                    int* first_child /* nullable */, int* next_sibling /* nullable */,
                    void* stream);

/* ------------------------------------------------------------------------- *
 * tree_attention -- [HB] forward_with_mask (full mask = all-visible prefix
 * columns followed by the tree mask; grouped KV heads repeated over the query
 * heads; default softmax scale), [E2] section 4 tree_decoding.
 *
 * For request b, query head h and node i < T_b (T_b = tree_size[b], or 1 when
 * status[b] != 0): keys = cache rows 0..P_b-1 (P_b = prefix_len[b]) and rows
 * P_b + j for every node j whose bit is set in tree_mask row i, of kv head
 * g = h / (Hq/Hkv).  O[b][i][h] = softmax(scale * q . k) . v.
 * Layouts (elements of dtype: bf16 or float32, row-major):
 *   Q, O  [B][T_max][Hq][d];  Kc, Vc  [B][Hkv][S_cap][d], tree node j's K/V at
 *   row P_b + j (already written by the caller's projection of the tree).
 * scale <= 0 selects 1/sqrt(d).  bf16 inputs accumulate in float32; the softmax
 * is computed online in float32.  Rows i >= T_b of O are not written.  A request
 * whose prefix does not fit the cache (prefix_len < 0 or prefix_len + T_b >
 * S_cap) reads no K/V and gets O rows 0..T_b-1 set to zero (status is read,
 * never written, by this call).
 * Requires d in {64, 128}, Hq % Hkv == 0 (any group size), T_max <= 256,
 * S_cap <= 2^30.  Every buffer must be allocated to its full layout size: rows
 * past a request's keys or nodes may be read, but their contents (any bits,
 * NaN included) never reach the output.
 * Workspace: tree_attention_workspace_bytes(...) with the same shape arguments.
 * ------------------------------------------------------------------------- */
size_t tree_attention_workspace_bytes(int dtype, int B, int T_max, int Hq, int Hkv, int d,
                                      long long S_cap);
int tree_attention(int dtype, int B, int T_max, int Hq, int Hkv, int d,
                   const void* Q, const void* Kc, const void* Vc, long long S_cap,
                   const int* prefix_len, const int* tree_size, const uint32_t* tree_mask,
                   const int* status, float scale, void* O,
                   void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * tree_attention_noalloc -- tree_attention for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, checks and results as
 * tree_attention, without the workspace: the split-KV partials go to a scratch
 * array the library holds in device memory, one per GPU, of
 * tree_attention_noalloc_max_bytes() bytes (64 MiB), kept until the process
 * ends.  A shape whose tree_attention_workspace_bytes(...) exceeds that is
 * refused with TV_EWORKSPACE before any device call.  The call allocates
 * nothing; its first call on a device looks up that device's scratch address
 * (TV_ELAUNCH if the runtime cannot).  Every call on one GPU shares the array:
 * calls that overlap on one GPU (concurrent streams, or threads) race on it and
 * must be serialised by the caller.  Nothing in the scratch needs clearing
 * between calls.
 * ------------------------------------------------------------------------- */
size_t tree_attention_noalloc_max_bytes(void);
int tree_attention_noalloc(int dtype, int B, int T_max, int Hq, int Hkv, int d,
                           const void* Q, const void* Kc, const void* Vc, long long S_cap,
                           const int* prefix_len, const int* tree_size,
                           const uint32_t* tree_mask, const int* status, float scale, void* O,
                           void* stream);

/* ------------------------------------------------------------------------- *
 * tree_attention_rope -- tree_attention with the rotary position embedding of
 * the queries fused in ([HB] forward_with_mask rotates the tree's queries and
 * keys at position prefix + depth, siblings sharing a position).
 *
 * Q holds the queries BEFORE their rotary embedding; the kernel rotates query
 * row (node i, head h) at position P_b + depth_i (depth_i = the number of node
 * i's ancestors in its tree_mask row, i.e. tree_position_ids), in the
 * rotate-half layout: pair (j, j + d/2) turns by the angle
 * pos * rope_theta^(-2j/d) (out_j = q_j cos - q_(j+d/2) sin, out_(j+d/2) =
 * q_(j+d/2) cos + q_j sin), in float32 with the angle reduced to revolutions
 * with ~1e-7 accuracy, then rounds to bf16 for the products.  The cache holds
 * keys after their rotary embedding (prefix rows and tree rows alike).
 * Everything else is tree_attention's.  Requires rope_theta > 1 and
 * S_cap <= 2^24 (positions exact in float32).
 * ------------------------------------------------------------------------- */
int tree_attention_rope(int dtype, int B, int T_max, int Hq, int Hkv, int d,
                        const void* Q, const void* Kc, const void* Vc, long long S_cap,
                        const int* prefix_len, const int* tree_size, const uint32_t* tree_mask,
                        const int* status, float rope_theta, float scale, void* O,
                        void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * tree_accept -- [TRT] greedy verification (walk from the root: accept the child
 * whose token equals the target's argmax, else stop; path <= depth + 1), [HB]
 * tree_speculative_generate (first matching child by index; next root = target
 * argmax at the path end), [E2] section 5 (same result as the longest
 * cumprod-accepted retrieve row when sibling tokens are distinct).
 *
 * In:  draft_tokens, parents, target_predict [B][T_max] (the target's argmax at
 *      every node), tree_size [B], status [B].
 * Out: accept_len [B] = accepted draft nodes (0..dcap), accept_path
 *      [B][dcap+1] = node ids root first, -1 padded, bonus_token [B] =
 *      target_predict at the last node of the path.
 * ------------------------------------------------------------------------- */
int tree_accept(int B, int T_max, int dcap, const int* draft_tokens, const int* parents,
                const int* tree_size, const int* target_predict, const int* status,
                int* accept_len, int* accept_path, int* bonus_token, void* stream);

/* ------------------------------------------------------------------------- *
 * tree_accept_sample -- non-greedy acceptance: [TRT] target-only rejection
 * sampling (one probability test per node instead of an argmax comparison, and
 * a correction token sampled from the target distribution at the point of
 * rejection), [HB] exercise "trees when sampling" (children in order, accept
 * with min(1, p/q), continue with norm(max(0, p - q)), sample the correction
 * from the last residual when every child is rejected).
 *
 * The tree's candidates are the drafter's deterministic top-K picks, so a
 * candidate's draft distribution q is the point mass on its token.  From the
 * root: at node n with target row p = target_probs[b][n] (Z = sum of the row,
 * float64), try the children in ascending id; child c with token x is accepted
 * iff uniforms[b][c] * (Z - R) < p(x), R being the mass of the tokens already
 * rejected at n (a token already rejected, or outside [0, V), has p(x) = 0);
 * on acceptance move to c.  The walk stops when every child is rejected, at
 * depth dcap, or at once when status != 0.  bonus_token = the correction at the
 * last node: with r = p minus the rejected tokens' mass, the smallest v whose
 * cumulative sum of r (float64, token order) exceeds uniforms[b][0] * sum(r);
 * if rounding leaves none, the last v with r(v) > 0; if sum(r) = 0, the row's
 * best token (probability desc, token asc).
 * In:  draft_tokens, parents [B][T_max], tree_size [B], status [B];
 *      target_probs float32 [B][T_max][V] (the target's distribution at every
 *      node after the caller's temperature / top-k / top-p filtering; rows
 *      i >= T_b are never read); uniforms float32 [B][T_max] in [0, 1): entry
 *      c >= 1 is the draw for child c's test, entry 0 the draw for the
 *      correction token.
 * Out: accept_len, accept_path, bonus_token as tree_accept.
 * Workspace (optional): NULL, or at least tree_accept_sample_workspace_bytes(B,
 *      T_max) bytes (8-byte aligned, contents arbitrary, overwritten).  With it,
 *      a call whose rows total at most 32 MB first sums every row i < T_b on
 *      its own workgroup (as many CUs as rows), so the walk's decisions read Z
 *      instead of passing over each visited row; the results are the same
 *      either way (each row is summed in the same order).  A workspace that is
 *      too small or misaligned gives TV_EWORKSPACE.
 * Requires 1 <= T_max <= 256, 0 <= dcap < T_max, 1 <= V <= 262144, B <= 65535.
 * ------------------------------------------------------------------------- */
size_t tree_accept_sample_workspace_bytes(int B, int T_max);
int tree_accept_sample(int B, int T_max, int dcap, int V, const int* draft_tokens, const int* parents,
                       const int* tree_size, const float* target_probs, const float* uniforms,
                       const int* status, int* accept_len, int* accept_path, int* bonus_token,
                       void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * tree_sampling_probs -- [TRT] "non-greedy: rejection from the target
 * distribution alone": before the rejection step the target's logits at every
 * tree node are turned into probabilities with the request's sampling
 * parameters (temperature, top-k, top-p, min-p), the per-request parameters
 * repeated over the request's nodes and each node filtered on its own.
 *
 * For request b and node i < T_b (T_b = tree_size[b], or 1 when status[b] != 0
 * or the size is out of range), row probs[b][i] is computed from logits[b][i]:
 *   - tokens rank by (logit descending, token ascending); NaN ranks as -inf,
 *     -0.0 equals +0.0;
 *   - temperature[b] <= 0 (or NaN), top_k[b] == 1 or top_p[b] <= 0: 1.0 on the
 *     first-ranked token, 0 elsewhere;
 *   - otherwise the weight of token v is w = float32(exp((l_v - l_max) /
 *     temperature)) computed in float64, exactly 1 where l_v equals the largest
 *     logit; then, in this order: top-k (1 < top_k < V) keeps the first top_k
 *     ranks; top-p (top_p < 1) keeps the shortest rank prefix of those whose
 *     cumulative weight reaches top_p x their total weight (sums in float64);
 *     min-p (min_p > 0) drops tokens with w < min_p, the first-ranked token
 *     always kept; the output is w / (sum of kept w) in float64, rounded to
 *     float32, and 0 for dropped tokens.
 * Rows i >= T_b are not written.  The result feeds tree_accept_sample (target
 * only) or tree_accept_sample_draft.
 * In:  logits float32 [B][T_max][V]; tree_size [B]; status [B] (nullable = all
 *      TV_ST_OK); temperature, top_p, min_p float32 [B]; top_k int32 [B]
 *      (<= 0 or >= V: no top-k).
 * Out: probs float32 [B][T_max][V] (must not overlap logits).
 * Requires 1 <= T_max <= 256, 1 <= V <= 262144, B <= 65535.
 * ------------------------------------------------------------------------- */
int tree_sampling_probs(int B, int T_max, int V, const float* logits, const int* tree_size,
                        const int* status, const float* temperature, const int* top_k,
                        const float* top_p, const float* min_p, float* probs, void* stream);

/* ------------------------------------------------------------------------- *
 * tree_accept_sample_draft -- tree rejection sampling with the drafter's
 * distribution: [HB] exercise "trees when sampling" (at a node try its
 * children in order, accept each with min(1, p(x)/q(x)); after a rejection the
 * target becomes norm(max(0, p - q)) and q is adjusted to how the candidates
 * were drawn; when every child is rejected the correction token comes from the
 * last residual).
 *
 * draft_probs[b][n] is q at node n: the drafter's distribution that node n's
 * children were proposed from.  On entering node n, R = target_probs[b][n] and
 * Q = draft_probs[b][n] (float64), ZR, ZQ their sums.  Children in ascending
 * id: child c with token x, r = R(x), s = Q(x) (0 outside [0, V)), is accepted
 * iff r > 0 and (s == 0 or uniforms[b][c] * s * ZR < r * ZQ), each product
 * rounded on its own; on acceptance move to c.  On rejection, if ZQ > 0:
 * R <- max(0, R * ZQ - Q * ZR) elementwise (the residual up to a positive
 * factor), ZR <- sum(R); with without_replacement != 0 (candidates drawn
 * without replacement) Q(x) <- 0 and ZQ <- sum(Q), otherwise Q is kept
 * (independent draws).  The walk stops when every child is rejected, at depth
 * dcap, or at once when status != 0.  bonus_token: the smallest v whose
 * cumulative R (float64, token order; R = the node's row p when nothing was
 * rejected there) exceeds uniforms[b][0] * sum(R); if rounding leaves none, the
 * last v with R(v) > 0; if sum(R) = 0, the node's best token (p descending,
 * token ascending).  With draft rows that are the point mass on a chain node's
 * only child this is tree_accept_sample; with one-hot target rows it is
 * tree_accept.
 * In:  as tree_accept_sample, plus draft_probs float32 [B][T_max][V] (rows of
 *      nodes the walk does not reach are not read).
 * Out: accept_len, accept_path, bonus_token as tree_accept.
 * Workspace: tree_accept_sample_draft_workspace_bytes(B, V) bytes (B x V
 *   float64 words per request, any contents, 8-byte aligned): the residual
 *   rows, or, when few requests share a large vocabulary and several
 *   workgroups split each row between them, the slots through which they
 *   exchange their partial sums.  Those workgroups wait for each other with
 *   bounded waits; a request whose wait runs out (all of a call's workgroups
 *   are sized to be resident at once, so this does not happen unless other
 *   work holds the device's CUs for seconds) gets accept_len = bonus_token = -1.
 * Requires 1 <= T_max <= 256, 0 <= dcap < T_max, 1 <= V <= 262144.
 * ------------------------------------------------------------------------- */
size_t tree_accept_sample_draft_workspace_bytes(int B, int V);
int tree_accept_sample_draft(int B, int T_max, int dcap, int V, const int* draft_tokens,
                             const int* parents, const int* tree_size, const float* target_probs,
                             const float* draft_probs, const float* uniforms, const int* status,
                             int without_replacement, int* accept_len, int* accept_path,
                             int* bonus_token, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * kv_compact -- [TRT] "after acceptance: KV from tree layout back to linear",
 * [HB] note after tree_spec.py (accepted KV is reused, not recomputed; it is
 * compacted into the sequence's positions, rejected slots are dropped).
 *
 * Kc, Vc: n_layers blocks of [B][Hkv][S_cap][d] elements of elem_bytes (2 or
 * 4), block l at element offset l * layer_stride_elems.  For every layer, kv
 * head and k = 1..L (L = accept_len[b]) row P_b + k receives the old row
 * P_b + accept_path[b][k]; all sources of a (request, head, layer) are read
 * before any destination is written, so overlapping paths are safe.  Other rows
 * are untouched.  new_prefix_len[b] = P_b + L + 1 (nullable); it must not
 * overlap prefix_len, accept_len or accept_path (TV_EINVAL: the workgroups of a
 * request read those while one of them writes new_prefix_len, so a prefix grown
 * in place would move the wrong rows -- write it to a buffer of its own).  Requires
 * d*elem_bytes to be a multiple of 16 and <= 1024, dcap < 64, and
 * 2 * dcap * d * elem_bytes <= 65536 (the K and V rows of one path are staged
 * in on-chip memory; TV_EUNSUPPORTED otherwise).
 * ------------------------------------------------------------------------- */
int kv_compact(int B, int n_layers, int Hkv, int d, int elem_bytes, void* Kc, void* Vc,
               long long S_cap, long long layer_stride_elems, const int* prefix_len,
               const int* accept_path, const int* accept_len, int dcap,
               int* new_prefix_len /* nullable */, void* stream);

/* ------------------------------------------------------------------------- *
 * tree_accept_compact -- tree_accept followed by kv_compact, in one launch.
 * Same arguments, outputs and checks as the two calls (tree_accept's first,
 * then kv_compact's; accept_path and accept_len are outputs here, and the walk
 * is taken from draft_tokens/parents/target_predict directly).  Results equal
 * tree_accept then kv_compact on the same inputs.  For a step that runs both
 * calls back to back: each (request, kv head, layer) workgroup repeats the
 * request's walk, which saves one kernel boundary.  new_prefix_len must not
 * overlap prefix_len (TV_EINVAL), as in kv_compact.
 * ------------------------------------------------------------------------- */
int tree_accept_compact(int B, int T_max, int dcap, const int* draft_tokens, const int* parents,
                        const int* tree_size, const int* target_predict, const int* status,
                        int* accept_len, int* accept_path, int* bonus_token, int n_layers, int Hkv,
                        int d, int elem_bytes, void* Kc, void* Vc, long long S_cap,
                        long long layer_stride_elems, const int* prefix_len,
                        int* new_prefix_len /* nullable */, void* stream);

/* ------------------------------------------------------------------------- *
 * Paged K/V cache -- [TRT] "after acceptance: KV from tree layout back to
 * linear" (the cache is paged: a token's physical slot is given by its request's
 * block table and its offset inside the block; the relocation kernel walks the
 * block table and copies inside blocks), [HB] "implementing it in an engine"
 * (compact the accepted slots, or only update the block table).
 *
 * K_pool, V_pool: [num_blocks][Hkv][tokens_per_block][d] elements (kv head g's
 *   rows of one block are contiguous); for the compaction calls, n_layers such
 *   pools at element offsets l * layer_stride_elems.
 * block_table: int32 [B][max_blocks_per_seq]; logical row s of request b (the
 *   row the linear calls call s) lives in block block_table[b][s /
 *   tokens_per_block] at offset s % tokens_per_block.  tokens_per_block is a
 *   power of two in [1, 1024].  A request holds at most S_cap = max_blocks_per_seq
 *   * tokens_per_block rows, which takes the place of the linear calls' S_cap
 *   everywhere (workspace size included).
 * Table entries must lie in [0, num_blocks) for every logical row a call reads
 *   or writes (rows below prefix_len + tree_size, resp. the accepted path's
 *   rows).  Entries past those rows are never read.  An entry outside the pool
 *   is never dereferenced: tree_attention_paged clamps it into the pool (that
 *   request's output is then unspecified, other requests are unaffected) and
 *   the compaction calls leave that request untouched (new_prefix_len = P_b + 1,
 *   as for a path that does not fit).
 * Everything else -- arguments, results, checks, workspace -- is that of
 * tree_attention, kv_compact and tree_accept_compact; results equal those calls
 * on the linear cache the table describes.
 * ------------------------------------------------------------------------- */
int tree_attention_paged(int dtype, int B, int T_max, int Hq, int Hkv, int d,
                         const void* Q, const void* K_pool, const void* V_pool,
                         long long num_blocks, int tokens_per_block,
                         const int* block_table, int max_blocks_per_seq,
                         const int* prefix_len, const int* tree_size, const uint32_t* tree_mask,
                         const int* status, float scale, void* O,
                         void* workspace, size_t ws_bytes, void* stream);
int kv_compact_paged(int B, int n_layers, int Hkv, int d, int elem_bytes,
                     void* K_pool, void* V_pool, long long num_blocks, int tokens_per_block,
                     const int* block_table, int max_blocks_per_seq, long long layer_stride_elems,
                     const int* prefix_len, const int* accept_path, const int* accept_len, int dcap,
                     int* new_prefix_len /* nullable */, void* stream);
int tree_accept_compact_paged(int B, int T_max, int dcap, const int* draft_tokens, const int* parents,
                              const int* tree_size, const int* target_predict, const int* status,
                              int* accept_len, int* accept_path, int* bonus_token, int n_layers,
                              int Hkv, int d, int elem_bytes, void* K_pool, void* V_pool,
                              long long num_blocks, int tokens_per_block, const int* block_table,
                              int max_blocks_per_seq, long long layer_stride_elems,
                              const int* prefix_len, int* new_prefix_len /* nullable */,
                              void* stream);

/* human-readable names for return codes and status codes */
const char* tv_error_string(int code);
const char* tv_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* TREEVERIFY_H */
