/*
 * kdtree_verify.h -- C ABI of the MI355X (gfx950) tree-verify MLA-absorb attention.
 *
 * The operation ("The Milestone Commit: Cementing Phase 1 ...", section "The
 * Context", item 2): every draft-tree node of a request is a query row in the
 * absorbed MLA latent space (H heads x (512 latent + 64 rope) dims).  It attends,
 * with a masked softmax, over one latent KV stream shared by all heads: the
 * request's prefix followed by its tree tail.  Prefix keys are visible to every
 * node; a tail key is visible only to the node it belongs to and that node's
 * descendants, i.e. each node sees its ancestors-or-self ("Strategic Pivots in CUDA
 * Kernel Engineering ...", section "The Message": a tree visibility mask from the
 * builder).  The result is a 512-dim latent output per (node, head) plus the row's
 * log-sum-exp, produced on the device with no host round trips.  The library shape
 * (extern "C" wrappers in one shared library, a MAX_QLEN query, a Python ctypes
 * bridge passing raw device pointers and the caller's stream) follows "The Capstone
 * Commit: Validating a Native CUDA DDTree Inference Engine", section "The Message
 * Itself" (commit body) and section "Output Knowledge Created".
 *
 * Math, per request b, node i, head h (natural log, fp32 output):
 *   K_k = [kv_lat_k | k_rope_k] (576), V_k = kv_lat_k (512), Q = [q_lat | q_rope]
 *   s_k = scale * (Q . K_k) for visible keys k
 *   out_lat = sum_k softmax(s)_k V_k,   out_lse = ln sum_k exp(s_k)
 *
 * Packed layout (all device memory, row-major, contiguous, no padding):
 *   q_lat  [total_q, H, 512]  q_rope [total_q, H, 64]   (dtype: fp32 or bf16)
 *   kv_lat [total_kv, 512]    k_rope [total_kv, 64]     (same dtype)
 *   prefix_len [batch], q_len [batch]  int32
 *   tree_parent [total_q] int32: local node index of each node's parent; -1 at the
 *       root (node 0); parent[i] in [0, i) for i >= 1 (best-first pop order).
 *   out_lat [total_q, H, 512] fp32, out_lse [total_q, H] fp32.
 *   Request b owns query rows [qoff_b, qoff_b + q_len[b]) and KV rows
 *   [kvoff_b, kvoff_b + prefix_len[b] + q_len[b]): prefix_len[b] prefix rows, then
 *   q_len[b] tail rows in node order (tail row j = node j).  qoff / kvoff are the
 *   exclusive prefix sums of q_len and prefix_len + q_len; the kernels compute them
 *   on the device.
 *
 * Ownership: the caller owns every buffer and keeps it alive until the work
 * enqueued on `stream` has finished.  The library never allocates, never reads
 * device memory on the host and never synchronises: calls are asynchronous and
 * HIP-graph capturable.  Outputs are fully overwritten for valid requests.
 *
 * Threads: calls are re-entrant; concurrent calls must not share output or
 * workspace buffers.
 */
#ifndef KDTREE_VERIFY_H
#define KDTREE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest q_len (draft budget 64 + root) accepted: "The Capstone Commit ...",
 * section "The Message Itself" (the bridge reports MAX_QLEN=65) and "Strategic
 * Pivots ...", section "Why This Message Was Written" (max budget 64, q_len 65). */
#define KDTREE_MAX_QLEN 65

#define KDTREE_DTYPE_FP32 0
#define KDTREE_DTYPE_BF16 1

/* Return codes (nothing is enqueued unless the result is KDTREE_OK). */
#define KDTREE_OK 0
#define KDTREE_ERR_NULL (-1)        /* a required pointer is NULL */
#define KDTREE_ERR_SHAPE (-2)       /* batch < 1, num_heads < 1, total_q < batch,
                                       total_kv < total_q, or a size overflows */
#define KDTREE_ERR_QLEN (-3)        /* max_q_len outside [1, KDTREE_MAX_QLEN] */
#define KDTREE_ERR_DTYPE (-4)       /* dtype not FP32 / BF16 */
#define KDTREE_ERR_SPLITS (-5)      /* num_splits < 1 or > 256, split_ratio outside (0, 1],
                                       or workspace NULL / smaller than
                                       kdtree_verify_attn_workspace_bytes */
#define KDTREE_ERR_SCALE (-6)       /* scale not finite */
#define KDTREE_ERR_LAUNCH (-7)      /* HIP launch failure */
#define KDTREE_ERR_SCRATCH (-8)     /* kdtree_verify_attn_noalloc: the call needs more
                                       scratch than KDTREE_NOALLOC_SCRATCH_BYTES */

/* Device status bits OR-ed into *status (if non-NULL) by the kernels. */
#define KDTREE_STATUS_BAD_QLEN 1u     /* some q_len[b] outside [1, max_q_len] */
#define KDTREE_STATUS_BAD_PREFIX 2u   /* some prefix_len[b] < 0 */
#define KDTREE_STATUS_BAD_PARENT 4u   /* parent[0] != -1 or parent[i] outside [0, i) */
#define KDTREE_STATUS_OVERFLOW 8u     /* packed offsets exceed total_q / total_kv, or a
                                         request has prefix_len + q_len > 2^24 */
#define KDTREE_STATUS_NONFINITE 16u   /* a non-finite output row was produced (with the
                                         bf16 last-round cut, such a row of a cut row
                                         tile may be left unwritten instead) */
#define KDTREE_STATUS_RANGE 32u       /* bf16 inputs: a q_lat or kv_lat value is not
                                         finite or has |x| >= 65504, outside the fp16
                                         range of the latent contractions.  The call
                                         still completes; the rows of the affected
                                         request (every row that sees such a key, or
                                         whose query holds such a value) are then
                                         meaningless, typically inf or NaN. */

/* MAX_QLEN (65). */
int32_t kdtree_max_qlen(void);

/* Workspace bytes kdtree_verify_attn needs (0 = none).  Returns 0 for invalid sizes.
 * Regions (each rounded up to 256 bytes):
 *   bf16 inputs: the request schedule (one 64-byte record per request: its index in
 *     longest-first order, packed offsets and status) and fp16 copies of the latent
 *     rows, key-major in 32-key tiles, both written by a pre-pass of the same call:
 *     batch * 64 and (total_kv / 32 + batch + 1) * 32 KB bytes;
 *   one region of the larger of
 *     num_splits > 1: split partial outputs num_splits * total_q * num_heads * 512 * 4
 *       bytes, then their log-sum-exps num_splits * total_q * num_heads * 4 bytes;
 *     bf16 inputs: 256 * 128 * (512 + 1) * 4 + 256 * 16 bytes, used with num_splits
 *       == 1 by the last-round cut (when each of the 8 XCDs' queues holds at most two
 *       whole rounds of 32 workgroups, the row tiles left over after them run as key
 *       pieces over all of the XCD's CUs, and a merge pass combines the pieces; same
 *       result up to rounding).
 * The size never decreases with num_splits, so a workspace sized for some split count
 * also serves every smaller one. */
size_t kdtree_verify_attn_workspace_bytes(int64_t total_q, int64_t total_kv, int32_t batch,
                                          int32_t num_heads, int32_t num_splits, int32_t dtype);

/*
 * Tree-verify MLA-absorb attention (see the top of this file).
 *
 *   q_lat, q_rope, kv_lat, k_rope   device inputs, dtype `dtype` (fp32 / bf16).
 *       bf16 contract: values must be finite with |x| < 65504 in q_lat and kv_lat
 *       (the latent contractions run as fp16 MFMAs with fp32 accumulation; bf16 ->
 *       fp16 is exact for 2^-17 <= |x| < 65504, smaller magnitudes round with an
 *       absolute error <= 2^-25).  A value outside it sets KDTREE_STATUS_RANGE.
 *   prefix_len, tree_parent, q_len  device int32 arrays (layout above).
 *   scale        softmax scale applied to q . k (finite; e.g. 1/sqrt(192)).
 *   out_lat      device fp32 [total_q, H, 512];  out_lse device fp32 [total_q, H].
 *   stream       hipStream_t to enqueue on (NULL = the default stream).
 *   batch        number of requests (>= 1).
 *   num_heads    H (>= 1).
 *   max_q_len    upper bound of every q_len[b], in [1, 65]; sizes the launch.
 *   total_q      rows of q_lat / q_rope / tree_parent / outputs the caller allocated
 *                (>= sum q_len).   total_kv: rows of kv_lat / k_rope (>= sum of
 *                prefix_len + q_len).  The kernels never access rows beyond these;
 *                a request whose packed offsets exceed them is skipped and flagged.
 *   dtype        KDTREE_DTYPE_FP32 or KDTREE_DTYPE_BF16 (all four inputs).
 *   num_splits   split-KV factor (1..256).  With S > 1 each request's prefix is cut
 *                into S chunks of whole 32-key tiles (the tail goes with the last
 *                chunk; chunks may be empty); each chunk's partial output + lse is
 *                written to `workspace` and a merge pass combines them ("The Milestone
 *                Commit ...", section "What to defer": flash partial outputs merged for
 *                long prefixes).
 *   split_ratio  chunk sizes, in (0, 1].  1: S equal chunks of ceil(P/S) keys rounded
 *                up to a multiple of 32.  r < 1: geometric chunks, chunk s holding about
 *                r^s (1 - r) / (1 - r^S) of the prefix (boundaries rounded up to whole
 *                tiles), and the work is handed out largest chunks first, so that a
 *                launch whose workgroups overrun a whole number of rounds over the CUs
 *                ends on small pieces.  The result is the same up to rounding; with
 *                S = 1 the ratio has no effect.
 *   workspace    device buffer of at least kdtree_verify_attn_workspace_bytes(...)
 *                bytes (may be NULL when that is 0: fp32 inputs with num_splits == 1).
 *                Its contents are scratch; calls sharing a workspace must not overlap.
 *   status       optional device int32; the kernels OR KDTREE_STATUS_* bits into it
 *                on malformed device inputs (the caller zeroes it).  Rows of a
 *                flagged request are left unwritten.
 *
 * Returns KDTREE_OK after enqueueing, or a negative KDTREE_ERR_* code with nothing
 * enqueued.
 */
int32_t kdtree_verify_attn(const void* q_lat, const void* q_rope, const void* kv_lat,
                           const void* k_rope, const int32_t* prefix_len,
                           const int32_t* tree_parent, const int32_t* q_len, float scale,
                           float* out_lat, float* out_lse, void* stream, int32_t batch,
                           int32_t num_heads, int32_t max_q_len, int64_t total_q,
                           int64_t total_kv, int32_t dtype, int32_t num_splits,
                           float split_ratio, void* workspace, size_t workspace_bytes,
                           int32_t* status);

/*
 * The same call in two phases, for callers that time or schedule them apart.  Both
 * take exactly the arguments of kdtree_verify_attn and validate them the same way.
 *
 *   kdtree_verify_attn_prepare   enqueues the bf16 pre-pass: it writes the request
 *       schedule and the fp16 key-major copies of kv_lat into `workspace`
 *       (nothing for fp32 inputs, where it only validates).  It reads kv_lat,
 *       prefix_len and q_len only; the other pointers must still be valid values.
 *   kdtree_verify_attn_attend    enqueues the attention (and, with num_splits > 1,
 *       the merge), reading the workspace that a prepare call with the same
 *       kv_lat, prefix_len, q_len, batch, max_q_len, total_q, total_kv and dtype
 *       filled.  Until
 *       any of those inputs change, one prepare may serve several attend calls.
 *
 * kdtree_verify_attn(args) == kdtree_verify_attn_prepare(args) followed by
 * kdtree_verify_attn_attend(args) on the same stream.  Returns as kdtree_verify_attn.
 */
int32_t kdtree_verify_attn_prepare(const void* q_lat, const void* q_rope, const void* kv_lat,
                                   const void* k_rope, const int32_t* prefix_len,
                                   const int32_t* tree_parent, const int32_t* q_len,
                                   float scale, float* out_lat, float* out_lse, void* stream,
                                   int32_t batch, int32_t num_heads, int32_t max_q_len,
                                   int64_t total_q, int64_t total_kv, int32_t dtype,
                                   int32_t num_splits, float split_ratio, void* workspace,
                                   size_t workspace_bytes, int32_t* status);

int32_t kdtree_verify_attn_attend(const void* q_lat, const void* q_rope, const void* kv_lat,
                                  const void* k_rope, const int32_t* prefix_len,
                                  const int32_t* tree_parent, const int32_t* q_len,
                                  float scale, float* out_lat, float* out_lse, void* stream,
                                  int32_t batch, int32_t num_heads, int32_t max_q_len,
                                  int64_t total_q, int64_t total_kv, int32_t dtype,
                                  int32_t num_splits, float split_ratio, void* workspace,
                                  size_t workspace_bytes, int32_t* status);

/*
 * kdtree_verify_attn for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments
 * and result as kdtree_verify_attn, without the workspace: the scratch it needs (the
 * amount kdtree_verify_attn_workspace_bytes reports) comes from one static device array
 * of KDTREE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until
 * the process ends.  The call never calls hipMalloc, hipFree or any other allocating
 * routine; on its first call on a device it looks up that device's array address.
 *
 *   Limit: calls whose workspace need exceeds KDTREE_NOALLOC_SCRATCH_BYTES (128 MiB)
 *   return KDTREE_ERR_SCRATCH with nothing enqueued (for example the batch-8 workload
 *   with 4096-key prefixes needs about 101 MB and fits; batch 64 with prefixes up to
 *   8192 keys needs about 390 MB and does not).
 *   Sharing: every call on one GPU uses that GPU's one array, and a call leaves its
 *   contents behind; calls whose work overlaps on one GPU (other streams, other host
 *   threads) race on it and must be serialised by the caller.  Nothing in the array has
 *   to start at zero: each call writes every scratch value it later reads.
 */
#define KDTREE_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int32_t kdtree_verify_attn_noalloc(const void* q_lat, const void* q_rope, const void* kv_lat,
                                   const void* k_rope, const int32_t* prefix_len,
                                   const int32_t* tree_parent, const int32_t* q_len,
                                   float scale, float* out_lat, float* out_lse, void* stream,
                                   int32_t batch, int32_t num_heads, int32_t max_q_len,
                                   int64_t total_q, int64_t total_kv, int32_t dtype,
                                   int32_t num_splits, float split_ratio, int32_t* status);

/* ------------------------------------------------------------------------------------
 * The steps on either side of verify attention in one greedy DDTree step.
 * ------------------------------------------------------------------------------------ */

/* Limits of kdtree_build_ddtree. */
#define KDTREE_MAX_BUDGET 64     /* drafted nodes per tree: q_len <= 65 */
#define KDTREE_MAX_DEPTH 64      /* draft positions per request */
#define KDTREE_MAX_TABLE 4096    /* depth * top_k of one request's candidate table */
#define KDTREE_MAX_ACCEPT_NODES 4096  /* max_nodes of kdtree_tree_accept */

/*
 * Best-first draft-tree builder on the device, one wavefront per request ("The Milestone
 * Commit: Cementing Phase 1 ...", section "The Context", item 1: the builder runs on the
 * GPU in place of a per-request host heap; "Strategic Pivots in CUDA Kernel Engineering
 * ...", sections "The Message" and "Why This Message Was Written": trees from the
 * drafter's top-k log-probabilities and token ids, budgets up to 64, exact agreement with
 * the host heap including its tie-breaks and float32 accumulation).
 *
 *   logp        device fp32 [batch, depth, top_k]: for draft position d (0-based row) the
 *               drafter's top_k log-probabilities, sorted descending; -inf marks an absent
 *               candidate (rows shorter than top_k).  No NaN.
 *   token_ids   device int32 [batch, depth, top_k]: the token of each candidate.
 *   root_token  device int32 [batch]: token of node 0 (the last verified token).
 *   batch >= 1; 1 <= depth <= 64; 1 <= top_k <= 4095; depth * top_k <= 4096;
 *   0 <= budget <= 64 (drafted nodes besides the root).
 *
 * The tree: node 0 is the root with score 0.  A node at depth d >= 1 taking rank r
 * carries token_ids[b][d-1][r] and the score parent + logp[b][d-1][r], added in float32.
 * Nodes are popped from a frontier by highest score, ties to the earliest pushed; popping
 * (d, r) under parent p pushes (d, r+1) under p and (d+1, 0) under the new node; node
 * index = pop order.  The tree stops at budget drafted nodes or an empty frontier, so
 * q_len[b] = drafted nodes + 1 <= budget + 1, and parent[i] < i (the layout
 * kdtree_verify_attn takes, once packed).
 *
 * Outputs, device int32 [batch, budget + 1] (row b of request b; entries at and past
 * q_len[b] are -1):
 *   tree_parent   parent node (-1 for the root);
 *   tree_token    token (root: root_token[b]);
 *   tree_depth    depth (root: 0);
 *   first_child   lowest-index child, or -1;
 *   next_sibling  next-higher-index node with the same parent, or -1;
 *   tree_score    optional (NULL = not written) fp32 [batch, budget + 1]: the node
 *                 scores, -inf past q_len[b].
 *   q_len         device int32 [batch].
 * Ownership and stream rules as for kdtree_verify_attn; no workspace.  Returns
 * KDTREE_OK after enqueueing, KDTREE_ERR_NULL for a missing required pointer,
 * KDTREE_ERR_SHAPE for sizes outside the limits, KDTREE_ERR_LAUNCH on a launch failure.
 */
int32_t kdtree_build_ddtree(const float* logp, const int32_t* token_ids,
                            const int32_t* root_token, int32_t batch, int32_t depth,
                            int32_t top_k, int32_t budget, int32_t* q_len, int32_t* tree_parent,
                            int32_t* tree_token, int32_t* tree_depth, int32_t* first_child,
                            int32_t* next_sibling, float* tree_score, void* stream);

/*
 * Pack the builder's padded rows into the packed node-order layout kdtree_verify_attn
 * reads, on the device (the verify step consumes the builder's output without a host
 * round trip: "The Capstone Commit ...", section "The Message Itself", the on-device
 * build -> accept composition and the bridge that takes the builder's device output).
 *
 *   q_len        device int32 [batch]: nodes per tree (clamped to [0, width]).
 *   tree_parent  device int32 [batch, width]; tree_token the same or NULL.
 *   total_q      rows of the packed outputs (>= sum of q_len; a request that would end
 *                past total_q is not written).
 *   packed_parent device int32 [total_q]: request b's nodes at rows
 *                [q_offsets[b], q_offsets[b] + q_len[b]) (local indices, as given).
 *   packed_token device int32 [total_q] or NULL (then tree_token may be NULL).
 *   q_offsets    device int64 [batch + 1] or NULL: exclusive prefix sums of the clamped
 *                q_len, q_offsets[batch] = their total.
 * Returns KDTREE_OK, KDTREE_ERR_NULL, KDTREE_ERR_SHAPE (batch < 1, width outside
 * [1, 2^20], total_q < 1) or KDTREE_ERR_LAUNCH.
 */
int32_t kdtree_pack_tree(const int32_t* q_len, const int32_t* tree_parent,
                         const int32_t* tree_token, int32_t batch, int32_t width, int64_t total_q,
                         int32_t* packed_parent, int32_t* packed_token, int64_t* q_offsets,
                         void* stream);

/*
 * Greedy follow-verified-tree accept ("The Milestone Commit ...", section "The Context",
 * item 3: a walk over the verified tree's next-token and next-sibling pointers, one
 * thread per request there; here one wavefront per request stages the tree in LDS and
 * resolves every node's matching child in parallel before the walk).
 *
 *   tree_token, first_child, next_sibling   device int32 [batch, max_nodes], as written
 *               by kdtree_build_ddtree (max_nodes = budget + 1).
 *   q_len       device int32 [batch]: nodes of each tree (clamped to [1, max_nodes]).
 *   target_next device int32 [batch, max_nodes]: the target model's greedy next token
 *               after node i (the argmax of its logits at query row i).
 *   max_accept  columns of the outputs (>= 1); at most max_accept - 1 draft nodes are
 *               accepted, so that the bonus token always fits.
 *
 * From the root, the walk moves to the first child (in sibling order) whose token equals
 * target_next at the current node, and stops at the first node with no such child,
 * emitting target_next there as the bonus token.  Pointers that leave [1, q_len) or do
 * not increase the node index end the walk as "no such child".
 *
 * Outputs:
 *   accept_len     device int32 [batch]: accepted draft nodes + 1 (the bonus token).
 *   accept_tokens  device int32 [batch, max_accept]: the accepted tokens, then the bonus
 *                  token, then -1.
 *   accept_nodes   device int32 [batch, max_accept]: node index of each accepted token,
 *                  -1 for the bonus token and the padding.
 * Returns as kdtree_build_ddtree (KDTREE_ERR_SHAPE: batch < 1, max_nodes outside
 * [1, KDTREE_MAX_ACCEPT_NODES] or max_accept outside [1, 2^20]).
 */
int32_t kdtree_tree_accept(const int32_t* tree_token, const int32_t* first_child,
                           const int32_t* next_sibling, const int32_t* q_len,
                           const int32_t* target_next, int32_t batch, int32_t max_nodes,
                           int32_t max_accept, int32_t* accept_len, int32_t* accept_tokens,
                           int32_t* accept_nodes, void* stream);

/*
 * The target model's next token at every tree node, drawn at temperature T: the input of
 * kdtree_tree_accept on the temperature path of the accept step ("The Milestone Commit
 * ...", sections "Why This Message Was Written" and "How Decisions Were Made" name that
 * sampling path without giving it).  The tree's candidates are the drafter's top-k,
 * chosen rather than sampled, so the lossless accept draws the target's token at a node
 * and follows the child that carries it: kdtree_tree_accept with these tokens as
 * target_next.  T = 0 gives the greedy (argmax) tokens.
 *
 *   logits      device [rows, row_stride] of dtype KDTREE_DTYPE_FP32 or _BF16: the
 *               target's logits at each node (entries [0, vocab) of a row are used).
 *   rows        1 .. 2^31 - 1;  vocab >= 1;  row_stride >= vocab (elements).
 *   temperature finite, >= 0.
 *   seed, offset the generator key; draws of one (seed, offset) are reproducible, and
 *               a caller advances offset per decoding step.
 *   tokens      device int32 [rows]: the drawn token, or -1 if every logit is -inf.
 *
 * Draw of row r, T > 0: entry i takes u_i in (0, 1) from Philox4x64-10 (Salmon et al.,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) with counter (i / 8, r, 0, 0)
 * and key (seed, offset): word (i / 2) % 4 of the block, low 32 bits for even i and high
 * for odd i, x32 -> (2 (x32 >> 9) + 1) 2^-24.  With each step rounded in float32,
 * z_i = logit_i * (log2(e) / T) - log2(-log2(u_i)), and the token is the argmax of z,
 * lowest index on ties.  z is log2(e) times the Gumbel-max key logit / T - ln(-ln u)
 * less a constant, so the token follows softmax(logit / T).  The logarithms are within
 * about an ulp of the correctly rounded ones (the inner one relative to its value, as
 * u near 1 decides the argmax).  T = 0: the argmax of the logits.  NaN logits are not
 * allowed.
 *
 * Returns KDTREE_OK, KDTREE_ERR_NULL, KDTREE_ERR_SHAPE, KDTREE_ERR_DTYPE,
 * KDTREE_ERR_SCALE (temperature negative or not finite) or KDTREE_ERR_LAUNCH.
 */
int32_t kdtree_sample_tokens(const void* logits, int32_t dtype, int64_t rows, int32_t vocab,
                             int64_t row_stride, float temperature, uint64_t seed,
                             uint64_t offset, int32_t* tokens, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDTREE_VERIFY_H */
