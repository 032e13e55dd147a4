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
#define KDTREE_ERR_SPLITS (-5)      /* num_splits < 1 or > 256, or workspace NULL /
                                       smaller than kdtree_verify_attn_workspace_bytes */
#define KDTREE_ERR_SCALE (-6)       /* scale not finite */
#define KDTREE_ERR_LAUNCH (-7)      /* HIP launch failure */

/* Device status bits OR-ed into *status (if non-NULL) by the kernels. */
#define KDTREE_STATUS_BAD_QLEN 1u     /* some q_len[b] outside [1, max_q_len] */
#define KDTREE_STATUS_BAD_PREFIX 2u   /* some prefix_len[b] < 0 */
#define KDTREE_STATUS_BAD_PARENT 4u   /* parent[0] != -1 or parent[i] outside [0, i) */
#define KDTREE_STATUS_OVERFLOW 8u     /* packed offsets exceed total_q / total_kv, or a
                                         request has prefix_len + q_len > 2^24 */
#define KDTREE_STATUS_NONFINITE 16u   /* a non-finite output row was produced */

/* MAX_QLEN (65). */
int32_t kdtree_max_qlen(void);

/* Workspace bytes kdtree_verify_attn needs (0 = none).  Returns 0 for invalid sizes.
 * Regions (each rounded up to 256 bytes):
 *   bf16 inputs: the request schedule (batch int32) and fp16 copies of the latent rows,
 *     key-major in 32-key tiles, both written by a pre-pass of the same call:
 *     batch * 4 and (total_kv / 32 + batch + 1) * 32 KB bytes;
 *   num_splits > 1: split partial outputs num_splits * total_q * num_heads * 512 * 4
 *     bytes and their log-sum-exps num_splits * total_q * num_heads * 4 bytes. */
size_t kdtree_verify_attn_workspace_bytes(int64_t total_q, int64_t total_kv, int32_t batch,
                                          int32_t num_heads, int32_t num_splits, int32_t dtype);

/*
 * Tree-verify MLA-absorb attention (see the top of this file).
 *
 *   q_lat, q_rope, kv_lat, k_rope   device inputs, dtype `dtype` (fp32 / bf16).
 *       bf16 contract: values must be finite with |x| < 65504 in q_lat and kv_lat
 *       (the latent contractions run as fp16 MFMAs with fp32 accumulation; bf16 ->
 *       fp16 is exact for 2^-17 <= |x| < 65504, smaller magnitudes round with an
 *       absolute error <= 2^-25).
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
 *                into S chunks of ceil(P/S) keys rounded up to a multiple of 32 (the
 *                tail goes with the last chunk; trailing chunks may be empty);
 *                each chunk's partial output + lse is written to `workspace` and a
 *                merge pass combines them ("The Milestone Commit ...", section "What
 *                to defer": flash partial outputs merged for long prefixes).
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
                           void* workspace, size_t workspace_bytes, int32_t* status);

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
 *       kv_lat, prefix_len, q_len, batch, max_q_len, total_kv and dtype filled.  Until
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
                                   int32_t num_splits, void* workspace, size_t workspace_bytes,
                                   int32_t* status);

int32_t kdtree_verify_attn_attend(const void* q_lat, const void* q_rope, const void* kv_lat,
                                  const void* k_rope, const int32_t* prefix_len,
                                  const int32_t* tree_parent, const int32_t* q_len,
                                  float scale, float* out_lat, float* out_lse, void* stream,
                                  int32_t batch, int32_t num_heads, int32_t max_q_len,
                                  int64_t total_q, int64_t total_kv, int32_t dtype,
                                  int32_t num_splits, void* workspace, size_t workspace_bytes,
                                  int32_t* status);

#ifdef __cplusplus
}
#endif

#endif /* KDTREE_VERIFY_H */
