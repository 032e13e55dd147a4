// C ABI of the tree-verify MLA-absorb attention library (declarations and contract in
// include/kdtree_verify.h).  Host code only: validates host arguments, sizes the
// launches from host scalars (device arrays are never read on the host) and enqueues
// the kernels on the caller's stream.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include "../../include/kdtree_verify.h"

#include "common.h"

namespace kdt {
// The allocation-free entry point's scratch: one static device array per GPU the library
// runs on, held until the process ends.  Its name is only a host-side stand-in for the
// symbol: host code takes the array's address on each device through hipGetSymbolAddress
// (with that device current) and passes that pointer to the kernels, never the name.
__device__ __align__(256) unsigned char scratch[KDTREE_NOALLOC_SCRATCH_BYTES];
}  // namespace kdt

namespace {

constexpr int32_t kMaxSplits = kdt::MAX_SPLITS;
constexpr int kCutMaxRounds = 2;  // cut only when every XCD's queue has at most 2 whole rounds

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// KDTREE_DISABLE_CUT=1 in the environment switches the last-round cut off (a switch for
// testing and timing the uncut launch; results agree up to rounding either way).
bool cut_disabled() {
  const char* v = getenv("KDTREE_DISABLE_CUT");
  return v && v[0] && v[0] != '0';
}

struct WorkspaceLayout {
  size_t req_bytes, k16_bytes, part_o_bytes, part_lse_bytes, piece_bytes, total;
  int64_t k16_tiles;
};

// Workspace: [request records + fp16 latent tiles (bf16 inputs)] [split partial outputs +
// split lse, or (bf16, one split) the last-round cut pieces], each region 256-byte
// aligned.  Latent tiles: one 32 KB tile per 32 keys
// of every request, bounded by total_kv / 32 + batch (each request adds at most one
// partial tile).
bool workspace_layout(int64_t total_q, int64_t total_kv, int32_t batch, int32_t num_heads,
                      int32_t num_splits, int32_t dtype, WorkspaceLayout* w) {
  if (total_q < 1 || total_kv < 1 || batch < 1 || num_heads < 1 || num_splits < 1 ||
      num_splits > kMaxSplits || (dtype != KDTREE_DTYPE_FP32 && dtype != KDTREE_DTYPE_BF16))
    return false;
  if (total_q > ((int64_t)1 << 40) || total_kv > ((int64_t)1 << 40)) return false;
  w->k16_tiles = dtype == KDTREE_DTYPE_BF16 ? total_kv / kdt::TILE_KEYS + batch + 1 : 0;
  w->req_bytes = dtype == KDTREE_DTYPE_BF16 ? round_up((size_t)batch * sizeof(kdt::ReqRec), 256) : 0;
  w->k16_bytes = round_up((size_t)w->k16_tiles * (size_t)kdt::TILE_BYTES, 256);
  const size_t rows = (size_t)total_q * (size_t)num_heads;
  w->part_o_bytes = num_splits > 1 ? round_up((size_t)num_splits * rows * kdt::DL * sizeof(float), 256) : 0;
  w->part_lse_bytes = num_splits > 1 ? round_up((size_t)num_splits * rows * sizeof(float), 256) : 0;
  // Last-round cut pieces (bf16, one split): outputs, lse, and two int64 per unit.  They
  // share one region with the split partials (a launch uses one or the other), sized for
  // the larger, so a workspace sized for more splits also serves fewer.
  const size_t slots = (size_t)kdt::cut_piece_slots(batch);
  w->piece_bytes = dtype == KDTREE_DTYPE_BF16
                       ? slots * kdt::PIECE_ROWS * (kdt::DL + 1) * sizeof(float) +
                             slots * 2 * sizeof(int64_t)
                       : 0;
  const size_t shared = std::max(w->part_o_bytes + w->part_lse_bytes, w->piece_bytes);
  w->total = w->req_bytes + w->k16_bytes + shared;
  return true;
}

// Host validation shared by the entry points; fills the launch parameters.
int32_t setup(const void* q_lat, const void* q_rope, const void* kv_lat, const void* k_rope,
              const int32_t* prefix_len, const int32_t* tree_parent, const int32_t* q_len,
              float scale, float* out_lat, float* out_lse, int32_t batch, int32_t num_heads,
              int32_t max_q_len, int64_t total_q, int64_t total_kv, int32_t dtype,
              int32_t num_splits, float split_ratio, void* workspace, size_t workspace_bytes,
              int32_t* status, kdt::VerifyParams* pp, WorkspaceLayout* wp) {
  if (!q_lat || !q_rope || !kv_lat || !k_rope || !prefix_len || !tree_parent || !q_len ||
      !out_lat || !out_lse)
    return KDTREE_ERR_NULL;
  if (batch < 1 || num_heads < 1 || total_q < batch || total_kv < total_q)
    return KDTREE_ERR_SHAPE;
  if (max_q_len < 1 || max_q_len > KDTREE_MAX_QLEN) return KDTREE_ERR_QLEN;
  if ((int64_t)max_q_len * num_heads > (1 << 24) || total_q > ((int64_t)1 << 40) ||
      total_kv > ((int64_t)1 << 40))
    return KDTREE_ERR_SHAPE;
  if (dtype != KDTREE_DTYPE_FP32 && dtype != KDTREE_DTYPE_BF16) return KDTREE_ERR_DTYPE;
  if (!isfinite(scale)) return KDTREE_ERR_SCALE;
  if (!(split_ratio > 0.0f && split_ratio <= 1.0f)) return KDTREE_ERR_SPLITS;
  WorkspaceLayout& w = *wp;
  if (!workspace_layout(total_q, total_kv, batch, num_heads, num_splits, dtype, &w))
    return KDTREE_ERR_SPLITS;
  if (w.total > 0 && (!workspace || workspace_bytes < w.total)) return KDTREE_ERR_SPLITS;

  kdt::VerifyParams& p = *pp;
  p.q_lat = q_lat;
  p.q_rope = q_rope;
  p.kv_lat = kv_lat;
  p.k_rope = k_rope;
  p.prefix_len = prefix_len;
  p.tree_parent = tree_parent;
  p.q_len = q_len;
  p.out_lat = out_lat;
  p.out_lse = out_lse;
  char* ws = (char*)workspace;
  p.req = w.req_bytes ? (kdt::ReqRec*)ws : nullptr;
  p.k16 = w.k16_bytes ? ws + w.req_bytes : nullptr;
  p.k16_tiles = w.k16_tiles;
  p.part_o = num_splits > 1 ? (float*)(ws + w.req_bytes + w.k16_bytes) : nullptr;
  p.part_lse =
      num_splits > 1 ? (float*)(ws + w.req_bytes + w.k16_bytes + w.part_o_bytes) : nullptr;
  char* pw = ws + w.req_bytes + w.k16_bytes;  // the region shared with the partials
  const bool pieces = w.piece_bytes && num_splits == 1;
  const size_t slots = (size_t)kdt::cut_piece_slots(batch);
  p.piece_slots = pieces ? (int32_t)slots : 0;
  p.piece_o = pieces ? (float*)pw : nullptr;
  p.piece_lse = pieces ? (float*)pw + slots * kdt::PIECE_ROWS * kdt::DL : nullptr;
  p.piece_desc =
      pieces ? (int64_t*)(pw + slots * kdt::PIECE_ROWS * (kdt::DL + 1) * sizeof(float)) : nullptr;
  p.status = status;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  p.split_ratio = split_ratio;
  p.batch = batch;
  p.num_heads = num_heads;
  p.max_q_len = max_q_len;
  p.num_splits = num_splits;
  p.total_q = total_q;
  p.total_kv = total_kv;
  const int bm = dtype == KDTREE_DTYPE_BF16 ? kdt::rows_per_block_bf16() : kdt::rows_per_block_f32();
  p.m_tiles = (max_q_len * num_heads + bm - 1) / bm;
  if ((int64_t)p.m_tiles * num_splits * batch > 0x7fffffff) return KDTREE_ERR_SHAPE;
  // Cut the last, partly filled round of each XCD's queue into key pieces when whole
  // rounds are few (there the leftover round is a large share of the launch); with more
  // rounds the longest-first order already fills it.
  p.cut = 0;
  if (pieces && !cut_disabled()) {
    for (int x = 0; x < kdt::NUM_XCD; ++x) {
      const kdt::XcdCut c = kdt::xcd_cut(batch, p.m_tiles, x);
      if (c.whole > kCutMaxRounds * kdt::CUS_PER_XCD) { p.cut = 0; break; }
      p.cut = std::max(p.cut, c.left);
    }
  }
  return KDTREE_OK;
}

int32_t launch_prepare(const kdt::VerifyParams& p, const WorkspaceLayout& w, int32_t dtype,
                       hipStream_t s) {
  if (dtype != KDTREE_DTYPE_BF16) return KDTREE_OK;
  return kdt::launch_prepass(p, w.k16_tiles, s) == hipSuccess ? KDTREE_OK : KDTREE_ERR_LAUNCH;
}

int32_t launch_attend(const kdt::VerifyParams& p, int32_t dtype, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (p.num_splits > 1) {
    // partial lse = NaN until an attention kernel writes it: the merge leaves rows that
    // no kernel wrote (skipped requests, rows past the packed total) unwritten
    e = kdt::launch_fill_nan(p.part_lse, (int64_t)p.num_splits * p.total_q * p.num_heads, s);
    if (e != hipSuccess) return KDTREE_ERR_LAUNCH;
  }
  if (p.cut) {
    // piece lse = NaN until a piece writes it: the piece merge leaves rows no piece wrote
    e = kdt::launch_fill_nan(p.piece_lse, (int64_t)p.piece_slots * kdt::PIECE_ROWS, s);
    if (e != hipSuccess) return KDTREE_ERR_LAUNCH;
  }
  e = dtype == KDTREE_DTYPE_BF16 ? kdt::launch_verify_bf16(p, s) : kdt::launch_verify_f32(p, s);
  if (e != hipSuccess) return KDTREE_ERR_LAUNCH;
  if (p.cut) {
    e = kdt::launch_piece_merge(p, s);
    if (e != hipSuccess) return KDTREE_ERR_LAUNCH;
  }
  if (p.num_splits > 1) {
    e = kdt::launch_lse_merge(p.part_o, p.part_lse, p.out_lat, p.out_lse,
                              p.total_q * p.num_heads, p.num_splits, s);
    if (e != hipSuccess) return KDTREE_ERR_LAUNCH;
  }
  return KDTREE_OK;
}

constexpr size_t kScratchBytes = (size_t)KDTREE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up once per device), or NULL on error.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(kdt::scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int32_t kdtree_max_qlen(void) { return KDTREE_MAX_QLEN; }

size_t kdtree_verify_attn_workspace_bytes(int64_t total_q, int64_t total_kv, int32_t batch,
                                          int32_t num_heads, int32_t num_splits, int32_t dtype) {
  WorkspaceLayout w;
  if (!workspace_layout(total_q, total_kv, batch, num_heads, num_splits, dtype, &w)) return 0;
  return w.total;
}

#define KDTREE_SETUP_ARGS                                                                  \
  q_lat, q_rope, kv_lat, k_rope, prefix_len, tree_parent, q_len, scale, out_lat, out_lse,  \
      batch, num_heads, max_q_len, total_q, total_kv, dtype, num_splits, split_ratio,      \
      workspace, workspace_bytes, status

int32_t kdtree_verify_attn(const void* q_lat, const void* q_rope, const void* kv_lat,
                           const void* k_rope, const int32_t* prefix_len,
                           const int32_t* tree_parent, const int32_t* q_len, float scale,
                           float* out_lat, float* out_lse, void* stream, int32_t batch,
                           int32_t num_heads, int32_t max_q_len, int64_t total_q,
                           int64_t total_kv, int32_t dtype, int32_t num_splits,
                           float split_ratio, void* workspace, size_t workspace_bytes,
                           int32_t* status) {
  kdt::VerifyParams p;
  WorkspaceLayout w;
  int32_t rc = setup(KDTREE_SETUP_ARGS, &p, &w);
  if (rc != KDTREE_OK) return rc;
  rc = launch_prepare(p, w, dtype, (hipStream_t)stream);
  if (rc != KDTREE_OK) return rc;
  return launch_attend(p, dtype, (hipStream_t)stream);
}

int32_t kdtree_verify_attn_prepare(const void* q_lat, const void* q_rope, const void* kv_lat,
                                   const void* k_rope, const int32_t* prefix_len,
                                   const int32_t* tree_parent, const int32_t* q_len,
                                   float scale, float* out_lat, float* out_lse, void* stream,
                                   int32_t batch, int32_t num_heads, int32_t max_q_len,
                                   int64_t total_q, int64_t total_kv, int32_t dtype,
                                   int32_t num_splits, float split_ratio, void* workspace,
                                   size_t workspace_bytes, int32_t* status) {
  kdt::VerifyParams p;
  WorkspaceLayout w;
  int32_t rc = setup(KDTREE_SETUP_ARGS, &p, &w);
  if (rc != KDTREE_OK) return rc;
  return launch_prepare(p, w, dtype, (hipStream_t)stream);
}

int32_t kdtree_verify_attn_attend(const void* q_lat, const void* q_rope, const void* kv_lat,
                                  const void* k_rope, const int32_t* prefix_len,
                                  const int32_t* tree_parent, const int32_t* q_len,
                                  float scale, float* out_lat, float* out_lse, void* stream,
                                  int32_t batch, int32_t num_heads, int32_t max_q_len,
                                  int64_t total_q, int64_t total_kv, int32_t dtype,
                                  int32_t num_splits, float split_ratio, void* workspace,
                                  size_t workspace_bytes, int32_t* status) {
  kdt::VerifyParams p;
  WorkspaceLayout w;
  int32_t rc = setup(KDTREE_SETUP_ARGS, &p, &w);
  if (rc != KDTREE_OK) return rc;
  return launch_attend(p, dtype, (hipStream_t)stream);
}

int32_t kdtree_verify_attn_noalloc(const void* q_lat, const void* q_rope, const void* kv_lat,
                                   const void* k_rope, const int32_t* prefix_len,
                                   const int32_t* tree_parent, const int32_t* q_len,
                                   float scale, float* out_lat, float* out_lse, void* stream,
                                   int32_t batch, int32_t num_heads, int32_t max_q_len,
                                   int64_t total_q, int64_t total_kv, int32_t dtype,
                                   int32_t num_splits, float split_ratio, int32_t* status) {
  // The workspace need is known from host scalars alone: reject what does not fit before
  // touching the device.
  WorkspaceLayout need;
  if (workspace_layout(total_q, total_kv, batch, num_heads, num_splits, dtype, &need) &&
      need.total > kScratchBytes)
    return KDTREE_ERR_SCRATCH;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  if (q_lat && q_rope && kv_lat && k_rope && prefix_len && tree_parent && q_len && out_lat &&
      out_lse && batch >= 1 && num_heads >= 1) {
    workspace = device_scratch();
    if (!workspace) return KDTREE_ERR_LAUNCH;
    workspace_bytes = kScratchBytes;
  }
  kdt::VerifyParams p;
  WorkspaceLayout w;
  int32_t rc = setup(KDTREE_SETUP_ARGS, &p, &w);
  if (rc != KDTREE_OK) return rc;
  rc = launch_prepare(p, w, dtype, (hipStream_t)stream);
  if (rc != KDTREE_OK) return rc;
  return launch_attend(p, dtype, (hipStream_t)stream);
}

int32_t kdtree_build_ddtree(const float* logp, const int32_t* token_ids,
                            const int32_t* root_token, int32_t batch, int32_t depth,
                            int32_t top_k, int32_t budget, int32_t* q_len, int32_t* tree_parent,
                            int32_t* tree_token, int32_t* tree_depth, int32_t* first_child,
                            int32_t* next_sibling, float* tree_score, void* stream) {
  if (!logp || !token_ids || !root_token || !q_len || !tree_parent || !tree_token ||
      !tree_depth || !first_child || !next_sibling)
    return KDTREE_ERR_NULL;
  if (batch < 1 || depth < 1 || depth > kdt::MAX_DDTREE_DEPTH || top_k < 1 || top_k > 4095 ||
      (int64_t)depth * top_k > kdt::MAX_DDTREE_TABLE || budget < 0 ||
      budget > kdt::MAX_DDTREE_BUDGET)
    return KDTREE_ERR_SHAPE;
  kdt::DdtreeBuildParams p{logp, token_ids, root_token, batch, depth, top_k, budget, q_len,
                           tree_parent, tree_token, tree_depth, first_child, next_sibling,
                           tree_score};
  return kdt::launch_build_ddtree(p, (hipStream_t)stream) == hipSuccess ? KDTREE_OK
                                                                         : KDTREE_ERR_LAUNCH;
}

int32_t kdtree_tree_accept(const int32_t* tree_token, const int32_t* first_child,
                           const int32_t* next_sibling, const int32_t* q_len,
                           const int32_t* target_next, int32_t batch, int32_t max_nodes,
                           int32_t max_accept, int32_t* accept_len, int32_t* accept_tokens,
                           int32_t* accept_nodes, void* stream) {
  if (!tree_token || !first_child || !next_sibling || !q_len || !target_next || !accept_len ||
      !accept_tokens || !accept_nodes)
    return KDTREE_ERR_NULL;
  if (batch < 1 || max_nodes < 1 || max_nodes > kdt::MAX_ACCEPT_NODES || max_accept < 1 ||
      max_accept > (1 << 20))
    return KDTREE_ERR_SHAPE;
  kdt::AcceptParams p{tree_token, first_child, next_sibling, q_len, target_next, batch,
                      max_nodes, max_accept, accept_len, accept_tokens, accept_nodes};
  return kdt::launch_tree_accept(p, (hipStream_t)stream) == hipSuccess ? KDTREE_OK
                                                                        : KDTREE_ERR_LAUNCH;
}

int32_t kdtree_pack_tree(const int32_t* q_len, const int32_t* tree_parent,
                         const int32_t* tree_token, int32_t batch, int32_t width, int64_t total_q,
                         int32_t* packed_parent, int32_t* packed_token, int64_t* q_offsets,
                         void* stream) {
  if (!q_len || !tree_parent || !packed_parent || (packed_token && !tree_token))
    return KDTREE_ERR_NULL;
  if (batch < 1 || width < 1 || width > (1 << 20) || total_q < 1) return KDTREE_ERR_SHAPE;
  kdt::PackParams p{q_len,   tree_parent,   tree_token,   batch,    width,
                    total_q, packed_parent, packed_token, q_offsets};
  return kdt::launch_pack_tree(p, (hipStream_t)stream) == hipSuccess ? KDTREE_OK
                                                                      : KDTREE_ERR_LAUNCH;
}

int32_t kdtree_sample_tokens(const void* logits, int32_t dtype, int64_t rows, int32_t vocab,
                             int64_t row_stride, float temperature, uint64_t seed,
                             uint64_t offset, int32_t* tokens, void* stream) {
  if (!logits || !tokens) return KDTREE_ERR_NULL;
  if (rows < 1 || rows > 0x7fffffff || vocab < 1 || row_stride < vocab ||
      row_stride > ((int64_t)1 << 40) / (rows > 0 ? rows : 1))
    return KDTREE_ERR_SHAPE;
  if (dtype != KDTREE_DTYPE_FP32 && dtype != KDTREE_DTYPE_BF16) return KDTREE_ERR_DTYPE;
  if (!(temperature >= 0.0f) || !(temperature < INFINITY)) return KDTREE_ERR_SCALE;
  kdt::SampleParams p{logits, rows, row_stride, vocab, temperature, seed, offset, tokens};
  return kdt::launch_sample_tokens(p, dtype == KDTREE_DTYPE_BF16, (hipStream_t)stream) ==
                 hipSuccess
             ? KDTREE_OK
             : KDTREE_ERR_LAUNCH;
}

}  // extern "C"
