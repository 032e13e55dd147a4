// C ABI of the tree-verify MLA-absorb attention library (declarations and contract in
// include/kdtree_verify.h).  Host code only: validates host arguments, sizes the
// launches from host scalars (device arrays are never read on the host) and enqueues
// the kernels on the caller's stream.
#include <math.h>

#include "../../include/kdtree_verify.h"
#include "common.h"

namespace {

constexpr int32_t kMaxSplits = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bytes of the per-split partial outputs and log-sum-exps; 0 when not needed.
bool workspace_layout(int64_t total_q, int32_t num_heads, int32_t num_splits, size_t* o_bytes,
                      size_t* total) {
  if (total_q < 1 || num_heads < 1 || num_splits < 1 || num_splits > kMaxSplits) return false;
  if (num_splits == 1) {
    *o_bytes = 0;
    *total = 0;
    return true;
  }
  const double est = (double)num_splits * (double)total_q * num_heads * (kdt::DL + 1) * 4.0;
  if (est > 9.0e18) return false;
  const size_t rows = (size_t)total_q * (size_t)num_heads;
  *o_bytes = round_up((size_t)num_splits * rows * kdt::DL * sizeof(float), 256);
  *total = round_up(*o_bytes + (size_t)num_splits * rows * sizeof(float), 256);
  return true;
}

}  // namespace

extern "C" {

int32_t kdtree_max_qlen(void) { return KDTREE_MAX_QLEN; }

size_t kdtree_verify_attn_workspace_bytes(int64_t total_q, int32_t num_heads, int32_t num_splits) {
  size_t o_bytes = 0, total = 0;
  if (!workspace_layout(total_q, num_heads, num_splits, &o_bytes, &total)) return 0;
  return total;
}

int32_t kdtree_verify_attn(const void* q_lat, const void* q_rope, const void* kv_lat,
                           const void* k_rope, const int32_t* prefix_len,
                           const int32_t* tree_parent, const int32_t* q_len, float scale,
                           float* out_lat, float* out_lse, void* stream, int32_t batch,
                           int32_t num_heads, int32_t max_q_len, int64_t total_q,
                           int64_t total_kv, int32_t dtype, int32_t num_splits,
                           void* workspace, size_t workspace_bytes, int32_t* status) {
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
  size_t o_bytes = 0, need = 0;
  if (!workspace_layout(total_q, num_heads, num_splits, &o_bytes, &need)) return KDTREE_ERR_SPLITS;
  if (num_splits > 1 && (!workspace || workspace_bytes < need)) return KDTREE_ERR_SPLITS;

  kdt::VerifyParams p;
  p.q_lat = q_lat;
  p.q_rope = q_rope;
  p.kv_lat = kv_lat;
  p.k_rope = k_rope;
  p.prefix_len = prefix_len;
  p.tree_parent = tree_parent;
  p.q_len = q_len;
  p.out_lat = out_lat;
  p.out_lse = out_lse;
  p.part_o = num_splits > 1 ? (float*)workspace : nullptr;
  p.part_lse = num_splits > 1 ? (float*)((char*)workspace + o_bytes) : nullptr;
  p.status = status;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  p.batch = batch;
  p.num_heads = num_heads;
  p.max_q_len = max_q_len;
  p.num_splits = num_splits;
  p.total_q = total_q;
  p.total_kv = total_kv;
  const int bm = dtype == KDTREE_DTYPE_BF16 ? kdt::rows_per_block_bf16() : kdt::rows_per_block_f32();
  p.m_tiles = (max_q_len * num_heads + bm - 1) / bm;
  if ((int64_t)p.m_tiles * num_splits * batch > 0x7fffffff) return KDTREE_ERR_SHAPE;

  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == KDTREE_DTYPE_BF16 ? kdt::launch_verify_bf16(p, s) : kdt::launch_verify_f32(p, s);
  if (e != hipSuccess) return KDTREE_ERR_LAUNCH;
  if (num_splits > 1) {
    e = kdt::launch_lse_merge(p.part_o, p.part_lse, out_lat, out_lse, total_q * num_heads,
                              num_splits, s);
    if (e != hipSuccess) return KDTREE_ERR_LAUNCH;
  }
  return KDTREE_OK;
}

}  // extern "C"
