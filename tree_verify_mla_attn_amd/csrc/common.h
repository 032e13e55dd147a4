// Shared definitions of the gfx950 tree-verify MLA-absorb attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kdt {

constexpr int DL = 512;          // latent dims (value vector and output)
constexpr int DR = 64;           // rope dims (scores only)
constexpr int DK = DL + DR;      // score contraction depth
constexpr int MAX_QLEN = 65;     // draft budget 64 + root
constexpr int MAX_REQUEST_KEYS = 1 << 24;  // prefix_len + q_len of one request
constexpr int TILE_KEYS = 32;              // keys per pre-converted fp16 latent tile
constexpr int64_t TILE_BYTES = DL * TILE_KEYS * 2;
constexpr int ORDER_MAX_BATCH = 4096;      // larger batches keep the request order as given
constexpr int NUM_XCD = 8;                 // MI355X: workgroup i runs on XCD i % 8
constexpr int CUS_PER_XCD = 32;
constexpr int PIECE_SLOTS = NUM_XCD * CUS_PER_XCD;  // cut pieces per launch, at most
constexpr int PIECE_ROWS = 128;                     // rows of one bf16 row tile
constexpr int MAX_SPLITS = 256;            // split-KV factor limit
constexpr float LN2 = 0.69314718055994530942f;

// Status bits (mirrors include/kdtree_verify.h).
constexpr int ST_BAD_QLEN = 1, ST_BAD_PREFIX = 2, ST_BAD_PARENT = 4, ST_OVERFLOW = 8,
              ST_NONFINITE = 16, ST_RANGE = 32;

// One request as the bf16 attention kernel needs it, written by the pre-pass at the
// request's rank (longest KV first): one record per workgroup prologue instead of a
// prefix sum over the earlier requests.  `flag` holds the status bits the kernel reports
// for the request: a malformed request and every request after it in index order (whose
// packed offsets are then unknown) are flagged, and 0 means the offsets are in range.
struct ReqRec {
  int32_t b;           // request index
  int32_t q_len, prefix_len;
  int32_t flag;
  int64_t qoff;        // sum of q_len over earlier requests
  int64_t kvoff;       // sum of prefix_len + q_len over earlier requests
  int64_t tbase;       // first fp16 latent tile of the request
  int64_t pad[3];
};
static_assert(sizeof(ReqRec) == 64, "one record per 64 bytes");

struct VerifyParams {
  const void* q_lat;
  const void* q_rope;
  const void* kv_lat;
  const void* k_rope;
  const int32_t* prefix_len;
  const int32_t* tree_parent;
  const int32_t* q_len;
  float* out_lat;    // [total_q, H, 512] (num_splits == 1)
  float* out_lse;    // [total_q, H]
  float* part_o;     // [num_splits, total_q*H, 512] (num_splits > 1)
  float* part_lse;   // [num_splits, total_q*H]
  int32_t* status;   // nullable
  void* k16;         // bf16 path: fp16 latent tiles (32 keys each) written by the pre-pass
  ReqRec* req;       // bf16 path: [batch] by rank, longest KV first (written by the pre-pass)
  float scale_log2;  // scale * log2(e)
  float split_ratio; // 1: equal splits; < 1: geometric splits, largest first
  int32_t batch, num_heads, max_q_len, num_splits, m_tiles;
  int64_t total_q, total_kv;
  int64_t k16_tiles; // capacity of `k16` in tiles
  // Last-round cut (bf16, one split): each XCD's units after its whole rounds of
  // CUS_PER_XCD run as key pieces, written here and merged by launch_piece_merge.
  int32_t cut;         // 0: off; else the most units any XCD's queue has cut (1..16)
  int32_t piece_slots; // piece slots of the area below: CUS_PER_XCD per XCD that has work
  float* piece_o;      // [piece_slots pieces, 128 rows, 512]
  float* piece_lse;    // [piece_slots pieces, 128 rows]
  int64_t* piece_desc; // [piece_slots units] x {first global row, rows}
};

// Draft-tree builder and accept.
constexpr int MAX_DDTREE_BUDGET = 64;     // drafted nodes per tree (q_len <= 65)
constexpr int MAX_DDTREE_DEPTH = 64;
constexpr int MAX_DDTREE_TABLE = 4096;    // depth * top_k entries of one request's table
constexpr int MAX_ACCEPT_NODES = 4096;    // nodes per tree the accept stages in LDS

struct DdtreeBuildParams {
  const float* logp;          // [batch, depth, top_k]
  const int32_t* token_ids;   // [batch, depth, top_k]
  const int32_t* root_token;  // [batch]
  int32_t batch, depth, top_k, budget;
  int32_t* q_len;             // [batch]
  int32_t* tree_parent;       // [batch, budget + 1] (all five)
  int32_t* tree_token;
  int32_t* tree_depth;
  int32_t* first_child;
  int32_t* next_sibling;
  float* tree_score;          // nullable
};

struct AcceptParams {
  const int32_t* tree_token;    // [batch, max_nodes] (also the two pointer arrays)
  const int32_t* first_child;
  const int32_t* next_sibling;
  const int32_t* q_len;         // [batch]
  const int32_t* target_next;   // [batch, max_nodes]
  int32_t batch, max_nodes, max_accept;
  int32_t* accept_len;          // [batch]
  int32_t* accept_tokens;       // [batch, max_accept]
  int32_t* accept_nodes;        // [batch, max_accept]
};

struct PackParams {
  const int32_t* q_len;         // [batch]
  const int32_t* tree_parent;   // [batch, width]
  const int32_t* tree_token;    // [batch, width] (nullable, with packed_token)
  int32_t batch, width;
  int64_t total_q;              // rows of the packed outputs
  int32_t* packed_parent;       // [total_q]
  int32_t* packed_token;        // [total_q] (nullable)
  int64_t* q_offsets;           // [batch + 1] (nullable)
};

struct SampleParams {
  const void* logits;   // [rows, row_stride] fp32 or bf16
  int64_t rows, row_stride;
  int32_t vocab;
  float temperature;    // >= 0 (0 = argmax)
  uint64_t seed, offset;
  int32_t* tokens;      // [rows]
};

// First key of split s (0..S) of a request with P prefix keys.  Splits cover whole
// 32-key tiles (every split after the first starts on a tile boundary), and the tree tail
// goes with split S-1.  ratio 1: S equal chunks of ceil(P/S) keys rounded up to 32.
// ratio r < 1: split s holds about r^s (1 - r) / (1 - r^S) of the prefix, largest first,
// so that when the launch's last round is short it holds the smallest pieces.  Both ends of
// a split come from this one function, so neighbouring splits meet exactly.
__device__ __forceinline__ int split_begin(int P, int S, float r, int s) {
  if (s <= 0) return 0;
  if (s >= S) return P;
  int64_t b;
  if (!(r < 1.0f)) {
    const int64_t chunk = (((int64_t)P + S - 1) / S + 31) / 32 * 32;
    b = (int64_t)s * chunk;
  } else {
    const float f = (1.0f - __builtin_powf(r, (float)s)) / (1.0f - __builtin_powf(r, (float)S));
    b = ((int64_t)((float)P * f) + 31) / 32 * 32;
  }
  return (int)(b < P ? b : P);
}

// Last-round cut of one XCD's queue (bf16 kernel, one split).  The kernel deals groups
// of m_tiles row tiles to the XCDs in snake order; XCD x's queue then holds n units, the
// first `whole` of them in whole rounds of CUS_PER_XCD.  Each of the `left` units after
// them is cut into `pieces` key pieces (0 when there is nothing to cut).
struct XcdCut {
  int whole, left, pieces;
};
// XCDs that receive work from a one-split launch of `batch` requests (groups are dealt
// to XCDs 0, 1, ... first), and so the piece slots a cut can use.
__host__ __device__ inline int cut_piece_slots(int batch) {
  return (batch < NUM_XCD ? batch : NUM_XCD) * CUS_PER_XCD;
}
__host__ __device__ inline XcdCut xcd_cut(int groups, int m_tiles, int xcd) {
  const int full_rounds = groups / NUM_XCD, rem = groups % NUM_XCD;
  const int pos = (full_rounds & 1) ? NUM_XCD - 1 - xcd : xcd;  // in the partial round
  const int n = (full_rounds + (pos < rem ? 1 : 0)) * m_tiles;
  XcdCut c;
  c.whole = n / CUS_PER_XCD * CUS_PER_XCD;
  c.left = n - c.whole;
  c.pieces = c.left ? CUS_PER_XCD / c.left : 0;
  if (c.pieces < 2) c.left = c.pieces = 0;
  return c;
}

// Host-side launchers (defined in the .hip files).
hipError_t launch_sample_tokens(const SampleParams& p, bool bf16, hipStream_t stream);
hipError_t launch_pack_tree(const PackParams& p, hipStream_t stream);
hipError_t launch_build_ddtree(const DdtreeBuildParams& p, hipStream_t stream);
hipError_t launch_tree_accept(const AcceptParams& p, hipStream_t stream);
hipError_t launch_verify_bf16(const VerifyParams& p, hipStream_t stream);
hipError_t launch_verify_f32(const VerifyParams& p, hipStream_t stream);
hipError_t launch_prepass(const VerifyParams& p, int64_t n_tiles_bound, hipStream_t stream);
hipError_t launch_fill_nan(float* p, int64_t n, hipStream_t stream);
hipError_t launch_lse_merge(const float* part_o, const float* part_lse, float* out_lat,
                            float* out_lse, int64_t rows, int32_t num_splits, hipStream_t stream);
hipError_t launch_piece_merge(const VerifyParams& p, hipStream_t stream);
int rows_per_block_bf16();
int rows_per_block_f32();

}  // namespace kdt
