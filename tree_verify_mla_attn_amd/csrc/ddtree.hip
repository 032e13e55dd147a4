// The two steps around verify attention in a greedy DDTree step, on the device:
//
// * best-first draft-tree builder ("The Milestone Commit: Cementing Phase 1 ...", section
//   "The Context", item 1: a device tree builder in place of a per-request host heap;
//   "Strategic Pivots in CUDA Kernel Engineering ...", sections "The Message" and "Why
//   This Message Was Written": trees from the drafter's top-k log-probabilities and token
//   ids, bit-exact with the host heap including its tie-breaks and float32 accumulation);
// * greedy follow-verified-tree accept ("The Milestone Commit ...", section "The
//   Context", item 3: a walk over next-token / next-sibling pointers, one thread per
//   request).
//
// Builder semantics: a node at depth d taking rank r scores parent + logp[d-1][r],
// added in float32 from the root down (root = 0); the frontier pops the highest score,
// ties to the earliest push; popping (d, r) under p pushes its next sibling (d, r+1)
// under p and its first child (d+1, 0) under itself; -inf marks an absent candidate;
// node index = pop order.
//
// A third kernel packs the builder's padded rows into the node-order packed layout of
// verify attention, so that build -> verify -> accept chain on the device.
#include "common.h"

namespace kdt {
namespace {

constexpr int BUILD_THREADS = 64;  // one wave per request
constexpr int MAX_FRONTIER = 2 * MAX_DDTREE_BUDGET + 1;

__global__ __launch_bounds__(BUILD_THREADS) void build_ddtree_kernel(DdtreeBuildParams p) {
  __shared__ float s_lp[MAX_DDTREE_TABLE];
  __shared__ float f_score[MAX_FRONTIER];   // frontier entry e = e-th push
  __shared__ int32_t f_meta[MAX_FRONTIER];  // depth << 20 | rank << 8 | parent
  __shared__ int32_t f_alive[MAX_FRONTIER];
  __shared__ float n_score[MAX_DDTREE_BUDGET + 1];
  __shared__ int32_t n_parent[MAX_DDTREE_BUDGET + 1];
  __shared__ int32_t n_depth[MAX_DDTREE_BUDGET + 1];
  __shared__ int32_t n_rank[MAX_DDTREE_BUDGET + 1];
  __shared__ int32_t s_count[2];  // [0] frontier entries pushed, [1] nodes

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int D = p.depth, K = p.top_k, width = p.budget + 1;
  const float* lp_g = p.logp + (int64_t)b * D * K;
  for (int i = lane; i < D * K; i += BUILD_THREADS) s_lp[i] = lp_g[i];
  for (int i = lane; i < MAX_FRONTIER; i += BUILD_THREADS) f_alive[i] = 0;
  if (lane == 0) {
    n_score[0] = 0.0f;
    n_parent[0] = -1;
    n_depth[0] = 0;
    n_rank[0] = -1;
    s_count[0] = 0;
    s_count[1] = 1;
  }
  __syncthreads();
  // (d, r) exists and is a candidate (-inf = absent)
  auto candidate = [&](int d, int r) { return d <= D && r < K && s_lp[(d - 1) * K + r] > -INFINITY; };
  if (lane == 0 && p.budget >= 1 && candidate(1, 0)) {
    f_score[0] = n_score[0] + s_lp[0];
    f_meta[0] = (1 << 20) | (0 << 8) | 0;
    f_alive[0] = 1;
    s_count[0] = 1;
  }
  __syncthreads();

  for (int step = 0; step < p.budget; ++step) {
    // arg max over live entries: higher score, then lower push index
    const int pushed = s_count[0];
    float best = -INFINITY;
    int best_e = 0x7fffffff;
    for (int e = lane; e < pushed; e += BUILD_THREADS) {
      if (!f_alive[e]) continue;
      const float sc = f_score[e];
      if (best_e == 0x7fffffff || sc > best || (sc == best && e < best_e)) {
        best = sc;
        best_e = e;
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const float ob = __shfl_xor(best, off);
      const int oe = __shfl_xor(best_e, off);
      if (oe != 0x7fffffff &&
          (best_e == 0x7fffffff || ob > best || (ob == best && oe < best_e))) {
        best = ob;
        best_e = oe;
      }
    }
    if (best_e == 0x7fffffff) break;  // frontier empty: underfull tree (uniform)
    if (lane == 0) {
      const int meta = f_meta[best_e];
      const int d = meta >> 20, r = (meta >> 8) & 0xfff, par = meta & 0xff;
      f_alive[best_e] = 0;
      const int node = s_count[1];
      const float sc = n_score[par] + s_lp[(d - 1) * K + r];
      n_score[node] = sc;
      n_parent[node] = par;
      n_depth[node] = d;
      n_rank[node] = r;
      int e = s_count[0];
      if (candidate(d, r + 1)) {
        f_score[e] = n_score[par] + s_lp[(d - 1) * K + r + 1];
        f_meta[e] = (d << 20) | ((r + 1) << 8) | par;
        f_alive[e] = 1;
        ++e;
      }
      if (candidate(d + 1, 0)) {
        f_score[e] = sc + s_lp[d * K];
        f_meta[e] = ((d + 1) << 20) | (0 << 8) | node;
        f_alive[e] = 1;
        ++e;
      }
      s_count[0] = e;
      s_count[1] = node + 1;
    }
    __syncthreads();
  }
  __syncthreads();

  // outputs, padded to `width` with -1 (score: -inf)
  const int n = s_count[1];
  const int64_t row = (int64_t)b * width;
  const int32_t* ids = p.token_ids + (int64_t)b * D * K;
  if (lane == 0) p.q_len[b] = n;
  for (int i = lane; i < width; i += BUILD_THREADS) {
    int par = -1, tok = -1, dep = -1, fc = -1, ns = -1;
    float sc = -INFINITY;
    if (i < n) {
      par = n_parent[i];
      dep = n_depth[i];
      sc = n_score[i];
      tok = i == 0 ? p.root_token[b] : ids[(dep - 1) * K + n_rank[i]];
      for (int j = i + 1; j < n; ++j) {  // children and siblings in index order
        if (fc < 0 && n_parent[j] == i) fc = j;
        if (ns < 0 && i > 0 && n_parent[j] == par) ns = j;
      }
    }
    p.tree_parent[row + i] = par;
    p.tree_token[row + i] = tok;
    p.tree_depth[row + i] = dep;
    p.first_child[row + i] = fc;
    p.next_sibling[row + i] = ns;
    if (p.tree_score) p.tree_score[row + i] = sc;
  }
}

__global__ __launch_bounds__(256) void tree_accept_kernel(AcceptParams p) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= p.batch) return;
  const int64_t row = (int64_t)b * p.max_nodes;
  const int n = min(max(p.q_len[b], 1), p.max_nodes);
  int32_t* toks = p.accept_tokens + (int64_t)b * p.max_accept;
  int32_t* nodes = p.accept_nodes + (int64_t)b * p.max_accept;
  int len = 0, cur = 0;
  // every step moves to a larger node index, so n steps bound the walk (also for
  // malformed pointers, which can only end it early)
  for (int it = 0; it < n; ++it) {
    const int want = p.target_next[row + cur];
    int c = p.first_child[row + cur];
    // follow the sibling chain to the child carrying the target's next token
    int guard = 0;
    while (c > 0 && c < n && p.tree_token[row + c] != want && ++guard <= n)
      c = p.next_sibling[row + c];
    const bool take = c > 0 && c < n && p.tree_token[row + c] == want && len + 1 < p.max_accept;
    if (!take || c <= cur) {
      toks[len] = want;  // bonus token
      nodes[len] = -1;
      ++len;
      break;
    }
    toks[len] = want;
    nodes[len] = c;
    ++len;
    cur = c;
  }
  p.accept_len[b] = len;
  for (int i = len; i < p.max_accept; ++i) {
    toks[i] = -1;
    nodes[i] = -1;
  }
}

// Padded per-request tree rows -> the packed node-order rows verify attention reads.
// Workgroup b sums the clamped q_len of requests 0..b-1 itself (no cross-workgroup
// dependency), so the offsets need no separate scan launch.
__global__ __launch_bounds__(64) void pack_tree_kernel(PackParams p) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  auto clamp_len = [&](int i) { return min(max(p.q_len[i], 0), p.width); };
  int64_t part = 0;
  for (int i = lane; i < b; i += 64) part += clamp_len(i);
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  const int64_t qoff = part;
  const int n = clamp_len(b);
  if (lane == 0) {
    if (p.q_offsets) {
      p.q_offsets[b] = qoff;
      if (b == p.batch - 1) p.q_offsets[p.batch] = qoff + n;
    }
  }
  if (qoff + n > p.total_q) return;  // capacity exceeded: nothing written for b
  const int64_t src = (int64_t)b * p.width;
  for (int i = lane; i < n; i += 64) {
    p.packed_parent[qoff + i] = p.tree_parent[src + i];
    if (p.packed_token) p.packed_token[qoff + i] = p.tree_token[src + i];
  }
}

}  // namespace

hipError_t launch_pack_tree(const PackParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(pack_tree_kernel, dim3((unsigned)p.batch), dim3(64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_build_ddtree(const DdtreeBuildParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(build_ddtree_kernel, dim3((unsigned)p.batch), dim3(BUILD_THREADS), 0, stream,
                     p);
  return hipGetLastError();
}

hipError_t launch_tree_accept(const AcceptParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(tree_accept_kernel, dim3((unsigned)((p.batch + 255) / 256)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace kdt
