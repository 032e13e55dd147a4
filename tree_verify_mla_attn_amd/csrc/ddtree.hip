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

constexpr int WAVE = 64;  // one wavefront per request

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Largest value over the wavefront (no NaN): DPP swaps within each row of 16 lanes
// (xor 1, xor 2, half-row mirror, row mirror), then the four row results.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
               fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

// One wavefront builds one request's tree.  The frontier holds one entry per lane: before
// pop k at most k entries are live, and the last pop pushes nothing, so 64 lanes suffice
// for budgets up to 64.  A pop is a wave max over the live scores, a ballot of the lanes
// holding it (the earliest push among them wins a tie), and two pushes: the next sibling
// reuses the popped lane, the first child takes the lowest free lane.  Node i < 64 is
// recorded in lane i's registers, node 64 in scalars.
__global__ __launch_bounds__(WAVE) void build_ddtree_kernel(DdtreeBuildParams p) {
  __shared__ float s_lp[MAX_DDTREE_TABLE];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int D = p.depth, K = p.top_k, budget = p.budget, width = budget + 1;
  const float* lp_g = p.logp + (int64_t)b * D * K;
  for (int i = lane; i < D * K; i += WAVE) s_lp[i] = lp_g[i];
  __syncthreads();
  // log-probability of (depth d, rank r); -inf where there is no candidate
  auto lp_at = [&](int d, int r) { return (d <= D && r < K) ? s_lp[(d - 1) * K + r] : -INFINITY; };
  // lane d: rank 0 at depth d + 1, the first child of any depth-d node
  const float lp_first = lane < D ? s_lp[lane * K] : -INFINITY;

  bool alive = false;                           // frontier entry of this lane
  float f_sc = -INFINITY, f_lpsib = -INFINITY;  // its score; log-prob of its next sibling
  int f_meta = 0, f_push = 0;                   // depth << 20 | rank << 8 | parent; push index
  int m_par = -1, m_dep = 0, m_rank = -1;       // node `lane` (lane 0: the root)
  float m_sc = 0.0f;
  int l_par = -1, l_dep = -1, l_rank = -1;      // node 64
  float l_sc = -INFINITY;
  int pushed = 0, n = 1;

  if (budget >= 1) {
    const float lp0 = readlane_f(lp_first, 0);
    if (lp0 > -INFINITY) {
      if (lane == 0) {
        alive = true;
        f_sc = 0.0f + lp0;
        f_meta = 1 << 20;
        f_push = 0;
        f_lpsib = lp_at(1, 1);
      }
      pushed = 1;
    }
  }
  for (int step = 0; step < budget; ++step) {
    const float mx = wave_max(alive ? f_sc : -INFINITY);
    uint64_t cand = __builtin_amdgcn_ballot_w64(alive && f_sc == mx);
    if (cand == 0) break;  // frontier empty: underfull tree
    int w = __builtin_ctzll(cand);
    cand &= cand - 1;
    if (cand) {  // equal scores: the earliest push wins
      int best = __builtin_amdgcn_readlane(f_push, w);
      while (cand) {
        const int l = __builtin_ctzll(cand);
        cand &= cand - 1;
        const int pl = __builtin_amdgcn_readlane(f_push, l);
        if (pl < best) {
          best = pl;
          w = l;
        }
      }
    }
    const float sc = readlane_f(f_sc, w);
    const int meta = __builtin_amdgcn_readlane(f_meta, w);
    const float lpsib = readlane_f(f_lpsib, w);
    const int d = meta >> 20, r = (meta >> 8) & 0xfff, par = meta & 0xff;
    const int node = n++;
    if (node < WAVE) {
      if (lane == node) {
        m_par = par;
        m_dep = d;
        m_rank = r;
        m_sc = sc;
      }
    } else {
      l_par = par;
      l_dep = d;
      l_rank = r;
      l_sc = sc;
    }
    if (lane == w) alive = false;
    if (step + 1 == budget) break;  // the last pop: nothing more is popped
    // here node <= budget - 1 <= 63 and par < node, so both are lanes
    int tgt = w;
    if (lpsib > -INFINITY) {
      const float ssc = readlane_f(m_sc, par) + lpsib;
      if (lane == w) {
        alive = true;
        f_sc = ssc;
        f_meta = (d << 20) | ((r + 1) << 8) | par;
        f_push = pushed;
        f_lpsib = lp_at(d, r + 2);
      }
      ++pushed;
      tgt = __builtin_ctzll(~__builtin_amdgcn_ballot_w64(alive));
    }
    const float lpc = d < D ? readlane_f(lp_first, d) : -INFINITY;
    if (lpc > -INFINITY) {
      const float csc = sc + lpc;
      if (lane == tgt) {
        alive = true;
        f_sc = csc;
        f_meta = ((d + 1) << 20) | node;
        f_push = pushed;
        f_lpsib = lp_at(d + 1, 1);
      }
      ++pushed;
    }
  }

  // first child / next sibling of node `lane`: the lowest later node with this parent
  int fc = -1, ns = -1;
  for (int j = 1; j < n; ++j) {
    const int pj = j < WAVE ? __builtin_amdgcn_readlane(m_par, j) : l_par;
    if (j > lane) {
      if (fc < 0 && pj == lane) fc = j;
      if (ns < 0 && lane > 0 && pj == m_par) ns = j;
    }
  }
  // outputs, padded to `width` with -1 (score: -inf)
  const int64_t row = (int64_t)b * width;
  const int32_t* ids = p.token_ids + (int64_t)b * D * K;
  if (lane == 0) p.q_len[b] = n;
  for (int i = lane; i < width; i += WAVE) {
    int par = -1, tok = -1, dep = -1, c = -1, sib = -1;
    float sc = -INFINITY;
    if (i < n && i < WAVE) {
      par = m_par;
      dep = m_dep;
      sc = m_sc;
      c = fc;
      sib = ns;
      tok = i == 0 ? p.root_token[b] : ids[(m_dep - 1) * K + m_rank];
    } else if (i < n) {  // node 64: a leaf, the last node
      par = l_par;
      dep = l_dep;
      sc = l_sc;
      tok = ids[(l_dep - 1) * K + l_rank];
    }
    p.tree_parent[row + i] = par;
    p.tree_token[row + i] = tok;
    p.tree_depth[row + i] = dep;
    p.first_child[row + i] = c;
    p.next_sibling[row + i] = sib;
    if (p.tree_score) p.tree_score[row + i] = sc;
  }
}

// One wavefront per request.  The request's tokens and sibling pointers are staged in
// LDS; each lane then finds, for its nodes i, the child matching target_next[i] (the
// first in sibling order; a pointer that leaves (i, n) ends the search); the walk from
// the root follows those matches.
__global__ __launch_bounds__(WAVE) void tree_accept_kernel(AcceptParams p) {
  extern __shared__ int32_t s_dyn[];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t row = (int64_t)b * p.max_nodes;
  const int n = min(max(p.q_len[b], 1), p.max_nodes);
  int32_t* s_tok = s_dyn;
  int32_t* s_ns = s_dyn + p.max_nodes;
  int32_t* s_match = s_dyn + 2 * p.max_nodes;
  for (int i = lane; i < n; i += WAVE) {
    s_tok[i] = p.tree_token[row + i];
    s_ns[i] = p.next_sibling[row + i];
  }
  __syncthreads();
  for (int i = lane; i < n; i += WAVE) {
    const int want = p.target_next[row + i];
    int c = p.first_child[row + i];
    for (int guard = 0; c > i && c < n && s_tok[c] != want && guard < n; ++guard) c = s_ns[c];
    s_match[i] = (c > i && c < n && s_tok[c] == want) ? c : -1;
  }
  __syncthreads();
  int32_t* toks = p.accept_tokens + (int64_t)b * p.max_accept;
  int32_t* nodes = p.accept_nodes + (int64_t)b * p.max_accept;
  int len = 0, cur = 0;
  while (true) {  // every step moves to a larger node index: at most n steps
    const int m = s_match[cur];
    if (m < 0 || len + 1 >= p.max_accept) break;
    if (lane == 0) {
      toks[len] = s_tok[m];
      nodes[len] = m;
    }
    ++len;
    cur = m;
  }
  if (lane == 0) {
    toks[len] = p.target_next[row + cur];  // bonus token
    nodes[len] = -1;
    p.accept_len[b] = len + 1;
  }
  for (int i = len + 1 + lane; i < p.max_accept; i += WAVE) {
    toks[i] = -1;
    nodes[i] = -1;
  }
}

// Padded per-request tree rows -> the packed node-order rows verify attention reads.
// Workgroup b sums the clamped q_len of requests 0..b-1 itself (no cross-workgroup
// dependency), so the offsets need no separate scan launch.
__global__ __launch_bounds__(WAVE) void pack_tree_kernel(PackParams p) {
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
  hipLaunchKernelGGL(build_ddtree_kernel, dim3((unsigned)p.batch), dim3(WAVE), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_tree_accept(const AcceptParams& p, hipStream_t stream) {
  const size_t lds = (size_t)3 * p.max_nodes * sizeof(int32_t);
  hipLaunchKernelGGL(tree_accept_kernel, dim3((unsigned)p.batch), dim3(WAVE), lds, stream, p);
  return hipGetLastError();
}

}  // namespace kdt
