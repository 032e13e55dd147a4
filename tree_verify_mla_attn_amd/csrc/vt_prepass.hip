// V^T pre-pass for the bf16 path: the latent rows of every request's KV stream,
// converted once to fp16 and laid out feature-major in 32-key tiles, exactly as the
// attention kernel's PV contraction reads them from LDS.
//
// Why: the softmax-weighted sum of latent rows runs as an fp16 MFMA (P must be fp16:
// bf16 P is too coarse for a 2e-3 relative bound), so V must be fp16 too, and the MFMA
// operand wants 8 consecutive keys of one feature.  Converting here, once per call,
// keeps the conversion and its LDS traffic out of the attention loop, where each KV
// tile is consumed by every row tile of its request.
//
// Workgroup 0 also ranks the requests by KV length (longest first; ties by index) into
// p.order, which the attention kernel uses to hand out work longest-first.
//
// Tile t of request b covers keys [32t, 32t+32) of that request's stream (prefix, then
// tail); keys past the end repeat the last key (their probabilities are zero).  Tile
// layout (u32x4 = 8 fp16 keys of one feature): feature f, key chunk q at slot
// f*4 + (q ^ ((f >> 2) & 3)); chunk q holds keys {b..b+3, b+8..b+11} with
// b = 16(q/2) + 4(q%2), in the k-slot order of the PV MFMA.  Tiles of request b start at
// tile index sum_{b' < b} ceil((P_b' + T_b') / 32).
#include "common.h"

namespace kdt {
namespace {

constexpr int NTHR = 256;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// order[rank] = request, ranks by descending (prefix_len + q_len), ties by index
// (malformed requests count as empty).  O(B^2 / 256) work, bounded by ORDER_MAX_BATCH.
__device__ void rank_requests(const VerifyParams& p) {
  __shared__ int s_cost[ORDER_MAX_BATCH];
  const int B = p.batch;
  if (B > ORDER_MAX_BATCH) {
    for (int b = threadIdx.x; b < B; b += NTHR) p.order[b] = b;
    return;
  }
  for (int b = threadIdx.x; b < B; b += NTHR) {
    const int t = p.q_len[b], pl = p.prefix_len[b];
    const bool bad = t < 1 || t > p.max_q_len || pl < 0 || pl > MAX_REQUEST_KEYS - t;
    s_cost[b] = bad ? 0 : pl + t;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += NTHR) {
    const int cb = s_cost[b];
    int rank = 0;
    for (int i = 0; i < B; ++i) {
      const int ci = s_cost[i];
      rank += (ci > cb) || (ci == cb && i < b);
    }
    p.order[rank] = b;
  }
}

__global__ __launch_bounds__(NTHR) void vt_prepass_kernel(VerifyParams p) {
  __shared__ int64_t s_kvoff, s_tbase;
  __shared__ int s_b, s_flag;
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x;  // global tile index
  // Find the request owning tile g (scan over requests, 256 at a time).
  if (tid == 0) {
    s_b = -1;
    s_flag = 0;
  }
  __syncthreads();
  int64_t kv_run = 0, t_run = 0;
  for (int b0 = 0; b0 < p.batch; b0 += NTHR) {
    const int b = b0 + tid;
    int64_t kv_len = 0, tiles = 0;
    bool bad = false;
    if (b < p.batch) {
      const int t = p.q_len[b], pl = p.prefix_len[b];
      bad = t < 1 || t > p.max_q_len || pl < 0 || pl > MAX_REQUEST_KEYS - t;
      kv_len = bad ? 0 : (int64_t)pl + t;
      tiles = (kv_len + 31) / 32;
    }
    if (bad) atomicOr(&s_flag, 1);
    // inclusive scans of kv_len and tiles across the block
    __shared__ int64_t s_scan_kv[NTHR], s_scan_t[NTHR];
    s_scan_kv[tid] = kv_len;
    s_scan_t[tid] = tiles;
    __syncthreads();
    for (int off = 1; off < NTHR; off <<= 1) {
      const int64_t a = tid >= off ? s_scan_kv[tid - off] : 0;
      const int64_t c = tid >= off ? s_scan_t[tid - off] : 0;
      __syncthreads();
      s_scan_kv[tid] += a;
      s_scan_t[tid] += c;
      __syncthreads();
    }
    const int64_t t_excl = t_run + s_scan_t[tid] - tiles;
    if (b < p.batch && tiles > 0 && g >= t_excl && g < t_excl + tiles) {
      s_b = b;
      s_kvoff = kv_run + s_scan_kv[tid] - kv_len;
      s_tbase = t_excl;
    }
    kv_run += s_scan_kv[NTHR - 1];
    t_run += s_scan_t[NTHR - 1];
    __syncthreads();
  }
  if (g == 0) rank_requests(p);
  // Malformed inputs: the attention kernel flags them; nothing sensible to convert.
  if (s_flag || s_b < 0) return;
  const int b = s_b;
  const int64_t kvoff = s_kvoff;
  if (kvoff + p.prefix_len[b] + p.q_len[b] > p.total_kv) return;
  const int n_keys = p.prefix_len[b] + p.q_len[b];
  const int key0 = (int)(g - s_tbase) * 32;

  const int q = tid & 3, fg = tid >> 2;
  const int kb = 16 * (q >> 1) + 4 * (q & 1);
  const uint4* src = (const uint4*)p.kv_lat;  // bf16 rows of 64 x 16 B
  uint4 w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = min(key0 + kb + (e >> 2) * 8 + (e & 3), n_keys - 1);
    w[e] = src[(kvoff + k) * 64 + fg];
  }
  uint4* dst = (uint4*)p.vt + g * (DL * 4);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    unsigned o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const unsigned* a = (const unsigned*)&w[2 * d];
      const unsigned* c = (const unsigned*)&w[2 * d + 1];
      const unsigned x = a[j >> 1], y = c[j >> 1];
      const float fx = __uint_as_float((j & 1) ? (x & 0xffff0000u) : (x << 16));
      const float fy = __uint_as_float((j & 1) ? (y & 0xffff0000u) : (y << 16));
      o[d] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){fx, fy}, f16x2));
    }
    const int f = fg * 8 + j;
    dst[f * 4 + (q ^ ((f >> 2) & 3))] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t launch_vt_prepass(const VerifyParams& p, int64_t n_tiles_bound, hipStream_t stream) {
  if (n_tiles_bound <= 0 || n_tiles_bound > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vt_prepass_kernel, dim3((unsigned)n_tiles_bound), dim3(NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kdt
