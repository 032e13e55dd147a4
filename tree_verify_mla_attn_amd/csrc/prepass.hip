// Pre-pass of the bf16 path: the latent rows of every request's KV stream, converted once
// per call to fp16 and laid out in 32-key tiles exactly as the attention kernel keeps
// them in LDS, where each tile serves both contractions: the scores read its rows (8
// latent features per lane) and the softmax-weighted sum reads it through the transposing
// LDS load (4 keys per lane).
//
// Why fp16: the weighted sum of latent rows runs as an fp16 MFMA (P must be fp16: bf16 P
// is too coarse for a 2e-3 relative bound), so V must be fp16; the scores then use the
// same copy.  bf16 -> fp16 is exact for 2^-17 <= |x| < 65504 (fp16 normals carry 11
// significant bits, its subnormals reach every bf16 value down to 2^-17); smaller
// magnitudes round with an absolute error <= 2^-25.  Converting here, once per call,
// keeps the conversion out of the attention loop, where each tile is consumed by every
// row tile of its request.
//
// Workgroup 0 also ranks the requests by KV length (longest first; ties by index) and
// writes one record per rank into p.req: the attention kernel hands out work in that
// order and takes each request's offsets and status from its record.
//
// Tile t of request b covers keys [32t, 32t+32) of that request's stream (prefix, then
// tail); keys past the end repeat the last key (their probabilities are zero, their
// values stay finite).  Tile image: row r (key 32t + r) = 1 KB = 64 chunks of 8 fp16
// features; slot s of row r holds chunk s ^ ((r >> 2) & 3).  Tiles of request b start at
// tile index sum_{b' < b} ceil((P_b' + T_b') / 32).
#include "common.h"

namespace kdt {
namespace {

constexpr int NTHR = 256;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// req[rank]: ranks by descending (prefix_len + q_len), ties by index (malformed requests
// count as empty), each with the request's packed offsets (exclusive prefix sums over the
// requests before it in index order) and the status bits the attention kernel reports
// for it.  O(B^2 / 256) work for the ranks, bounded by ORDER_MAX_BATCH; larger batches
// keep the index order.
__device__ void index_requests(const VerifyParams& p) {
  __shared__ int s_cost[ORDER_MAX_BATCH];
  __shared__ int64_t s_q[NTHR], s_kv[NTHR], s_t[NTHR];
  __shared__ int s_f[NTHR];
  const int B = p.batch;
  const int tid = threadIdx.x;
  const bool ranked = B <= ORDER_MAX_BATCH;
  if (ranked) {
    for (int b = tid; b < B; b += NTHR) {
      const int t = p.q_len[b], pl = p.prefix_len[b];
      const bool bad = t < 1 || t > p.max_q_len || pl < 0 || pl > MAX_REQUEST_KEYS - t;
      s_cost[b] = bad ? 0 : pl + t;
    }
  }
  __syncthreads();
  int64_t q_run = 0, kv_run = 0, t_run = 0;
  int f_run = 0;
  for (int b0 = 0; b0 < B; b0 += NTHR) {
    const int b = b0 + tid;
    int t = 0, pl = 0, own = 0, later = 0;
    int64_t kvl = 0, tiles = 0;
    if (b < B) {
      t = p.q_len[b];
      pl = p.prefix_len[b];
      own = (t < 1 || t > p.max_q_len ? ST_BAD_QLEN : 0) | (pl < 0 ? ST_BAD_PREFIX : 0);
      // what this request means for every later one: their offsets are unknown, or (key
      // count over the limit) the pre-pass stops converting tiles here
      later = own | (!own && pl > MAX_REQUEST_KEYS - t ? ST_OVERFLOW : 0);
      kvl = (int64_t)pl + t;
      tiles = (kvl + TILE_KEYS - 1) / TILE_KEYS;
    }
    // inclusive scans across the block (Hillis-Steele)
    s_q[tid] = t;
    s_kv[tid] = kvl;
    s_t[tid] = tiles;
    s_f[tid] = later;
    __syncthreads();
    for (int off = 1; off < NTHR; off <<= 1) {
      const int64_t aq = tid >= off ? s_q[tid - off] : 0;
      const int64_t akv = tid >= off ? s_kv[tid - off] : 0;
      const int64_t at = tid >= off ? s_t[tid - off] : 0;
      const int af = tid >= off ? s_f[tid - off] : 0;
      __syncthreads();
      s_q[tid] += aq;
      s_kv[tid] += akv;
      s_t[tid] += at;
      s_f[tid] |= af;
      __syncthreads();
    }
    if (b < B) {
      ReqRec r;
      r.b = b;
      r.q_len = t;
      r.prefix_len = pl;
      r.qoff = q_run + s_q[tid] - t;
      r.kvoff = kv_run + s_kv[tid] - kvl;
      r.tbase = t_run + s_t[tid] - tiles;
      int flag = f_run | (tid > 0 ? s_f[tid - 1] : 0) | own;
      if (!flag && (r.qoff + t > p.total_q || r.kvoff + kvl > p.total_kv ||
                    pl > MAX_REQUEST_KEYS - t))
        flag |= ST_OVERFLOW;
      if (!flag && r.tbase + tiles > p.k16_tiles) flag |= ST_OVERFLOW;
      r.flag = flag;
      r.pad[0] = r.pad[1] = r.pad[2] = 0;
      int rank = b;
      if (ranked) {
        const int cb = s_cost[b];
        rank = 0;
        for (int i = 0; i < B; ++i) {
          const int ci = s_cost[i];
          rank += (ci > cb) || (ci == cb && i < b);
        }
      }
      p.req[rank] = r;
    }
    q_run += s_q[NTHR - 1];
    kv_run += s_kv[NTHR - 1];
    t_run += s_t[NTHR - 1];
    f_run |= s_f[NTHR - 1];
    __syncthreads();
  }
}

__global__ __launch_bounds__(NTHR) void prepass_kernel(VerifyParams p) {
  __shared__ int64_t s_kvoff, s_tbase;
  __shared__ int s_b, s_first_bad;
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x;  // global tile index
  // Find the request owning tile g (scan over requests, 256 at a time).
  if (tid == 0) {
    s_b = -1;
    s_first_bad = p.batch;
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
    if (bad) atomicMin(&s_first_bad, b);
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
  if (g == 0) index_requests(p);
  // Malformed inputs: the attention kernel flags a malformed request and skips it and
  // every request after it (their packed offsets are unknown), but runs the requests
  // before it; so tiles are converted exactly for the requests before the first
  // malformed one.
  if (s_b < 0 || s_b >= s_first_bad) return;
  const int b = s_b;
  const int64_t kvoff = s_kvoff;
  if (kvoff + p.prefix_len[b] + p.q_len[b] > p.total_kv) return;
  const int n_keys = p.prefix_len[b] + p.q_len[b];
  const int key0 = (int)(g - s_tbase) * 32;

  // wave w converts rows 8w..8w+7, one contiguous 1 KB row per instruction: lane l reads
  // chunk l (8 bf16) and writes it, as 8 fp16, to slot l ^ ((row >> 2) & 3)
  const int lane = tid & 63, wave = tid >> 6;
  const uint4* src = (const uint4*)p.kv_lat;  // bf16 rows: 64 x 16 B
  uint4* dst = (uint4*)p.k16 + g * (DL * 2 / 16 * 32);
  uint4 w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = min(key0 + wave * 8 + e, n_keys - 1);
    w[e] = src[(kvoff + k) * 64 + lane];
  }
  unsigned range = 0;  // bit 15 / 31: an fp16 half with an all-ones exponent (inf or NaN)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = wave * 8 + e;
    unsigned o[4];
    const unsigned* x = (const unsigned*)&w[e];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // bf16 pair -> fp32 pair (exact) -> fp16 pair, round to nearest even
      const f16x2 hp = {(_Float16)__uint_as_float(x[d] << 16),
                        (_Float16)__uint_as_float(x[d] & 0xffff0000u)};
      o[d] = __builtin_bit_cast(unsigned, hp);
      range |= (o[d] & 0x7c007c00u) + 0x04000400u;
    }
    dst[row * 64 + (lane ^ ((row >> 2) & 3))] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  // A latent value outside fp16's range (|x| >= 65504: no bf16 value lies in
  // [65504, 65536), and 65536 and up round to inf) or not finite: the contract of the bf16
  // path is broken, and the rows that see this key are not meaningful.
  if (__builtin_amdgcn_ballot_w64((range & 0x80008000u) != 0) && lane == 0 && p.status)
    atomicOr(p.status, ST_RANGE);
}

}  // namespace

hipError_t launch_prepass(const VerifyParams& p, int64_t n_tiles_bound, hipStream_t stream) {
  if (n_tiles_bound <= 0 || n_tiles_bound > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prepass_kernel, dim3((unsigned)n_tiles_bound), dim3(NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kdt
