// LSE merge of split-KV partial results ("The Milestone Commit: Cementing Phase 1 ...",
// section "What to defer": flash partial outputs merged for long prefixes).
//
// For each query row, split s holds a normalised partial output O_s (512 fp32) and its
// log-sum-exp lse_s (-inf when the split saw no key).  With L = max_s lse_s and
// w_s = exp(lse_s - L):  out = sum_s w_s O_s / sum_s w_s,  lse = L + ln sum_s w_s.
//
// Before the attention kernels run, every partial lse is set to NaN.  The attention
// kernels overwrite it for every row of every request they process, so a row whose lse
// is still NaN in some split belongs to a request they skipped (flagged in the status
// word) or to no request (rows past the packed total).  The merge leaves such rows
// unwritten, as the single-split path does.
//
// HBM-bound: one pass over the partials.  One wavefront per row: lane l holds the lse of
// splits l, l + 64, ...; the weights are formed once per row and read back with lane
// reads; each lane accumulates features [4l, 4l + 4) and [256 + 4l, 256 + 4l + 4), so
// every load instruction of the wave covers 1 KB contiguous; four splits' loads are in
// flight at a time.
#include "common.h"

namespace kdt {
namespace {

constexpr int MERGE_ROWS = 4;  // rows (wavefronts) per 256-thread workgroup
constexpr int MERGE_UNROLL = 4;
constexpr int PIECE_UNROLL = 8;
static_assert(PIECE_ROWS % MERGE_ROWS == 0, "whole row tiles per piece-merge grid");

__device__ __forceinline__ float wave_max_f(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(256) void fill_nan_kernel(float* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = __builtin_nanf("");
}

__global__ __launch_bounds__(256) void lse_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_lse,
                                                        float* __restrict__ out_lat,
                                                        float* __restrict__ out_lse, int64_t rows,
                                                        int num_splits) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * MERGE_ROWS + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wavefront
  float ls[MAX_SPLITS / 64];
  float big = -INFINITY;
  bool unset = false;
#pragma unroll
  for (int k = 0; k < MAX_SPLITS / 64; ++k) {
    const int s = 64 * k + lane;
    ls[k] = s < num_splits ? part_lse[(int64_t)s * rows + row] : -INFINITY;
    unset |= __builtin_isnan(ls[k]);
    big = fmaxf(big, ls[k]);
  }
  if (__builtin_amdgcn_ballot_w64(unset)) return;  // skipped by the attention kernels
  big = wave_max_f(big);
  const float bref = big == -INFINITY ? 0.0f : big;
  float w[MAX_SPLITS / 64];
  float wpart = 0.0f;
#pragma unroll
  for (int k = 0; k < MAX_SPLITS / 64; ++k) {
    w[k] = ls[k] == -INFINITY ? 0.0f : __expf(ls[k] - bref);
    wpart += w[k];
  }
  const float wsum = wave_sum_f(wpart);

  const float* src = part_o + row * DL + lane * 4;
  const int64_t split_stride = rows * DL;
  float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
  for (int s0 = 0; s0 < num_splits; s0 += MERGE_UNROLL) {
    float4 v0[MERGE_UNROLL], v1[MERGE_UNROLL];
    float ws[MERGE_UNROLL];
#pragma unroll
    for (int u = 0; u < MERGE_UNROLL; ++u) {
      const int s = s0 + u;  // uniform
      ws[u] = 0.0f;
      v0[u] = v1[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < num_splits) {
        const int k = s >> 6;
        const float wk = k == 0 ? w[0] : (k == 1 ? w[1] : (k == 2 ? w[2] : w[3]));
        ws[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), s & 63));
        v0[u] = *(const float4*)(src + s * split_stride);
        v1[u] = *(const float4*)(src + s * split_stride + 256);
      }
    }
#pragma unroll
    for (int u = 0; u < MERGE_UNROLL; ++u) {
      a0.x += ws[u] * v0[u].x; a0.y += ws[u] * v0[u].y;
      a0.z += ws[u] * v0[u].z; a0.w += ws[u] * v0[u].w;
      a1.x += ws[u] * v1[u].x; a1.y += ws[u] * v1[u].y;
      a1.z += ws[u] * v1[u].z; a1.w += ws[u] * v1[u].w;
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  float* dst = out_lat + row * DL + lane * 4;
  *(float4*)dst = make_float4(a0.x * inv, a0.y * inv, a0.z * inv, a0.w * inv);
  *(float4*)(dst + 256) = make_float4(a1.x * inv, a1.y * inv, a1.z * inv, a1.w * inv);
  if (lane == 0) out_lse[row] = wsum > 0.0f ? big + logf(wsum) : -INFINITY;
}

// Piece merge of the last-round cut: one wavefront per (XCD, cut unit, row), for units
// 0 .. max_left - 1 of each XCD (max_left: the most units any XCD cut).  Lane k < K
// holds the lse of piece k; the same weights as above combine the K pieces' outputs into
// the unit's output row (the pieces cover the request's whole key range).  A row whose
// piece lse is still NaN in some piece was not computed (a skipped request, or a row past
// the request's rows) and is left unwritten.
__global__ __launch_bounds__(256) void piece_merge_kernel(const float* __restrict__ piece_o,
                                                          const float* __restrict__ piece_lse,
                                                          const int64_t* __restrict__ desc,
                                                          float* __restrict__ out_lat,
                                                          float* __restrict__ out_lse,
                                                          int32_t* __restrict__ status,
                                                          int groups, int m_tiles,
                                                          int max_left, int64_t total_rows) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * MERGE_ROWS + (threadIdx.x >> 6);  // (xcd, unit, row)
  const int row = w % PIECE_ROWS;
  const int unit = (w / PIECE_ROWS) % max_left;
  const int xcd = w / (PIECE_ROWS * max_left);
  if (xcd >= NUM_XCD) return;
  const XcdCut cut = xcd_cut(groups, m_tiles, xcd);
  if (unit >= cut.left) return;
  const int k_n = cut.pieces;  // 2..32
  const int64_t s0 = (int64_t)xcd * CUS_PER_XCD + (int64_t)unit * k_n;  // first piece slot
  const float ls = lane < k_n ? piece_lse[(s0 + lane) * PIECE_ROWS + row] : -INFINITY;
  if (__builtin_amdgcn_ballot_w64(__builtin_isnan(ls))) return;
  const int64_t d = (int64_t)xcd * CUS_PER_XCD + unit;
  const int64_t grow = desc[2 * d] + row;
  if (row >= desc[2 * d + 1] || desc[2 * d] < 0 || grow >= total_rows) return;
  const float big = wave_max_f(ls);
  const float bref = big == -INFINITY ? 0.0f : big;
  const float wl = ls == -INFINITY ? 0.0f : __expf(ls - bref);
  const float wsum = wave_sum_f(wl);
  const float* src = piece_o + (s0 * PIECE_ROWS + row) * DL + lane * 4;
  float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
  // PIECE_UNROLL pieces' loads in flight at a time (one at a time, the wave would wait a
  // full memory latency per piece); the sum still runs over the pieces in order
  for (int k0 = 0; k0 < k_n; k0 += PIECE_UNROLL) {
    float4 v0[PIECE_UNROLL], v1[PIECE_UNROLL];
    float ws[PIECE_UNROLL];
#pragma unroll
    for (int u = 0; u < PIECE_UNROLL; ++u) {
      const int k = k0 + u;  // uniform
      ws[u] = 0.0f;
      v0[u] = v1[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < k_n) {
        ws[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k));
        v0[u] = *(const float4*)(src + (int64_t)k * PIECE_ROWS * DL);
        v1[u] = *(const float4*)(src + (int64_t)k * PIECE_ROWS * DL + 256);
      }
    }
#pragma unroll
    for (int u = 0; u < PIECE_UNROLL; ++u) {
      a0.x += ws[u] * v0[u].x; a0.y += ws[u] * v0[u].y;
      a0.z += ws[u] * v0[u].z; a0.w += ws[u] * v0[u].w;
      a1.x += ws[u] * v1[u].x; a1.y += ws[u] * v1[u].y;
      a1.z += ws[u] * v1[u].z; a1.w += ws[u] * v1[u].w;
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  float* dst = out_lat + grow * DL + lane * 4;
  *(float4*)dst = make_float4(a0.x * inv, a0.y * inv, a0.z * inv, a0.w * inv);
  *(float4*)(dst + 256) = make_float4(a1.x * inv, a1.y * inv, a1.z * inv, a1.w * inv);
  if (lane == 0) {
    const float lse = wsum > 0.0f ? big + logf(wsum) : -INFINITY;
    out_lse[grow] = lse;
    if (!(fabsf(lse) < INFINITY) && status) atomicOr(status, ST_NONFINITE);
  }
}

}  // namespace

hipError_t launch_piece_merge(const VerifyParams& p, hipStream_t stream) {
  if (!p.cut) return hipSuccess;
  if (p.piece_slots <= 0 || p.piece_slots > PIECE_SLOTS) return hipErrorInvalidValue;
  if (p.cut < 1 || p.cut > CUS_PER_XCD / 2) return hipErrorInvalidValue;  // >= 2 pieces a unit
  const int xcds = p.piece_slots / CUS_PER_XCD;  // the XCDs that received work
  const int blocks = xcds * p.cut * (PIECE_ROWS / MERGE_ROWS);
  hipLaunchKernelGGL(piece_merge_kernel, dim3(blocks), dim3(256), 0, stream, p.piece_o,
                     p.piece_lse, p.piece_desc, p.out_lat, p.out_lse, p.status, p.batch,
                     p.m_tiles, (int)p.cut, p.total_q * p.num_heads);
  return hipGetLastError();
}

hipError_t launch_fill_nan(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_nan_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* part_o, const float* part_lse, float* out_lat,
                            float* out_lse, int64_t rows, int32_t num_splits, hipStream_t stream) {
  const int64_t blocks = (rows + MERGE_ROWS - 1) / MERGE_ROWS;
  if (blocks <= 0 || blocks > 0x7fffffff || num_splits < 1 || num_splits > MAX_SPLITS)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part_o,
                     part_lse, out_lat, out_lse, rows, num_splits);
  return hipGetLastError();
}

}  // namespace kdt
