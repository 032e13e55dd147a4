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

}  // namespace

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
