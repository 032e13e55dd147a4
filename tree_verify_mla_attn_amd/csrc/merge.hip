// LSE merge of split-KV partial results ("The Milestone Commit: Cementing Phase 1 ...",
// section "What to defer": flash partial outputs merged for long prefixes).
//
// For each query row, split s holds a normalised partial output O_s (512 fp32) and its
// log-sum-exp lse_s (-inf when the split saw no key).  With L = max_s lse_s and
// w_s = exp(lse_s - L):  out = sum_s w_s O_s / sum_s w_s,  lse = L + ln sum_s w_s.
// HBM-bound: one pass over the partials; 128 threads per row, float4 per thread.
#include "common.h"

namespace kdt {
namespace {

constexpr int ROWS_PER_BLOCK = 2;

__global__ __launch_bounds__(256) void lse_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_lse,
                                                        float* __restrict__ out_lat,
                                                        float* __restrict__ out_lse, int64_t rows,
                                                        int num_splits) {
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 7);
  const int t = threadIdx.x & 127;
  if (row >= rows) return;
  float big = -INFINITY;
  for (int s = 0; s < num_splits; ++s) big = fmaxf(big, part_lse[(int64_t)s * rows + row]);
  const float bref = big == -INFINITY ? 0.0f : big;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.0f;
  for (int s = 0; s < num_splits; ++s) {
    const float ls = part_lse[(int64_t)s * rows + row];
    const float w = ls == -INFINITY ? 0.0f : __expf(ls - bref);
    wsum += w;
    if (w != 0.0f) {
      const float4 v = *(const float4*)(part_o + ((int64_t)s * rows + row) * DL + t * 4);
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  *(float4*)(out_lat + row * DL + t * 4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (t == 0) out_lse[row] = wsum > 0.0f ? big + logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_lse_merge(const float* part_o, const float* part_lse, float* out_lat,
                            float* out_lse, int64_t rows, int32_t num_splits, hipStream_t stream) {
  const int64_t blocks = (rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part_o,
                     part_lse, out_lat, out_lse, rows, num_splits);
  return hipGetLastError();
}

}  // namespace kdt
