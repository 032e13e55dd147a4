// The target model's next token at every tree node, drawn at temperature T: the input of
// the accept walk on the temperature path ("The Milestone Commit: Cementing Phase 1 ...",
// sections "Why This Message Was Written" and "How Decisions Were Made": a sampling path
// of the accept step, named but not given).  The tree's candidates are the drafter's
// top-k, chosen rather than sampled, so the lossless accept draws the target's token at a
// node and follows the child that carries it; this kernel does the draws, the walk is
// the greedy accept kernel.
//
// Draw of row r (T > 0): entry i gets u_i in (0, 1) from Philox4x64-10 (Salmon et al.,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) with counter (i / 8, r, 0, 0)
// and key (seed, offset): word (i / 2) % 4 of the block, its low 32 bits for even i and
// high 32 bits for odd i, x32 -> (2 (x32 >> 9) + 1) 2^-24.  Then, rounding each step in
// float32, z_i = logit_i * (log2(e) / T) - L(-L(u_i)), with L the float32 base-2
// logarithm log2_seq below (a fixed sequence of rounded operations, so the draws are
// reproducible bit for bit on the host), and the token is the argmax of z, lowest index
// on ties.  z is log2(e) times the Gumbel-max key logit / T - ln(-ln u)
// less a constant, so token ~ softmax(logit / T).  T = 0: argmax of the logits.  A row
// whose logits are all -inf yields -1.
//
// One workgroup per row streams the row once; a thread takes 8 consecutive entries per
// step (one generator block), so every step of the workgroup reads a contiguous 8 KB
// (fp32) or 4 KB (bf16).  The generator dominates on flat logits; on peaked ones the
// blocks that cannot hold the winner skip it (exact pruning, below).
#include "common.h"

namespace kdt {
namespace {

constexpr int SAMPLE_THREADS = 256;

// The 128-bit product a * m as (lo, hi) from four 32 x 32 -> 64 multiply-adds:
// x = a0 m0, y = a1 m0 + x1, z = a0 m1 + y (65 bits: z + 2^64 c), so that
// a*m = x0 + 2^32 z0 + 2^64 (a1 m1 + z1 + 2^32 c).  The carry c comes from the
// multiply-add's own carry-out mask, which saves the zero-extended register pair (two
// moves) and the add with carry that the compiler builds for an explicit 65-bit sum; a
// VALU write of a lane mask takes two wait states before a VALU reads it as a select.
__device__ __forceinline__ void mul_wide(uint64_t a, uint32_t m0, uint32_t m1, uint64_t& lo,
                                         uint64_t& hi) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
  const uint64_t x = (uint64_t)a0 * m0;
  const uint64_t y = (uint64_t)a1 * m0 + (x >> 32);
  uint64_t z;
  uint32_t c;
  uint64_t cm;
  asm("v_mad_u64_u32 %0, %1, %3, %4, %5\n\t"
      "s_nop 1\n\t"
      "v_cndmask_b32_e64 %2, 0, 1, %1"
      : "=&v"(z), "=&s"(cm), "=v"(c)
      : "v"(a0), "s"(m1), "v"(y));
  hi = (uint64_t)a1 * m1 + (((uint64_t)c << 32) | (z >> 32));
  lo = (uint32_t)x | (z << 32);
}

// a ^ b ^ c in one instruction (gfx950 three-input bit operation, truth table 0x96)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(c));
  return r;
}

__device__ __forceinline__ uint64_t xor3_64(uint64_t a, uint64_t b, uint64_t c) {
  return (uint64_t)xor3((uint32_t)a, (uint32_t)b, (uint32_t)c) |
         ((uint64_t)xor3((uint32_t)(a >> 32), (uint32_t)(b >> 32), (uint32_t)(c >> 32)) << 32);
}

__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint32_t M0L = 0xE14C6C93u, M0H = 0xD2E7470Eu;
  constexpr uint32_t M1L = 0x95121157u, M1H = 0xCA5A8263u;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    uint64_t lo0, hi0, lo1, hi1;
    mul_wide(c[0], M0L, M0H, lo0, hi0);
    mul_wide(c[2], M1L, M1H, lo1, hi1);
    const uint64_t n0 = xor3_64(hi1, c[1], k0), n2 = xor3_64(hi0, c[3], k1);
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
  return __uint_as_float((unsigned)b << 16);
}

// 8 logits starting at entry i0 (entries at or past `vocab` read as -inf).
template <bool BF16, bool VEC>
__device__ __forceinline__ void load8(const void* row, int64_t i0, int vocab, float (&x)[8]) {
  if (VEC && i0 + 8 <= vocab) {
    if constexpr (BF16) {
      const uint4 v = *(const uint4*)((const unsigned short*)row + i0);
      const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(w[k] << 16);
        x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    } else {
      const float4 a = *(const float4*)((const float*)row + i0);
      const float4 b = *(const float4*)((const float*)row + i0 + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t i = i0 + k;
    if (i < vocab)
      x[k] = BF16 ? bf16_to_f32(((const unsigned short*)row)[i]) : ((const float*)row)[i];
    else
      x[k] = -INFINITY;
  }
}

// a * b - g with both operations rounded (never fused into one fma)
__device__ __forceinline__ float mul_sub_rounded(float a, float b, float g) {
#pragma clang fp contract(off)
  const float ab = a * b;
  return ab - g;
}

template <int CTRL>
__device__ __forceinline__ float dpp_max_step(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf,
                                                             false)));
}

// Largest value over the wavefront (no NaN).
__device__ __forceinline__ float wave_max_f(float v) {
  v = dpp_max_step<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141>(v);  // row_half_mirror
  v = dpp_max_step<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The uniform of a 32-bit generator word: (2 (x32 >> 9) + 1) 2^-24, formed as
// (1 + (x32 >> 9) 2^-23) - (1 - 2^-24), where the first operand is the bits
// 0x3f800000 | (x32 >> 9) and the subtraction is exact (Sterbenz).
__device__ __forceinline__ float uniform_of(unsigned x32) {
  return __uint_as_float(__builtin_amdgcn_alignbit(0x7fu, x32, 9)) - 0x1.fffffep-1f;
}

// Base-2 logarithm of a positive normal float as a fixed sequence of float32 operations,
// each rounded to nearest, none fused, so that any other evaluation of the same sequence
// (the host's) gets the same bits:
//   x = 2^e m, m in [1, 2) from the bits; if m > sqrt(2): m = m / 2, e = e + 1 (exact);
//   f = m - 1 (exact), s = f / (2 + f) (correctly rounded division), z = s s;
//   p = (((A4 z + A3) z + A2) z + A1) z + A0, with A_k = 2 / ((2k + 1) ln 2) in float32;
//   log2 x = e + s p.
// This is the classical series ln z = 2 (s + s^3/3 + s^5/5 + ...), s = (z-1)/(z+1), in
// base 2.  |s| <= 0.172 keeps the truncation after s^9 below 2e-9 relative; the result is
// within a few ulp of log2 x (relative near x = 1, where f is exact), and exact at powers
// of two.
__device__ __forceinline__ float log2_seq(float x) {
#pragma clang fp contract(off)
  constexpr float A0 = 0x1.715476p+1f, A1 = 0x1.ec709ep-1f, A2 = 0x1.2776c6p-1f,
                  A3 = 0x1.a61762p-2f, A4 = 0x1.484b14p-2f;
  const unsigned bits = __float_as_uint(x);
  int e = (int)((bits >> 23) & 0xffu) - 127;
  unsigned mb = (bits & 0x7fffffu) | 0x3f800000u;
  if (mb > 0x3fb504f3u) {  // m > sqrt(2) (float32 sqrt(2) rounds down)
    mb -= 0x00800000u;
    e += 1;
  }
  const float f = __uint_as_float(mb) - 1.0f;
  const float s = f / (2.0f + f);  // correctly rounded: HIP's default float division
  const float z = s * s;
  float p = A4 * z + A3;
  p = p * z + A2;
  p = p * z + A1;
  p = p * z + A0;
  return (float)e + s * p;
}

// log2(-log2(u)) for u in [2^-24, 1 - 2^-24]: both arguments are normal numbers.  It falls
// as u rises, up to the few-ulp rounding of the two logarithms.
__device__ __forceinline__ float gumbel_log2(float u) { return log2_seq(-log2_seq(u)); }

// The same with the hardware base-2 logarithm (v_log_f32, within about an ulp), for the
// pruning bound only: it never enters a key.
__device__ __forceinline__ float gumbel_log2_hw(float u) {
  return __builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));
}

__device__ __forceinline__ float mul_rounded(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// Whether a key RN(RN(x cs) - gumbel_log2(u)) can reach `best`, given sx >= RN(x cs) and
// gh = gumbel_log2_hw(u') with u' >= u (u' = u for one entry, the block's largest
// uniform for a block; the exact log2(-log2 u) falls as u rises).  False only when every
// such key is strictly below `best`.  The margin covers, with a factor of two to spare,
// the error of gumbel_log2 against the exact value (its inner logarithm within 3.6e-7
// relative, which moves the outer one by at most 5.2e-7, plus 3 ulp of the result; the
// bound is pinned over every uniform the draw can produce), the error of gumbel_log2_hw
// (2 ulp each way assumed: 3.5e-7 plus 2 ulp), and the rounding of the key's subtraction
// and of this expression: in all, less than 8.7e-7 + 2^-20 |gh| + 2^-22 |sx|.
__device__ __forceinline__ bool could_reach(float sx, float gh, float best) {
  return sx - gh + (fabsf(sx) + fabsf(gh)) * 0x1p-19f + 0x1p-19f >= best;
}

// u <= 1 - 2^-24 gives -log2(-log2 u) <= 23.47, so no key exceeds its scaled logit by more
// than this (plus a relative margin for the rounding of large scaled logits).
constexpr float KEY_HEADROOM = 24.0f;

// (value, index) of the larger; equal values -> lower index; index -1 = nothing yet.
__device__ __forceinline__ void keep_best(float& bz, int& bi, float z, int i) {
  if (i < 0) return;
  if (bi < 0 || z > bz || (z == bz && i < bi)) {
    bz = z;
    bi = i;
  }
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(SAMPLE_THREADS) void sample_tokens_kernel(SampleParams p) {
  __shared__ float s_z[SAMPLE_THREADS / 64];
  __shared__ int s_i[SAMPLE_THREADS / 64];
  __shared__ float s_bound;  // a key some lane of the workgroup has reached
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int vocab = p.vocab;
  const void* row = (const char*)p.logits + r * p.row_stride * (BF16 ? 2 : 4);
  float bz = -INFINITY;
  int bi = -1;
  const bool greedy = p.temperature == 0.0f;
  if (tid == 0) s_bound = -INFINITY;
  __syncthreads();
  const float cs = greedy ? 1.0f : __fdiv_rn(1.4426950408889634f, p.temperature);
  // Lower bound of the winning key: the largest key the lanes of the workgroup have seen,
  // shared through one LDS word without synchronisation (every value written is some
  // lane's key, so a stale or overwritten value is still a lower bound).  A block of 8
  // entries whose largest scaled logit plus the headroom is below it cannot hold the
  // winner (its keys are strictly smaller), so its generator block and logarithms are
  // skipped.  A second test after the generator, with the block's largest uniform, skips
  // the logarithms of most blocks that pass the first.  Neither changes the result.
  // The trip count is uniform per wavefront (all lanes take part in the wave maximum);
  // entries past the vocabulary read as -inf.
  float wave_best = -INFINITY;
  const int64_t n_blocks = ((int64_t)vocab + 7) / 8;
  int step = 0;
  for (int64_t g = tid; g - (tid & 63) < n_blocks; g += SAMPLE_THREADS, ++step) {
    float x[8];
    load8<BF16, VEC>(row, g * 8, vocab, x);
    if (greedy) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (x[k] > bz) {  // entries rise within a thread: strict keeps the lowest index
          bz = x[k];
          bi = (int)(g * 8 + k);
        }
      continue;
    }
    // A stale bound is still a bound: it is refreshed every step at first, while it is
    // far below the winner (the first step prunes nothing), then every eighth step.
    if (step < 8 || (step & 7) == 0) {
      wave_best = fmaxf(wave_max_f(bz), s_bound);
      if ((tid & 63) == 0 && wave_best > s_bound) s_bound = wave_best;
    }
    const float best = fmaxf(bz, wave_best);
    const float xm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                           fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    const float sm = xm * cs;
    // skip unless some key of the block could reach the bound (an all -inf block gives
    // NaN here and is skipped; the bound starts at -inf, which never skips)
    if (!(sm + KEY_HEADROOM + fabsf(sm) * 0x1p-20f >= best)) continue;
    uint64_t c[4] = {(uint64_t)g, (uint64_t)r, 0ull, 0ull};
    philox4x64_10(c, p.seed, p.offset);
    unsigned w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = (unsigned)(c[k >> 1] >> (32 * (k & 1)));
    // Second test, with the block's own uniforms: u rises with its word, so with u_max
    // the uniform of the largest word every key of the block is at most sm - g(u_max)
    // plus rounding (could_reach).  A skipped block holds only keys strictly below the
    // bound, and the draw is the same as without the test.
    const unsigned wmax = max(max(max(w[0], w[1]), max(w[2], w[3])),
                              max(max(w[4], w[5]), max(w[6], w[7])));
    const float gmin = gumbel_log2_hw(uniform_of(wmax));
    if (!could_reach(sm, gmin, best)) continue;
    // The same test per entry, with its own uniform (no monotonicity step needed): only
    // entries that could reach the bound get the exact key, whose two fixed-sequence
    // logarithms cost about ten times the hardware ones.
    unsigned need = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      need |= could_reach(mul_rounded(x[k], cs), gumbel_log2_hw(uniform_of(w[k])), best) ? 1u << k
                                                                                     : 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (!(need & (1u << k))) continue;
      const float z = mul_sub_rounded(x[k], cs, gumbel_log2(uniform_of(w[k])));
      if (z > bz) {
        bz = z;
        bi = (int)(g * 8 + k);
      }
    }
  }
  // -inf entries never win (bz starts at -inf, comparisons are strict)
  for (int off = 32; off > 0; off >>= 1) {
    const float oz = __shfl_xor(bz, off);
    const int oi = __shfl_xor(bi, off);
    keep_best(bz, bi, oz, oi);
  }
  if ((tid & 63) == 0) {
    s_z[tid >> 6] = bz;
    s_i[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < SAMPLE_THREADS / 64; ++w) keep_best(bz, bi, s_z[w], s_i[w]);
    p.tokens[r] = bi;
  }
}

}  // namespace

hipError_t launch_sample_tokens(const SampleParams& p, bool bf16, hipStream_t stream) {
  const size_t esize = bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)p.logits % 16 == 0) && ((p.row_stride * esize) % 16 == 0);
  const dim3 grid((unsigned)p.rows), block(SAMPLE_THREADS);
  if (bf16) {
    if (vec) hipLaunchKernelGGL((sample_tokens_kernel<true, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((sample_tokens_kernel<true, false>), grid, block, 0, stream, p);
  } else {
    if (vec) hipLaunchKernelGGL((sample_tokens_kernel<false, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((sample_tokens_kernel<false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace kdt
