// Tree-verify MLA-absorb attention, fp32 inputs, gfx950.
//
// Same operation as the bf16 kernel ("The Milestone Commit: Cementing Phase 1 ...",
// section "The Context", item 2), computed with fp32 MFMA (v_mfma_f32_16x16x4_f32) so
// that products and sums stay in fp32.  One workgroup = 4 waves = 64 query rows; each
// wave owns 16 rows with its Q fragment (16 x 576 fp32) in AGPRs, as the B operand of the
// score MFMAs, which leaves the VGPRs to the 512-wide O accumulator.  Per 16-key tile:
//   S^T = K Q^T  (16 keys x 16 rows per wave; each lane holds one query row),
//   online softmax in the log2 domain with a lazy rescale,
//   O^T += V^T P^T with V read straight from the fp32 tile (V = latent part of K).
// The tiles arrive by 16-byte global->LDS DMA into two LDS stages: the next tile's copy is
// in flight while the current tile is processed, and no VGPR stages it.
#include "common.h"

namespace kdt {
namespace {

constexpr int BM = 64;
constexpr int BN = 16;
constexpr int NTHR = 256;
constexpr float RESCALE_THRESHOLD = 8.0f;

typedef __attribute__((ext_vector_type(4))) float f32x4;

#define LDS_AS __attribute__((address_space(3)))

// LDS stage (floats): latent rows [16 keys][512 + 4 pad] (a 2064-byte stride, so each row
// is two contiguous 1 KB copies and a row's 16-byte chunk c sits in bank group
// (key + c) mod 16), then rope rows [16 keys][64] whose chunk c of key k sits at slot
// c ^ k.  Score reads (16 keys, one chunk), value reads (4 keys x 16 consecutive floats)
// and rope reads are all bank-conflict free.
constexpr int LSTRIDE = DL + 4;
constexpr int STAGE_LAT = BN * LSTRIDE;
constexpr int STAGE_FLOATS = STAGE_LAT + BN * DR;
// Output staging in the finished tile stages: 16 rows x 256 fp32 features per wave, rows
// padded by 16 bytes (conflict-free row-per-lane writes); two waves' blocks per stage.
constexpr int EPI_ROW_BYTES = 256 * 4 + 16;
constexpr int EPI_WAVE_BYTES = 16 * EPI_ROW_BYTES;
static_assert(2 * EPI_WAVE_BYTES <= STAGE_FLOATS * 4, "two output blocks per stage");
// Separate objects per stage: the compiler's wait-count insertion can then tell that a
// copy into one stage does not alias reads of the other.
__shared__ __attribute__((aligned(1024))) float sK0[STAGE_FLOATS];
__shared__ __attribute__((aligned(1024))) float sK1[STAGE_FLOATS];
__shared__ int32_t sParent32[MAX_QLEN];
__shared__ int64_t sRed32[8];
__shared__ int32_t sFlag32;

template <int STAGE> __device__ __forceinline__ float* ktile() { return STAGE ? sK1 : sK0; }

// 16-byte global -> LDS copies (64 lanes fill 1 KB at `lds`) through a buffer descriptor
// on a wave-uniform base; lane and row offsets stay below 32 KB.
__device__ __forceinline__ void dma16(const __amdgpu_buffer_rsrc_t& rsrc, float* lds,
                                      unsigned lane_off, unsigned row_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)lds, 16, (int)lane_off,
                                           (int)row_off, 0, 0);
}

// Copy tile keys [key0, key0 + 16) (clamped to key_last; both relative to the request's
// first row) into stage STAGE.  Wave w moves latent rows 4w..4w+3 (two 1 KB halves each)
// and rope rows 4w..4w+3 (one instruction): nine copies per wave.
template <int STAGE>
__device__ __forceinline__ void issue_tile(const float* kv_lat_req, const float* k_rope_req,
                                           int key0, int key_last, int wave, int lane) {
  float* kt = ktile<STAGE>();
  const __amdgpu_buffer_rsrc_t lat = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kv_lat_req + (int64_t)key0 * DL), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rope = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(k_rope_req + (int64_t)key0 * DR), (short)0, -1, 0x00020000);
  const int last = key_last - key0;  // >= 0
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int row = wave * 4 + (n >> 1), half = n & 1;
    const int src = min(row, last);
    dma16(lat, kt + row * LSTRIDE + half * 256, (unsigned)lane * 16u,
          (unsigned)(src * DL * 4 + half * 1024));
  }
  const int row = wave * 4 + (lane >> 4), slot = lane & 15;
  dma16(rope, kt + STAGE_LAT + wave * 4 * DR,
        (unsigned)(min(row, last) * DR * 4 + ((slot ^ row) & 15) * 16), 0u);
}

// K fragment kb of this lane (16 bytes: key lane & 15, floats 16 kb + 4 g .. + 3).
template <int STAGE>
__device__ __forceinline__ float4 k_frag(int kb, int key, int g) {
  const float* kt = ktile<STAGE>();
  const float* kr = kt + STAGE_LAT;
  return kb < 32 ? *(const float4*)(kt + key * LSTRIDE + 16 * kb + 4 * g)
                 : *(const float4*)(kr + key * DR + (((kb - 32) * 4 + g) ^ key) * 4);
}

template <int STAGE>
__device__ __forceinline__ f32x4 qk_tile(const float4 (&qf)[36], int lane) {
  const int key = lane & 15, g = lane >> 4;
  // Four independent accumulation chains (one per float of the 16-byte operand), summed
  // pairwise at the end: each chain adds 144 products, which keeps the fp32 rounding of
  // the 576-term score well inside the 1e-5 output bound.
  f32x4 s0 = {}, s1 = {}, s2 = {}, s3 = {};
  // K fragments are read two k-steps ahead: the MFMAs are asm statements, which the
  // compiler does not move loads across, so a fragment read just before its MFMAs would
  // wait out the whole LDS latency at every k-step.
  constexpr int KA = 2;
  float4 ka[KA + 1];
#pragma unroll
  for (int i = 0; i < KA; ++i) ka[i] = k_frag<STAGE>(i, key, g);
#pragma unroll
  for (int kb = 0; kb < 36; ++kb) {
    if (kb + KA < 36) ka[(kb + KA) % (KA + 1)] = k_frag<STAGE>(kb + KA, key, g);
    const float4 a = ka[kb % (KA + 1)];
    // Q is an AGPR operand of these MFMAs, so the register allocator keeps all 144 Q
    // values in the AGPR file for the whole loop.  Q and O together (272 values) exceed
    // the 256 VGPRs; with Q in VGPRs, O moved between the two files every tile.
    asm volatile("v_mfma_f32_16x16x4_f32 %0, %4, %8, %0\n\t"
                 "v_mfma_f32_16x16x4_f32 %1, %5, %9, %1\n\t"
                 "v_mfma_f32_16x16x4_f32 %2, %6, %10, %2\n\t"
                 "v_mfma_f32_16x16x4_f32 %3, %7, %11, %3"
                 : "+v"(s0), "+v"(s1), "+v"(s2), "+v"(s3)
                 : "v"(a.x), "v"(a.y), "v"(a.z), "v"(a.w),
                   "a"(qf[kb].x), "a"(qf[kb].y), "a"(qf[kb].z), "a"(qf[kb].w));
  }
  // wait states between the last MFMAs and VALU reads of their results
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3");
  return (s0 + s1) + (s2 + s3);
}

template <int STAGE>
__device__ __forceinline__ void pv_tile(f32x4 (&o)[32], const f32x4& pr, int lane) {
  const float* kt = ktile<STAGE>();
  const int fl = lane & 15, g = lane >> 4;
#pragma unroll
  for (int fb = 0; fb < 32; ++fb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a = kt[(4 * g + r) * LSTRIDE + fb * 16 + fl];
      o[fb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, pr[r], o[fb], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(uint64_t)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

struct RowState32 {
  float m, l;
};

__device__ __forceinline__ float row_max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ void softmax_tile(f32x4& s, f32x4 (&o)[32], RowState32& st, float c,
                                             bool masked, int tile_key0, int key_end, int prefix,
                                             int node, uint64_t anc, int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    bool vis = true;
    if (masked) {
      const int k = tile_key0 + 4 * g + r;
      vis = k < key_end;
      if (k >= prefix) {
        const int j = k - prefix;
        vis = vis && (j == node || (j < 64 && ((anc >> j) & 1ull)));
      }
    }
    s[r] = vis ? s[r] * c : -INFINITY;
  }
  float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  mx = row_max4(mx);
  const bool need = mx > st.m + RESCALE_THRESHOLD;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float mnew = need ? mx : st.m;
    const float alpha = need ? __builtin_amdgcn_exp2f(st.m - mnew) : 1.0f;
    st.m = mnew;
    st.l *= alpha;
#pragma unroll
    for (int fb = 0; fb < 32; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[fb][r] *= alpha;
  }
  const float mref = st.m == -INFINITY ? 0.0f : st.m;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s[r] = __builtin_amdgcn_exp2f(s[r] - mref);
    st.l += s[r];
  }
}

__global__ __attribute__((amdgpu_flat_work_group_size(NTHR, NTHR), amdgpu_waves_per_eu(1, 1)))
void verify_attn_f32_kernel(VerifyParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;

  // Row tiles fastest; then request-major for equal splits, split-major (every request's
  // largest split first) for geometric ones.
  int bid = blockIdx.x;
  const int mt = bid % p.m_tiles;
  bid /= p.m_tiles;
  const bool geo = p.split_ratio < 1.0f;
  const int split = geo ? bid / p.batch : bid % p.num_splits;
  const int b = geo ? bid % p.batch : bid / p.num_splits;

  int64_t qoff = 0, kvoff = 0;
  int bad = 0;
  for (int i = tid; i < b; i += NTHR) {
    const int t = p.q_len[i], pl = p.prefix_len[i];
    bad |= (t < 1 || t > p.max_q_len) ? ST_BAD_QLEN : 0;
    bad |= pl < 0 ? ST_BAD_PREFIX : 0;
    qoff += t;
    kvoff += (int64_t)pl + t;
  }
  for (int off = 32; off > 0; off >>= 1) {
    qoff += __shfl_xor(qoff, off);
    kvoff += __shfl_xor(kvoff, off);
    bad |= __shfl_xor(bad, off);
  }
  if (tid == 0) sFlag32 = 0;
  __syncthreads();
  if (lane == 0) {
    sRed32[wave] = qoff;
    sRed32[4 + wave] = kvoff;
    if (bad) atomicOr(&sFlag32, bad);
  }
  __syncthreads();
  // The same in every lane; said so explicitly, or the copies' buffer descriptors built
  // from them would be treated as per-lane and each copy run in a waterfall loop.
  qoff = uniform64(sRed32[0] + sRed32[1] + sRed32[2] + sRed32[3]);
  kvoff = uniform64(sRed32[4] + sRed32[5] + sRed32[6] + sRed32[7]);
  const int T = p.q_len[b];
  const int P = p.prefix_len[b];
  int flag = sFlag32;
  if (T < 1 || T > p.max_q_len) flag |= ST_BAD_QLEN;
  if (P < 0) flag |= ST_BAD_PREFIX;
  if (!flag && (qoff + T > p.total_q || kvoff + P + T > p.total_kv || P > MAX_REQUEST_KEYS - T))
    flag |= ST_OVERFLOW;
  if (flag) {
    if (tid == 0 && p.status) atomicOr(p.status, flag);
    return;
  }
  const int H = p.num_heads;
  const int rows = T * H;
  const int m0 = mt * BM;
  if (m0 >= rows) return;

  __syncthreads();
  if (tid == 0) sFlag32 = 0;
  __syncthreads();
  if (tid < T) {
    const int pa = p.tree_parent[qoff + tid];
    const bool ok = tid == 0 ? pa == -1 : (pa >= 0 && pa < tid);
    sParent32[tid] = ok ? pa : -1;
    if (!ok) atomicOr(&sFlag32, ST_BAD_PARENT);
  }
  __syncthreads();
  if (sFlag32) {
    if (tid == 0 && p.status) atomicOr(p.status, sFlag32);
    return;
  }

  const int row = m0 + wave * 16 + (lane & 15);
  const bool row_ok = row < rows;
  const int crow = row_ok ? row : rows - 1;
  const int node = crow / H;
  uint64_t anc = 0;
  for (int x = node, hops = 0; x >= 0 && hops <= MAX_QLEN; ++hops) {
    if (x < 64) anc |= 1ull << x;
    x = sParent32[x];
  }

  const int S = p.num_splits;
  const int k_begin = split_begin(P, S, p.split_ratio, split);
  const int k_end = (split == S - 1) ? P + T : split_begin(P, S, p.split_ratio, split + 1);
  const int64_t grow = qoff * H + crow;
  if (k_end <= k_begin) {
    if (row_ok) {
      float* po = p.part_o + ((int64_t)split * p.total_q * H + grow) * DL;
      for (int f = g * 4; f < DL; f += 16) *(float4*)(po + f) = make_float4(0.f, 0.f, 0.f, 0.f);
      if (g == 0) p.part_lse[(int64_t)split * p.total_q * H + grow] = -INFINITY;
    }
    return;
  }

  float4 qf[36];
  {
    const float* ql = (const float*)p.q_lat + grow * DL;
    const float* qr = (const float*)p.q_rope + grow * DR;
#pragma unroll
    for (int kb = 0; kb < 36; ++kb) {
      const int f = 16 * kb + 4 * g;
      qf[kb] = kb < 32 ? *(const float4*)(ql + f) : *(const float4*)(qr + f - DL);
    }
  }

  const float* kv_lat = (const float*)p.kv_lat;
  const float* k_rope = (const float*)p.k_rope;
  const int key_last = k_end - 1;
  const int n_tiles = (k_end - k_begin + BN - 1) / BN;
  const int mask_from = min(P, k_end);
  const float c = p.scale_log2;

  f32x4 o[32];
#pragma unroll
  for (int fb = 0; fb < 32; ++fb) o[fb] = f32x4{};
  RowState32 st{-INFINITY, 0.0f};

  // Tile j sits in stage j % 2; the copy of tile j+1 into the other stage (read by tile
  // j-1 before the previous barrier) is in flight while tile j is processed.
  const float* kv_lat_req = kv_lat + kvoff * DL;
  const float* k_rope_req = k_rope + kvoff * DR;
  issue_tile<0>(kv_lat_req, k_rope_req, k_begin, key_last, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; j += 2) {
    {
      const int key0 = k_begin + j * BN;
      if (j + 1 < n_tiles) issue_tile<1>(kv_lat_req, k_rope_req, key0 + BN, key_last, wave, lane);
      f32x4 s = qk_tile<0>(qf, lane);
      softmax_tile(s, o, st, c, key0 + BN > mask_from, key0, k_end, P, node, anc, lane);
      pv_tile<0>(o, s, lane);
      if (j + 1 >= n_tiles) break;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    {
      const int key0 = k_begin + (j + 1) * BN;
      if (j + 2 < n_tiles) issue_tile<0>(kv_lat_req, k_rope_req, key0 + BN, key_last, wave, lane);
      f32x4 s = qk_tile<1>(qf, lane);
      softmax_tile(s, o, st, c, key0 + BN > mask_from, key0, k_end, P, node, anc, lane);
      pv_tile<1>(o, s, lane);
      if (j + 2 >= n_tiles) break;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  float l_tot = st.l + __shfl_xor(st.l, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = 1.0f / l_tot;
  const float lse = st.m * LN2 + logf(l_tot);
  // A wave's 16 rows are consecutive global rows, so its output block is contiguous.
  const int wrow0 = m0 + wave * 16;
  const int wrows = min(16, rows - wrow0);  // rows of this wave that exist (may be <= 0)
  const int64_t gbase = qoff * H + wrow0;
  float* const out = S == 1 ? p.out_lat + gbase * DL
                            : p.part_o + ((int64_t)split * p.total_q * H + gbase) * DL;
  // Each lane holds 16-byte pieces of one row, so direct stores would touch 16 rows per
  // instruction.  Each wave passes its block through LDS (the tile stages, free once every
  // wave has finished the last tile), 256 features at a time; every store instruction then
  // writes 1 KB of one row.  No tile copy is in flight here (the last trips issue none).
  __syncthreads();
  if (wrows > 0) {
    LDS_AS char* stage =
        (LDS_AS char*)(LDS_AS void*)((wave < 2) ? sK0 : sK1) + (wave & 1) * EPI_WAVE_BYTES;
    const int r = lane & 15;
#pragma unroll
    for (int chunk = 0; chunk < 2; ++chunk) {
#pragma unroll
      for (int f = 0; f < 16; ++f) {
        const f32x4 a = o[chunk * 16 + f];
        *(LDS_AS f32x4*)(stage + r * EPI_ROW_BYTES + (f * 16 + g * 4) * 4) =
            f32x4{a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv};
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      f32x4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = *(const LDS_AS f32x4*)(stage + i * EPI_ROW_BYTES + lane * 16);
      float* dst = out + chunk * 256 + lane * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < wrows) *(f32x4*)(dst + (int64_t)i * DL) = v[i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  if (row_ok && g == 0) {
    if (S == 1)
      p.out_lse[grow] = lse;
    else
      p.part_lse[(int64_t)split * p.total_q * H + grow] = lse;
    if (!(fabsf(lse) < INFINITY) && p.status) atomicOr(p.status, ST_NONFINITE);
  }
}

}  // namespace

int rows_per_block_f32() { return BM; }

hipError_t launch_verify_f32(const VerifyParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.m_tiles * p.num_splits * p.batch;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(verify_attn_f32_kernel, dim3((unsigned)blocks), dim3(NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kdt
