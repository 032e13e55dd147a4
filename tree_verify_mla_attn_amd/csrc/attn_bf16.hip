// Tree-verify MLA-absorb attention, bf16 inputs, gfx950.
//
// Operation ("The Milestone Commit: Cementing Phase 1 ...", section "The Context",
// item 2; "Strategic Pivots in CUDA Kernel Engineering ...", section "The Message"):
// each draft-tree node x head is a query row in the absorbed latent space; it attends
// over the request's prefix + tree tail (ancestor-or-self visibility in the tail) and
// yields a 512-dim latent output and the row's log-sum-exp.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one request and one
// KV split).  Rows are packed node-major, head-minor, so all heads of a node share its
// ancestor mask and all 128 rows share every KV tile.  Each wave owns 32 rows:
//   * Q fragment (32 rows x 576, bf16) lives in VGPRs for the whole KV loop;
//   * S^T = K Q^T per 32-key tile: bf16 MFMA 32x32x16, so each lane holds one query
//     row and the softmax row reductions are in-register plus one lane swap;
//   * online softmax in the log2 domain with a lazy rescale (the running max is only
//     raised when a tile beats it by more than 2^8);
//   * O^T += V^T P^T: fp16 MFMA 32x32x16 with P in fp16 (bf16 P is too coarse for a
//     2e-3 relative bound) against an fp16, feature-major copy of the latent tile.
// KV tiles (32 keys x 576 bf16) and the matching fp16 V^T tiles (converted once per
// call by the pre-pass) arrive by 16-byte global->LDS DMA into double-buffered LDS.
#include "common.h"

namespace kdt {
namespace {

constexpr int BM = 128;     // query rows per workgroup
constexpr int BN = 32;      // keys per tile
constexpr int NTHR = 256;   // 4 waves
constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

#define LDS_AS __attribute__((address_space(3)))

// LDS tiles, two stages, one buffer.  Per stage (u32x4 = 16 B units):
//   K latent [32 keys][64 chunks + 1 pad]: chunk c of key k at slot k*65 + c (the pad
//            staggers rows across banks and keeps every k-step a constant offset);
//   K rope   [32 keys][8 chunks]:  chunk c of key k at slot k*8 + (c ^ rswz(k));
//   V^T fp16 [512 features][4 chunks of 8 keys]: chunk q of feature f at
//            vt_slot(f, q) = f*4 + (q ^ ((f >> 2) & 3)) -- the pre-pass's tile image; the
//            swizzle keeps the PV reads (32 consecutive features) bank-conflict free.
constexpr int KLAT_ROW = 65;
constexpr int KLAT_U4 = BN * KLAT_ROW, KROPE_U4 = BN * 8, VT_U4 = DL * 4;
// Separate objects per stage: the compiler's wait-count insertion can then tell that a
// DMA into one stage does not alias LDS reads of the other, and does not stall the
// compute of tile j on the in-flight copy of tile j+2.
__shared__ __attribute__((aligned(1024))) u32x4 sKlat0[KLAT_U4];
__shared__ __attribute__((aligned(1024))) u32x4 sKlat1[KLAT_U4];
__shared__ __attribute__((aligned(1024))) u32x4 sKrope0[KROPE_U4];
__shared__ __attribute__((aligned(1024))) u32x4 sKrope1[KROPE_U4];
__shared__ __attribute__((aligned(1024))) u32x4 sVt0[VT_U4];
__shared__ __attribute__((aligned(1024))) u32x4 sVt1[VT_U4];
__shared__ int32_t sParent[MAX_QLEN];
__shared__ int64_t sRed[3 * 4];
__shared__ int32_t sFlag;

__device__ __forceinline__ int rswz(int k) { return (k ^ (k >> 3)) & 7; }
__device__ __forceinline__ int vt_slot(int f, int q) { return f * 4 + (q ^ ((f >> 2) & 3)); }

template <int STAGE> __device__ __forceinline__ u32x4* klat() { return STAGE ? sKlat1 : sKlat0; }
template <int STAGE> __device__ __forceinline__ u32x4* krope() { return STAGE ? sKrope1 : sKrope0; }
template <int STAGE> __device__ __forceinline__ u32x4* vt() { return STAGE ? sVt1 : sVt0; }

__device__ __forceinline__ void dma16(const char* uniform_base, unsigned lane_off, u32x4* lds_base) {
  __builtin_amdgcn_global_load_lds((const void*)(uniform_base + lane_off), (LDS_AS void*)lds_base, 16,
                                   0, 0);
}

// Issue the DMA of keys [key0, key0+32) of this request (rows clamped to key_last) into
// a stage.  Wave w moves latent rows 8w..8w+7 (one contiguous 1 KB row per instruction)
// and rope rows 8w..8w+7 (one instruction).  Row pointers are wave-uniform; lanes only
// add a 32-bit offset.
template <int STAGE>
__device__ __forceinline__ void issue_tile(const char* kv_lat_req, const char* k_rope_req,
                                           int key0, int key_last, int wave, int lane) {
  u32x4* kl = klat<STAGE>();
  u32x4* kr = krope<STAGE>();
  // Re-materialise the lane id here so the per-lane offsets are recomputed per tile
  // instead of being hoisted out of the KV loop as eight long-lived registers.
  asm volatile("" : "+v"(lane));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int key = wave * 8 + i;
    const int k = __builtin_amdgcn_readfirstlane(min(key0 + key, key_last));
    dma16(kv_lat_req + (int64_t)k * (DL * 2), (unsigned)lane * 16u, kl + key * KLAT_ROW);
  }
  {
    const int key = wave * 8 + (lane >> 3);
    const int k = min(key0 + key, key_last);
    const unsigned off = (unsigned)k * (DR * 2) + (unsigned)((lane & 7) ^ rswz(key)) * 16u;
    dma16(k_rope_req, off, kr + wave * 64);
  }
}

// DMA of the pre-converted V^T tile `tile` into a stage (wave w moves 1 KB blocks
// 8w..8w+7 of the 32 KB tile image).
template <int STAGE>
__device__ __forceinline__ void issue_vt(const char* vt_req, int tile, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = wave * 8 + i;
    dma16(vt_req + (int64_t)tile * VT_TILE_BYTES + blk * 1024, (unsigned)lane * 16u,
          vt<STAGE>() + blk * 64);
  }
}

// S^T (32 keys x 32 rows of this wave) for the tile in a stage.  K fragments are read
// four MFMAs ahead of use.
template <int STAGE>
__device__ __forceinline__ f32x16 qk_tile(const u32x4 (&qf)[36], int lane) {
  const u32x4* kl = klat<STAGE>();
  const u32x4* kr = krope<STAGE>();
  const int key = lane & 31, h = lane >> 5;
  auto frag = [&](int ks) -> u32x4 {
    const int c = 2 * ks + h;
    return ks < 32 ? kl[key * KLAT_ROW + c] : kr[key * 8 + ((c - 64) ^ rswz(key))];
  };
  u32x4 a[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = frag(i);
  f32x16 s = {};
#pragma unroll
  for (int ks = 0; ks < 36; ++ks) {
    if (ks + 4 < 36) a[(ks + 4) & 7] = frag(ks + 4);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[ks & 7]),
                                                __builtin_bit_cast(bf16x8, qf[ks]), s, 0, 0, 0);
  }
  return s;
}

// Scores of the next tile fused with the copies that must be in flight meanwhile: the
// K tile j+2 into stage SC and the V^T tile j+1 into stage SN.  One 1 KB DMA is
// spliced after every two score MFMAs, so the copy engine's queue drains in the shadow
// of the matrix pipe instead of stalling the wave in one burst.
template <int SC, int SN>
__device__ __forceinline__ f32x16 qk_dma(const u32x4 (&qf)[36], int lane, const char* kv_lat_req,
                                         const char* k_rope_req, const char* vt_req, int k_key0,
                                         int key_last, int vt_tile, int wave) {
  const u32x4* kl = klat<SN>();
  const u32x4* kr = krope<SN>();
  const int key = lane & 31, h = lane >> 5;
  auto frag = [&](int ks) -> u32x4 {
    const int c = 2 * ks + h;
    return ks < 32 ? kl[key * KLAT_ROW + c] : kr[key * 8 + ((c - 64) ^ rswz(key))];
  };
  u32x4 a[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = frag(i);
  f32x16 s = {};
  int dl = lane;
  asm volatile("" : "+v"(dl));  // per-tile lane offsets, not hoisted out of the KV loop
  auto dma = [&](int n) {
    if (n < 8) {          // K latent row wave*8 + n
      const int kk = wave * 8 + n;
      const int k = __builtin_amdgcn_readfirstlane(min(k_key0 + kk, key_last));
      dma16(kv_lat_req + (int64_t)k * (DL * 2), (unsigned)dl * 16u, klat<SC>() + kk * KLAT_ROW);
    } else if (n == 8) {  // K rope rows wave*8 .. +7
      const int kk = wave * 8 + (dl >> 3);
      const int k = min(k_key0 + kk, key_last);
      dma16(k_rope_req, (unsigned)k * (DR * 2) + (unsigned)((dl & 7) ^ rswz(kk)) * 16u,
            krope<SC>() + wave * 64);
    } else {              // V^T tile: 1 KB blocks wave*8 + (n - 9)
      const int blk = wave * 8 + (n - 9);
      dma16(vt_req + (int64_t)vt_tile * VT_TILE_BYTES + blk * 1024, (unsigned)dl * 16u,
            vt<SN>() + blk * 64);
    }
  };
#pragma unroll
  for (int ks = 0; ks < 36; ++ks) {
    if (ks + 4 < 36) a[(ks + 4) & 7] = frag(ks + 4);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[ks & 7]),
                                                __builtin_bit_cast(bf16x8, qf[ks]), s, 0, 0, 0);
    if ((ks & 1) && (ks >> 1) < 17) dma(ks >> 1);
  }
  return s;
}

// O^T += V^T P^T for one 32-key tile: 16 feature blocks x 2 key steps of fp16 MFMA
// 32x32x16.  Written as one asm block so that the 16 output accumulators stay in the
// AGPR file (256 registers) across the KV loop while Q, S and P use VGPRs.  V^T
// fragments stream through eight rotating VGPR buffers, each LDS read issued four
// MFMAs ahead of its use; LDS reads return in order, so lgkmcnt(n) proves the oldest
// of this block's reads has landed.  The leading s_nop covers VALU writes of P / O
// (softmax, rescale) feeding the first MFMA; the trailing ones cover MFMA results
// read by VALU code after the block.
template <int STAGE>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[16], const f16x8 (&pk)[2], int lane) {
  const int fl = lane & 31, h = lane >> 5;
  // feature 32*fb + fl lives at byte vt_slot(fl, .)*16 + fb*2048
  const unsigned base = (unsigned)(size_t)(LDS_AS void*)vt<STAGE>();
  const unsigned v0 = base + (unsigned)(vt_slot(fl, 0 + h) * 16);
  const unsigned v1 = base + (unsigned)(vt_slot(fl, 2 + h) * 16);
  u32x4 t0, t1, t2, t3, t4, t5, t6, t7;
  asm volatile(
      "s_nop 4\n"
      "ds_read_b128 %[a0], %[v0] offset:0\n"
      "ds_read_b128 %[a1], %[v1] offset:0\n"
      "ds_read_b128 %[a2], %[v0] offset:2048\n"
      "ds_read_b128 %[a3], %[v1] offset:2048\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o0], %[a0], %[p0], %[o0]\n"
      "ds_read_b128 %[a4], %[v0] offset:4096\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o0], %[a1], %[p1], %[o0]\n"
      "ds_read_b128 %[a5], %[v1] offset:4096\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o1], %[a2], %[p0], %[o1]\n"
      "ds_read_b128 %[a6], %[v0] offset:6144\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o1], %[a3], %[p1], %[o1]\n"
      "ds_read_b128 %[a7], %[v1] offset:6144\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o2], %[a4], %[p0], %[o2]\n"
      "ds_read_b128 %[a0], %[v0] offset:8192\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o2], %[a5], %[p1], %[o2]\n"
      "ds_read_b128 %[a1], %[v1] offset:8192\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o3], %[a6], %[p0], %[o3]\n"
      "ds_read_b128 %[a2], %[v0] offset:10240\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o3], %[a7], %[p1], %[o3]\n"
      "ds_read_b128 %[a3], %[v1] offset:10240\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o4], %[a0], %[p0], %[o4]\n"
      "ds_read_b128 %[a4], %[v0] offset:12288\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o4], %[a1], %[p1], %[o4]\n"
      "ds_read_b128 %[a5], %[v1] offset:12288\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o5], %[a2], %[p0], %[o5]\n"
      "ds_read_b128 %[a6], %[v0] offset:14336\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o5], %[a3], %[p1], %[o5]\n"
      "ds_read_b128 %[a7], %[v1] offset:14336\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o6], %[a4], %[p0], %[o6]\n"
      "ds_read_b128 %[a0], %[v0] offset:16384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o6], %[a5], %[p1], %[o6]\n"
      "ds_read_b128 %[a1], %[v1] offset:16384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o7], %[a6], %[p0], %[o7]\n"
      "ds_read_b128 %[a2], %[v0] offset:18432\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o7], %[a7], %[p1], %[o7]\n"
      "ds_read_b128 %[a3], %[v1] offset:18432\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o8], %[a0], %[p0], %[o8]\n"
      "ds_read_b128 %[a4], %[v0] offset:20480\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o8], %[a1], %[p1], %[o8]\n"
      "ds_read_b128 %[a5], %[v1] offset:20480\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o9], %[a2], %[p0], %[o9]\n"
      "ds_read_b128 %[a6], %[v0] offset:22528\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o9], %[a3], %[p1], %[o9]\n"
      "ds_read_b128 %[a7], %[v1] offset:22528\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o10], %[a4], %[p0], %[o10]\n"
      "ds_read_b128 %[a0], %[v0] offset:24576\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o10], %[a5], %[p1], %[o10]\n"
      "ds_read_b128 %[a1], %[v1] offset:24576\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o11], %[a6], %[p0], %[o11]\n"
      "ds_read_b128 %[a2], %[v0] offset:26624\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o11], %[a7], %[p1], %[o11]\n"
      "ds_read_b128 %[a3], %[v1] offset:26624\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o12], %[a0], %[p0], %[o12]\n"
      "ds_read_b128 %[a4], %[v0] offset:28672\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o12], %[a1], %[p1], %[o12]\n"
      "ds_read_b128 %[a5], %[v1] offset:28672\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o13], %[a2], %[p0], %[o13]\n"
      "ds_read_b128 %[a6], %[v0] offset:30720\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o13], %[a3], %[p1], %[o13]\n"
      "ds_read_b128 %[a7], %[v1] offset:30720\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %[o14], %[a4], %[p0], %[o14]\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_32x32x16_f16 %[o14], %[a5], %[p1], %[o14]\n"
      "s_waitcnt lgkmcnt(1)\n"
      "v_mfma_f32_32x32x16_f16 %[o15], %[a6], %[p0], %[o15]\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_32x32x16_f16 %[o15], %[a7], %[p1], %[o15]\n"
      "s_nop 7\n s_nop 7\n s_nop 3\n"
      : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]), [o4] "+a"(o[4]),
        [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]), [o8] "+a"(o[8]), [o9] "+a"(o[9]),
        [o10] "+a"(o[10]), [o11] "+a"(o[11]), [o12] "+a"(o[12]), [o13] "+a"(o[13]),
        [o14] "+a"(o[14]), [o15] "+a"(o[15]), [a0] "=&v"(t0), [a1] "=&v"(t1), [a2] "=&v"(t2),
        [a3] "=&v"(t3), [a4] "=&v"(t4), [a5] "=&v"(t5), [a6] "=&v"(t6), [a7] "=&v"(t7)
      : [v0] "v"(v0), [v1] "v"(v1), [p0] "v"(pk[0]), [p1] "v"(pk[1])
      : "memory");
}

// max / sum of x over the lane pair (l, l ^ 32) that shares a query row, without an
// LDS round trip: v_permlane32_swap exchanges the upper half of one copy with the lower
// half of the other, so every lane ends up with both values of its pair.
__device__ __forceinline__ float pair_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// The output accumulators live in AGPRs for the whole kernel.  Any VALU arithmetic on
// them goes through an explicit copy to fresh VGPRs (the empty asm makes the copy a
// distinct value), so the register allocator never gives the accumulators themselves a
// VGPR home.
__device__ __forceinline__ f32x16 read_acc(const f32x16& acc) {
  f32x16 t = acc;
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ f32x16 scale_acc(const f32x16& acc, float alpha) {
  f32x16 t = read_acc(acc) * alpha;
  asm volatile("" : "+a"(t));
  return t;
}

// A value known to be equal in every lane, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(uint64_t)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

struct RowState {
  float m;      // running max (log2 units, scale folded in)
  float l;      // this lane's partial sum of fp16-rounded probabilities
  float alpha;  // factor O must be scaled by before this tile's PV (1 = none)
  bool rescale; // some row of the wave needs the O rescale
};

// Visibility of keys [key0, key0 + 32) for this lane's row as a bit mask (bit kt set =
// key key0 + kt visible): keys outside [key_begin, key_end) are out of range; prefix keys are
// visible; tail key P + j is visible iff node j is an ancestor-or-self of the row's
// node ("Strategic Pivots ...", section "The Message": tree visibility mask).  `anc`
// holds bits 0..63 of the ancestor-or-self set; node 64 can only be its own ancestor.
__device__ __forceinline__ uint32_t tile_visibility(int key0, int key_begin, int key_end,
                                                    int prefix, int node, uint64_t anc) {
  uint32_t vis = 0xffffffffu;
  const int nvalid = key_end - key0;
  if (nvalid < 32) vis = nvalid <= 0 ? 0u : (0xffffffffu >> (32 - nvalid));
  const int nskip = key_begin - key0;  // keys before this split's range
  if (nskip > 0) vis &= nskip >= 32 ? 0u : (0xffffffffu << nskip);
  const int t0 = prefix - key0;  // tile index of tail node 0
  if (t0 < 32) {
    const uint32_t tail_pos = t0 <= 0 ? 0xffffffffu : (0xffffffffu << t0);
    uint32_t anc_bits = t0 >= 0 ? (uint32_t)(anc << t0) : (-t0 >= 64 ? 0u : (uint32_t)(anc >> -t0));
    const int self64 = t0 + 64;
    if (node == 64 && self64 >= 0 && self64 < 32) anc_bits |= 1u << self64;
    vis &= ~tail_pos | anc_bits;
  }
  return vis;
}

// Online softmax of one tile: S^T (raw scores, register r <-> key 8(r/4) + 4h + r%4)
// -> P (fp16) and the running max / sum.  `vis` = visibility bits (see above).
__device__ __forceinline__ void softmax_tile(f32x16& s, f16x8 (&pk)[2], RowState& st, float c,
                                             bool masked, uint32_t vis, int lane) {
  const int h = lane >> 5;
  if (masked) {
    const uint32_t vh = vis >> (4 * h);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      s[r] = ((vh >> (8 * (r >> 2) + (r & 3))) & 1u) ? s[r] * c : -INFINITY;
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = s[r] * c;
  }
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx = pair_max(mx);
  // Lazy rescale: the running max only moves when this tile beats it by more than
  // 2^RESCALE_THRESHOLD; the caller then scales O by `alpha` (rare after the first tile).
  const bool need = mx > st.m + RESCALE_THRESHOLD;  // also true when st.m == -inf
  st.alpha = 1.0f;
  st.rescale = __builtin_amdgcn_ballot_w64(need) != 0;
  if (need) {
    st.alpha = __builtin_amdgcn_exp2f(st.m - mx);
    st.m = mx;
    st.l *= st.alpha;
  }
  const float mref = st.m == -INFINITY ? 0.0f : st.m;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    u32x4 packed;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float p0 = __builtin_amdgcn_exp2f(s[8 * kk + 2 * d] - mref);
      const float p1 = __builtin_amdgcn_exp2f(s[8 * kk + 2 * d + 1] - mref);
      // round to nearest even (one v_cvt_pk_f16_f32); l sums the rounded values
      const f16x2 hp = __builtin_convertvector((f32x2){p0, p1}, f16x2);
      st.l = __builtin_amdgcn_fdot2(hp, ones, st.l, false);
      packed[d] = __builtin_bit_cast(unsigned, hp);
    }
    pk[kk] = __builtin_bit_cast(f16x8, packed);
  }
}

// One pipelined trip of the KV loop for tile j held in stage STAGE = j & 1: softmax and
// PV of tile j, scores and V^T conversion of tile j+1, DMA of tile j+2 into the other
// stage's K buffer.  One barrier per tile.
struct TileLoop {
  const char* kv_lat;
  const char* k_rope;
  const char* vt;  // this split's first V^T tile
  int k_begin;     // first key of tile 0 (32-aligned)
  int k_first;     // first key of the split's range (>= k_begin)
  int k_end, key_last, n_tiles, mask_from, prefix, node;
  uint64_t anc;
  float c;
  int tid, wave, lane;

  template <int STAGE>
  __device__ __forceinline__ void iteration(int j, f32x16& s_cur, f32x16 (&o)[16], RowState& st,
                                            const u32x4 (&qf)[36]) const {
    const int key0 = k_begin + j * BN;
    const bool masked = key0 < k_first || key0 + BN > mask_from;
    const uint32_t vis = masked ? tile_visibility(key0, k_first, k_end, prefix, node, anc)
                                : 0xffffffffu;
    f16x8 pk[2];
    softmax_tile(s_cur, pk, st, c, masked, vis, lane);
    if (__builtin_expect(st.rescale, 0)) {
#pragma unroll
      for (int fb = 0; fb < 16; ++fb) o[fb] = scale_acc(o[fb], st.alpha);
    }
    const bool more = j + 1 < n_tiles;
    if (more) {
      // Past the last tile the DMA is clamped to the last key: a harmless refill of a
      // buffer nobody reads any more.
      s_cur = qk_dma<STAGE, STAGE ^ 1>(qf, lane, kv_lat, k_rope, vt, key0 + 2 * BN, key_last,
                                       j + 1, wave);
    }
    pv_tile<STAGE>(o, pk, lane);
    if (more) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
};

__global__ __launch_bounds__(NTHR, 1) void verify_attn_bf16_kernel(VerifyParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;

  // ---- which (request, split, row tile) ------------------------------------------
  // Workgroup i runs on XCD i % 8.  Work comes in groups of m_tiles row tiles that share
  // one (request, split) KV range; groups are ranked by request (longest KV first, from
  // the pre-pass) then split, and dealt to the XCDs in snake order (ranks 0..7 to XCDs
  // 0..7, ranks 8..15 to XCDs 7..0, ...), so every XCD gets an even, longest-first share
  // of the work, and the row tiles of a group share that XCD's L2.
  const int slot = blockIdx.x / NUM_XCD;
  const int xcd = (int)(blockIdx.x % NUM_XCD);
  const int round = slot / p.m_tiles;
  const int grank = NUM_XCD * round + ((round & 1) ? NUM_XCD - 1 - xcd : xcd);
  if (grank >= p.batch * p.num_splits) return;
  const int mt = slot % p.m_tiles;
  const int rank = grank / p.num_splits;
  const int split = grank % p.num_splits;
  int b = p.order ? p.order[rank] : rank;
  if (b < 0 || b >= p.batch) b = rank;
  b = __builtin_amdgcn_readfirstlane(b);

  // ---- packed offsets: exclusive prefix sums over earlier requests ---------------
  int64_t qoff = 0, kvoff = 0, tbase = 0;
  int bad = 0;
  for (int i = tid; i < b; i += NTHR) {
    const int t = p.q_len[i], pl = p.prefix_len[i];
    bad |= (t < 1 || t > p.max_q_len) ? ST_BAD_QLEN : 0;
    bad |= pl < 0 ? ST_BAD_PREFIX : 0;
    qoff += t;
    kvoff += (int64_t)pl + t;
    tbase += ((int64_t)pl + t + VT_TILE_KEYS - 1) / VT_TILE_KEYS;
  }
  for (int off = 32; off > 0; off >>= 1) {
    qoff += __shfl_xor(qoff, off);
    kvoff += __shfl_xor(kvoff, off);
    tbase += __shfl_xor(tbase, off);
    bad |= __shfl_xor(bad, off);
  }
  if (tid == 0) sFlag = 0;
  __syncthreads();
  if (lane == 0) {
    sRed[wave] = qoff;
    sRed[4 + wave] = kvoff;
    sRed[8 + wave] = tbase;
    if (bad) atomicOr(&sFlag, bad);
  }
  __syncthreads();
  qoff = uniform64(sRed[0] + sRed[1] + sRed[2] + sRed[3]);
  kvoff = uniform64(sRed[4] + sRed[5] + sRed[6] + sRed[7]);
  tbase = uniform64(sRed[8] + sRed[9] + sRed[10] + sRed[11]);
  const int T = p.q_len[b];
  const int P = p.prefix_len[b];
  int flag = __builtin_amdgcn_readfirstlane(sFlag);
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

  // ---- parents -> LDS, validated -------------------------------------------------
  __syncthreads();
  if (tid == 0) sFlag = 0;
  __syncthreads();
  if (tid < T) {
    const int pa = p.tree_parent[qoff + tid];
    const bool ok = tid == 0 ? pa == -1 : (pa >= 0 && pa < tid);
    sParent[tid] = ok ? pa : -1;
    if (!ok) atomicOr(&sFlag, ST_BAD_PARENT);
  }
  __syncthreads();
  const int pflag = __builtin_amdgcn_readfirstlane(sFlag);
  if (pflag) {
    if (tid == 0 && p.status) atomicOr(p.status, pflag);
    return;
  }

  // ---- this lane's query row, node and ancestor-or-self mask ----------------------
  const int row = m0 + wave * 32 + (lane & 31);
  const bool row_ok = row < rows;
  const int crow = row_ok ? row : rows - 1;
  const int node = crow / H;
  uint64_t anc = 0;
  for (int x = node, hops = 0; x >= 0 && hops <= MAX_QLEN; ++hops) {
    if (x < 64) anc |= 1ull << x;
    x = sParent[x];
  }

  // ---- key range of this split ---------------------------------------------------
  const int S = p.num_splits;
  int k_begin, k_end;
  {
    // chunks of whole 32-key tiles, so every split starts on a V^T tile boundary
    const int chunk = ((P + S - 1) / S + BN - 1) / BN * BN;
    k_begin = min(P, split * chunk);
    k_end = (split == S - 1) ? P + T : min(P, (split + 1) * chunk);
  }
  const int64_t grow = qoff * H + crow;  // global query row
  if (k_end <= k_begin) {
    // empty split: partial = (0, -inf)
    if (row_ok) {
      float* po = p.part_o + ((int64_t)split * p.total_q * H + grow) * DL;
      for (int f = h * 4; f < DL; f += 8) *(float4*)(po + f) = make_float4(0.f, 0.f, 0.f, 0.f);
      if (h == 0) p.part_lse[(int64_t)split * p.total_q * H + grow] = -INFINITY;
    }
    return;
  }

  // ---- Q fragment -> VGPRs (B operand of S^T = K Q^T) ----------------------------
  u32x4 qf[36];
  {
    const char* ql = (const char*)p.q_lat + grow * (DL * 2);
    const char* qr = (const char*)p.q_rope + grow * (DR * 2);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      const int c = 2 * ks + h;
      qf[ks] = ks < 32 ? *(const u32x4*)(ql + c * 16) : *(const u32x4*)(qr + (c - 64) * 16);
    }
  }

  const char* kv_lat = (const char*)p.kv_lat + kvoff * (DL * 2);  // this request's rows
  const char* k_rope = (const char*)p.k_rope + kvoff * (DR * 2);
  // Tiles are 32-aligned in the request's key stream (the V^T tiles are); a split whose
  // range starts mid-tile (only the last split, when the prefix is short) masks the keys
  // before its range.
  const int k_first = k_begin;
  k_begin &= ~(BN - 1);
  const int key_last = k_end - 1;
  const int n_tiles = (k_end - k_begin + BN - 1) / BN;
  const int mask_from = min(P, k_end);  // tiles ending at or before this key are unmasked
  const float c = p.scale_log2;

  f32x16 o[16];
#pragma unroll
  for (int fb = 0; fb < 16; ++fb) o[fb] = f32x16{};
  RowState st{-INFINITY, 0.0f, 1.0f, false};

  // Pipeline: iteration j runs the softmax and PV of tile j while the scores of tile
  // j+1 are computed and its V^T converted; the DMA of tile j+2 is in flight.  One
  // barrier per tile.  Stage j&1 holds K(j) / V^T(j).
  if (tbase + (P + T + BN - 1) / BN > p.vt_tiles) {  // cannot happen for valid offsets
    if (tid == 0 && p.status) atomicOr(p.status, ST_OVERFLOW);
    return;
  }
  const char* vt_split = (const char*)p.vt + (tbase + k_begin / BN) * VT_TILE_BYTES;
  issue_tile<0>(kv_lat, k_rope, k_begin, key_last, wave, lane);
  issue_vt<0>(vt_split, 0, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (n_tiles > 1) issue_tile<1>(kv_lat, k_rope, k_begin + BN, key_last, wave, lane);
  f32x16 s_cur = qk_tile<0>(qf, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  TileLoop tl{kv_lat, k_rope, vt_split, k_begin, k_first, k_end, key_last, n_tiles, mask_from,
              P, node, anc, c, tid, wave, lane};
  for (int j = 0; j < n_tiles; j += 2) {
    tl.iteration<0>(j, s_cur, o, st, qf);
    if (j + 1 >= n_tiles) break;
    tl.iteration<1>(j + 1, s_cur, o, st, qf);
  }

  // ---- finalize -------------------------------------------------------------------
  const float l_tot = pair_sum(st.l);
  const float inv = 1.0f / l_tot;
  const float lse = st.m * LN2 + logf(l_tot);
  if (!row_ok) return;
  float* out;
  float* lse_out;
  if (S == 1) {
    out = p.out_lat + grow * DL;
    lse_out = p.out_lse + grow;
  } else {
    out = p.part_o + ((int64_t)split * p.total_q * H + grow) * DL;
    lse_out = p.part_lse + (int64_t)split * p.total_q * H + grow;
  }
#pragma unroll
  for (int fb = 0; fb < 16; ++fb) {
    const f32x16 t = read_acc(o[fb]);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 v = make_float4(t[4 * q4] * inv, t[4 * q4 + 1] * inv, t[4 * q4 + 2] * inv,
                             t[4 * q4 + 3] * inv);
      *(float4*)(out + fb * 32 + q4 * 8 + h * 4) = v;
    }
  }
  if (h == 0) {
    *lse_out = lse;
    if (!(fabsf(lse) < INFINITY) && p.status) atomicOr(p.status, ST_NONFINITE);
  }
}

}  // namespace

int rows_per_block_bf16() { return BM; }

hipError_t launch_verify_bf16(const VerifyParams& p, hipStream_t stream) {
  const int64_t groups = (int64_t)p.batch * p.num_splits;
  const int64_t blocks = (int64_t)NUM_XCD * ((groups + NUM_XCD - 1) / NUM_XCD) * p.m_tiles;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(verify_attn_bf16_kernel, dim3((unsigned)blocks), dim3(NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kdt
