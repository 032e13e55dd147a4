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
// ancestor mask and all 128 rows share every KV tile.
//   * Scores and softmax by rows: wave w owns rows 32w..32w+31.  Its Q fragment (32 rows x
//     576: latent part converted to fp16, rope part bf16) lives in VGPRs for the whole
//     KV loop; S^T = K Q^T per 32-key tile runs as fp16 MFMA 32x32x16 over the latent dims
//     and bf16 over the rope dims, so each lane holds one query row and the softmax row
//     reductions are in-register plus one lane swap; online softmax in the log2 domain
//     with a lazy rescale (the running max is only raised when a tile beats it by more
//     than 2^8).
//   * PV by features: wave w owns features 128w..128w+127 of all 128 rows, O^T += V^T P^T
//     as fp16 MFMA 32x32x16 with P in fp16 (bf16 P is too coarse for a 2e-3 relative
//     bound).  Each V^T operand, read once from the fp16 latent tile through the
//     transposing LDS load, feeds four row blocks' MFMAs; the P operands come from the
//     softmax lanes of their owner waves through a double-buffered LDS area.
//   * One barrier per 32-key tile.  After it, one interleaved stream of 68 MFMAs: the
//     scores of the next tile, the PV of this tile, the copy of the tile after next, and,
//     between the last 22 PV MFMAs, the next tile's softmax (VALU work that costs almost
//     nothing next to independent MFMAs of the same wave, and stalls the matrix pipe when
//     run on its own).
// The fp16 latent tiles (converted once per call by the pre-pass) and the bf16 rope rows
// arrive by 16-byte global->LDS DMA into a three-stage LDS ring.
#include "common.h"

namespace kdt {
namespace {

constexpr int BM = 128;     // query rows per workgroup
static_assert(BM == PIECE_ROWS, "cut pieces hold one row tile");
constexpr int BN = 32;      // keys per tile
constexpr int NTHR = 256;   // 4 waves
constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

#define LDS_AS __attribute__((address_space(3)))

// LDS tiles, three stages.  Per stage (u32x4 = 16 B units):
//   K16    [32 keys][64 chunks + 4 pad] fp16 latent rows, 8 features per chunk: chunk c
//          of key k at slot k*68 + (c ^ ksw(k)), ksw(k) = (k >> 2) & 3.  The score reads
//          (16 consecutive keys, one chunk each) and the transposing value reads (4
//          consecutive keys x 4 chunks) are both bank-conflict free, and both address
//          streams stay affine (two base registers each);
//   K rope [8 chunks][32 keys] bf16, chunk-major: chunk c of key k at slot 32c + k, so
//          a score read (32 keys x one chunk per half-wave) is 1 KB contiguous and the
//          four rope k-steps are one affine stream (slot 64 (ks - 32) + lane).
// Tile j serves the scores (loop trip j-1) and the values (trip j) while tile j+2 is in
// flight: three stages.
constexpr int K16_ROW = 68;
constexpr int K16_U4 = BN * K16_ROW, KROPE_U4 = BN * 8;
constexpr int K16_STEP16 = 16 * K16_ROW * 16;  // bytes between key rows r and r + 16
// Output staging in the finished tile ring: 32 rows x 128 fp32 features per wave, rows
// padded by 16 bytes so that both the row-per-lane writes and the row-contiguous reads are
// free of bank conflicts; two waves' blocks fit in one latent tile buffer.
constexpr int EPI_ROW_BYTES = 128 * 4 + 16;
constexpr int EPI_WAVE_BYTES = 32 * EPI_ROW_BYTES;
static_assert(2 * EPI_WAVE_BYTES <= K16_U4 * 16, "two output blocks per tile buffer");
// Separate objects per stage: the compiler's wait-count insertion can then tell that a
// DMA into one stage does not alias LDS reads of another, and does not stall the
// compute of tile j on the in-flight copy of tile j+2.
__shared__ __attribute__((aligned(1024))) u32x4 sK16a[K16_U4];
__shared__ __attribute__((aligned(1024))) u32x4 sK16b[K16_U4];
__shared__ __attribute__((aligned(1024))) u32x4 sK16c[K16_U4];
__shared__ __attribute__((aligned(1024))) u32x4 sKropeA[KROPE_U4];
__shared__ __attribute__((aligned(1024))) u32x4 sKropeB[KROPE_U4];
__shared__ __attribute__((aligned(1024))) u32x4 sKropeC[KROPE_U4];
__shared__ int32_t sParent[MAX_QLEN];
__shared__ int32_t sFlag;
// What the softmax of one trip hands to the feature-split PV of every wave, in buffers of
// trip parity j & 1: each wave's fp16 P tile ([row block][key step][lane], 16 B each: the
// PV B operand of that lane as the softmax left it in registers), each row's O scale for
// the trip, and the number of the last trip in which some row's running max moved.
__shared__ __attribute__((aligned(1024))) u32x4 sP[2][4 * 2 * 64];
__shared__ float sAlpha[2][BM];
__shared__ int32_t sResc[2];
__shared__ float sInv[BM];

__device__ __forceinline__ int ksw(int k) { return (k >> 2) & 3; }

template <int S> __device__ __forceinline__ u32x4* k16() {
  return S == 0 ? sK16a : (S == 1 ? sK16b : sK16c);
}
template <int S> __device__ __forceinline__ u32x4* krope() {
  return S == 0 ? sKropeA : (S == 1 ? sKropeB : sKropeC);
}

// 16-byte global -> LDS copy per lane (64 lanes fill 1 KB at lds_base) through a buffer
// descriptor on the wave-uniform base (lane offsets below 2^31).  The buffer form, unlike
// global_load_lds, is counted by the compiler's wait insertion as a vector-memory
// operation only, so LDS reads issued while copies are in flight keep exact lgkmcnt
// waits instead of draining every outstanding LDS read.
__device__ __forceinline__ void dma16(const char* uniform_base, unsigned lane_off, u32x4* lds_base,
                                      bool live = true) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)uniform_base, (short)0, live ? -1 : 0, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)lds_base, 16, (int)lane_off, 0, 0,
                                           0);
}

// One fp16 latent row (1 KB, already in its LDS image) per DMA: row 8w + n of the tile
// behind `rsrc` (one descriptor per tile), selected by the scalar offset (8w + n) KB.
// (The immediate offset of an LDS-destination load moves the LDS address too, so it
// stays 0.)  A copy that is not `live` gets a zero-sized buffer: every lane is out of
// range, so it reads no memory and completes at once.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* uniform_tile,
                                                            bool live = true) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)uniform_tile, (short)0, live ? -1 : 0,
                                           0x00020000);
}
template <int S, int N>
__device__ __forceinline__ void dma_k16_row(__amdgpu_buffer_rsrc_t rsrc, int wave, unsigned lane_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(k16<S>() + (wave * 8 + N) * K16_ROW),
                                           16, (int)lane_off, (wave * 8 + N) * 1024, 0, 0);
}

// Rope chunks 2w, 2w+1 of keys [key0, key0+32) (clamped to key_last), one instruction per
// wave: lane l moves chunk 2w + (l >> 5) of key l & 31 into slot 64w + l.
template <int S>
__device__ __forceinline__ void dma_rope(const char* k_rope_req, int key0, int key_last, int wave,
                                         int lane, bool live = true) {
  // recomputed from an opaque lane id on every call: kept live across the KV loop, the
  // key index would be spilled, and its reload's vmcnt(0) would wait for this tile's copies
  asm volatile("" : "+v"(lane));
  const int k = min(key0 + (lane & 31), key_last);
  dma16(k_rope_req, (unsigned)k * (DR * 2) + (unsigned)(2 * wave + (lane >> 5)) * 16u,
        krope<S>() + wave * 64, live);
}

// Issue the DMA of tile `tile` (keys [key0, key0+32)) into stage S.  Wave w moves fp16
// latent rows 8w..8w+7 and rope chunks 2w, 2w+1.
template <int S>
__device__ __forceinline__ void issue_tile(const char* tile, const char* k_rope_req, int key0,
                                           int key_last, int wave, int lane) {
  // Re-materialise the lane id here so the per-lane offsets are recomputed per tile
  // instead of being hoisted out of the KV loop as long-lived registers.
  asm volatile("" : "+v"(lane));
  const __amdgpu_buffer_rsrc_t rsrc = tile_rsrc(tile);
  dma_k16_row<S, 0>(rsrc, wave, (unsigned)lane * 16u);
  dma_k16_row<S, 1>(rsrc, wave, (unsigned)lane * 16u);
  dma_k16_row<S, 2>(rsrc, wave, (unsigned)lane * 16u);
  dma_k16_row<S, 3>(rsrc, wave, (unsigned)lane * 16u);
  dma_k16_row<S, 4>(rsrc, wave, (unsigned)lane * 16u);
  dma_k16_row<S, 5>(rsrc, wave, (unsigned)lane * 16u);
  dma_k16_row<S, 6>(rsrc, wave, (unsigned)lane * 16u);
  dma_k16_row<S, 7>(rsrc, wave, (unsigned)lane * 16u);
  dma_rope<S>(k_rope_req, key0, key_last, wave, lane);
}

// Score fragment ks of the tile in stage S for this lane (key = lane & 31, half h):
// latent k-steps 0..31 read chunk 2ks + h of the key's fp16 row, rope k-steps 32..35
// read chunk 2 (ks - 32) + h of its bf16 rope row.  Three affine read streams.
struct ScoreFrags {
  int be, bo, rl;
  __device__ __forceinline__ ScoreFrags(int lane) {
    const int key = lane & 31, h = lane >> 5, sw = ksw(key);
    // chunk 2ks + h lands in slot 4 (ks >> 1) + ((2 (ks & 1) + h) ^ sw) of the row
    be = key * K16_ROW + (h ^ sw);
    bo = key * K16_ROW + ((2 + h) ^ sw);
    rl = lane;
  }
  template <int S>
  __device__ __forceinline__ u32x4 get(int ks, int h) const {
    if (ks < 32) return k16<S>()[((ks & 1) ? bo : be) + 4 * (ks >> 1)];
    return krope<S>()[rl + 64 * (ks - 32)];
  }
};

__device__ __forceinline__ f32x16 mfma_qk(int ks, const u32x4& a, const u32x4& q, const f32x16& s) {
  if (ks < 32)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, q), s, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, q), s, 0, 0, 0);
}

// o[FB] += a * p (fp16 MFMA 32x32x16).  Every accumulator is an operand of every such
// statement, which pins all 16 to fixed AGPRs for the whole loop; naming only o[FB]
// lets the allocator route them through one AGPR tuple with copies.
#define KDT_PV_OPERANDS                                                                    \
  : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]), [o4] "+a"(o[4]),   \
    [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]), [o8] "+a"(o[8]), [o9] "+a"(o[9]),   \
    [o10] "+a"(o[10]), [o11] "+a"(o[11]), [o12] "+a"(o[12]), [o13] "+a"(o[13]),            \
    [o14] "+a"(o[14]), [o15] "+a"(o[15])                                                   \
  : [a] "v"(a), [p] "v"(p)
#define KDT_PV_CASE(N)                                                                      \
  if constexpr (FB == N)                                                                    \
  asm volatile("v_mfma_f32_32x32x16_f16 %[o" #N "], %[a], %[p], %[o" #N "]" KDT_PV_OPERANDS)
template <int FB>
__device__ __forceinline__ void mfma_pv(f32x16 (&o)[16], const f16x8& a, const f16x8& p) {
  KDT_PV_CASE(0); KDT_PV_CASE(1); KDT_PV_CASE(2); KDT_PV_CASE(3);
  KDT_PV_CASE(4); KDT_PV_CASE(5); KDT_PV_CASE(6); KDT_PV_CASE(7);
  KDT_PV_CASE(8); KDT_PV_CASE(9); KDT_PV_CASE(10); KDT_PV_CASE(11);
  KDT_PV_CASE(12); KDT_PV_CASE(13); KDT_PV_CASE(14); KDT_PV_CASE(15);
}
#undef KDT_PV_CASE
#undef KDT_PV_OPERANDS

// V^T operand of feature block fb, key step ks: eight fp16 of feature 32fb + (lane & 31)
// at the k-slots 8h..8h+7 of the P operand (keys 16ks + 4h + {0..3, 8..11}), as two
// transposing 8-byte loads of four consecutive key rows each.
struct ValueFrags {
  const LDS_AS char* base;
  unsigned off0, off1;
  // foff: byte offset of this wave's first feature block (4 blocks of 64 B per wave).
  __device__ __forceinline__ ValueFrags(const u32x4* tile, int lane, int foff) {
    base = (const LDS_AS char*)(LDS_AS void*)tile;
    const int g = (lane >> 4) & 1, r = (lane >> 2) & 3, q = lane & 3, h = lane >> 5;
    // lane 4r + q of a 16-lane group reads 4 features (8 B) of key row 4h + 8j + r; the
    // row swizzle ksw = h + 2j there, chunk 4fb + 2g + (q >> 1).  The swizzle only moves
    // chunk bits 0-1, so a feature block is a plain 64-byte offset.
    off0 = (unsigned)((4 * h + r) * K16_ROW * 16 + 16 * ((2 * g + (q >> 1)) ^ h) + 8 * (q & 1) +
                      foff);
    off1 = (unsigned)((4 * h + 8 + r) * K16_ROW * 16 + 16 * ((2 * g + (q >> 1)) ^ (h + 2)) +
                      8 * (q & 1) + foff);
    // opaque per-lane offsets: every read stays base + offset + constant, a short address
    // chain from the stage's LDS object, so the compiler's wait insertion keeps telling
    // these reads apart from the copies into other stages
    asm("" : "+v"(off0), "+v"(off1));
  }
  template <int FB, int KS>
  __device__ __forceinline__ f16x8 get() const {
    constexpr unsigned step = (unsigned)(KS * K16_STEP16 + FB * 64);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(base + off0 + step));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(base + off1 + step));
    const f16x4 l4 = __builtin_bit_cast(f16x4, lo), h4 = __builtin_bit_cast(f16x4, hi);
    return f16x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
  }
};

// Wait states between the last PV MFMA and VALU reads of the accumulators.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n s_nop 7\n s_nop 3"); }

// Orders one wave's LDS writes before its later LDS reads (and the reverse): the wave's
// LDS instructions execute in order, so only the compiler has to be kept from moving them.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
// The same copy, pinned after everything before it in program order: the first empty asm
// keeps the value in AGPRs up to this point, so the register allocator cannot hoist the
// copy (and its 16 VGPRs) above earlier barriers.
__device__ __forceinline__ f32x16 read_acc_here(const f32x16& acc) {
  f32x16 t = acc;
  asm volatile("" : "+a"(t));
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
  float l;      // this lane's partial sum of the probabilities (fp32, before rounding)
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

// This wave's P tile of tile `jt` (two 16-byte fragments per lane), its rows' O scales
// and, when some row's running max moved, the rescale flag, into the buffers of parity
// jt & 1 that the feature-split PV of every wave reads after the next barrier.
__device__ __forceinline__ void publish_p(int kk, const u32x4& packed, int wave, int lane, int jt) {
  sP[jt & 1][(wave * 2 + kk) * 64 + lane] = packed;
}
__device__ __forceinline__ void publish_scale(const RowState& st, int wave, int lane, int jt) {
  if (lane < 32) sAlpha[jt & 1][wave * 32 + lane] = st.alpha;
  if (st.rescale && lane == 0) sResc[jt & 1] = jt;
}

// Online softmax of one tile: S^T (raw scores, register r <-> key 8(r/4) + 4h + r%4)
// -> P (fp16, published to LDS) and the running max / sum.  `vis` = visibility bits (see
// tile_visibility).  The scale c (> 0: the prologue folds a sign or a zero scale into Q)
// is applied inside the exponent's argument, exp2(s c - m) as one fma.  The row max of the
// raw scores times c is exactly the max of the rounded products, since rounding is
// monotone; masked keys stay -inf.
//
// The work is cut into 22 steps so that it can sit between independent MFMAs: on gfx950
// up to three or four VALU instructions per 32-cycle MFMA of the same wave cost almost
// nothing, while the same work run on its own leaves the matrix pipe idle.
struct SoftmaxSteps {
  f32x16& s;
  RowState& st;
  const float c;
  const bool masked;
  const uint32_t vis;
  const int lane, wave, jt;
  float mx, mref, p_even;
  u32x4 packed;

  template <int K>
  __device__ __forceinline__ void step() {
    if constexpr (K == 0) {
      if (masked) {
        int ol = lane;  // the half's shift, recomputed rather than kept live in the loop
        asm volatile("" : "+v"(ol));
        const uint32_t vh = vis >> (4 * (ol >> 5));
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[r] = ((vh >> (8 * (r >> 2) + (r & 3))) & 1u) ? s[r] : -INFINITY;
      }
    } else if constexpr (K == 1) {
      mx = s[0];
#pragma unroll
      for (int r = 1; r < 8; ++r) mx = fmaxf(mx, s[r]);
    } else if constexpr (K == 2) {
#pragma unroll
      for (int r = 8; r < 16; ++r) mx = fmaxf(mx, s[r]);
    } else if constexpr (K == 3) {
      mx = pair_max(mx) * c;
    } else if constexpr (K == 4) {
      // Lazy rescale: the running max only moves when this tile beats it by more than
      // 2^RESCALE_THRESHOLD (also when st.m == -inf); O is then scaled by alpha before
      // this tile's PV (rare after the first tile).
      const bool need = mx > st.m + RESCALE_THRESHOLD;
      st.alpha = 1.0f;
      st.rescale = __builtin_amdgcn_ballot_w64(need) != 0;
      if (need) {
        st.alpha = __builtin_amdgcn_exp2f(st.m - mx);
        st.m = mx;
        st.l *= st.alpha;
      }
      mref = st.m == -INFINITY ? 0.0f : st.m;
    } else if constexpr (K == 5) {
      publish_scale(st, wave, lane, jt);
    } else if constexpr (K >= 6 && K < 22) {
      constexpr int E = K - 6;  // score register E: p = exp2(s c - m)
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[E], c, -mref));
      // l sums the fp32 values with plain adds (a v_dot2 next to the MFMAs would stall
      // the matrix pipe ~20 cycles each); P for the MFMA is rounded to nearest even
      st.l += pe;
      if constexpr (E % 2 == 0) {
        p_even = pe;
      } else {
        const f16x2 hp = {(_Float16)p_even, (_Float16)pe};
        packed[(E % 8) / 2] = __builtin_bit_cast(unsigned, hp);
        if constexpr (E % 8 == 7) publish_p(E / 8, packed, wave, lane, jt);
      }
    }
  }
};

// The MFMA stream of one trip, after its barrier: the scores of tile j+1 (stage SQ), the
// PV of tile j (stage SV), the copy of tile j+2 into stage SD, and the softmax of tile
// j+1.  PV is split by features: this wave owns feature blocks 4w..4w+3 (128 features) of
// all 128 rows, accumulator 4 fbl + rb = local feature block fbl of row block rb.  Its B
// operands (P) come from the LDS copies every wave's softmax wrote before the barrier; each
// V^T operand, read once, feeds the four row blocks' MFMAs.
//
// 68 MFMA slots in two parts.  Part A (36 + PA slots): the 36 score MFMAs, the first Q0
// alone, then with PV MFMAs 0..PA-1 spread evenly between them, so that tile j+1's scores
// are complete at its end.  Part B: PV MFMAs PA..31, with the 22 steps of tile j+1's
// softmax spread evenly over them.  PV MFMAs run in the order (key step, feature block,
// row block).  K fragments are read three score MFMAs ahead, V^T fragments three PV MFMAs
// ahead, the P fragments of key step 1 four ahead (each replaces the key-step-0 fragment
// of its row block after that one's last use).  The nine copies are spread over the
// first DMA_SPAN slots, so that they have most of a trip to land before the next barrier
// waits for them.
#ifndef KDT_SCHED_Q0
#define KDT_SCHED_Q0 6
#endif
#ifndef KDT_SCHED_PA
#define KDT_SCHED_PA 10
#endif
#ifndef KDT_SCHED_DMA_SPAN
#define KDT_SCHED_DMA_SPAN 45
#endif
struct Sched {
  static constexpr int Q0 = KDT_SCHED_Q0, PA = KDT_SCHED_PA, LA = 36 + PA, NB = 32 - PA;
  static constexpr int DMA_SPAN = KDT_SCHED_DMA_SPAN;
  static_assert(Q0 >= 1 && Q0 <= 36 && PA >= 1 && PA <= 31, "schedule shape");
  // part A, slot t >= Q0: PV MFMAs placed by an even (Bresenham) spread
  static constexpr int pv_done(int t) { return t < Q0 ? 0 : ((t - Q0 + 1) * PA) / (LA - Q0); }
  static constexpr int qk(int T) {
    return T < Q0 ? T
         : (T < LA ? (pv_done(T) > pv_done(T - 1) ? -1 : T - pv_done(T)) : -1);
  }
  static constexpr int pv(int T) {
    return T < Q0 ? -1 : (T < LA ? (pv_done(T) > pv_done(T - 1) ? pv_done(T) - 1 : -1)
                                 : PA + (T - LA));
  }
  // softmax steps [sm_begin, sm_end) run in part-B slot T
  static constexpr int sm_begin(int T) { return T < LA ? 0 : ((T - LA) * 22) / NB; }
  static constexpr int sm_end(int T) { return T < LA ? 0 : ((T - LA + 1) * 22) / NB; }
  // copy N (0..8) goes in slot dma_slot(N)
  static constexpr int dma_slot(int N) { return 1 + (N * (DMA_SPAN - 1)) / 8; }
  static constexpr int dma_at(int T) {
    for (int n = 0; n < 9; ++n)
      if (dma_slot(n) == T) return n;
    return -1;
  }
};

template <int SQ, int SD, int SV>
struct TripStream {
  static constexpr int KA = 3;  // K fragments read this many score MFMAs ahead
  f32x16& s;
  f32x16 (&o)[16];
  const u32x4 (&qf)[36];
  const ScoreFrags fr;
  const ValueFrags vf;
  const __amdgpu_buffer_rsrc_t rsrc;
  const char* k_rope_req;
  const int key0s, lasts, wave, lane, dl, j, par;
  const bool live;  // the copy is of a tile the loop still needs
  SoftmaxSteps& sm;
  int resc;
  u32x4 ka[KA + 1];
  f16x8 va[2];
  f16x8 pf[4];

  __device__ __forceinline__ TripStream(f32x16& s_, f32x16 (&o_)[16], const u32x4 (&qf_)[36],
                                        int lane_, int wave_, const char* dma_tile,
                                        const char* k_rope_req_, int k_key0, int key_last,
                                        int j_, bool live_, SoftmaxSteps& sm_)
      : s(s_), o(o_), qf(qf_), fr(lane_), vf(k16<SV>(), lane_, wave_ * 256),
        rsrc(tile_rsrc(dma_tile, live_)), k_rope_req(k_rope_req_),
        key0s(__builtin_amdgcn_readfirstlane(k_key0)),
        lasts(__builtin_amdgcn_readfirstlane(key_last)), wave(wave_), lane(lane_),
        dl(lane_), j(j_), par(j_ & 1), live(live_), sm(sm_), resc(-1) {}

  // P fragment (key step ks, row block rb): lane `lane` of the owner wave's softmax.
  __device__ __forceinline__ f16x8 pfrag(int ks, int rb) const {
    return __builtin_bit_cast(f16x8, sP[par][(rb * 2 + ks) * 64 + lane]);
  }

  __device__ __forceinline__ void run() {
    const int h = lane >> 5;
    // LDS reads return in order: the first score MFMA's operand goes first
#pragma unroll
    for (int i = 0; i < KA; ++i) ka[i] = fr.get<SQ>(i, h);
    va[0] = vf.get<0, 0>();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) pf[rb] = pfrag(0, rb);
    resc = sResc[par];
    __builtin_amdgcn_sched_barrier(0);
    slot<0>();
  }

  // O *= alpha for every row whose running max moved with tile j (rare after the first
  // tiles).  Trip 0 needs none: O is still zero.
  __device__ __forceinline__ void rescale() {
    if (__builtin_expect(__builtin_amdgcn_readfirstlane(resc) == j, 0) && j > 0) {
      mfma_drain();
      int ol = lane;  // recomputed address: nothing of this rare path stays live
      asm volatile("" : "+v"(ol));
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const float a = sAlpha[par][rb * 32 + (ol & 31)];
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) o[4 * fb + rb] = scale_acc(o[4 * fb + rb], a);
      }
      // wait states between the VALU writes of the accumulators and the MFMAs reading them
      asm volatile("s_nop 4");
    }
  }

  template <int K, int KE>
  __device__ __forceinline__ void sm_steps() {
    if constexpr (K < KE) {
      sm.step<K>();
      sm_steps<K + 1, KE>();
    }
  }

  template <int T>
  __device__ __forceinline__ void slot() {
    if constexpr (T < 68) {
      constexpr int QK = Sched::qk(T);
      constexpr int PV = Sched::pv(T);
      if constexpr (PV == 0) {
        rescale();
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (QK >= 0 && QK + KA < 36) ka[(QK + KA) % (KA + 1)] = fr.get<SQ>(QK + KA, lane >> 5);
      if constexpr (PV >= 0 && PV % 4 == 1 && PV / 4 + 1 < 8) {
        constexpr int V = PV / 4 + 1;  // next V^T fragment (key step V / 4, block V % 4)
        va[V & 1] = vf.get<V % 4, V / 4>();
      }
      if constexpr (Sched::dma_at(T) >= 0) {
        constexpr int N = Sched::dma_at(T);  // copies 0..8
        if constexpr (N < 8)
          dma_k16_row<SD, N>(rsrc, wave, (unsigned)dl * 16u);
        else
          dma_rope<SD>(k_rope_req, key0s, lasts, wave, dl, live);
      }
      // the score chain starts from zero: s held tile j's scores, consumed last trip
      if constexpr (QK >= 0) s = mfma_qk(QK, ka[QK % (KA + 1)], qf[QK], QK == 0 ? f32x16{} : s);
      if constexpr (PV >= 0) {
        constexpr int V = PV / 4;
        mfma_pv<(V % 4) * 4 + PV % 4>(o, va[V & 1], pf[PV % 4]);
        // the last key-step-0 use of this row block's P: fetch its key-step-1 fragment
        if constexpr (PV >= 12 && PV < 16) pf[PV % 4] = pfrag(1, PV % 4);
      }
      sm_steps<Sched::sm_begin(T), Sched::sm_end(T)>();
      __builtin_amdgcn_sched_barrier(0);
      slot<T + 1>();
    }
  }
};

// One trip of the KV loop for tile j, held in stage ST = j % 3.  On entry every wave has
// published tile j's P (the previous trip, or the prologue for tile 0).  The trip's one
// barrier then makes those visible and vouches for tile j+1's copy and for every wave
// being done with tile j-1's stage; the stream then runs the scores of tile j+1, the PV of
// tile j, the copy of tile j+2 into the stage tile j-1 used, and tile j+1's softmax,
// which publishes its P for the next trip.
struct TileLoop {
  const char* k_rope;
  const char* k16;  // this split's first fp16 latent tile
  int k_begin;      // first key of tile 0 (32-aligned)
  int k_first;      // first key of the split's range (>= k_begin)
  int k_end, key_last, n_tiles, mask_from, prefix, node;
  uint64_t anc;
  float c;
  int tid, wave, lane;

  __device__ __forceinline__ bool tile_masked(int key0) const {
    return key0 < k_first || key0 + BN > mask_from;
  }

  template <int ST>
  __device__ __forceinline__ void iteration(int j, f32x16& s_cur, f32x16 (&o)[16], RowState& st,
                                            const u32x4 (&qf)[36]) const {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Tile j+1's softmax.  On the last trip the stream's scores are of a stale stage: every
    // key is masked, which leaves the running max and sum as they are (and publishes a P
    // nobody reads).
    const int key1 = k_begin + (j + 1) * BN;
    const bool last = j + 1 >= n_tiles;
    const bool masked = last || tile_masked(key1);
    const uint32_t vis = last ? 0u
                       : (masked ? tile_visibility(key1, k_first, k_end, prefix, node, anc)
                                 : 0xffffffffu);
    SoftmaxSteps sm{s_cur, st, c, masked, vis, lane, wave, j + 1};
    // One stream for every trip (a second PV call site would cost the accumulators their
    // fixed AGPRs).  On the last two trips there is no tile j+2: the copy goes through a
    // zero-sized buffer, so it reads nothing and completes at once (it zero-fills a stage
    // nobody reads any more), and neither the next barrier nor the epilogue waits on memory.
    const int jd = min(j + 2, n_tiles - 1);
    TripStream<(ST + 1) % 3, (ST + 2) % 3, ST> ts(s_cur, o, qf, lane, wave,
                                                  k16 + (int64_t)jd * TILE_BYTES, k_rope,
                                                  k_begin + (j + 2) * BN, key_last, j,
                                                  __builtin_amdgcn_readfirstlane(j + 2 < n_tiles) != 0,
                                                  sm);
    ts.run();
  }
};

// LDS writes of this workgroup before its later LDS reads: LDS traffic only, so copies
// into LDS and global loads in flight stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The latent part of one wave's 32 query rows, moved through LDS.  Loaded directly in the
// fragment layout, each 16-byte load would take 32 bytes from each of 32 rows; here each
// 16-byte global->LDS copy instruction moves 512 contiguous bytes of two rows (whole
// cache lines), in two halves of the 1 KB rows (half PS = bytes [512 PS, 512 PS + 512)).
// Area of wave w: the latent buffer of stage 1 (waves 0, 1) or stage 2 (waves 2, 3), at
// (w & 1) * 16640 bytes.  Copy i puts row i's half at 1040 i and row i + 16's at
// 1040 i + 512; the 16-byte pad between copies keeps the fragment reads (16 rows of one
// chunk per 16 lanes) free of bank conflicts.  Rows past the row tile's end repeat its
// last row.
struct QStage {
  static constexpr int COPY_BYTES = 1040;
  static_assert(2 * 16 * COPY_BYTES <= K16_U4 * 16, "two waves' areas per latent buffer");
  const char* wave_row0;  // the wave's first row (clamped to the last row)
  int rel_last;           // the last row, relative to wave_row0
  int lane;
  u32x4* area;

  __device__ __forceinline__ QStage(const void* q_lat, int64_t req_row0, int wave_row, int rows,
                                    int wave, int lane_)
      : lane(lane_) {
    const int first = min(wave_row, rows - 1);
    wave_row0 = (const char*)q_lat + (req_row0 + first) * (DL * 2);
    rel_last = rows - 1 - first;
    area = ((wave < 2) ? sK16b : sK16c) + (wave & 1) * (16 * COPY_BYTES / 16);
  }
  template <int PS>
  __device__ __forceinline__ void issue() const {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = min(i + 16 * (lane >> 5), rel_last);
      dma16(wave_row0, (unsigned)(r * (DL * 2) + PS * 512 + (lane & 31) * 16),
            area + i * (COPY_BYTES / 16));
    }
  }
  // fragments 16 PS .. 16 PS + 15: lane (row r = lane & 31, half h) takes chunk 2 ks + h
  template <int PS>
  __device__ __forceinline__ void read(u32x4 (&qf)[36]) const {
    const int r = lane & 31, h = lane >> 5;
    const LDS_AS char* base = (const LDS_AS char*)(LDS_AS void*)area + (r & 15) * COPY_BYTES +
                              (r >> 4) * 512 + h * 16;
#pragma unroll
    for (int k = 0; k < 16; ++k) qf[16 * PS + k] = *(const LDS_AS u32x4*)(base + k * 32);
  }
};

// Latent fragments K0 .. K0 + 15 (bf16) to fp16, tracking the largest magnitude.  The
// scores contract them against the fp16 latent tiles; exact for 2^-17 <= |x| < 65504
// like the tiles themselves.  One fragment at a time: left to itself the scheduler widens
// all values to fp32 first and runs out of registers.
template <int K0>
__device__ __forceinline__ void q_to_fp16(u32x4 (&qf)[36], float& qmax) {
#pragma unroll
  for (int ks = K0; ks < K0 + 16; ++ks) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const unsigned x = qf[ks][d];
      const float lo = __uint_as_float(x << 16), hi = __uint_as_float(x & 0xffff0000u);
      qmax = fmaxf(qmax, fmaxf(fabsf(lo), fabsf(hi)));
      const f16x2 hp = {(_Float16)lo, (_Float16)hi};
      qf[ks][d] = __builtin_bit_cast(unsigned, hp);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

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
  int slot = blockIdx.x / NUM_XCD;
  const int xcd = (int)(blockIdx.x % NUM_XCD);
  // Last-round cut (one split): the units of this XCD's queue after its whole rounds of
  // CUS_PER_XCD are skipped here and run instead as key pieces, workgroups appended to
  // the grid (blockIdx = NUM_XCD * (normal_slots + j) + xcd, piece j of this XCD).
  int piece = -1, pieces = 0, pslot = 0, punit = 0;
  if (p.cut) {
    const int normal_slots = ((p.batch + NUM_XCD - 1) / NUM_XCD) * p.m_tiles;
    const XcdCut cut = xcd_cut(p.batch, p.m_tiles, xcd);
    if (slot >= normal_slots) {
      const int j = slot - normal_slots;
      if (j >= cut.left * cut.pieces) return;
      pieces = cut.pieces;
      punit = j / pieces;
      piece = j % pieces;
      pslot = xcd * CUS_PER_XCD + j;
      slot = cut.whole + punit;
    } else if (cut.left && slot >= cut.whole) {
      return;
    }
  }
  const int round = slot / p.m_tiles;
  const int grank = NUM_XCD * round + ((round & 1) ? NUM_XCD - 1 - xcd : xcd);
  if (grank >= p.batch * p.num_splits) return;
  const int mt = slot % p.m_tiles;
  // Equal splits: requests longest first, then their splits.  Geometric splits: every
  // request's split 0 (the largest) first, then every split 1, ...
  const bool geo = p.split_ratio < 1.0f;
  const int rank = geo ? grank % p.batch : grank / p.num_splits;
  const int split = geo ? grank / p.batch : grank % p.num_splits;
  // ---- this request: lengths, packed offsets and status, from its record ----------
  const ReqRec* const rec = p.req + rank;
  const int flag = __builtin_amdgcn_readfirstlane(rec->flag);
  if (flag) {
    if (tid == 0 && p.status) atomicOr(p.status, flag);
    return;
  }
  const int T = __builtin_amdgcn_readfirstlane(rec->q_len);
  const int P = __builtin_amdgcn_readfirstlane(rec->prefix_len);
  const int64_t qoff = uniform64(rec->qoff);
  const int64_t kvoff = uniform64(rec->kvoff);
  const int64_t tbase = uniform64(rec->tbase);
  const int H = p.num_heads;
  const int rows = T * H;
  const int m0 = mt * BM;
  if (m0 >= rows) return;

  // ---- this lane's query row and node ----------------------------------------------
  const int row = m0 + wave * 32 + (lane & 31);
  const bool row_ok = row < rows;
  const int crow = row_ok ? row : rows - 1;
  const int node = crow / H;

  // ---- key range of this split (or piece) --------------------------------------------
  const int S = p.num_splits;
  // whole 32-key tiles, so every split starts on a V^T tile boundary
  int k_begin, k_end;
  if (piece < 0) {
    k_begin = split_begin(P, S, p.split_ratio, split);
    k_end = (split == S - 1) ? P + T : split_begin(P, S, p.split_ratio, split + 1);
  } else {  // one split: piece `piece` of `pieces` equal runs of whole tiles
    const int per = ((P + T + BN - 1) / BN + pieces - 1) / pieces;
    k_begin = min(piece * per * BN, P + T);
    k_end = min((piece + 1) * per * BN, P + T);
    if (piece == 0 && tid == 0) {  // where the piece merge writes this unit's rows
      p.piece_desc[2 * (xcd * CUS_PER_XCD + punit)] = qoff * H + m0;
      p.piece_desc[2 * (xcd * CUS_PER_XCD + punit) + 1] = min(BM, rows - m0);
    }
  }
  const int64_t grow = qoff * H + crow;  // global query row
  if (piece >= 0 && k_end <= k_begin) {
    // empty piece: partial = (0, -inf)
    if (row_ok) {
      const int64_t prow = (int64_t)pslot * BM + (row - m0);
      float* po = p.piece_o + prow * DL;
      for (int f = h * 4; f < DL; f += 8) *(float4*)(po + f) = make_float4(0.f, 0.f, 0.f, 0.f);
      if (h == 0) p.piece_lse[prow] = -INFINITY;
    }
    return;
  }
  if (k_end <= k_begin) {
    // empty split: partial = (0, -inf)
    if (row_ok) {
      float* po = p.part_o + ((int64_t)split * p.total_q * H + grow) * DL;
      for (int f = h * 4; f < DL; f += 8) *(float4*)(po + f) = make_float4(0.f, 0.f, 0.f, 0.f);
      if (h == 0) p.part_lse[(int64_t)split * p.total_q * H + grow] = -INFINITY;
    }
    return;
  }

  const char* k_rope = (const char*)p.k_rope + kvoff * (DR * 2);  // this request's rows
  // Tiles are 32-aligned in the request's key stream (the fp16 latent tiles are); a split
  // whose range starts mid-tile (only the last split, when the prefix is short) masks the
  // keys before its range.
  const int k_first = k_begin;
  k_begin &= ~(BN - 1);
  const int key_last = k_end - 1;
  const int n_tiles = (k_end - k_begin + BN - 1) / BN;
  const int mask_from = min(P, k_end);  // tiles ending at or before this key are unmasked
  const float c = p.scale_log2 > 0.0f ? p.scale_log2 : (p.scale_log2 < 0.0f ? -p.scale_log2 : 1.0f);

  // ---- the prologue's memory traffic, all in flight together ----------------------
  // the rope part of Q straight into the fragments, the request's parents, tile 0 into
  // stage 0 and the first half of the latent part of this wave's Q rows into its staging
  // area.
  u32x4 qf[36];
  {
    const char* qr = (const char*)p.q_rope + grow * (DR * 2);
#pragma unroll
    for (int ks = 32; ks < 36; ++ks) qf[ks] = *(const u32x4*)(qr + (2 * ks + h - 64) * 16);
  }
  const int pa = tid < T ? p.tree_parent[qoff + tid] : -1;
  const char* k16_split = (const char*)p.k16 + (tbase + k_begin / BN) * TILE_BYTES;
  issue_tile<0>(k16_split, k_rope, k_begin, key_last, wave, lane);
  const QStage qs(p.q_lat, qoff * H, m0 + wave * 32, rows, wave, lane);
  qs.issue<0>();

  // ---- parents -> LDS, validated -------------------------------------------------
  if (tid == 0) sFlag = 0;
  lds_barrier();
  if (tid < T) {
    const bool ok = tid == 0 ? pa == -1 : (pa >= 0 && pa < tid);
    sParent[tid] = ok ? pa : -1;
    if (!ok) atomicOr(&sFlag, ST_BAD_PARENT);
  }
  lds_barrier();
  const int pflag = __builtin_amdgcn_readfirstlane(sFlag);
  if (pflag) {
    __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS may land after the workgroup ends
    if (tid == 0 && p.status) atomicOr(p.status, pflag);
    return;
  }

  // ---- Q fragments (B operand of S^T = K Q^T) ----------------------------------------
  // Read the first half of the latent Q, reload the area with the second half, and
  // convert the first half while that copy is in flight.  (Explicit waits: the copies
  // write LDS behind the compiler's back.)
  __builtin_amdgcn_s_waitcnt(0);
  qs.read<0>(qf);
  __builtin_amdgcn_s_waitcnt(0);  // LDS reads done before the area is refilled
  qs.issue<1>();
  float qmax = 0.0f;
  q_to_fp16<0>(qf, qmax);
  // this lane's node's ancestor-or-self mask, also while the copy is in flight
  uint64_t anc = 0;
  for (int x = node, hops = 0; x >= 0 && hops <= MAX_QLEN; ++hops) {
    if (x < 64) anc |= 1ull << x;
    x = sParent[x];
  }
  __builtin_amdgcn_s_waitcnt(0);
  qs.read<1>(qf);
  q_to_fp16<16>(qf, qmax);
  // a query value outside fp16's range: the bf16 path's contract is broken (the
  // pre-pass flags latent keys the same way)
  if (__builtin_amdgcn_ballot_w64(row_ok && !(qmax < 65504.0f)) && lane == 0 && p.status)
    atomicOr(p.status, ST_RANGE);
  // The softmax takes a positive scale.  A negative one is moved into Q by flipping
  // every sign bit (exact: each score is then exactly negated); a zero one by zeroing
  // Q (every score is then exactly 0) with scale 1.
  {
    const unsigned flip = p.scale_log2 < 0.0f ? 0x80008000u : 0u;
    const unsigned keep = p.scale_log2 == 0.0f ? 0u : 0xffffffffu;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks)
#pragma unroll
      for (int d = 0; d < 4; ++d) qf[ks][d] = (qf[ks][d] & keep) ^ flip;
  }

  f32x16 o[16];
#pragma unroll
  for (int fb = 0; fb < 16; ++fb) o[fb] = f32x16{};
  RowState st{-INFINITY, 0.0f, 1.0f, false};

  // Pipeline: trip j runs the softmax of tile j (stage j % 3), then the scores of tile
  // j+1 interleaved with the PV of tile j, while the DMA of tile j+2 is in flight.  One
  // barrier per tile (trip 0's waits for tile 1).
  // Trip -1 runs the same stream as every other trip: tile 0's scores and softmax, the copy
  // of tile 1, and a PV of zero P over a zeroed stage 2 (a no-op on O).  So tile 0 needs
  // no code of its own: a second copy of the softmax or of the PV would cost the output
  // accumulators their fixed AGPRs.  Stage 2 held Q staging areas: every wave is done
  // with them after this barrier.
  __syncthreads();
  for (int i = tid; i < K16_U4; i += NTHR) sK16c[i] = u32x4{0u, 0u, 0u, 0u};
  for (int i = tid; i < 4 * 2 * 64; i += NTHR) sP[1][i] = u32x4{0u, 0u, 0u, 0u};
  if (tid < 2) sResc[tid] = -1;

  TileLoop tl{k_rope, k16_split, k_begin, k_first, k_end, key_last, n_tiles, mask_from,
              P, node, anc, c, tid, wave, lane};
  f32x16 s_cur = {};
  // Trip j works on tile j in stage (j + 3) % 3.
  for (int j = -1; j < n_tiles; j += 3) {
    tl.iteration<2>(j, s_cur, o, st, qf);
    if (j + 1 >= n_tiles) break;
    tl.iteration<0>(j + 1, s_cur, o, st, qf);
    if (j + 2 >= n_tiles) break;
    tl.iteration<1>(j + 2, s_cur, o, st, qf);
  }
  mfma_drain();

  // ---- finalize -------------------------------------------------------------------
  // The softmax lanes of a row (its owner wave) hold l and m; every wave holds 128
  // features of all 128 rows of O.  1 / l goes to the other waves through LDS.
  const float l_tot = pair_sum(st.l);
  // A cut piece may hold only tree-tail keys that a row cannot see: its partial is then
  // (0, -inf), as for an empty split.  (A whole split always holds the node itself.)
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse = l_tot > 0.0f ? st.m * LN2 + logf(l_tot) : -INFINITY;
  if (lane < 32) sInv[wave * 32 + lane] = inv;
  // The tile ring is free once every wave has finished the last tile (the last trips'
  // copies read nothing and are done at once).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // The row's lse, before the output (no wait after it then holds the output stores
  // back), addressed from the tile's uniform base and a lane id recomputed here, so that
  // no per-lane 64-bit address stays live across the KV loop.
  int el = lane;  // the lane id, recomputed: lane-derived offsets are not kept across the loop
  asm volatile("" : "+v"(el));
  {
    const int rloc = wave * 32 + (el & 31);  // row within the row tile
    float* const lse_tile = (piece >= 0 ? p.piece_lse + (int64_t)pslot * BM
                             : S == 1  ? p.out_lse + qoff * H + m0
                                       : p.part_lse + (int64_t)split * p.total_q * H + qoff * H + m0);
    if (m0 + rloc < rows && (el >> 5) == 0) {
      lse_tile[rloc] = lse;
      // a piece's lse may be -inf (no visible key); NaN still means non-finite data, and
      // the piece merge leaves such rows unwritten
      if ((piece < 0 ? !(fabsf(lse) < INFINITY) : __builtin_isnan(lse)) && p.status)
        atomicOr(p.status, ST_NONFINITE);
    }
  }
  const int trows = min(BM, rows - m0);  // rows of this row tile that exist
  // The workgroup's rows are consecutive global rows; this wave writes features
  // [128 w, 128 w + 128) of each.
  float* const out = (piece >= 0 ? p.piece_o + (int64_t)pslot * BM * DL
                      : S == 1  ? p.out_lat + (qoff * H + m0) * DL
                                : p.part_o + ((int64_t)split * p.total_q * H + qoff * H + m0) * DL) +
                     wave * 128;
  // The accumulator layout gives each lane 16-byte pieces of one row, so direct stores
  // would touch 32 rows per instruction.  Instead each wave passes its block through LDS,
  // one row block (32 rows x 128 features) at a time, and every store instruction then
  // writes 512 contiguous bytes of two rows.
  LDS_AS char* stage = (LDS_AS char*)(LDS_AS void*)((wave < 2) ? sK16a : sK16b) + (wave & 1) * EPI_WAVE_BYTES;
  const int r = el & 31, eh = el >> 5;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if (rb * 32 >= trows) continue;
    // keep each row block's accumulator reads inside it: read all at once, the 256
    // values would not fit the VGPRs next to the accumulators
    __builtin_amdgcn_sched_barrier(0);
    const float ir = sInv[rb * 32 + r];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      const f32x16 t = read_acc_here(o[4 * fb + rb]);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = {t[4 * q4] * ir, t[4 * q4 + 1] * ir, t[4 * q4 + 2] * ir,
                         t[4 * q4 + 3] * ir};
        *(LDS_AS f32x4*)(stage + r * EPI_ROW_BYTES + (fb * 32 + q4 * 8 + eh * 4) * 4) = v;
      }
    }
    wave_sync();
    f32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v[i] = *(const LDS_AS f32x4*)(stage + (2 * i + eh) * EPI_ROW_BYTES + r * 16);
    float* dst = out + (int64_t)(rb * 32 + eh) * DL + r * 4;
    // streaming stores: the output is not read again by this kernel
    if (rb * 32 + 32 <= trows) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __builtin_nontemporal_store(v[i], (f32x4*)(dst + (int64_t)(2 * i) * DL));
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (rb * 32 + 2 * i + eh < trows)
          __builtin_nontemporal_store(v[i], (f32x4*)(dst + (int64_t)(2 * i) * DL));
    }
    wave_sync();
  }
}

}  // namespace

int rows_per_block_bf16() { return BM; }

hipError_t launch_verify_bf16(const VerifyParams& p, hipStream_t stream) {
  const int64_t groups = (int64_t)p.batch * p.num_splits;
  if (p.cut && (p.num_splits != 1 || !p.piece_o || !p.piece_lse || !p.piece_desc))
    return hipErrorInvalidValue;
  if (p.cut && p.piece_slots != cut_piece_slots(p.batch)) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)NUM_XCD * ((groups + NUM_XCD - 1) / NUM_XCD) * p.m_tiles +
                         (p.cut ? PIECE_SLOTS : 0);
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(verify_attn_bf16_kernel, dim3((unsigned)blocks), dim3(NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kdt
