// attn_fwd_kernel.h -- the tiled SageAttention kernel for gfx950 (templates;
// attn_fwd_d*_*.hip instantiate them per head dimension and P~V mode so that
// the variants compile in parallel, attn_fwd.hip dispatches).
//
// "SageAttention: Accurate 8-Bit Attention for Plug-and-Play Inference
// Acceleration" (paper detail page), §3 Algorithm 1 (SAGEAttn-B) and §4
// Eq. 4-5: for each query block, walk the KV tiles in ascending order,
// S = INT8 Q^ K^T (INT32) * delta_Q * delta_K, online softmax (running max m,
// running sum l, output rescaled by exp(m_old - m_new)), then P~V in FP16 --
// or in FP8 E4M3 with a static delta_P = 1/448 and a per-channel delta_V, as in
// the "8+8" variant of the "SageAttention2++ ..." review page (section 三) --
// accumulated in FP32 (gfx950 has no FP16-accumulator MFMA), and finally
// O = O / l.  The all-INT8 variant (detail page, §3 Figure 5) quantises P~
// with the static delta_P = 1/127 (§7) and V per channel to INT8.  Every
// tile's product P^ V^ then has the same scale delta_P delta_V, so while a
// row's max stands the products add up exactly in the INT32 accumulator; when
// the max grows the accumulator is rescaled by alpha (rounded to an integer),
// O = alpha O + P^ V^ as Eq. 4-5 write it.  Heads longer than 2^17 keys, where
// INT32 could overflow, convert each tile's product to float instead.
//
// MI355X mapping
// * Workgroup = 4 wavefronts = 128 query rows = one delta_Q block of one (b, h)
//   (FP16 P~V, non-causal, d = 128: 8 wavefronts, two blocks, sharing tiles).
//   Each wavefront owns 32 query rows for the whole KV walk.
// * Scores are computed transposed, S^T = K^ Q^T, with v_mfma_i32_32x32x32_i8:
//   in the 32x32 accumulator lane l holds query l%32 and keys
//   8*(r/4) + 4*(l/32) + r%4 (r = register 0..15).  That is exactly the B
//   operand layout of O^T = V^T P~^T (v_mfma_f32_32x32x16_f16, or
//   v_mfma_scale_f32_32x32x64_f8f6f4 for FP8, two v_mfma_i32_32x32x32_i8 over
//   the two 32-key halves for INT8), so P~ goes from the softmax to
//   the second MFMA without leaving registers; V is stored pre-permuted (see
//   sage_quant_v) so that its A operand is one 16-byte LDS read per lane.
// * Row reductions (max over keys) are in-lane over 32 values plus one
//   v_permlane32_swap between lanes l and l^32.  The max runs on the INT32
//   scores (exact, and monotone under the positive scale).
// * The dequantisation scale and log2(e) are folded into one scalar per KV
//   tile: P~ = exp2(s * c_j - m) with c_j = delta_Q delta_K[j] log2(e).  For
//   FP8, log2(448) is folded into the same subtraction so the MFMA operand is
//   448 P~ directly, and l is kept in the same units.
// * K^ and prepared-V tiles go from HBM straight into LDS (buffer_load ...
//   lds, XOR-swizzled rows; V double-buffered, K^ in three slots in FP16
//   mode), one step ahead of their use.  The copies are issued from inline
//   assembly: the compiler would otherwise make every LDS read of the current
//   tiles wait for them.
// * FP16 mode reads the INT32 accumulator as a float with no instruction
//   (it starts from the bit pattern of 1.5 * 2^23) and, in steady-state
//   steps, takes no max at all: the exps use the running max as it stands and
//   the row sum checks them (a rare recompute otherwise).
// * The output rescale by alpha is skipped when no row of the wavefront has a
//   new maximum (alpha == 1 exactly), which is bit-identical.
// * With Q smoothed per block (SQ, see smooth_q.hip), each K^ tile carries the
//   block's 64 compensation values C (INT32, 256 bytes) in its LDS slot, and
//   the INT32 accumulation of S starts from them instead of from a constant.
#pragma once

#include <type_traits>
#include <utility>

#include "sage_common.h"
#include "sage_launch.h"

namespace sage {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448)
constexpr float kLog2_127 = 6.988684686772166f;   // log2(127)

template <int D>
struct KTile {
  static constexpr int BYTES = kKvTile * D;   // 64 keys x d int8
  static constexpr int CHUNKS = BYTES / 16;
  static constexpr int CPR = D / 16;          // 16-byte chunks per key row
  __device__ static __forceinline__ int lds_off(int key, int kc) {
    return key * D + ((kc ^ row_swizzle<D>(key)) << 4);
  }
};

template <int D, int PV>
struct VTile {
  static constexpr int ROWB = PV == kPvFp16 ? 128 : 64;
  static constexpr int BYTES = D * ROWB;
  static constexpr int CHUNKS = BYTES / 16;
};

// Q^ B-operand fragment for the wavefront's 32 rows: lane (n = l%32, h = l/32)
// holds bytes [32 t + 16 h, +16) of query row q0 + n for each d-step t.
template <int D>
__device__ __forceinline__ void load_q_frag(v4i (&qf)[D / 32], const int8_t* __restrict__ q_bh,
                                            int qrow, int N, int hh) {
  const int8_t* qp = q_bh + (size_t)qrow * D + 16 * hh;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
    qf[t] = qrow < N ? *reinterpret_cast<const v4i*>(qp + 32 * t) : v4i{0, 0, 0, 0};
}

// One 32-key x 32-query block of S^T (INT32) from the K^ tile in LDS,
// accumulated onto `init` (zero, or the magic bias of FP16 mode).
template <int D>
__device__ __forceinline__ v16i qk_block(const v4i (&qf)[D / 32], const uint8_t* kb, int blk,
                                         int n, int hh, const v16i& init) {
  v16i acc = init;
  const int row = 32 * blk + n;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const v4i a = *reinterpret_cast<const v4i*>(kb + KTile<D>::lds_off(row, 2 * t + hh));
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[t], acc, 0, 0, 0);
  }
  return acc;
}

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource for gfx9: base address, stride 0, byte-addressed
// records, default data format word.  The record count and every offset
// into the buffer are unsigned 32-bit: a resource spans less than 4 GiB, so
// the callers keep each one to a head's K^ (N d <= 2^31 bytes for N <= 2^24)
// or to a single tile.
constexpr int kBufferFlags = 0x00020000;
// Byte sizes and offsets at the longest sequence: a head's K^ is at most
// 2^31 bytes, so every K^ row offset (< N d) fits a signed 32-bit int and the
// record count an unsigned one; prepared V is addressed one tile (at most
// 16 KiB) per resource from a 64-bit base; the smoothed-Q seeds of one query
// block are 256 bytes per tile.
static_assert((uint64_t)kMaxN * 128 <= (1ull << 31), "K^ head offsets fit 32 bits");
static_assert((uint64_t)(kMaxN / kKvTile) * kKvTile * 4 < (1ull << 32), "seed rows fit 32 bits");
static_assert((uint64_t)kMaxN / kKvTile * kKvTile * 128 * 2 >= (1ull << 32),
              "a head's FP16 V can pass 4 GiB: V is addressed per tile");
__device__ __forceinline__ v4i buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4i{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
             __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)), (int)bytes, kBufferFlags};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}

// PER buffer_load_dwordx4 ... lds copies in one block: copy i writes 1 KiB
// of LDS at m0[i] (64 lanes x 16 bytes) from byte offset voff[i] + soff of
// the buffer rsrc.  The compiler only sees opaque code with no register
// outputs: it does not count these loads, so a later LDS read of a
// different tile does not wait for them; the caller waits explicitly
// (wait_lds_loads) before the barrier that publishes the tile.  Hazards
// handled here: an SGPR written by a vector instruction must not be read
// by a buffer load within 5 wait states, and M0 written by a scalar move
// must not be read by an LDS copy in the next wait state.
// M0 is a reserved register; these kernels use it only for LDS copies, each
// of which sets it right before use, so clobbering it here is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int PER>
__device__ __forceinline__ void lds_copy_x4(v4i rsrc, int soff, const uint32_t (&m0)[PER],
                                            const int (&voff)[PER]) {
  static_assert(PER == 1 || PER == 2 || PER % 4 == 0, "copies per block");
  if constexpr (PER > 4) {
#pragma unroll
    for (int g = 0; g < PER; g += 4) {
      const uint32_t m4[4] = {m0[g], m0[g + 1], m0[g + 2], m0[g + 3]};
      const int v4[4] = {voff[g], voff[g + 1], voff[g + 2], voff[g + 3]};
      lds_copy_x4<4>(rsrc, soff, m4, v4);
    }
  } else if constexpr (PER == 1) {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(m0[0]), "v"(voff[0]), "s"(rsrc), "s"(soff)
        : "memory", "m0");
  } else if constexpr (PER == 2) {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %4, %5 offen lds\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %3, %4, %5 offen lds"
        :
        : "s"(m0[0]), "s"(m0[1]), "v"(voff[0]), "v"(voff[1]), "s"(rsrc), "s"(soff)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %4, %8, %9 offen lds\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %5, %8, %9 offen lds\n\t"
        "s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %6, %8, %9 offen lds\n\t"
        "s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %7, %8, %9 offen lds"
        :
        : "s"(m0[0]), "s"(m0[1]), "s"(m0[2]), "s"(m0[3]), "v"(voff[0]), "v"(voff[1]),
          "v"(voff[2]), "v"(voff[3]), "s"(rsrc), "s"(soff)
        : "memory", "m0");
  }
}
#pragma clang diagnostic pop

// HBM -> LDS copies with buffer_load_dwordx4 ... lds: every lane moves 16
// bytes straight into LDS (no VGPR staging, scalar base and LDS address, one
// 32-bit lane offset); a wavefront writes 1 KiB of contiguous LDS per
// instruction, so the K^ row swizzle is applied by choosing each lane's
// source offset.  NW wavefronts share the work; `wave` must be uniform.
template <int D, int NW>
struct KLoader {
  static constexpr int PER = KTile<D>::CHUNKS / (64 * NW);
  static_assert(PER * 64 * NW == KTile<D>::CHUNKS, "wavefronts must tile the K^ tile");
  int row[PER], off[PER];   // per-lane source row and byte offset within the tile
  __device__ __forceinline__ KLoader(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int P = (i * NW + wave) * 64 + lane;   // LDS chunk this lane writes
      row[i] = P / KTile<D>::CPR;
      const int kc = (P % KTile<D>::CPR) ^ row_swizzle<D>(row[i]);
      off[i] = row[i] * D + kc * 16;
    }
  }
  // rs: buffer resource of the head's K^ (N*D bytes); kb: LDS byte address of
  // the tile slot.  Rows at or beyond N re-read row N-1 (their scores are
  // masked).  Offsets are below N*D <= 2^31 (N <= 2^24, D <= 128), so the
  // int arithmetic does not wrap.
  template <bool CLAMP>
  __device__ __forceinline__ void issue(v4i rs, int key0, int N, uint32_t kb, int wave) const {
    uint32_t m0[PER];
    int vo[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      m0[i] = kb + (i * NW + wave) * 1024;
      vo[i] = CLAMP ? min(key0 + row[i], N - 1) * D + (off[i] - row[i] * D) : off[i];
    }
    lds_copy_x4<PER>(rs, CLAMP ? 0 : key0 * D, m0, vo);
  }
};

// Prepared-V tiles are stored pre-swizzled, so their copy is linear.
template <int D, int PV, int NW>
struct VLoader {
  static constexpr int PER = VTile<D, PV>::CHUNKS / (64 * NW);
  static_assert(PER * 64 * NW == VTile<D, PV>::CHUNKS, "wavefronts must tile the V tile");
  // v_bh: the head's prepared V (tile t starts at byte t * VTile::BYTES, a
  // 64-bit offset: a head of 2^24 keys holds 4 GiB of FP16 V); vb: LDS byte
  // address of the tile slot.  The buffer resource covers the one tile.
  __device__ __forceinline__ static void issue(const uint8_t* v_bh, int tile, uint32_t vb,
                                               int wave, int lane) {
    uint32_t m0[PER];
    int vo[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      m0[i] = vb + (i * NW + wave) * 1024;
      vo[i] = ((i * NW + wave) * 64 + lane) * 16;
    }
    lds_copy_x4<PER>(buffer_rsrc(v_bh + (size_t)tile * VTile<D, PV>::BYTES, VTile<D, PV>::BYTES),
                     0, m0, vo);
  }
};

// Wait until this wavefront's HBM -> LDS copies have landed.
__device__ __forceinline__ void wait_lds_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int OUT>
__device__ __forceinline__ void store4(void* out, size_t idx, float a, float b, float c, float d) {
  if constexpr (OUT == 2) {
    *reinterpret_cast<v4f*>(static_cast<float*>(out) + idx) = v4f{a, b, c, d};
  } else if constexpr (OUT == 0) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) =
        uint2{pack_f16x2(a, b), pack_f16x2(c, d)};
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) =
        uint2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
  }
}

// P~ of one tile as the B operand of the P~V MFMA: FP16 = four 8-half steps
// (16 keys each), FP8 = one 32-byte operand covering the 64 keys, INT8 = the
// same 32 bytes, split into the 16-byte operands of the two 32-key halves.
template <int PV>
struct PTile;
template <>
struct PTile<kPvFp16> {
  v4i w[4];
};
template <>
struct PTile<kPvFp8> {
  v8i w;
};
template <>
struct PTile<kPvInt8> {
  v8i w;
};

// Four floats in [0, 255] -> four u8 codes, round to nearest even
// (v_cvt_pk_u8_f32), first value in the low byte.
__device__ __forceinline__ uint32_t pack_u8x4(float a, float b, float c, float d) {
  // every byte is written below, so the register may be a's own
  uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(a, 0u, __builtin_bit_cast(uint32_t, a));
  w = __builtin_amdgcn_cvt_pk_u8_f32(b, 1u, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(c, 2u, w);
  return __builtin_amdgcn_cvt_pk_u8_f32(d, 3u, w);
}

// Smoothed Q: the compensation values of a tile follow its K^ in the LDS
// slot (64 INT32 per 128-row query block of the workgroup, already carrying
// FP16 mode's magic bias); sqo is the byte offset of the wavefront's block's
// values.  The start value of 32-key block blk in the accumulator layout:
// register r holds key 32 blk + 8 (r/4) + 4 hh + r%4.
constexpr int kSqTileBytes = kKvTile * 4;
template <int D>
__device__ __forceinline__ v16i sq_init(const uint8_t* kb, int blk, int hh, int sqo) {
  const int32_t* c =
      reinterpret_cast<const int32_t*>(kb + KTile<D>::BYTES + sqo) + 32 * blk + 4 * hh;
  v16i r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const v4i x = *reinterpret_cast<const v4i*>(c + 8 * j);
    r[4 * j] = x[0]; r[4 * j + 1] = x[1]; r[4 * j + 2] = x[2]; r[4 * j + 3] = x[3];
  }
  return r;
}

// S^T = K^ Q^T for one 64-key tile: two 32x32 INT32 blocks.
template <int D, bool SQ>
__device__ __forceinline__ void qk_tile(v16i (&s)[2], const v4i (&qf)[D / 32], const uint8_t* kb,
                                        int n, int hh, const v16i& init,
                                        int sqo) {
  s[0] = qk_block<D>(qf, kb, 0, n, hh, SQ ? sq_init<D>(kb, 0, hh, sqo) : init);
  s[1] = qk_block<D>(qf, kb, 1, n, hh, SQ ? sq_init<D>(kb, 1, hh, sqo) : init);
}

// FP16 mode converts scores to float without an instruction: the INT32
// accumulation starts from the bit pattern of 1.5 * 2^23, so the accumulator
// read as a float is exactly 1.5 * 2^23 + s (|s| <= 127^2 d < 2^22 keeps it in
// the binade where the float spacing is 1).  With c = delta_Q delta_K log2(e)
// rounded to 21 significant bits, K0 = 1.5 * 2^23 * c is exact, and the
// exponent argument s c - m becomes one fused multiply-add
// fma(x, c, -(K0 + m)); the running max m is kept on a grid of twice the
// float spacing at the workgroup's largest K0, which makes K0 + m exact, so
// the argument is the correctly rounded s c - m as before.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
constexpr int kNegInfBits = (int)0xFF800000u;   // -infinity

// Grid of the FP16-mode running max: step (a power of two) and 1/step.
struct MaxGrid {
  float step, inv;
};

struct TileScale {
  float c;    // delta_Q delta_K log2(e) (FP16 mode: rounded to 21 significant bits)
  float k0;   // FP16 mode: kMagic * c (exact); unused in FP8 mode
};

template <int PV>
__device__ __forceinline__ TileScale tile_scale(float cq, float dk) {
  if constexpr (PV == kPvFp16) {
    const float c = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, cq * dk) & ~7u);
    return TileScale{c, kMagic * c};
  } else {
    return TileScale{cq * dk, 0.f};
  }
}

// In FP16 mode the running max used for P~ is refreshed only when a tile's max
// exceeds it by more than this many log2 units; until then P~ may reach
// 2^kLazyMax (far inside FP16 range) and the output rescale is skipped.  The
// result is the same softmax up to rounding.  FP8 mode keeps the exact max
// because P^ = 448 P~ must not exceed the E4M3 range.
constexpr float kLazyMax = 8.0f;

// Steady-state FP16 tiles go further and skip the max: their exps use the
// running max as it stands, and the row sum, which is computed anyway, checks
// the result.  When some lane's sum over its 32 keys exceeds this bound (so a
// P~ of the tile may exceed it, or overflowed FP16 to infinity) the wavefront
// recomputes the tile's scores from K^ (still in LDS) and takes the max-based
// rule above; otherwise every P~ of the tile is at most 2^14, well inside FP16
// range, and the state changes by l += sum only.
constexpr float kOptimisticSum = 16384.0f;

// K^ tile slots in LDS: three in FP16 mode, so that the tile whose softmax a
// step runs is still resident when the step may have to recompute its scores.
template <int PV>
constexpr int kKSlots = PV == kPvFp16 ? 3 : 2;

// Visibility bits of a lane's 32 scores of a tile (bit 16 blk + r: key
// key0 + 32 blk + 8 (r/4) + 4 hh + r%4) for the keys at most `last`.
__device__ __forceinline__ uint32_t key_mask(int key0, int hh, int last) {
  uint32_t m = 0u;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      m |= (uint32_t)(key0 + 32 * blk + 8 * (r >> 2) + 4 * hh + (r & 3) <= last) << (16 * blk + r);
  return m;
}

// Online softmax of one tile: returns alpha = exp2(m_old - m_new) and writes
// P~ (FP8: 448 P~; INT8: round(127 P~)) into the MFMA operand.  MASK selects
// the variant that hides the keys whose bit in `keep` (key_mask layout) is
// clear (keys >= N, causal keys > query); a fully masked tile leaves the
// state unchanged (P~ = 0, alpha = 1).
template <int PV, bool MASK>
__device__ __forceinline__ float softmax_tile(v16i (&s)[2], float& m_run, float& l_run,
                                              PTile<PV>& pt, TileScale ts, MaxGrid grid,
                                              uint32_t keep, int hh) {
  constexpr bool F16 = PV == kPvFp16;
  if constexpr (MASK) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        // FP16: the biased scores are positive floats and a hidden one
        // becomes -infinity, below all of them as an integer too, whose exp
        // is exactly 0 (for c > 0, below)
        if (!((keep >> (16 * blk + r)) & 1u)) s[blk][r] = F16 ? kNegInfBits : INT32_MIN;
  }
  if constexpr (MASK && F16) {
    // c = 0 (an all-zero delta_Q or delta_K block) would turn -inf * c into
    // NaN; the smallest normal float gives the same exps to float precision
    ts.c = fmaxf(ts.c, __FLT_MIN__);
    ts.k0 = kMagic * ts.c;
  }
  // row max: chain of 3-input maxima over the lane's 32 scores, then the pair
  // (in FP16 mode on the bit patterns of positive floats, which order alike)
  int mx = max(s[0][0], s[0][1]);
#pragma unroll
  for (int i = 2; i < 32; i += 2) mx = max(mx, max(s[i >> 4][i & 15], s[i >> 4][(i & 15) + 1]));
  mx = pair_max_i32(mx);
  float m_new, nb;
  if constexpr (F16) {
    const float mt = (__builtin_bit_cast(float, mx) - kMagic) * ts.c;
    m_new = mt > m_run + kLazyMax ? __builtin_ceilf(mt * grid.inv) * grid.step : m_run;
    nb = -(ts.k0 + m_new);
  } else {
    const float mt = (float)mx * ts.c;
    m_new = fmaxf(m_run, mt);
    nb = (PV == kPvInt8 ? kLog2_127 : kLog2_448) - m_new;
    if constexpr (PV == kPvInt8) {
      // 127 P~ of the row's largest score must round to at most 127 (128
      // would read as -128 in the INT8 MFMA): when |m| is so large that the
      // float32 rounding of nb lifts it, lower nb by the excess.  Every other
      // score's argument is at most this one's (fma is monotone in s).
      const float tmax = __builtin_fmaf((float)mx, ts.c, nb);
      nb -= fmaxf(tmax - kLog2_127, 0.f);
    }
  }
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);

  float p[2][16];
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // copy the element to a scalar first: clang mis-lowers a bit_cast
      // whose operand is an ext_vector element (it reads element 0)
      const int si = s[blk][r];
      const float x = F16 ? __builtin_bit_cast(float, si) : (float)si;
      float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x, ts.c, nb));
      if constexpr (MASK && !F16) e = ((keep >> (16 * blk + r)) & 1u) ? e : 0.f;
      p[blk][r] = e;
      if constexpr (!F16) ls[r & 3] += e;
    }

  if constexpr (F16) {
    // step S (16 keys) = registers 8*(S%2) .. +7 of block S/2; the row sum
    // adds the fp16 values the MFMA consumes (v_dot2 with (1, 1): two keys
    // per instruction, float32 accumulation).
    const v2h one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int S = 0; S < 4; ++S) {
      const int blk = S >> 1, r0 = 8 * (S & 1);
      pt.w[S] = v4i{(int)pack_f16x2(p[blk][r0 + 0], p[blk][r0 + 1]),
                    (int)pack_f16x2(p[blk][r0 + 2], p[blk][r0 + 3]),
                    (int)pack_f16x2(p[blk][r0 + 4], p[blk][r0 + 5]),
                    (int)pack_f16x2(p[blk][r0 + 6], p[blk][r0 + 7])};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // copy the element to a scalar first: clang mis-lowers a bit_cast
        // whose operand is an ext_vector element (it reads element 0)
        const int pair = pt.w[S][i];
        ls[i] = __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, pair), one, ls[i], false);
      }
    }
  } else {
    // byte 16*blk + r <-> register r of block blk
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int blk = w >> 2, r0 = 4 * (w & 3);
      pt.w[w] = PV == kPvFp8
                    ? (int)pack_fp8x4(p[blk][r0], p[blk][r0 + 1], p[blk][r0 + 2], p[blk][r0 + 3])
                    : (int)pack_u8x4(p[blk][r0], p[blk][r0 + 1], p[blk][r0 + 2], p[blk][r0 + 3]);
    }
  }
  l_run = l_run * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
  m_run = m_new;
  return alpha;
}

// O^T += V^T P~^T for one tile, V from LDS.  INT8 with ACC: O holds the INT32
// sum of the products (bit patterns in the float registers) and the MFMAs add
// to it directly.  INT8 without ACC: O = alpha O + P^ V^ with the INT32
// product of the tile converted to float (|P^ V^| <= 64 127^2 < 2^24, exact),
// alpha being the rescale factor of this tile's softmax.
template <int D, int PV, bool ACC = false>
__device__ __forceinline__ void pv_tile(v16f (&o)[D / 32], const PTile<PV>& pt,
                                        const uint8_t* vb, int n, int hh, float alpha = 1.f) {
  constexpr int NCB = D / 32;
  if constexpr (PV == kPvFp16) {
#pragma unroll
    for (int S = 0; S < 4; ++S) {
      const v8h pb = __builtin_bit_cast(v8h, pt.w[S]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int row = 32 * cb + n;
        const v4i a = *reinterpret_cast<const v4i*>(
            vb + row * 128 + (((2 * S + hh) ^ row_swizzle<128>(row)) << 4));
        o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), pb, o[cb], 0,
                                                       0, 0);
      }
    }
  } else if constexpr (PV == kPvFp8) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int row = 32 * cb + n;
      const int sw = row_swizzle<64>(row);
      const v4i a0 = *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh) ^ sw) << 4));
      const v4i a1 = *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh + 1) ^ sw) << 4));
      const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      // scale operands 127 = E8M0 exponent of 1.0 (no block scaling)
      o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pt.w, o[cb], 0, 0, 0, 127, 0, 127);
    }
  } else if constexpr (ACC) {
    const v4i plo = {pt.w[0], pt.w[1], pt.w[2], pt.w[3]};
    const v4i phi = {pt.w[4], pt.w[5], pt.w[6], pt.w[7]};
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int row = 32 * cb + n;
      const int sw = row_swizzle<64>(row);
      const v4i a0 = *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh) ^ sw) << 4));
      const v4i a1 = *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh + 1) ^ sw) << 4));
      v16i r = __builtin_bit_cast(v16i, o[cb]);
      r = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, plo, r, 0, 0, 0);
      r = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, phi, r, 0, 0, 0);
      o[cb] = __builtin_bit_cast(v16f, r);
    }
  } else {
    const v4i plo = {pt.w[0], pt.w[1], pt.w[2], pt.w[3]};
    const v4i phi = {pt.w[4], pt.w[5], pt.w[6], pt.w[7]};
    // two channel blocks in flight: the MFMA pair of block cb + 1 is issued
    // before block cb's product is converted and added
    v16i acc[2];
    auto product = [&](int cb) __attribute__((always_inline)) {
      const int row = 32 * cb + n;
      const int sw = row_swizzle<64>(row);
      const v4i a0 = *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh) ^ sw) << 4));
      const v4i a1 = *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh + 1) ^ sw) << 4));
      v16i& r = acc[cb & 1];
      r = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, plo, v16i{}, 0, 0, 0);
      r = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, phi, r, 0, 0, 0);
    };
    product(0);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      if (cb + 1 < NCB) product(cb + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // copy the element to a scalar first (see softmax_tile)
        const int pr = acc[cb & 1][r];
        o[cb][r] = __builtin_fmaf(o[cb][r], alpha, (float)pr);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int D>
__device__ __forceinline__ void rescale(v16f (&o)[D / 32], float alpha) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) o[cb] *= alpha;
  }
}

// Nearest integer to f, halves rounded up (v_cvt_rpi_i32_f32: floor(f + 0.5)),
// one instruction; the compiler has no builtin for it.
__device__ __forceinline__ int round_half_up_i32(float f) {
  int r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(f));
  return r;
}

// INT8 with ACC: rescale the INT32 sums by alpha, rounded to the nearest
// integer.  Exact where alpha == 1 and |sum| < 2^24.  Three instructions per
// value: a wavefront pays this whenever one of its 32 rows gets a new max.
template <int D>
__device__ __forceinline__ void rescale_i32(v16f (&o)[D / 32], float alpha) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      v16i x = __builtin_bit_cast(v16i, o[cb]);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int xi = x[r];   // element to a scalar first (see softmax_tile)
        x[r] = round_half_up_i32((float)xi * alpha);
      }
      o[cb] = __builtin_bit_cast(v16f, x);
    }
  }
}

// ---------------------------------------------------------------------------
// The steady-state step as an explicit instruction schedule.
//
// A step issues NQK INT8 MFMAs (S(j+2)) and NPV P~V MFMAs (tile j), and runs
// the softmax of S(j+1), whose scores were produced one step earlier.  The
// MFMAs are spread over "slots"; every slot issues one MFMA (its LDS operand
// was read two slots earlier) followed by a slice of the softmax's vector
// micro-ops, and slots are separated by scheduling barriers.  Each wavefront
// thus alternates MFMA and VALU issue, keeping both units busy.  The order
// only affects timing: the arithmetic is the same as softmax_tile/qk_tile/
// pv_tile (unmasked tiles only).  INT8 P~V runs here only with O kept as the
// INT32 sum (pv_tile's ACC form): two MFMAs per channel block, the 32-key
// halves, issued for all blocks' first halves before any second half.
template <int D, int PV>
struct StepPlan {
  static constexpr int TD = D / 32;                              // d-steps per QK block
  static constexpr int NCB = D / 32;                             // output channel blocks
  static constexpr int NQK = 2 * TD;
  static constexpr int NPV = PV == kPvFp16 ? 4 * NCB : PV == kPvInt8 ? 2 * NCB : NCB;
  static constexpr int NM = NQK + NPV;                           // MFMA slots
  // slot k issues a P~V MFMA iff the running PV quota steps up at k
  static constexpr bool is_pv(int k) { return ((k + 1) * NPV) / NM > (k * NPV) / NM; }
  static constexpr int index(int k) {   // index of the MFMA among its kind
    int c = 0;
    for (int i = 0; i < k; ++i) c += is_pv(i) == is_pv(k);
    return c;
  }
  // softmax micro-ops: NPRE maxima with the conversions (FP8, INT8: FP16
  // steady-state tiles skip the max), one combine, then the exps and packs,
  // then the finish
  static constexpr int NPRE = PV == kPvFp16 ? 0 : 48;
  static constexpr int NPACK = PV == kPvFp16 ? 16 : 8;
  // FP16: the 48 exp/pack micro-ops of the 16 score pairs g run as a
  // three-stage pipeline, arguments (A_g: two fma), exps (B_g) and pack +
  // row sum (C_g), in the order A_s, B_s-1, C_s-2 for s = 0, 1, ..., so that
  // no micro-op waits on the one just before it.  op16(v) = (stage, g).
  struct StageOp { int stage, g; };
  static constexpr StageOp op16(int v) {
    int k = 0;
    for (int s = 0; s < 18; ++s)
      for (int st = 0; st < 3; ++st) {
        const int g = s - st;
        if (g < 0 || g >= 16) continue;
        if (k++ == v) return StageOp{st, g};
      }
    return StageOp{-1, -1};
  }
  static constexpr int NU = NPRE + 1 + 32 + NPACK + 1;
  // first micro-op of slot k (cumulative instruction weight, spread evenly)
  static constexpr int weight(int u) {
    return u < NPRE ? 1 : u == NPRE ? (PV == kPvFp16 ? 1 : 10) : u < NPRE + 1 + 32 + NPACK ? 2 : 3;
  }
  static constexpr int total_weight() {
    int w = 0;
    for (int u = 0; u < NU; ++u) w += weight(u);
    return w;
  }
  static constexpr int first_uop(int k) {
    const int target = (k * total_weight()) / NM;
    int w = 0, u = 0;
    while (u < NU && w + weight(u) / 2 < target) w += weight(u++);
    return u;
  }
};

template <int D, int PV>
using OpReg = std::conditional_t<PV == kPvFp8, v8i, v4i>;

template <int D, int PV, bool SQ>
__device__ __forceinline__ void fused_step(v16f (&o)[D / 32], const v4i (&qf)[D / 32],
                                            v16i (&s_cur)[2], v16i (&s_new)[2],
                                            const PTile<PV>& p_cur, PTile<PV>& p_new,
                                            const uint8_t* kb, const uint8_t* kb_prev,
                                            const uint8_t* vb, float& m_run,
                                            float& l_run, TileScale ts, MaxGrid grid,
                                            const v16i& init, int n, int hh, int sqo) {
  using Plan = StepPlan<D, PV>;
  using Op = OpReg<D, PV>;
  constexpr int LA = 2;   // operand read lookahead (slots)
  Op ops[LA + 1];
  v16i cin[2];            // SQ: start values of the two 32-key blocks of S(j+2)

  // ---- MFMA side
  auto read_op = [&]<int K>() __attribute__((always_inline)) {
    Op& r = ops[K % (LA + 1)];
    constexpr int i = Plan::index(K);
    if constexpr (!Plan::is_pv(K)) {
      constexpr int blk = i % 2, t = i / 2;
      const v4i a = *reinterpret_cast<const v4i*>(kb + KTile<D>::lds_off(32 * blk + n, 2 * t + hh));
      if constexpr (PV != kPvFp8) r = a;
      else r = Op{a[0], a[1], a[2], a[3], 0, 0, 0, 0};
      if constexpr (SQ && t == 0) cin[blk] = sq_init<D>(kb, blk, hh, sqo);
    } else if constexpr (PV == kPvFp16) {
      constexpr int S = i / Plan::NCB, cb = i % Plan::NCB;
      const int row = 32 * cb + n;
      r = *reinterpret_cast<const v4i*>(vb + row * 128 +
                                        (((2 * S + hh) ^ row_swizzle<128>(row)) << 4));
    } else if constexpr (PV == kPvInt8) {
      constexpr int cb = i % Plan::NCB, half = i / Plan::NCB;
      const int row = 32 * cb + n;
      r = *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh + half) ^ row_swizzle<64>(row)) << 4));
    } else {
      constexpr int cb = i;
      const int row = 32 * cb + n;
      const int sw = row_swizzle<64>(row);
      const v4i a0 = *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh) ^ sw) << 4));
      const v4i a1 = *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh + 1) ^ sw) << 4));
      r = Op{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
  };
  auto do_mfma = [&]<int K>() __attribute__((always_inline)) {
    const Op& r = ops[K % (LA + 1)];
    constexpr int i = Plan::index(K);
    if constexpr (!Plan::is_pv(K)) {
      constexpr int blk = i % 2, t = i / 2;
      v4i a;
      if constexpr (PV != kPvFp8) a = r;
      else a = v4i{r[0], r[1], r[2], r[3]};
      s_new[blk] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
          a, qf[t], t == 0 ? (SQ ? cin[blk] : init) : s_new[blk], 0, 0, 0);
    } else if constexpr (PV == kPvFp16) {
      constexpr int S = i / Plan::NCB, cb = i % Plan::NCB;
      o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, r),
                                                     __builtin_bit_cast(v8h, p_cur.w[S]), o[cb],
                                                     0, 0, 0);
    } else if constexpr (PV == kPvInt8) {
      constexpr int cb = i % Plan::NCB, half = i / Plan::NCB;
      const v4i pb = half ? v4i{p_cur.w[4], p_cur.w[5], p_cur.w[6], p_cur.w[7]}
                          : v4i{p_cur.w[0], p_cur.w[1], p_cur.w[2], p_cur.w[3]};
      o[cb] = __builtin_bit_cast(
          v16f, __builtin_amdgcn_mfma_i32_32x32x32_i8(r, pb, __builtin_bit_cast(v16i, o[cb]), 0,
                                                      0, 0));
    } else {
      constexpr int cb = i;
      // scale operands 127 = E8M0 exponent of 1.0 (no block scaling)
      o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(r, p_cur.w, o[cb], 0, 0, 0, 127,
                                                              0, 127);
    }
  };

  // ---- softmax side (same arithmetic as softmax_tile, unmasked)
  constexpr bool F16 = PV == kPvFp16;
  constexpr int NPRE = Plan::NPRE;
  int mpart[4];
  float f[32], e[32], t[32];
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
  float m_new = 0.f, alpha = 1.f, nb = 0.f, lsum = 0.f;
  auto sc = [&](int i) __attribute__((always_inline)) -> int { return s_cur[i >> 4][i & 15]; };
  auto uop = [&]<int U>() __attribute__((always_inline)) {
    if constexpr (U < NPRE) {
      // FP8, INT8: triples of (max of two scores into one of 4 partial
      // maxima, two conversions).  The maxima are written as explicit
      // 3-input instructions (one per score pair after the first four):
      // left to the compiler, the chains get re-associated into pairwise
      // maxima first and take about five more instructions per step.
      constexpr int g = U / 3, r = U % 3;
      if constexpr (r == 0) {
        if constexpr (g < 4) {
          mpart[g] = max(sc(2 * g), sc(2 * g + 1));
        } else {
          asm("v_max3_i32 %0, %1, %2, %3"
              : "=v"(mpart[g & 3])
              : "v"(mpart[g & 3]), "v"(sc(2 * g)), "v"(sc(2 * g + 1)));
        }
      } else {
        f[2 * g + r - 1] = (float)sc(2 * g + r - 1);
      }
    } else if constexpr (U == NPRE) {
      if constexpr (F16) {
        // exps against the running max as it stands; the row sum continues
        // from the running total
        nb = -(ts.k0 + m_run);
        lsum = l_run;
      } else {
        int mx;
        asm("v_max3_i32 %0, %1, %2, %3" : "=v"(mx) : "v"(mpart[0]), "v"(mpart[1]), "v"(mpart[2]));
        mx = pair_max_i32(max(mx, mpart[3]));
        const float mt = (float)mx * ts.c;
        // the larger of two finite-or-(-inf) floats (m_run starts at -inf;
        // neither is a NaN), without the NaN quieting fmaxf adds
        asm("v_max_f32 %0, %1, %2" : "=v"(m_new) : "v"(m_run), "v"(mt));
        nb = (PV == kPvInt8 ? kLog2_127 : kLog2_448) - m_new;
        if constexpr (PV == kPvInt8) {
          // the row's largest 127 P~ rounds to at most 127 (see softmax_tile)
          const float tmax = __builtin_fmaf((float)mx, ts.c, nb);
          nb -= fmaxf(tmax - kLog2_127, 0.f);
        }
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      }
    } else if constexpr (U < NPRE + 1 + 32 + Plan::NPACK) {
      if constexpr (F16) {
        constexpr auto op = Plan::op16(U - NPRE - 1);
        constexpr int g = op.g;
        if constexpr (op.stage == 0) {
          t[2 * g] = __builtin_fmaf(__builtin_bit_cast(float, sc(2 * g)), ts.c, nb);
          t[2 * g + 1] = __builtin_fmaf(__builtin_bit_cast(float, sc(2 * g + 1)), ts.c, nb);
        } else if constexpr (op.stage == 1) {
          e[2 * g] = __builtin_amdgcn_exp2f(t[2 * g]);
          e[2 * g + 1] = __builtin_amdgcn_exp2f(t[2 * g + 1]);
        } else {
          // pair (2g, 2g+1) -> step g/4, element g%4
          uint32_t pk = pack_f16x2(e[2 * g], e[2 * g + 1]);
          // pin: keep this micro-op in its slot (otherwise the backend sinks
          // the softmax below the branch, out of the MFMA slots)
          asm volatile("" : "+v"(pk));
          p_new.w[g >> 2][g & 3] = (int)pk;
          const v2h one = {(_Float16)1.0f, (_Float16)1.0f};
          lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, pk), one, lsum, false);
        }
      } else {
        // FP8, INT8: exp of score i, and after every 4 scores their pack
        constexpr int v = U - NPRE - 1;
        constexpr int grp = v / 5, pos = v % 5;   // 4 exps + pack
        if constexpr (pos < 4) {
          constexpr int i = grp * 4 + pos;
          e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[i], ts.c, nb));
          ls[i & 3] += e[i];
        } else {
          constexpr int w = grp;
          uint32_t pk = PV == kPvFp8
                            ? pack_fp8x4(e[4 * w], e[4 * w + 1], e[4 * w + 2], e[4 * w + 3])
                            : pack_u8x4(e[4 * w], e[4 * w + 1], e[4 * w + 2], e[4 * w + 3]);
          asm volatile("" : "+v"(pk));
          p_new.w[w] = (int)pk;
        }
      }
    } else if constexpr (F16) {
      asm volatile("" : "+v"(lsum));
    } else {
      l_run = l_run * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
      m_run = m_new;
      asm volatile("" : "+v"(l_run));
    }
  };
  auto uops = [&]<int U0, int U1>() __attribute__((always_inline)) {
    [&]<int... U>(std::integer_sequence<int, U...>) __attribute__((always_inline)) {
      (uop.template operator()<U0 + U>(), ...);
    }(std::make_integer_sequence<int, U1 - U0>{});
  };

  // ---- the schedule
  [&]<int... K>(std::integer_sequence<int, K...>) __attribute__((always_inline)) {
    (read_op.template operator()<K>(), ...);
  }(std::make_integer_sequence<int, LA>{});
  [&]<int... K>(std::integer_sequence<int, K...>) __attribute__((always_inline)) {
    ([&]() __attribute__((always_inline)) {
      if constexpr (K + LA < Plan::NM) read_op.template operator()<K + LA>();
      do_mfma.template operator()<K>();
      uops.template operator()<Plan::first_uop(K), Plan::first_uop(K + 1)>();
      __builtin_amdgcn_sched_barrier(0);
    }(), ...);
  }(std::make_integer_sequence<int, Plan::NM>{});
  uops.template operator()<Plan::first_uop(Plan::NM), Plan::NU>();
  if constexpr (F16) {
    // the tile's sum lsum - l_run bounds each of its P~ (infinity included)
    if (__builtin_amdgcn_ballot_w64(!(lsum - l_run <= kOptimisticSum))) {
      // rare: recompute the tile's scores (into the registers they came in,
      // free by now) and take the max-based rule
      qk_tile<D, SQ>(s_cur, qf, kb_prev, n, hh, init, sqo);
      rescale<D>(o, softmax_tile<PV, false>(s_cur, m_run, l_run, p_new, ts, grid, ~0u, hh));
    } else {
      l_run = lsum;
    }
  } else if constexpr (PV == kPvInt8) {
    rescale_i32<D>(o, alpha);
  } else {
    rescale<D>(o, alpha);
  }
}

// The debug instantiation (DUMP) of the kernel below stores every INT32
// score it computes inside a window of one head, exactly as the softmax then
// reads it, minus the accumulator's start bias (FP16 mode's 1.5 * 2^23; with
// Q smoothed the start values are the compensation C, which stays in): so
// the stored value is S = Q^ K^^T, or S + C.  It runs the query blocks qb0,
// qb0 + 1, ... of the head the kernel's pointers are offset to.
struct DumpWin {
  int32_t* s;   // int32 [nq, nk], row-major; entries not computed are untouched
  int q0, nq, k0, nk, qb0;
};

template <int PV>
__device__ __forceinline__ void dump_tile(const DumpWin& dw, const v16i (&s)[2], int tile,
                                          int qrow, int N, int hh) {
  const int qi = qrow - dw.q0;
  if (qrow >= N || qi < 0 || qi >= dw.nq) return;
  constexpr int bias = PV == kPvFp16 ? kMagicBits : 0;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = tile * kKvTile + 32 * blk + 8 * (r >> 2) + 4 * hh + (r & 3);
      const int kj = key - dw.k0;
      if (key < N && kj >= 0 && kj < dw.nk) {
        const int v = s[blk][r];   // element to a scalar first (see softmax_tile)
        dw.s[(size_t)qi * dw.nk + kj] = v - bias;
      }
    }
}

// Software pipeline over the KV tiles of one workgroup (NW wavefronts), two
// tiles deep.  Entering step j a wavefront holds P~(j) (MFMA operand) and the
// INT32 scores S(j+1); step j issues
//     S(j+2) = K^(j+2) Q^T          [INT8 MFMA]
//     O     += P~(j) V(j)           [FP16/FP8 MFMA]
//     softmax(S(j+1)) -> P~(j+1)    [VALU, independent of both]
// then rescales O by alpha(j+1).  K^ tile j+3 and V tile j+1 are loaded from
// HBM during step j straight into LDS (V double-buffered; K^ in three slots
// in FP16 mode, so K^(j+1) is still there if step j must recompute S(j+1);
// one barrier per step).  All wavefronts run every step of the workgroup; a
// causal tile beyond a wavefront's last row is fully masked and changes
// nothing.  ACC (INT8 P~V only): O is the INT32 sum of the tiles' P^ V^.
// NW wavefronts per workgroup (32 query rows each): 4, one delta_Q block, or
// 8 (two blocks; FP16 P~V, d = 128, non-causal), where every K^ and V tile
// copied into LDS serves twice the rows.
//
// Wavefronts per SIMD: two (up to 256 registers each), or three (168) for
// FP8 and INT8-sum P~V at d = 64 without smoothed Q, whose steps are
// VALU-bound (6 or 8 MFMAs against about 200 VALU instructions): a third
// wavefront fills more of the VALU's idle issue cycles (c4 -2%, c4i8 -4%).
// Their steady-state loops keep every value in registers; the spills are in
// the tail steps.
template <int D, int PV, bool ACC, bool SQ>
constexpr int kWavesPerSimd =
    D == 64 && !SQ && (PV == kPvFp8 || (PV == kPvInt8 && ACC)) ? 3 : 2;

template <int D, int PV, int OUT, bool CAUSAL, bool SQ, bool ACC, int NW, bool DUMP>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW),
                          amdgpu_waves_per_eu(kWavesPerSimd<D, PV, ACC, SQ>,
                                              kWavesPerSimd<D, PV, ACC, SQ>)))
void attn_fwd_kernel(const int8_t* __restrict__ q_i8, const int8_t* __restrict__ k_i8,
                     const uint8_t* __restrict__ v_t, const float* __restrict__ q_scale,
                     const float* __restrict__ k_scale, const float* __restrict__ v_scale,
                     const int32_t* __restrict__ comp, int BH, int N, int qb_begin, int nqb,
                     int ntiles,
                     int xcd_remap, int H, int nhd, void* __restrict__ out, DumpWin dw) {
  // K^ slot: the tile, then (SQ) its 64 compensation values
  constexpr int KB = KTile<D>::BYTES + (SQ ? kSqTileBytes * (NW / 4) : 0);
  constexpr int VB = VTile<D, PV>::BYTES;
  constexpr int NCB = D / 32;   // 32-channel blocks of the output
  constexpr int NKS = kKSlots<PV>;
  static_assert(NW == 4 || (NW == 8 && PV == kPvFp16 && D == 128 && !CAUSAL),
                "8-wavefront workgroups: FP16 P~V, d = 128, non-causal");
  constexpr int BQW = kWaveQ * NW;   // query rows per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[NKS][KB];
  __shared__ __attribute__((aligned(16))) uint8_t vbuf[2][VB];

  // Workgroup -> (b*h, query block).
  // Consecutive workgroups are dispatched round-robin over the 8 XCDs (each
  // with its own L2); the remap keeps the workgroups of a head on one XCD so
  // that its K^/V tiles are shared in that L2.
  int wg = blockIdx.x;
  if (xcd_remap) {
    // each XCD a contiguous range of (head, block) ids
    const int g8 = gridDim.x & ~7;
    if (wg < g8) wg = (wg & 7) * (g8 >> 3) + (wg >> 3);
  }
  int bh, qb;
  if constexpr (DUMP) {     // one head (pointers offset to it), blocks qb0, qb0 + 1, ...
    bh = 0;
    qb = dw.qb0 + (int)blockIdx.x;
  } else if constexpr (CAUSAL) {
    // heaviest query blocks first, over all heads.  (Keeping each head on
    // one XCD cut the HBM fetches of c2 threefold but not its time, and the
    // head-by-head order it needs balanced short grids worse.)
    qb = nqb - 1 - wg / BH;
    bh = wg % BH;
  } else {
    bh = wg / nqb;
    qb = wg % nqb;
  }
  // this launch covers query blocks [qb_begin, qb_begin + nqb) of each head
  if constexpr (!DUMP) qb += qb_begin;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wavefront
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int qrow = qb * BQW + wave * kWaveQ + n;   // this lane's query row

  const int8_t* q_bh = q_i8 + (size_t)bh * N * D;
  const int8_t* k_bh = k_i8 + (size_t)bh * N * D;
  const uint8_t* v_bh = v_t + (size_t)bh * ntiles * VB;
  const float* ks_bh = k_scale + (size_t)bh * ntiles;   // one delta_K per KV tile

  v4i qf[D / 32];
  load_q_frag<D>(qf, q_bh, qrow, N, hh);
  // delta_Q of this wavefront's 128-row block (rows past N: the last block)
  const int nq128 = (N + kQBlock - 1) / kQBlock;
  const int qblk = min((qb * BQW + wave * kWaveQ) / kQBlock, nq128 - 1);
  const float cq = q_scale[(size_t)bh * nq128 + qblk] * kLog2e;

  // FP16 mode: the accumulator start value (magic bias) and the grid of the
  // running max, twice the float spacing at the largest K0 of the head.
  v16i init = {};
  MaxGrid grid = {1.f, 1.f};
  if constexpr (PV == kPvFp16) {
    const int mb = __builtin_amdgcn_readfirstlane(kMagicBits + (N & 0x80000000));
#pragma unroll
    for (int r = 0; r < 16; ++r) init[r] = mb;
    float kmax = 0.f;
    for (int i = lane; i < ntiles; i += 64) kmax = fmaxf(kmax, ks_bh[i]);
    kmax = wave_max(kmax);
    const int e = (int)(__builtin_bit_cast(uint32_t, kMagic * (cq * kmax)) >> 23);
    const int ge = max(e - 22, 2);   // biased exponent of the grid step
    grid = MaxGrid{__builtin_bit_cast(float, (uint32_t)ge << 23),
                   __builtin_bit_cast(float, (uint32_t)(254 - ge) << 23)};
  }

  // Tiles of the workgroup; tiles [0, nt_full) need no mask for any row, the
  // rest (ragged tail, causal diagonal) run the masked softmax.
  const int kv_end = CAUSAL ? min(N, (qb + 1) * BQW) : N;
  const int nt = (kv_end + kKvTile - 1) / kKvTile;
  const int nt_full = CAUSAL ? min(2 * qb, N / kKvTile) : N / kKvTile;

  const KLoader<D, NW> kld(wave, lane);
  using VL = VLoader<D, PV, NW>;
  const v4i krs = buffer_rsrc(k_bh, (uint32_t)((size_t)N * D));
  // SQ: the row of compensation values of this wavefront's 128-row block,
  // ntiles * 64 INT32, and their place in each K^ slot
  v4i crs = {0, 0, 0, 0};
  // (a launch over part of the query blocks gets the rows of its own blocks:
  // 128-row blocks [q128_0, q128_0 + n128) of each head)
  if constexpr (SQ) {
    const int q128_0 = DUMP ? 0 : qb_begin * BQW / kQBlock;
    const int n128 = DUMP ? nq128 : (min(N, (qb_begin + nqb) * BQW) + kQBlock - 1) / kQBlock - q128_0;
    crs = buffer_rsrc(comp + ((size_t)bh * n128 + (qblk - q128_0)) * ntiles * kKvTile,
                      (uint32_t)ntiles * kSqTileBytes);
  }
  const int sqo = (wave / 4) * kSqTileBytes;
  // K^ tile `tile` into the slot at LDS address `dst`, with (SQ) the
  // compensation values of each 128-row block behind it (wavefronts 0 and 4,
  // lanes 0..15, 16 bytes each)
  auto issue_k = [&]<bool CLAMP>(int tile, uint32_t dst) __attribute__((always_inline)) {
    kld.template issue<CLAMP>(krs, tile * kKvTile, N, dst, wave);
    if constexpr (SQ) {
      if (wave % 4 == 0 && lane < 16) {
        const uint32_t m0[1] = {dst + KTile<D>::BYTES + sqo};
        const int vo[1] = {lane * 16};
        lds_copy_x4<1>(crs, tile * kSqTileBytes, m0, vo);
      }
    }
  };
  // K^ tile t lives in slot t % NKS (tile indices here are wavefront-uniform;
  // with two slots and an even j, the slot of tile j + u + c is (u + c) & 1)
  auto kslot = [&](int t, int u_plus_c) __attribute__((always_inline)) {
    return NKS == 2 ? (u_plus_c & 1) : t % NKS;
  };
  const uint32_t kl0 = lds_addr(kbuf[0]);
  const uint32_t vl[2] = {lds_addr(vbuf[0]), lds_addr(vbuf[1])};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  v16f o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = v16f{};
  v16i sA[2], sB[2];
  PTile<PV> pA, pB;
  // INT8 outside the fused steps: the rescale factor of the tile whose P^ V^
  // comes next, applied in the same fused multiply-add that adds the product,
  // or (ACC) to the INT32 sums just before the product's MFMAs (the fused
  // steps rescale at their end and leave it at 1)
  float alpha_pend = 1.f;
  static_assert(!ACC || PV == kPvInt8, "INT32 accumulation is for INT8 P~V only");

  // Masks of the tiles that need one.  Causal: the two tiles on the diagonal
  // of query block qb (2 qb + dd, dd = 0, 1) show key 64 dd + off of the tile
  // to row 32 wave + n of the block iff 64 dd + off <= 32 wave + n, the same
  // for every block, so both masks are formed once.  The tile holding key
  // N - 1 of a ragged N also hides the keys >= N.
  uint32_t kdiag0 = ~0u, kdiag1 = ~0u;
  if constexpr (CAUSAL) {
    kdiag0 = key_mask(0, hh, kWaveQ * wave + n);
    kdiag1 = key_mask(kKvTile, hh, kWaveQ * wave + n);
  }
  auto tile_keep = [&](int t) __attribute__((always_inline)) {
    uint32_t keep = ~0u;
    if constexpr (CAUSAL) {
      const int dd = t - 2 * qb;   // 0 or 1 for a masked tile of a causal block
      if (dd >= 0) keep = dd == 0 ? kdiag0 : kdiag1;
    }
    if ((t + 1) * kKvTile > N) keep &= key_mask(t * kKvTile, hh, N - 1);
    return keep;
  };
  auto softmax_any = [&](v16i (&sc)[2], PTile<PV>& pn, int t) __attribute__((always_inline)) {
    const TileScale ts = tile_scale<PV>(cq, ks_bh[t]);
    return t < nt_full ? softmax_tile<PV, false>(sc, m_run, l_run, pn, ts, grid, ~0u, hh)
                       : softmax_tile<PV, true>(sc, m_run, l_run, pn, ts, grid, tile_keep(t), hh);
  };

  // Prologue: S(0), S(1), P~(0).  K^(2) goes to its own third slot with the
  // first copies (FP16 mode), or into the slot of K^(0) once every wavefront
  // has read it (two slots).
  issue_k.template operator()<true>(0, kl0);
  VL::issue(v_bh, 0, vl[0], wave, lane);
  if (nt > 1) issue_k.template operator()<true>(1, kl0 + KB);
  if (NKS == 3 && nt > 2) issue_k.template operator()<true>(2, kl0 + 2 * KB);
  wait_lds_loads();
  __syncthreads();
  qk_tile<D, SQ>(sA, qf, kbuf[0], n, hh, init, sqo);
  if (nt > 1) qk_tile<D, SQ>(sB, qf, kbuf[1], n, hh, init, sqo);
  if constexpr (DUMP) {
    dump_tile<PV>(dw, sA, 0, qrow, N, hh);
    if (nt > 1) dump_tile<PV>(dw, sB, 1, qrow, N, hh);
  }
  softmax_any(sA, pA, 0);   // alpha irrelevant: O is still zero
  __syncthreads();          // every wave has read K^(0)
  if (NKS == 2) {
    if (nt > 2) issue_k.template operator()<true>(2, kl0 + kslot(2, 2) * KB);
    wait_lds_loads();
    __syncthreads();
  }

  // Steady state: no masking, every load and MFMA present.  Step jj writes
  // K^(jj+3) and V(jj+1) into the slots read before it (K^ slot sw, V slot
  // 1 - U%2), runs QK on K^(jj+2) (slot sr) and may recompute from K^(jj+1)
  // (slot sp); register roles alternate with U%2.
  // delta_K of the tile whose softmax the next step runs is loaded one step
  // ahead: a scalar load shares the LDS counter, so waiting for it inside a
  // step would also wait for every LDS read in flight.  Its wait is placed at
  // the end of the step instead, where no LDS read is outstanding.
  float dk_next = ks_bh[min(1, ntiles - 1)];
  auto steady = [&]<int U>(int jj, int sw, int sr, int sp) __attribute__((always_inline)) {
    issue_k.template operator()<false>(jj + 3, kl0 + sw * KB);
    VL::issue(v_bh, jj + 1, vl[1 - (U & 1)], wave, lane);
    v16i(&s_cur)[2] = (U & 1) == 0 ? sB : sA;
    v16i(&s_new)[2] = (U & 1) == 0 ? sA : sB;
    PTile<PV>& p_cur = (U & 1) == 0 ? pA : pB;
    PTile<PV>& p_new = (U & 1) == 0 ? pB : pA;
    const float dk = dk_next;
    dk_next = ks_bh[jj + 2];   // jj + 2 < nt: in range
    // FP16: keep the accumulator start value resident (not rebuilt every
    // step); in FP8 mode it is zero, an inline constant
    if constexpr (PV == kPvFp16 && !SQ) asm volatile("" : "+v"(init));
    fused_step<D, PV, SQ>(o, qf, s_cur, s_new, p_cur, p_new, kbuf[sr], kbuf[sp], vbuf[U & 1], m_run,
                      l_run, tile_scale<PV>(cq, dk), grid, init, n, hh, sqo);
    if constexpr (DUMP) dump_tile<PV>(dw, s_new, jj + 2, qrow, N, hh);
    asm volatile("" ::"s"(dk_next));
    wait_lds_loads();
    __syncthreads();
  };
  int j = 0;
  if constexpr (NKS == 3) {
    // six steps per trip: with j a multiple of 6 every K^ slot (t % 3) is a
    // constant, so all LDS addresses are immediates
    for (; j + 8 < nt && j + 6 < nt_full; j += 6) {
      steady.template operator()<0>(j + 0, 0, 2, 1);
      steady.template operator()<1>(j + 1, 1, 0, 2);
      steady.template operator()<2>(j + 2, 2, 1, 0);
      steady.template operator()<3>(j + 3, 0, 2, 1);
      steady.template operator()<4>(j + 4, 1, 0, 2);
      steady.template operator()<5>(j + 5, 2, 1, 0);
    }
  }
  if constexpr (PV != kPvInt8 || ACC) {
    for (; j + 4 < nt && j + 2 < nt_full; j += 2) {
      steady.template operator()<0>(j, kslot(j + 3, 3), kslot(j + 2, 2), kslot(j + 1, 1));
      steady.template operator()<1>(j + 1, kslot(j + 4, 4), kslot(j + 3, 3), kslot(j + 2, 2));
    }
  } else {
    // INT8 with O converted per tile: the same unmasked steps with every load
    // and MFMA present, in source order (P^ V^(jj), softmax(S(jj+1)), S(jj+2)),
    // so that the two score tiles and the tile's INT32 product are never live
    // together
    auto plain = [&]<int U>(int jj) __attribute__((always_inline)) {
      issue_k.template operator()<false>(jj + 3, kl0 + ((U + 3) & 1) * KB);
      VL::issue(v_bh, jj + 1, vl[1 - U], wave, lane);
      v16i(&s_cur)[2] = U == 0 ? sB : sA;
      v16i(&s_new)[2] = U == 0 ? sA : sB;
      PTile<PV>& p_cur = U == 0 ? pA : pB;
      PTile<PV>& p_new = U == 0 ? pB : pA;
      const float dk = dk_next;
      dk_next = ks_bh[jj + 2];
      pv_tile<D, PV>(o, p_cur, vbuf[U], n, hh, alpha_pend);
      alpha_pend = softmax_tile<PV, false>(s_cur, m_run, l_run, p_new, tile_scale<PV>(cq, dk),
                                           grid, ~0u, hh);
      qk_tile<D, SQ>(s_new, qf, kbuf[U], n, hh, init, sqo);
      if constexpr (DUMP) dump_tile<PV>(dw, s_new, jj + 2, qrow, N, hh);
      asm volatile("" ::"s"(dk_next));
      wait_lds_loads();
      __syncthreads();
    };
    for (; j + 4 < nt && j + 2 < nt_full; j += 2) {
      plain.template operator()<0>(j);
      plain.template operator()<1>(j + 1);
    }
  }
  // Tail: the last steps, with masking and missing tiles handled explicitly.
  // Causal: a tile whose first key lies past this wavefront's last row is
  // hidden from all of its rows (the second diagonal tile, for the first two
  // wavefronts of a block); its scores, softmax and P~V would change nothing
  // (P~ = 0, alpha = 1), so the wavefront skips them and only takes part in
  // the copies and barriers.  The debug instantiation computes them (its
  // scores are checked).
  const int last_row = qb * BQW + wave * kWaveQ + (kWaveQ - 1);
  auto dead = [&](int t) __attribute__((always_inline)) {
    return CAUSAL && !DUMP && t * kKvTile > last_row;
  };
  for (; j < nt; j += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int jj = j + u;
      if (jj < nt) {
        if (jj + 3 < nt)
          issue_k.template operator()<true>(jj + 3, kl0 + kslot(jj + 3, u + 3) * KB);
        if (jj + 1 < nt) VL::issue(v_bh, jj + 1, vl[1 - u], wave, lane);
        v16i(&s_cur)[2] = u == 0 ? sB : sA;
        v16i(&s_new)[2] = u == 0 ? sA : sB;
        PTile<PV>& p_cur = u == 0 ? pA : pB;
        PTile<PV>& p_new = u == 0 ? pB : pA;
        if constexpr (PV == kPvInt8) {
          // P^ V^, softmax, then the next scores: the two score tiles are
          // never live at once (the INT32 product needs the registers)
          if (!dead(jj)) {
            if constexpr (ACC) rescale_i32<D>(o, alpha_pend);
            pv_tile<D, PV, ACC>(o, p_cur, vbuf[u], n, hh, alpha_pend);
          }
          if (jj + 1 < nt) alpha_pend = dead(jj + 1) ? 1.f : softmax_any(s_cur, p_new, jj + 1);
          if (jj + 2 < nt && !dead(jj + 2)) {
            qk_tile<D, SQ>(s_new, qf, kbuf[kslot(jj + 2, u + 2)], n, hh, init, sqo);
            if constexpr (DUMP) dump_tile<PV>(dw, s_new, jj + 2, qrow, N, hh);
          }
        } else {
          if (jj + 2 < nt && !dead(jj + 2)) {
            qk_tile<D, SQ>(s_new, qf, kbuf[kslot(jj + 2, u + 2)], n, hh, init, sqo);
            if constexpr (DUMP) dump_tile<PV>(dw, s_new, jj + 2, qrow, N, hh);
          }
          if (!dead(jj)) pv_tile<D, PV>(o, p_cur, vbuf[u], n, hh, alpha_pend);
          if (jj + 1 < nt && !dead(jj + 1)) rescale<D>(o, softmax_any(s_cur, p_new, jj + 1));
        }
        wait_lds_loads();
        __syncthreads();
      }
    }
  }

  // Epilogue: O = O / l (FP8, INT8: l is in units of 448 P~ or 127 P~, and
  // delta_V per channel).
  const float l_tot = pair_sum_f32(l_run);
  const float inv = 1.0f / l_tot;
  if (qrow < N && (!DUMP || (qrow >= dw.q0 && qrow - dw.q0 < dw.nq))) {
    // O row of (b, h, qrow): [B,H,N,d] or token-major [B,N,H,d]; the dump
    // instantiation writes the rows of its window, [nq, d] from row q0
    const size_t orow = DUMP  ? (size_t)(qrow - dw.q0) * D
                        : nhd ? (((size_t)(bh / H) * N + qrow) * H + bh % H) * D
                              : ((size_t)bh * N + qrow) * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int c0 = 32 * cb + 8 * j4 + 4 * hh;
        float y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float ou = o[cb][4 * j4 + u];   // element to a scalar first
          y[u] = (ACC ? (float)__builtin_bit_cast(int, ou) : ou) * inv;
          if constexpr (PV != kPvFp16) y[u] *= v_scale[(size_t)bh * D + c0 + u];
        }
        store4<OUT>(out, orow + c0, y[0], y[1], y[2], y[3]);
      }
  }
}


// ---------------------------------------------------------------------------
// INT8 P~V keeps O as an INT32 sum of the tiles' products for heads of up to
// 2^17 keys: one 64-key tile adds at most 64 * 127^2 = 1032256 in magnitude
// (|P^| <= 127, |V^| <= 127), 2048 tiles at most 2114060288, and each rescale
// (alpha <= 1) rounds by at most 0.5 + 2^-24 |sum|, so the sum stays below 2^31.
constexpr int kInt8AccMaxKeys = 1 << 17;

// 8-wavefront workgroups halve the K^/V copies into LDS per query row (on c3
// the copies cost about a tenth of the kernel).  They pay off in FP16 mode,
// whose steps rarely rescale; with the exact max of FP8 and INT8 P~V the
// rescales of single wavefronts hold all eight at each step's barrier.  With
// Q smoothed each K^ slot carries the compensation values of both blocks.
template <int D, int PV, bool CAUSAL>
constexpr int kWaves = PV == kPvFp16 && D == 128 && !CAUSAL ? 8 : 4;

template <int D, int PV, int OUT, bool CAUSAL, bool SQ, bool DUMP>
static hipError_t attn_dispatch(const AttnArgs& a, hipStream_t s) {
  constexpr int NW = kWaves<D, PV, CAUSAL>;
  constexpr int BQW = kWaveQ * NW;
  const int ntiles = ceil_div(a.N, kKvTile);
  // query blocks of this launch: 128-row blocks [q128_begin, + q128_count)
  // (count 0: to the end), in workgroup blocks of BQW rows
  const int qb_begin = a.q128_begin * kQBlock / BQW;
  const int q_end = a.q128_count ? min(a.N, (a.q128_begin + a.q128_count) * kQBlock) : a.N;
  const int nqb = ceil_div(q_end, BQW) - qb_begin;
  int BH = a.B * a.H;
  long long grid = (long long)BH * nqb;
  DumpWin dw{};
  if constexpr (DUMP) {
    const int qb0 = a.dump_q0 / BQW;
    grid = ceil_div(a.dump_q0 + a.dump_nq, BQW) - qb0;
    BH = 1;
    dw = DumpWin{a.s_dump, a.dump_q0, a.dump_nq, a.dump_k0, a.dump_nk, qb0};
  }
  if (grid < 1 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int remap = CAUSAL || DUMP ? 0 : 1;
  auto go = [&](auto acc) {
    attn_fwd_kernel<D, PV, OUT, CAUSAL, SQ, decltype(acc)::value, NW, DUMP>
        <<<dim3((unsigned)grid), 64 * NW, 0, s>>>(a.q_i8, a.k_i8, a.v_t, a.q_scale, a.k_scale,
                                                  a.v_scale, a.comp, BH, a.N, qb_begin, nqb,
                                                  ntiles, remap,
                                                  a.H, a.nhd, a.out, dw);
    return hipGetLastError();
  };
  if constexpr (PV == kPvInt8) {
    if (a.N <= kInt8AccMaxKeys) return go(std::true_type{});
  }
  return go(std::false_type{});
}

// All variants of one head dimension and P~V mode (instantiated once per
// mode by the attn_fwd_d*_*.hip translation units).  The dump launch
// (a.s_dump set) writes float32 O.
template <int D, int PV>
hipError_t attn_launch_dp(const AttnArgs& a, hipStream_t s) {
  const bool sq = a.comp != nullptr;
#define SAGE_DISPATCH(OUT, DUMP)                                                         \
  {                                                                                     \
    if (a.causal) return sq ? attn_dispatch<D, PV, OUT, true, true, DUMP>(a, s)         \
                            : attn_dispatch<D, PV, OUT, true, false, DUMP>(a, s);       \
    return sq ? attn_dispatch<D, PV, OUT, false, true, DUMP>(a, s)                      \
              : attn_dispatch<D, PV, OUT, false, false, DUMP>(a, s);                    \
  }
  if (a.s_dump) {
    if (a.out_kind != 2) return hipErrorInvalidValue;
    SAGE_DISPATCH(2, true)
  }
  switch (a.out_kind) {
    case 0: SAGE_DISPATCH(0, false)
    case 1: SAGE_DISPATCH(1, false)
    case 2: SAGE_DISPATCH(2, false)
    default: return hipErrorInvalidValue;
  }
#undef SAGE_DISPATCH
}

}  // namespace sage
