// sage_launch.h -- host-side launchers of the HIP kernels (internal C++ API
// used by the C ABI in sage_api.cpp).  All arguments have been validated by
// the caller; the launchers only size grids and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sage {

// Blocking contract (the pages leave b_q, b_kv open; see sage_attn.h).
constexpr int kQBlock = 128;     // tokens per delta_Q block
constexpr int kKBlock = 64;      // tokens per delta_K block
constexpr int kKvTile = 64;      // keys per online-softmax step
constexpr int kMeanChunk = 256;  // tokens per float32 partial column sum
constexpr int kWaveQ = 32;       // query rows per wavefront (one 32x32 MFMA column block)
// Longest sequence the library accepts: (float)N is exact, and the byte
// offsets of one head's K^ (N d <= 2^31) fit the kernels' 32-bit buffer
// offsets (checked where they are formed, attn_fwd_kernel.h).
constexpr int kMaxN = 1 << 24;
static_assert(kQBlock % kWaveQ == 0, "a delta_Q block is whole wavefronts of rows");
static_assert(kKvTile == kKBlock, "one delta_K per KV tile");

constexpr int kPvFp16 = 0;
constexpr int kPvFp8 = 1;
constexpr int kPvInt8 = 2;

inline bool pv_valid(int pv) { return pv == kPvFp16 || pv == kPvFp8 || pv == kPvInt8; }
// FP8 and INT8 P~V quantise V per channel (delta_V = colmax|V| / range).
inline bool v_quantised(int pv) { return pv == kPvFp8 || pv == kPvInt8; }

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Bytes of one 64-key tile of prepared V (d rows of 64 keys).
inline size_t v_tile_bytes(int d, int pv_mode) {
  return (size_t)d * (pv_mode == kPvFp16 ? 128 : 64);
}

// Layout of q, k, v (and o) and the optional RoPE tables applied to Q and K
// ahead of smoothing and quantisation (float32 [N, d/2] cos and sin).
struct InLayout {
  int nhd;                  // 0: [B,H,N,d]; 1: token-major [B,N,H,d]
  const float* rope_cos;    // null: no RoPE
  const float* rope_sin;
};

// Prepass: column statistics of K (float32 partial sums per 256-token chunk)
// and, if v != nullptr, of |V| (partial maxima into part_max), then the
// finalised mean and, for V, delta_V and its reciprocal in the range of
// pv_mode (FP8 448, INT8 127).
// finalize = false: the partials only (launch_quant_qkv forms the statistics
// itself where quant_qkv_folds(N)).
hipError_t launch_colstats(const void* k, const void* v, int dtype, int B, int H, int N, int d,
                           int pv_mode, const InLayout& in, float* part_sum, float* part_max,
                           float* k_mean, float* v_scale, float* v_recip, hipStream_t s,
                           bool finalize = true);

// Prepass: INT8 quantisation of Q/sqrt(d) (128-token blocks) and of K - mean
// (64-token blocks).  Either q or k may be null to skip that tensor.
hipError_t launch_quant_qk(const void* q, const void* k, const float* k_mean, int dtype, int B,
                           int H, int N, int d, const InLayout& in, int8_t* q_i8, int8_t* k_i8,
                           float* q_scale, float* k_scale, hipStream_t s);

// Prepass: V -> fp16, E4M3 or INT8 in the tiled layout of the attention kernel.
hipError_t launch_prep_v(const void* v, const float* v_recip, int dtype, int B, int H, int N,
                         int d, int pv_mode, int nhd, uint8_t* v_out, hipStream_t s);

// launch_quant_qk and launch_prep_v as one launch (q may be null: K^ and V
// only; V in the layout in.nhd).  Where quant_qkv_folds(N) (at most 16
// 256-token chunks) the launch also forms the K mean and, with V quantised,
// delta_V and its reciprocal from the column partials (part_sum, part_max),
// storing them into k_mean, v_scale, v_recip: the column statistics are
// then launched without their finalisation.
bool quant_qkv_folds(int N);
hipError_t launch_quant_qkv(const void* q, const void* k, const void* v, float* k_mean,
                            float* v_recip, int dtype, int B, int H, int N, int d, int pv_mode,
                            const InLayout& in, int8_t* q_i8, int8_t* k_i8, float* q_scale,
                            float* k_scale, uint8_t* v_out, const float* part_sum,
                            const float* part_max, float* v_scale, hipStream_t s);

// Outputs of the one-launch prepass (any may be null when its stage is skipped).
struct PrepassOut {
  float* part_sum;   // float32 [B*H, ceil(N/256), d] column partial sums of K
  float* k_mean;
  float* v_scale;
  int8_t* q_i8;
  int8_t* k_i8;
  float* q_scale;
  float* k_scale;
  uint8_t* v_out;
};

// Sequences up to this length run the prepass in two launches: the first's
// workgroups take roles (one per 256-token K chunk for its column sums, one
// per Q^ block, one per V tile), the second forms each head's K mean and
// quantises one K^ block per wavefront.  A head of one chunk needs only the
// first launch.
constexpr int kHeadPrepassMaxN = 2048;

hipError_t launch_prepass_head(const void* q, const void* k, const void* v, int dtype, int B,
                               int H, int N, int d, int pv_mode, const InLayout& in,
                               const PrepassOut& o, hipStream_t s);

// Attention kernel.  out_kind: 0 = fp16, 1 = bf16, 2 = float32; nhd: o is
// token-major [B,N,H,d] instead of [B,H,N,d].  comp: null, or (Q smoothed per
// block) the compensation values int32 [B*H, ceil(N/128), ceil(N/64)*64],
// with FP16 mode's magic bias (kSqBiasFp16) already added in FP16 mode.
// q128_begin, q128_count: only the query rows of 128-row blocks [q128_begin,
// q128_begin + q128_count) of every head (count 0: to the last row); both
// multiples of 2 (the widest workgroup covers 256 rows) unless the range
// ends at N.  comp then holds those blocks only: [B*H, blocks in range, ld].
hipError_t launch_attn(const int8_t* q_i8, const int8_t* k_i8, const uint8_t* v_t,
                       const float* q_scale, const float* k_scale, const float* v_scale,
                       const int32_t* comp, int B, int H, int N, int d, int causal, int pv_mode,
                       int out_kind, int nhd, void* out, hipStream_t s, int q128_begin = 0,
                       int q128_count = 0);

// Debug: the attention kernel's own dump instantiation on head (b, h) for the
// query rows [q0, q0+nq): every INT32 score it computes for keys [k0, k0+nk)
// (minus the accumulator's start bias) into s_out int32 [nq, nk], and the
// float32 O of those rows into o_rows [nq, d].  Operands as for launch_attn.
hipError_t launch_attn_dump(const int8_t* q_i8, const int8_t* k_i8, const uint8_t* v_t,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            const int32_t* comp, int B, int H, int N, int d, int causal,
                            int pv_mode, int b, int h, int q0, int nq, int k0, int nk,
                            int32_t* s_out, float* o_rows, hipStream_t s);

// Arguments of one attention launch (attn_fwd_kernel.h).  The dump fields are
// used only when s_dump is set; the pointers then address one head.
struct AttnArgs {
  const int8_t* q_i8;
  const int8_t* k_i8;
  const uint8_t* v_t;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const int32_t* comp;
  int B, H, N, causal, out_kind, nhd;
  void* out;
  int32_t* s_dump;
  int dump_q0, dump_nq, dump_k0, dump_nk;
  int q128_begin, q128_count;
};

// Smoothed Q (smooth_q.hip): per 128-token block the mean qbar is removed
// before quantisation (q_i8, q_scale as for plain Q; q_mean float32 and q_w
// int32 [B*H, ceil(N/128), d]); the compensation C = rne((w . K^) / 2^8) + bias
// is written as int32 [B*H, ceil(N/128), ld] for keys t < ld.
hipError_t launch_smooth_q(const void* q, int dtype, int B, int H, int N, int d, int nhd,
                           int8_t* q_i8, float* q_scale, float* q_mean, int32_t* q_w,
                           hipStream_t s);
// Blocks [qb0, qb0 + nqr) only (nqr < 0: to the last block), written as
// int32 [B*H, nqr, ld].
hipError_t launch_sq_comp(const int8_t* k_i8, const int32_t* q_w, int B, int H, int N, int d,
                          int ld, int bias, int32_t* comp, hipStream_t s, int qb0 = 0,
                          int nqr = -1);
// The FP16-mode accumulator start (bit pattern of 1.5 * 2^23) that the
// compensation carries when it seeds the attention kernel's INT32 product.
constexpr int kSqBiasFp16 = 0x4B400000;

// Float32 softmax attention on selected query rows (reference for profiling).
hipError_t launch_ref_rows(const void* q, const void* k, const void* v, int dtype, int B, int H,
                           int N, int d, int causal, const int32_t* rows, int nrows, float* out,
                           hipStream_t s);

// Debug: INT32 S = Q^ K^T on a rectangle of one (b, h).
hipError_t launch_debug_s(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d,
                          int b, int h, int q0, int nq, int k0, int nk, int32_t* s_out,
                          hipStream_t s);

}  // namespace sage
