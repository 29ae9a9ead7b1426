/*
 * sage_attn.h -- C ABI of the MI355X (gfx950) SageAttention forward pass.
 *
 * Pages defining the operations (cited by title and section):
 *   [SA]    "SageAttention: Accurate 8-Bit Attention for Plug-and-Play Inference
 *           Acceleration", paper detail page (arXiv 2410.02367).
 *   [SA2pp] "SageAttention2++: A More Efficient Implementation of
 *           SageAttention2", paper review page (arXiv 2505.21136).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are caller-owned DEVICE pointers (HIP device memory of the current
 * device).  The library never allocates, frees or retains memory and keeps no
 * global mutable state; calls on different streams may run concurrently.
 *
 * q, k, v, o are contiguous [B, H, N, d] tensors ("HND": batch, head, token,
 * channel) of 16-bit elements (dtype SAGE_DT_F16 or SAGE_DT_BF16); element
 * offsets are 64-bit.  Base pointers must be 16-byte aligned and o must not
 * alias an input.  Supported: d in {64, 128}; 1 <= N <= 2^24; B, H >= 1;
 * causal in {0, 1} (key j visible to query i iff j <= i); the softmax scale
 * is fixed at 1/sqrt(d).  Inputs must be finite; for SAGE_PV_FP16 every V
 * value must also be finite in FP16 (|v| <= 65504).
 *
 * `stream` is a hipStream_t (NULL = the default stream).  All work is
 * enqueued on it; no call synchronises the host.  Every call validates all of
 * its arguments before it enqueues anything, so a call that returns an error
 * enqueued nothing.  A HIP launch error detected after enqueue is returned as
 * SAGE_ERR_HIP; device faults surface at the caller's next synchronisation.
 * No C++ exception crosses this interface.
 */
#ifndef SAGE_ATTN_H
#define SAGE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAGE_OK = 0,
  SAGE_ERR_INVALID_ARG = 1,   /* a pointer, size, flag or alignment is invalid */
  SAGE_ERR_UNSUPPORTED = 2,   /* valid request this library does not implement (e.g. d = 96, not gfx950) */
  SAGE_ERR_WORKSPACE = 3,     /* workspace / scratch smaller than required */
  SAGE_ERR_HIP = 4,           /* the HIP runtime reported an error */
  SAGE_ERR_NO_DEVICE = 5      /* no HIP device is visible */
} sage_status;

/* P~V precision: FP16, FP8 E4M3 ("8+8"), or INT8 (the all-INT8 kernel variant,
 * [SA] §3 Figure 5, chosen per layer in [SA] §6 step 4) */
enum { SAGE_PV_FP16 = 0, SAGE_PV_FP8 = 1, SAGE_PV_INT8 = 2 };
enum { SAGE_DT_F16 = 0, SAGE_DT_BF16 = 1 };   /* element type of q, k, v and o */
enum { SAGE_OUT_F32 = 2 };                     /* float32 output (sage_attn_fwd_quantized only) */
enum { SAGE_LAYOUT_HND = 0,                    /* q, k, v, o as [B,H,N,d] */
       SAGE_LAYOUT_NHD = 1 };                  /* token-major [B,N,H,d] */

/* Human-readable name of a status code (static string, never NULL). */
const char* sage_status_str(int status);

/*
 * Blocking constants of this library, which define the numerics of the method
 * ([SA] §3 Algorithm 1 leaves the block sizes b_q, b_kv open):
 *   q_block    tokens per delta_Q quantisation block (128)
 *   k_block    tokens per delta_K quantisation block (64)
 *   kv_tile    keys per online-softmax step, visited in ascending order (64)
 *   mean_chunk tokens per float32 partial sum of the K column mean (256)
 * Any output pointer may be NULL.  Returns SAGE_ERR_UNSUPPORTED for d outside
 * {64, 128} or an unknown pv_mode.
 */
int sage_attn_get_tiling(int d, int causal, int pv_mode, int* q_block, int* k_block,
                         int* kv_tile, int* mean_chunk);

/* Workspace bytes sage_attn_fwd needs for this shape (0 if the shape is invalid). */
size_t sage_attn_workspace_bytes(int B, int H, int N, int d, int pv_mode);

/*
 * The SageAttention forward pass ([SA] §3 Algorithm 1, kernel "SAGEAttn-B";
 * FP8 P~V as in [SA2pp] section 三, core formulas):
 *   1. K~ = K - mean_t(K) per (b, h, channel)               ([SA] §4 Eq. 6)
 *   2. Q^, delta_Q = psi(Q / sqrt(d)) per 128-token block;
 *      K^, delta_K = psi(K~) per 64-token block, where psi gives
 *      delta = max|X|/127 and X^ = round-to-nearest-even(X * 127/max|X|)
 *   3. for each 64-key tile j, ascending: S = (Q^ K^_j^T as INT32) delta_Q delta_K,
 *      online softmax (running max m, running sum l of the unquantised P~,
 *      rescale of the accumulator by exp(m_old - m_new))      ([SA] §4 Eq. 4-5)
 *   4. pv_mode SAGE_PV_FP16: O += fp16(P~) V'_j with V' = fp16(V);
 *      pv_mode SAGE_PV_FP8:  O += E4M3(448 P~) V^_j with the static delta_P = 1/448
 *      and V^ = E4M3(V * 448/colmax|V|), delta_V = colmax|V|/448 per channel;
 *      FP32 accumulation in both these modes;
 *      pv_mode SAGE_PV_INT8: O = alpha O + (P^ V^_j as INT32) with P^ =
 *      rne(127 P~) in [0, 127] (static delta_P = 1/127, [SA] §7 key
 *      implementation details) and V^ = clamp(rne(V * 127/colmax|V|), -127,
 *      127), delta_V = colmax|V|/127 per channel; every tile's product has
 *      the scale delta_P delta_V, so while a row's max stands the products add
 *      up exactly as INT32, and a rescale rounds that sum to the nearest
 *      integer (heads longer than 2^17 keys, where INT32 could overflow,
 *      convert each tile's product to float32, exactly, and add it instead)
 *   5. O = O / l (FP8, INT8: times delta_V / 448 or / 127), rounded to the
 *      input dtype (RNE).
 * In FP16 mode the kernel keeps the running max lazily (P~ may reach 2^14
 * before m is refreshed; softmax is invariant under the shift) and l sums the
 * fp16 values of P~ that enter the product; FP8 mode keeps the exact max and
 * the unquantised sum; so does INT8 mode.  Results agree with the definition
 * above to rounding.
 *
 * q, k, v: inputs [B,H,N,d] of `dtype`; o: output [B,H,N,d] of `dtype`.
 * workspace: device memory of at least sage_attn_workspace_bytes(B,H,N,d,pv_mode)
 * bytes, 256-byte aligned; its contents on entry are irrelevant and on return
 * hold the quantised operands (layout private).  The call is asynchronous.
 */
int sage_attn_fwd(const void* q, const void* k, const void* v, void* o,
                  int B, int H, int N, int d, int causal, int pv_mode, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/* As sage_attn_fwd, with o written as float32 [B,H,N,d] before the final
 * rounding to the input dtype (same kernels and arithmetic otherwise).
 * Used to check the forward pass at float32 output precision. */
int sage_attn_fwd_f32out(const void* q, const void* k, const void* v, float* o,
                         int B, int H, int N, int d, int causal, int pv_mode, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_attn_fwd with two options of the inputs:
 *   layout   SAGE_LAYOUT_HND ([B,H,N,d]) or SAGE_LAYOUT_NHD (token-major
 *            [B,N,H,d], contiguous); o is written in the same layout.
 *   rope_cos, rope_sin  NULL, or float32 device tables [N, d/2] (16-byte
 *            aligned): Q and K are rotated before smoothing and quantisation,
 *            in the same kernels that quantise them ([SA] §7 key implementation
 *            details, item 1: RoPE fused with the quantisation).  Rotate-half
 *            form: channel i < d/2 pairs with i + d/2, and with c = cos[t][i],
 *            s = sin[t][i] of token t, (x_i, x_{i+d/2}) -> (x_i c - x_{i+d/2} s,
 *            x_{i+d/2} c + x_i s), each product and sum rounded to float32.
 *            V is not rotated.  Both tables or neither.
 *   out_f32  0: o in `dtype`; 1: o float32 (as sage_attn_fwd_f32out).
 * Same workspace as sage_attn_fwd.  SAGE_ERR_INVALID_ARG for an unknown
 * layout, one table without the other, or a misaligned table.
 */
int sage_attn_fwd_ex(const void* q, const void* k, const void* v, void* o,
                     int B, int H, int N, int d, int causal, int pv_mode, int dtype,
                     int layout, const float* rope_cos, const float* rope_sin, int out_f32,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward pass with Q smoothed per 128-token block as well as K
 * (SageAttention2's smoothing of Q: "SageAttention2" abstract page, Q
 * smoothing improves the quantised QK^T; [SA2pp] 三 smooths Q and K before
 * quantising).  The pages print no formula; this library's reading, step 2 of
 * sage_attn_fwd replaced for Q by:
 *   qbar = the block's token mean of Q' = fp32(Q * fp32(1/sqrt(d))) (float32,
 *          tokens in order from 0.0f, one IEEE division by their count);
 *   Q~ = fp32(Q' - qbar), a = max|Q~|, r = fp32(127/a),
 *   Q~^ = clamp(rne(fp32(Q~ r)), -127, 127), delta_Q = fp32(a/127);
 *   w = rne(fp32(qbar r) * 2^8) per channel (the mean on a grid 2^8 finer);
 *   C[t] = rne((w . K^[t]) / 2^8) per block and key (exact integer product,
 *          ties to even), and step 3 uses S = (Q~^ K^^T + C) delta_Q delta_K.
 * A block is smoothed only if a > 0 and 127 sum_c |w_c| <= 2^29 (so that
 * |C| <= 2^21); any other block is quantised as in sage_attn_fwd (w = 0).
 * Arguments as sage_attn_fwd_ex without RoPE (layout SAGE_LAYOUT_HND or
 * SAGE_LAYOUT_NHD; out_f32 0/1); the workspace must hold
 * sage_attn_sq_workspace_bytes(...) bytes.  It adds ceil(N/64) * 64 int32
 * compensation values per head and 128-row query block, about N^2/32 bytes per
 * head (8 MiB at N = 16384), up to 256 MiB in all (or two query blocks of
 * every head where that is more): beyond that the pass computes them, and runs the
 * attention kernel, in chunks of query blocks (N = 131072 on one head: two
 * chunks of 512 blocks instead of a 512 MiB table).
 */
size_t sage_attn_sq_workspace_bytes(int B, int H, int N, int d, int pv_mode);
int sage_attn_fwd_sq(const void* q, const void* k, const void* v, void* o,
                     int B, int H, int N, int d, int causal, int pv_mode, int dtype,
                     int layout, int out_f32, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ---- The stages of the pass, exposed for testing and reuse -------------- */

/* Scratch bytes sage_smooth_quant_qk needs (float32 partial column sums). */
size_t sage_smooth_quant_qk_scratch_bytes(int B, int H, int N, int d);

/*
 * Steps 1-2 above.  Outputs (device, caller-owned, natural layouts):
 *   q_i8, k_i8 int8 [B,H,N,d]; q_scale float32 [B,H,ceil(N/128)];
 *   k_scale float32 [B,H,ceil(N/64)]; k_mean float32 [B,H,d].
 * The column mean is a float32 sum in a fixed order: per 256-token chunk a
 * sequential sum from 0.0f in increasing token order, then the chunk sums
 * sequentially in increasing chunk order from 0.0f, then one IEEE division by
 * N.  K~ = fp32(K - mean); per block a = max|X|, r = fp32(127/a),
 * X^ = clamp(rne(fp32(X * r)), -127, 127), delta = fp32(a/127); an all-zero
 * block gets delta = 0 and codes 0.  Q is first scaled: X = fp32(Q * fp32(1/sqrt(d))).
 * scratch: >= sage_smooth_quant_qk_scratch_bytes(...) bytes, 16-byte aligned.
 */
int sage_smooth_quant_qk(const void* q, const void* k, int dtype, int B, int H, int N, int d,
                         int8_t* q_i8, int8_t* k_i8, float* q_scale, float* k_scale,
                         float* k_mean, void* scratch, size_t scratch_bytes, void* stream);

/* sage_smooth_quant_qk with the input layout and the optional RoPE tables of
 * sage_attn_fwd_ex (the mean is then the mean of the rotated K).  Outputs are
 * in the [B,H,N,d] layout whatever the input layout. */
int sage_smooth_quant_qk_ex(const void* q, const void* k, int dtype, int layout,
                            const float* rope_cos, const float* rope_sin, int B, int H, int N,
                            int d, int8_t* q_i8, int8_t* k_i8, float* q_scale, float* k_scale,
                            float* k_mean, void* scratch, size_t scratch_bytes, void* stream);

/*
 * The smoothed-Q stage of sage_attn_fwd_sq on [B,H,N,d] q and the K^ codes of
 * sage_smooth_quant_qk (k_i8 int8 [B,H,N,d]): q_i8 int8 [B,H,N,d] (Q~^, or the
 * unsmoothed codes of a block left unsmoothed), q_scale float32
 * [B,H,ceil(N/128)], q_mean float32 and q_w int32 [B,H,ceil(N/128),d] (qbar
 * and w; 0 for a block left unsmoothed), and q_comp:
 *   seed_pv_mode = -1: C itself, int32 [B,H,ceil(N/128),N];
 *   seed_pv_mode = a SAGE_PV_* mode: the attention kernel's INT32 accumulator
 *     seeds for that mode, int32 [B,H,ceil(N/128),ceil(N/64)*64] (keys >= N
 *     get C = 0): C plus the bit pattern of 1.5 * 2^23 (0x4B400000) in
 *     SAGE_PV_FP16 mode, whose kernel reads the accumulator as a float; C
 *     itself in the other modes.  Input of sage_attn_fwd_quantized_sq.
 * q, k_i8, q_i8, q_w, q_comp 16-byte aligned; the others 4-byte aligned.
 */
int sage_smooth_q(const void* q, const int8_t* k_i8, int dtype, int B, int H, int N, int d,
                  int seed_pv_mode, int8_t* q_i8, float* q_scale, float* q_mean, int32_t* q_w,
                  int32_t* q_comp, void* stream);

/* Bytes of the prepared V (v_out of sage_quant_v) and of its scratch. */
size_t sage_quant_v_bytes(int B, int H, int N, int d, int pv_mode);
size_t sage_quant_v_scratch_bytes(int B, int H, int N, int d, int pv_mode);

/*
 * Step 4's V preparation.  v_out is written in the tiled layout the attention
 * kernel reads: for each (b, h) and each 64-key tile t (the last one padded
 * with zeros), d rows of 64 keys, row c holding channel c:
 *
 *   SAGE_PV_FP16: row = 128 bytes = eight 16-byte chunks of 8 fp16 values.
 *     Logical chunk kk (0..7), element e (0..7) holds key
 *       64 t + 16 (kk / 2) + 8 (e / 4) + 4 (kk % 2) + (e % 4),
 *     stored at physical chunk kk ^ ((c / 2) % 8).  Values: fp16_rne(V).
 *   SAGE_PV_FP8: row = 64 bytes = four 16-byte chunks of 16 E4M3 codes.
 *     Byte p (0..63) of the logical row holds key
 *       64 t + 32 ((p / 16) % 2) + 8 ((p % 16) / 4) + 4 (p / 32) + (p % 4),
 *     and logical chunk p / 16 is stored at physical chunk (p / 16) ^ ((c / 4) % 4).
 *     Codes: OCP E4M3FN of fp32(V * r_c), round to nearest even, with
 *     r_c = fp32(448 / colmax_t |V[t, c]|) (0 for an all-zero channel).
 *   SAGE_PV_INT8: the FP8 layout, with int8 codes
 *     clamp(rne(fp32(V * r_c)), -127, 127), r_c = fp32(127 / colmax_t |V[t, c]|).
 *
 * Tile (b, h, t) starts at byte ((b*H + h) * ceil(N/64) + t) * d * rowbytes.
 * v_scale (FP8 and INT8, else may be NULL): float32 [B,H,d] = fp32(colmax / 448)
 * or fp32(colmax / 127).  scratch: >= sage_quant_v_scratch_bytes(...) bytes,
 * 16-byte aligned
 * (FP16 mode needs none).  v_out: >= sage_quant_v_bytes(...), 16-byte aligned.
 */
int sage_quant_v(const void* v, int dtype, int B, int H, int N, int d, int pv_mode,
                 void* v_out, float* v_scale, void* scratch, size_t scratch_bytes,
                 void* stream);

/* sage_quant_v reading v in `layout` (SAGE_LAYOUT_HND or SAGE_LAYOUT_NHD);
 * the output layout is unchanged. */
int sage_quant_v_ex(const void* v, int dtype, int layout, int B, int H, int N, int d,
                    int pv_mode, void* v_out, float* v_scale, void* scratch,
                    size_t scratch_bytes, void* stream);

/*
 * Steps 3-5 alone: the attention kernel on operands already prepared by
 * sage_smooth_quant_qk and sage_quant_v (e.g. K and V quantised once and
 * reused).  q_i8, k_i8, q_scale, k_scale: as written by sage_smooth_quant_qk;
 * v_prep (and v_scale for SAGE_PV_FP8 and SAGE_PV_INT8, else may be NULL): as written by
 * sage_quant_v with the same pv_mode.  o: [B,H,N,d] of out_dtype
 * (SAGE_DT_F16, SAGE_DT_BF16 or SAGE_OUT_F32).  Same numerics as sage_attn_fwd.
 */
int sage_attn_fwd_quantized(const int8_t* q_i8, const int8_t* k_i8, const void* v_prep,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            void* o, int B, int H, int N, int d, int causal, int pv_mode,
                            int out_dtype, void* stream);

/* sage_attn_fwd_quantized with Q smoothed per block: q_i8 and q_scale from
 * sage_smooth_q, q_seed its q_comp for the same pv_mode (16-byte aligned);
 * the other operands as for sage_attn_fwd_quantized.  Same numerics as
 * sage_attn_fwd_sq. */
int sage_attn_fwd_quantized_sq(const int8_t* q_i8, const int8_t* k_i8, const void* v_prep,
                               const float* q_scale, const float* k_scale, const float* v_scale,
                               const int32_t* q_seed, void* o, int B, int H, int N, int d,
                               int causal, int pv_mode, int out_dtype, void* stream);

/*
 * Full-precision reference for selected query rows: float32 softmax
 * attention O[b,h,i,:] = softmax(q_i K^T / sqrt(d)) V (causal: keys <= i) with
 * no quantisation, for every (b, h) and every row index in `rows` (device
 * int32 [nrows]).  o: float32 [B,H,nrows,d].  A row index outside [0, N)
 * yields NaN outputs for that row (nothing is read for it).  This is the
 * reference against which a layer's quantised output is profiled when the
 * P~V precision is chosen per layer by cosine similarity ([SA] §2 Q2 item 3:
 * layers above 99.8% use the faster kernel).
 */
int sage_attn_ref_rows_f32(const void* q, const void* k, const void* v, int dtype, int B, int H,
                           int N, int d, int causal, const int32_t* rows, int nrows, float* o,
                           void* stream);

/*
 * Debug: the INT32 product S = Q^ K^T of one (b, h) on the rectangle
 * queries [q0, q0+nq) x keys [k0, k0+nk), computed by the same device code
 * (operand staging, LDS layout, INT8 MFMA tile) as the attention kernel.
 * q_i8, k_i8: int8 [B,H,N,d] as produced by sage_smooth_quant_qk.
 * s_out: int32 [nq, nk] row-major.  q0, k0, nq, nk must be multiples of 32
 * and the rectangle must lie inside [0, ceil32(N)); rows or columns >= N are
 * written as 0.
 */
int sage_attn_debug_s_i32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d,
                          int b, int h, int q0, int nq, int k0, int nk, int32_t* s_out,
                          void* stream);

/*
 * The prepass of sage_attn_fwd alone ([SA] §4 Eq. 6 and §3 Algorithm 1 up to
 * the quantised operands: K smoothed by its column mean, Q^ and K^ in INT8 per
 * block with delta_Q, delta_K, and V prepared for the P~V mode): fills the
 * private workspace exactly as sage_attn_fwd does before its attention kernel,
 * and launches no attention.  For sage_attn_debug_s_fwd on shapes where the
 * whole attention would take too long to run just to fill the workspace (a
 * head of 2^24 tokens).  Arguments, validation and errors as sage_attn_fwd
 * (SAGE_LAYOUT_HND, no output pointer, causal irrelevant).
 */
int sage_attn_prepare(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                      int pv_mode, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * The rest of sage_attn_fwd: its attention kernel ([SA] §3 Algorithm 1 from
 * the INT8 product on: dequantisation, online softmax, P~V in the pv_mode
 * precision, O = O / l) on the operands a preceding sage_attn_prepare with the
 * same B, H, N, d, pv_mode left in `workspace` (stream-ordered: launch both
 * on the same stream, or wait between them).  o: [B,H,N,d] of out_dtype
 * (SAGE_DT_F16, SAGE_DT_BF16 or SAGE_OUT_F32), caller-owned, 16-byte aligned.
 * sage_attn_prepare followed by sage_attn_attend computes exactly what
 * sage_attn_fwd computes (the same launches, bit for bit); the split lets a
 * caller time or schedule the two halves.  The workspace is only read.
 * Errors: SAGE_ERR_INVALID_ARG (null or misaligned pointers, bad flags),
 * SAGE_ERR_UNSUPPORTED (shape), SAGE_ERR_WORKSPACE (smaller than
 * sage_attn_workspace_bytes(B, H, N, d, pv_mode)).  Workspace contents not
 * written by such a sage_attn_prepare give undefined output (no fault: every
 * read stays inside the documented layout).
 */
int sage_attn_attend(const void* workspace, size_t workspace_bytes, void* o, int B, int H,
                     int N, int d, int causal, int pv_mode, int out_dtype, void* stream);

/*
 * Debug: the INT32 scores of the timed attention kernel itself ([SA] §3
 * Algorithm 1: S = Q^ K^^T in INT32).  Re-runs the attention kernel's debug
 * instantiation -- the same source, instruction schedule, LDS staging and
 * accumulator start values as the kernel sage_attn_fwd times (FP16 mode
 * starts every INT32 accumulation at the bit pattern of 1.5 * 2^23; with Q
 * smoothed, at the compensation values of sage_attn_fwd_sq) -- for head (b, h)
 * and the query rows [q0, q0 + nq), on the operands that a preceding
 * sage_attn_fwd / sage_attn_fwd_ex / sage_attn_prepare (smooth_q = 0) or
 * sage_attn_fwd_sq (smooth_q = 1) call with the same B, H, N, d, pv_mode (and
 * causal, for the forward calls) left in `workspace`.  Writes
 *   s_out  int32 [nq, nk] row-major: for query q0 + i and key k0 + j of a KV
 *          tile the kernel computes for that row, the accumulator minus its
 *          start bias, i.e. S = Q^ K^^T (S + C with Q smoothed, C as in
 *          sage_attn_fwd_sq).  Entries the kernel does not compute (keys >= N;
 *          with causal, the tiles past the diagonal of the row's query block)
 *          are left as they were;
 *   o_rows float32 [nq, d]: O of those rows, from the same launch.
 * 0 <= q0 < N, 1 <= nq <= N - q0, 0 <= k0 < N, 1 <= nk <= N - k0; s_out
 * 4-byte and o_rows 16-byte aligned; workspace as for the forward call
 * (SAGE_ERR_WORKSPACE if smaller than that call needs).  With smooth_q the
 * forward pass must have kept its whole compensation table in one chunk
 * (at most 256 MiB, see sage_attn_fwd_sq), else SAGE_ERR_UNSUPPORTED.
 */
int sage_attn_debug_s_fwd(const void* workspace, size_t workspace_bytes, int B, int H, int N,
                          int d, int causal, int pv_mode, int smooth_q, int b, int h, int q0,
                          int nq, int k0, int nk, int32_t* s_out, float* o_rows, void* stream);

/*
 * sage_attn_fwd for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc:
 * the same forward pass (same kernels, same results bit for bit) with no
 * workspace argument.  The workspace is a fixed device array of
 * SAGE_NOALLOC_MAX_WORKSPACE bytes inside this library, one per device, held
 * from this library's load until the process ends; its address on the
 * current device is looked up on the first call on that device.  The call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).
 *   Limit: shapes whose sage_attn_workspace_bytes(B,H,N,d,pv_mode) exceeds
 *   SAGE_NOALLOC_MAX_WORKSPACE return SAGE_ERR_WORKSPACE (c3's 1x24x16384x128
 *   needs about 200 MB; 1x32x4096x128 fits).
 *   Sharing: every call on a device uses that device's one array and leaves
 *   its contents behind (nothing in it needs to start at zero).  Calls whose
 *   work overlaps on one device -- on different streams, or from several host
 *   threads -- race on it and give wrong results: order them on one stream.
 * Other arguments, validation and errors as sage_attn_fwd.
 */
#define SAGE_NOALLOC_MAX_WORKSPACE ((size_t)128 << 20)
int sage_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H,
                          int N, int d, int causal, int pv_mode, int dtype, void* stream);

/* The name this entry point has in the hot-path contract: identical to
 * sage_attn_fwd_f32out (float32 O of the whole pass). */
int sage_attn_debug_fwd_f32(const void* q, const void* k, const void* v, float* o, int B, int H,
                            int N, int d, int causal, int pv_mode, int dtype, void* workspace,
                            size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_ATTN_H */
