// attn_fwd.hip -- dispatch of the attention kernel (attn_fwd_kernel.h) over
// head dimension and P~V mode, its debug dump launch, and the debug kernel of
// the INT32 product alone.
#include "attn_fwd_kernel.h"

namespace sage {

// Instantiated in attn_fwd_d{64,128}_{fp16,fp8,int8}.hip.
extern template hipError_t attn_launch_dp<64, kPvFp16>(const AttnArgs&, hipStream_t);
extern template hipError_t attn_launch_dp<64, kPvFp8>(const AttnArgs&, hipStream_t);
extern template hipError_t attn_launch_dp<64, kPvInt8>(const AttnArgs&, hipStream_t);
extern template hipError_t attn_launch_dp<128, kPvFp16>(const AttnArgs&, hipStream_t);
extern template hipError_t attn_launch_dp<128, kPvFp8>(const AttnArgs&, hipStream_t);
extern template hipError_t attn_launch_dp<128, kPvInt8>(const AttnArgs&, hipStream_t);

static hipError_t attn_launch(const AttnArgs& a, int d, int pv_mode, hipStream_t s) {
  if (d == 64) {
    if (pv_mode == kPvFp16) return attn_launch_dp<64, kPvFp16>(a, s);
    if (pv_mode == kPvFp8) return attn_launch_dp<64, kPvFp8>(a, s);
    if (pv_mode == kPvInt8) return attn_launch_dp<64, kPvInt8>(a, s);
  } else if (d == 128) {
    if (pv_mode == kPvFp16) return attn_launch_dp<128, kPvFp16>(a, s);
    if (pv_mode == kPvFp8) return attn_launch_dp<128, kPvFp8>(a, s);
    if (pv_mode == kPvInt8) return attn_launch_dp<128, kPvInt8>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn(const int8_t* q_i8, const int8_t* k_i8, const uint8_t* v_t,
                       const float* q_scale, const float* k_scale, const float* v_scale,
                       const int32_t* comp, int B, int H, int N, int d, int causal, int pv_mode,
                       int out_kind, int nhd, void* out, hipStream_t s, int q128_begin,
                       int q128_count) {
  const AttnArgs a{q_i8,   k_i8,     v_t, q_scale, k_scale, v_scale, comp, B, H,          N,
                   causal, out_kind, nhd, out,     nullptr, 0,       0,    0, 0, q128_begin,
                   q128_count};
  return attn_launch(a, d, pv_mode, s);
}

hipError_t launch_attn_dump(const int8_t* q_i8, const int8_t* k_i8, const uint8_t* v_t,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            const int32_t* comp, int B, int H, int N, int d, int causal,
                            int pv_mode, int b, int h, int q0, int nq, int k0, int nk,
                            int32_t* s_out, float* o_rows, hipStream_t s) {
  // offset every operand to head (b, h); the kernel then sees one head
  const size_t bh = (size_t)b * H + h;
  const size_t nt = (size_t)ceil_div(N, kKvTile), nq128 = (size_t)ceil_div(N, kQBlock);
  const AttnArgs a{q_i8 + bh * N * d,
                   k_i8 + bh * N * d,
                   v_t + bh * nt * v_tile_bytes(d, pv_mode),
                   q_scale + bh * nq128,
                   k_scale + bh * nt,
                   v_scale ? v_scale + bh * d : nullptr,
                   comp ? comp + bh * nq128 * nt * kKvTile : nullptr,
                   1, 1, N, causal, 2, 0, o_rows, s_out, q0, nq, k0, nk, 0, 0};
  (void)B;
  return attn_launch(a, d, pv_mode, s);
}

// ---------------------------------------------------------------------------
// Debug kernel: one wavefront per 32-query x 64-key block, using the same
// Q^ fragment load, K^ staging/LDS layout and INT8 MFMA block as the
// attention kernel, accumulating from zero.
template <int D>
__global__ __launch_bounds__(64) void debug_s_kernel(const int8_t* __restrict__ q_bh,
                                                     const int8_t* __restrict__ k_bh, int N,
                                                     int q0, int nq, int k0, int nk,
                                                     int32_t* __restrict__ s_out) {
  __shared__ __attribute__((aligned(16))) uint8_t kb[KTile<D>::BYTES];
  const int lane = threadIdx.x;
  const int n = lane & 31, hh = lane >> 5;
  const int qbase = q0 + 32 * blockIdx.x;
  const int kbase = k0 + 64 * blockIdx.y;
  v4i qf[D / 32];
  load_q_frag<D>(qf, q_bh, qbase + n, N, hh);
  const KLoader<D, 1> kld(0, lane);
  kld.template issue<true>(buffer_rsrc(k_bh, (uint32_t)((size_t)N * D)), kbase, N, lds_addr(kb),
                           0);
  wait_lds_loads();
  __syncthreads();
  const int query = qbase + n;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const v16i s = qk_block<D>(qf, kb, blk, n, hh, v16i{});
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kbase + 32 * blk + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (key < k0 + nk) {
        const int32_t val = (query < N && key < N) ? s[r] : 0;
        s_out[(size_t)(query - q0) * nk + (key - k0)] = val;
      }
    }
  }
}

hipError_t launch_debug_s(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d,
                          int b, int h, int q0, int nq, int k0, int nk, int32_t* s_out,
                          hipStream_t s) {
  const size_t bh = (size_t)b * H + h;
  dim3 grid(nq / 32, ceil_div(nk, 64));
  if (d == 64)
    debug_s_kernel<64><<<grid, 64, 0, s>>>(q_i8 + bh * N * 64, k_i8 + bh * N * 64, N, q0, nq, k0,
                                          nk, s_out);
  else if (d == 128)
    debug_s_kernel<128><<<grid, 64, 0, s>>>(q_i8 + bh * N * 128, k_i8 + bh * N * 128, N, q0, nq,
                                           k0, nk, s_out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sage
