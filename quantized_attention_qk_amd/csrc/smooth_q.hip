// smooth_q.hip -- smoothing of Q per 128-token block, the optional step of
// SageAttention2 ("SageAttention2" abstract page: smoothing Q improves the
// quantised QK^T; "SageAttention2++ ..." review page, section 三: Q and K are
// smoothed before quantisation).  The pages print no formula; this file
// implements the reading documented in sage_attn.h (sage_smooth_q):
//
//   qbar  = block mean of Q' = fp32(Q * fp32(1/sqrt(d)))  (float32, token order)
//   Q~    = fp32(Q' - qbar);  a = max|Q~|;  r = fp32(127/a)
//   Q~^   = clamp(rne(fp32(Q~ r)), -127, 127);  delta = fp32(a/127)
//   w     = rne(fp32(qbar r) * 2^8)               (per channel, an integer)
//   C[t]  = rne((w . K^[t]) / 2^8)                (per block and key)
//   S     = delta_Q delta_K (Q~^ K^^T + C)
//
// A block is smoothed only if a > 0 and 127 sum|w| <= 2^29; otherwise it is
// quantised as without smoothing (w = 0, C = 0).  Built without FP
// contraction (the decisions are reproducible bit for bit).
#include "sage_common.h"
#include "sage_launch.h"

namespace sage {

constexpr int kSqFracBits = 8;
constexpr double kSqLimit = 536870912.0;   // 2^29

// One workgroup (256 threads) per (b*h, Q block).  The block's raw 16-bit
// rows are staged in LDS; thread c < d sums channel c over the block's tokens
// in order; every thread then owns 8-channel chunks as in the plain
// quantiser.
template <int DT, int D>
__global__ __launch_bounds__(256) void smooth_q_kernel(
    const uint16_t* __restrict__ q, int N, int H, int nhd, int nqb, float inv_sqrt_d,
    int8_t* __restrict__ q_i8, float* __restrict__ q_scale, float* __restrict__ q_mean,
    int32_t* __restrict__ q_w) {
  constexpr int CPR = D / 8;                        // 16-byte chunks per token row
  constexpr int MAXC = kQBlock * CPR / 256;         // chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t tile[kQBlock * D];
  __shared__ float qbar[D];
  __shared__ float red_s[4], red_p[4];
  __shared__ double red_w[4];
  const int qb = blockIdx.x, bh = blockIdx.y;
  const int tok0 = qb * kQBlock;
  const int ntok = min(kQBlock, N - tok0);
  const int nchunk = ntok * CPR;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  for (int c = tid; c < kQBlock * CPR; c += 256) {
    uint4 w = {0u, 0u, 0u, 0u};
    if (c < nchunk)
      w = *reinterpret_cast<const uint4*>(q + row_off<D>(bh, tok0 + c / CPR, H, N, nhd) +
                                           (c % CPR) * 8);
    *reinterpret_cast<uint4*>(&tile[c * 8]) = w;
  }
  __syncthreads();
  // block mean of Q' per channel: sequential in token order from 0.0f, then
  // one IEEE division by the token count
  if (tid < D) {
    float acc = 0.f;
#pragma unroll 16
    for (int t = 0; t < ntok; ++t) acc += in_to_f32<DT>(tile[t * D + tid]) * inv_sqrt_d;
    qbar[tid] = acc / (float)ntok;
  }
  __syncthreads();

  const int ch0 = (tid * 8) % D;   // every chunk of this thread: channels ch0..ch0+7
  float xs[MAXC][8], xp[MAXC][8];
  float amax_s = 0.f, amax_p = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + i * 256;
    const bool live = c < nchunk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = in_to_f32<DT>(tile[c * 8 + e]) * inv_sqrt_d;
      const float sm = f - qbar[ch0 + e];
      xp[i][e] = live ? f : 0.f;
      xs[i][e] = live ? sm : 0.f;
      amax_p = fmaxf(amax_p, fabsf(xp[i][e]));
      amax_s = fmaxf(amax_s, fabsf(xs[i][e]));
    }
  }
  amax_s = wave_max(amax_s);
  amax_p = wave_max(amax_p);
  if (lane == 0) {
    red_s[wave] = amax_s;
    red_p[wave] = amax_p;
  }
  __syncthreads();
  const float a_s = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
  const float a_p = fmaxf(fmaxf(red_p[0], red_p[1]), fmaxf(red_p[2], red_p[3]));
  const float r_s = a_s > 0.f ? 127.f / a_s : 0.f;
  const float r_p = a_p > 0.f ? 127.f / a_p : 0.f;
  // the mean on the fine grid; |w| summed exactly in double (integers below
  // 2^53, or far above the limit)
  float wf = 0.f;
  double aw = 0.0;
  if (tid < D) {
    wf = __builtin_rintf((qbar[tid] * r_s) * 256.f);
    aw = fabs((double)wf);
  }
  for (int off = 32; off >= 1; off >>= 1) aw += __shfl_xor(aw, off, 64);
  if (lane == 0) red_w[wave] = aw;
  __syncthreads();
  const double sum_w = (red_w[0] + red_w[1]) + (red_w[2] + red_w[3]);
  const bool ok = a_s > 0.f && 127.0 * sum_w <= kSqLimit;

  const float r = ok ? r_s : r_p;
  int8_t* dst = q_i8 + ((size_t)bh * N + tok0) * D;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + i * 256;
    if (c < nchunk) {
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t = __builtin_rintf((ok ? xs[i][e] : xp[i][e]) * r);
        t = fminf(fmaxf(t, -127.f), 127.f);
        packed[e >> 2] |= ((uint32_t)(uint8_t)(int8_t)(int)t) << ((e & 3) * 8);
      }
      *reinterpret_cast<uint2*>(dst + (size_t)c * 8) = uint2{packed[0], packed[1]};
    }
  }
  const size_t mo = ((size_t)bh * nqb + qb) * D;
  if (tid < D) {
    q_mean[mo + tid] = ok ? qbar[tid] : 0.f;
    q_w[mo + tid] = ok ? (int32_t)wf : 0;
  }
  if (tid == 0) q_scale[(size_t)bh * nqb + qb] = (ok ? a_s : a_p) / 127.f;
}

// The compensation C[bh][qb][t] = rne((w[bh][qb] . K^[bh][t]) / 2^8) + bias
// for t < ld (keys at or beyond N have K^ = 0), as an INT8 MFMA product: w
// is split into four signed base-128 digits in [-64, 63] (|w| <= 2^29/127 <
// 2^22 leaves the top digit in [-2, 2]), each digit plane multiplied with K^
// (v_mfma_i32_32x32x32_i8, A = 32 keys of K^, B = 32 blocks' digits), and the
// planes combined with weights 1, 2^7, 2^14, 2^21 in wrapping 32-bit
// arithmetic, which is exact because |w . K^| <= 2^29.  Workgroup = one
// (b, h) and a chunk of kSqChunk keys; its four wavefronts take four groups
// of 32 Q blocks (more groups in turn when there are more than 128 blocks),
// build their blocks' digit operands once and walk the chunk's 32-key tiles,
// so each K^ tile comes from HBM once and is shared in L2 by the wavefronts.
constexpr int kSqChunk = 256;
// Blocks [qb0, qb0 + nqr) of the nqb of each head; comp holds nqr rows of ld
// values per head.
template <int D>
__global__ __launch_bounds__(256) void sq_comp_kernel(const int8_t* __restrict__ k_i8,
                                                      const int32_t* __restrict__ q_w, int N,
                                                      int nqb, int qb0, int nqr, int ld, int bias,
                                                      int32_t* __restrict__ comp) {
  constexpr int KT = D / 32;
  const int bh = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int c0 = blockIdx.x * kSqChunk;
  const int c1 = min(c0 + kSqChunk, ld);
  const bool vec = (ld & 3) == 0;   // rows 16-byte aligned: 16-byte stores
  for (int g = wave; g * 32 < nqr; g += 4) {
    const int qr = g * 32 + n;      // B column of this lane: block qb0 + qr
    const bool in = qr < nqr;
    const int qb = qb0 + qr;
    // the digit operands of this lane's block: plane p, d-step kt
    v4i dig[4][KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      uint32_t dd[4][4] = {};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i x = in ? *reinterpret_cast<const v4i*>(
                                     q_w + ((size_t)bh * nqb + qb) * D + 32 * kt + 16 * hh + 4 * j)
                               : v4i{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int v = x[u];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int dp = p < 3 ? ((v + 64) & 127) - 64 : v;
            v = (v - dp) >> 7;
            dd[p][j] |= ((uint32_t)(uint8_t)(int8_t)dp) << (8 * u);
          }
        }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
        dig[p][kt] = v4i{(int)dd[p][0], (int)dd[p][1], (int)dd[p][2], (int)dd[p][3]};
    }
    int32_t* out = comp + ((size_t)bh * nqr + qr) * ld;
    // A operand (this lane's key row of K^) of a 32-key tile; the next
    // tile's is loaded while the current one is multiplied
    auto load_a = [&](int t0, v4i (&a)[KT]) __attribute__((always_inline)) {
      const int key = t0 + n;
      const int8_t* krow = k_i8 + ((size_t)bh * N + key) * D + 16 * hh;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        a[kt] = key < N ? *reinterpret_cast<const v4i*>(krow + 32 * kt) : v4i{0, 0, 0, 0};
    };
    v4i a_next[KT];
    load_a(c0, a_next);
    for (int t0 = c0; t0 < c1; t0 += 32) {
      v4i a[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) a[kt] = a_next[kt];
      if (t0 + 32 < c1) load_a(t0 + 32, a_next);
      v16i acc[4] = {};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int p = 0; p < 4; ++p)
          acc[p] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[kt], dig[p][kt], acc[p], 0, 0, 0);
      if (!in) continue;
      int cv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // copy the elements to scalars first (clang mis-lowers some
        // ext_vector element uses)
        const uint32_t p0 = (uint32_t)acc[0][r], p1 = (uint32_t)acc[1][r];
        const uint32_t p2 = (uint32_t)acc[2][r], p3 = (uint32_t)acc[3][r];
        const int P = (int)(p0 + (p1 << 7) + (p2 << 14) + (p3 << 21));
        int c = P >> kSqFracBits;                           // floor
        const int rem = P - (c << kSqFracBits);             // 0 .. 255
        c += (rem > 128 || (rem == 128 && (c & 1))) ? 1 : 0;
        cv[r] = c + bias;
      }
      // register r holds key t0 + 8 (r/4) + 4 hh + r%4
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + 8 * j + 4 * hh;
        if (vec && t + 3 < ld) {
          *reinterpret_cast<v4i*>(out + t) = v4i{cv[4 * j], cv[4 * j + 1], cv[4 * j + 2],
                                                 cv[4 * j + 3]};
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (t + u < ld) out[t + u] = cv[4 * j + u];
        }
      }
    }
  }
}

hipError_t launch_smooth_q(const void* q, int dtype, int B, int H, int N, int d, int nhd,
                           int8_t* q_i8, float* q_scale, float* q_mean, int32_t* q_w,
                           hipStream_t s) {
  const int nqb = ceil_div(N, kQBlock);
  const float isd = (float)(1.0 / __builtin_sqrt((double)d));
  dim3 grid(nqb, B * H);
  auto qp = static_cast<const uint16_t*>(q);
#define SAGE_SQ(DT, D)                                                                       \
  if (dtype == DT && d == D) {                                                               \
    smooth_q_kernel<DT, D><<<grid, 256, 0, s>>>(qp, N, H, nhd, nqb, isd, q_i8, q_scale,      \
                                                q_mean, q_w);                                \
    return hipGetLastError();                                                                \
  }
  SAGE_SQ(0, 64) SAGE_SQ(0, 128) SAGE_SQ(1, 64) SAGE_SQ(1, 128)
#undef SAGE_SQ
  return hipErrorInvalidValue;
}

hipError_t launch_sq_comp(const int8_t* k_i8, const int32_t* q_w, int B, int H, int N, int d,
                          int ld, int bias, int32_t* comp, hipStream_t s, int qb0, int nqr) {
  const int nqb = ceil_div(N, kQBlock);
  if (nqr < 0) nqr = nqb - qb0;
  dim3 grid(ceil_div(ld, kSqChunk), B * H);
  if (d == 64)
    sq_comp_kernel<64><<<grid, 256, 0, s>>>(k_i8, q_w, N, nqb, qb0, nqr, ld, bias, comp);
  else if (d == 128)
    sq_comp_kernel<128><<<grid, 256, 0, s>>>(k_i8, q_w, N, nqb, qb0, nqr, ld, bias, comp);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sage
