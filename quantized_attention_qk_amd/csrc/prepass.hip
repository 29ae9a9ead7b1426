// prepass.hip -- the HBM-bound stages before the attention kernel:
//   smoothing of K ("SageAttention: Accurate 8-Bit Attention ..." detail page,
//   §4 Eq. 6: subtract the per-channel token mean), per-block INT8 quantisation
//   of Q/sqrt(d) and of the smoothed K (§3 Algorithm 1; the SageAttention2++
//   review page, section 三 core formulas: delta = max|X|/127), and the
//   preparation of V: fp16, or E4M3 with delta_V = colmax|V|/448 (same
//   section of the SageAttention2++ review page).
//
// Every quantisation decision is taken in float32 in a fixed order so that the
// codes and scales are reproducible bit for bit: no FP contraction (this file
// is built with -ffp-contract=off), IEEE division, round-to-nearest-even.
#include "sage_common.h"
#include "sage_launch.h"

namespace sage {

// ---------------------------------------------------------------------------
// Column statistics.  One thread owns a pair of channels of one 256-token
// chunk of one (b, h) and adds the tokens in increasing order from 0.0f.
// Workgroups of 256 threads cover 256/(d/2) chunks.
template <int DT, int D, bool DO_K, bool DO_V>
__global__ __launch_bounds__(256) void colstats_kernel(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, int N,
                                                       int nchunks, float* __restrict__ part_sum,
                                                       float* __restrict__ part_max) {
  constexpr int P = D / 2;
  constexpr int CPW = 256 / P;
  const int bh = blockIdx.y;
  const int p = threadIdx.x % P;
  const int chunk = blockIdx.x * CPW + threadIdx.x / P;
  if (chunk >= nchunks) return;
  const int t0 = chunk * kMeanChunk;
  const int cnt = min(kMeanChunk, N - t0);
  const size_t base = ((size_t)bh * N + t0) * D + 2 * p;
  const size_t out = ((size_t)bh * nchunks + chunk) * D + 2 * p;
  if constexpr (DO_K) {
    const uint32_t* kp = reinterpret_cast<const uint32_t*>(k + base);
    float s0 = 0.f, s1 = 0.f;
    if (cnt == kMeanChunk) {
#pragma unroll 16
      for (int t = 0; t < kMeanChunk; ++t) {
        const uint32_t w = kp[(size_t)t * P];
        s0 += in_to_f32<DT>((uint16_t)(w & 0xffffu));
        s1 += in_to_f32<DT>((uint16_t)(w >> 16));
      }
    } else {
      for (int t = 0; t < cnt; ++t) {
        const uint32_t w = kp[(size_t)t * P];
        s0 += in_to_f32<DT>((uint16_t)(w & 0xffffu));
        s1 += in_to_f32<DT>((uint16_t)(w >> 16));
      }
    }
    *reinterpret_cast<v2f*>(part_sum + out) = v2f{s0, s1};
  }
  if constexpr (DO_V) {
    const uint32_t* vp = reinterpret_cast<const uint32_t*>(v + base);
    float m0 = 0.f, m1 = 0.f;
#pragma unroll 16
    for (int t = 0; t < cnt; ++t) {
      const uint32_t w = vp[(size_t)t * P];
      m0 = fmaxf(m0, fabsf(in_to_f32<DT>((uint16_t)(w & 0xffffu))));
      m1 = fmaxf(m1, fabsf(in_to_f32<DT>((uint16_t)(w >> 16))));
    }
    *reinterpret_cast<v2f*>(part_max + out) = v2f{m0, m1};
  }
}

// Finalise: mean = (sequential sum of the chunk partials) / N; for FP8 V,
// colmax = max of the partial maxima, delta_V = colmax/448, r = 448/colmax.
template <int D, bool DO_K, bool DO_V>
__global__ __launch_bounds__(128) void finalize_kernel(const float* __restrict__ part_sum,
                                                       const float* __restrict__ part_max, int N,
                                                       int nchunks, float* __restrict__ k_mean,
                                                       float* __restrict__ v_scale,
                                                       float* __restrict__ v_recip) {
  const int bh = blockIdx.x;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    if constexpr (DO_K) {
      float tot = 0.f;
#pragma unroll 16
      for (int j = 0; j < nchunks; ++j) tot += part_sum[((size_t)bh * nchunks + j) * D + c];
      k_mean[(size_t)bh * D + c] = tot / (float)N;
    }
    if constexpr (DO_V) {
      float cm = 0.f;
#pragma unroll 16
      for (int j = 0; j < nchunks; ++j) cm = fmaxf(cm, part_max[((size_t)bh * nchunks + j) * D + c]);
      v_scale[(size_t)bh * D + c] = cm / 448.f;
      v_recip[(size_t)bh * D + c] = cm > 0.f ? 448.f / cm : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// INT8 block quantisation.  One workgroup per block (Q: 128 tokens, K: 64
// tokens) of one (b, h); a block is a contiguous run of ntok*d elements read
// as 16-byte chunks.  Values stay in registers between the absmax reduction
// and the encoding.
template <int DT, int D>
__global__ __launch_bounds__(256) void quant_qk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ k_mean, int N, int nqb, int nkb, int first_blk, float inv_sqrt_d,
    int8_t* __restrict__ q_i8, int8_t* __restrict__ k_i8, float* __restrict__ q_scale,
    float* __restrict__ k_scale) {
  constexpr int MAXC = kQBlock * D / 8 / 256;   // 16-byte chunks per thread (Q block)
  __shared__ float red[4];
  const int bh = blockIdx.y;
  const int bx = blockIdx.x + first_blk;
  const bool isq = bx < nqb;
  const int blk = isq ? bx : bx - nqb;
  const int btok = isq ? kQBlock : kKBlock;
  const int tok0 = blk * btok;
  const int ntok = min(btok, N - tok0);
  const int nchunk = ntok * (D / 8);
  const size_t base = ((size_t)bh * N + tok0) * D;
  const uint16_t* src = (isq ? q : k) + base;
  const float* mean = k_mean + (size_t)bh * D;

  // Every chunk of this thread covers the same 8 channels (256 * 8 is a
  // multiple of d); Q is scaled by 1/sqrt(d) and K has its mean subtracted,
  // each with one rounding: x = f * sc - mu with (sc, mu) = (1/sqrt(d), 0) for
  // Q and (1, mean) for K (multiplying by 1 and subtracting 0 are exact).
  const int ch0 = (threadIdx.x * 8) % D;
  const float sc = isq ? inv_sqrt_d : 1.0f;
  float mu[8];
  if (isq) {
#pragma unroll
    for (int e = 0; e < 8; ++e) mu[e] = 0.f;
  } else {
    const v4f m0 = *reinterpret_cast<const v4f*>(mean + ch0);
    const v4f m1 = *reinterpret_cast<const v4f*>(mean + ch0 + 4);
    mu[0] = m0[0]; mu[1] = m0[1]; mu[2] = m0[2]; mu[3] = m0[3];
    mu[4] = m1[0]; mu[5] = m1[1]; mu[6] = m1[2]; mu[7] = m1[3];
  }
  uint4 raw[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + i * 256;
    raw[i] = c < nchunk ? *reinterpret_cast<const uint4*>(src + (size_t)c * 8) : uint4{0u, 0u, 0u, 0u};
  }
  float x[MAXC][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const uint32_t ww[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    const bool live = threadIdx.x + i * 256 < nchunk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = in_to_f32<DT>((uint16_t)(ww[e >> 1] >> ((e & 1) * 16)));
      const float v = live ? f * sc - mu[e] : 0.f;
      x[i][e] = v;
      amax = fmaxf(amax, fabsf(v));
    }
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float r = a > 0.f ? 127.f / a : 0.f;
  int8_t* dst = (isq ? q_i8 : k_i8) + base;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + i * 256;
    if (c < nchunk) {
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t = __builtin_rintf(x[i][e] * r);
        t = fminf(fmaxf(t, -127.f), 127.f);
        packed[e >> 2] |= ((uint32_t)(uint8_t)(int8_t)(int)t) << ((e & 3) * 8);
      }
      *reinterpret_cast<uint2*>(dst + (size_t)c * 8) = uint2{packed[0], packed[1]};
    }
  }
  if (threadIdx.x == 0) {
    const float delta = a / 127.f;
    if (isq) q_scale[(size_t)bh * nqb + blk] = delta;
    else k_scale[(size_t)bh * nkb + blk] = delta;
  }
}

// ---------------------------------------------------------------------------
// V preparation.  One workgroup per 64-key tile of one (b, h): the tile is
// staged in LDS as raw 16-bit values, then every thread gathers the keys of
// one output 16-byte chunk (layout documented in sage_attn.h) and converts.
template <int DT, int D, int PV>
__global__ __launch_bounds__(256) void prep_v_kernel(const uint16_t* __restrict__ v,
                                                     const float* __restrict__ v_recip, int N,
                                                     int ntiles, uint8_t* __restrict__ v_out) {
  constexpr int LD = D + 8;   // halves per LDS row (16-byte aligned, rotated banks)
  __shared__ __attribute__((aligned(16))) uint16_t tile[kKvTile * LD];
  const int bh = blockIdx.y;
  const int t = blockIdx.x;
  const int key0 = t * kKvTile;
  constexpr int NCH = kKvTile * D / 8;
  for (int c = threadIdx.x; c < NCH; c += 256) {
    const int key = c / (D / 8);
    const int col = (c % (D / 8)) * 8;
    uint4 w = {0u, 0u, 0u, 0u};
    if (key0 + key < N)
      w = *reinterpret_cast<const uint4*>(v + ((size_t)bh * N + key0 + key) * D + col);
    *reinterpret_cast<uint4*>(&tile[key * LD + col]) = w;
  }
  __syncthreads();
  constexpr int ROWB = PV == kPvFp16 ? 128 : 64;
  uint8_t* out = v_out + ((size_t)bh * ntiles + t) * (size_t)(D * ROWB);
  if constexpr (PV == kPvFp16) {
    for (int g = threadIdx.x; g < D * 8; g += 256) {
      const int c = g >> 3;
      const int kk = (g & 7) ^ row_swizzle<128>(c);
      const int S = kk >> 1, h = kk & 1;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int key_a = 16 * S + 8 * (e >> 2) + 4 * h + (e & 3);
        const float fa = in_to_f32<DT>(tile[key_a * LD + c]);
        const float fb = in_to_f32<DT>(tile[(key_a + 1) * LD + c]);
        w[e >> 1] = pack_f16x2(fa, fb);
      }
      *reinterpret_cast<uint4*>(out + (size_t)g * 16) = uint4{w[0], w[1], w[2], w[3]};
    }
  } else {
    const float* rc = v_recip + (size_t)bh * D;
    for (int g = threadIdx.x; g < D * 4; g += 256) {
      const int c = g >> 2;
      const int lq = (g & 3) ^ row_swizzle<64>(c);
      const float r = rc[c];
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 16; e += 4) {
        float f[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int p = 16 * lq + e + u;
          const int key = 32 * ((p >> 4) & 1) + 8 * ((p & 15) >> 2) + 4 * (p >> 5) + (p & 3);
          f[u] = in_to_f32<DT>(tile[key * LD + c]) * r;
        }
        w[e >> 2] = pack_fp8x4(f[0], f[1], f[2], f[3]);
      }
      *reinterpret_cast<uint4*>(out + (size_t)g * 16) = uint4{w[0], w[1], w[2], w[3]};
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.
template <int DT, int D>
static hipError_t colstats_dispatch(const void* k, const void* v, int B, int H, int N,
                                    float* part_sum, float* part_max, float* k_mean,
                                    float* v_scale, float* v_recip, hipStream_t s) {
  const int nch = ceil_div(N, kMeanChunk);
  const int cpw = 256 / (D / 2);
  dim3 grid(ceil_div(nch, cpw), B * H);
  const bool dk = k != nullptr, dv = v != nullptr;
  auto kp = static_cast<const uint16_t*>(k);
  auto vp = static_cast<const uint16_t*>(v);
  if (dk && dv) {
    colstats_kernel<DT, D, true, true><<<grid, 256, 0, s>>>(kp, vp, N, nch, part_sum, part_max);
    finalize_kernel<D, true, true><<<B * H, 128, 0, s>>>(part_sum, part_max, N, nch, k_mean,
                                                         v_scale, v_recip);
  } else if (dk) {
    colstats_kernel<DT, D, true, false><<<grid, 256, 0, s>>>(kp, vp, N, nch, part_sum, part_max);
    finalize_kernel<D, true, false><<<B * H, 128, 0, s>>>(part_sum, part_max, N, nch, k_mean,
                                                          v_scale, v_recip);
  } else if (dv) {
    colstats_kernel<DT, D, false, true><<<grid, 256, 0, s>>>(kp, vp, N, nch, part_sum, part_max);
    finalize_kernel<D, false, true><<<B * H, 128, 0, s>>>(part_sum, part_max, N, nch, k_mean,
                                                          v_scale, v_recip);
  }
  return hipGetLastError();
}

hipError_t launch_colstats(const void* k, const void* v, int dtype, int B, int H, int N, int d,
                           float* part_sum, float* part_max, float* k_mean, float* v_scale,
                           float* v_recip, hipStream_t s) {
  if (dtype == 0 && d == 64) return colstats_dispatch<0, 64>(k, v, B, H, N, part_sum, part_max, k_mean, v_scale, v_recip, s);
  if (dtype == 0 && d == 128) return colstats_dispatch<0, 128>(k, v, B, H, N, part_sum, part_max, k_mean, v_scale, v_recip, s);
  if (dtype == 1 && d == 64) return colstats_dispatch<1, 64>(k, v, B, H, N, part_sum, part_max, k_mean, v_scale, v_recip, s);
  if (dtype == 1 && d == 128) return colstats_dispatch<1, 128>(k, v, B, H, N, part_sum, part_max, k_mean, v_scale, v_recip, s);
  return hipErrorInvalidValue;
}

template <int DT, int D>
static hipError_t quant_qk_dispatch(const void* q, const void* k, const float* k_mean, int B,
                                    int H, int N, int8_t* q_i8, int8_t* k_i8, float* q_scale,
                                    float* k_scale, hipStream_t s) {
  const int nqb = ceil_div(N, kQBlock), nkb = ceil_div(N, kKBlock);
  const float isd = (float)(1.0 / __builtin_sqrt((double)D));
  const int first = q ? 0 : nqb;
  const int count = (q ? nqb : 0) + (k ? nkb : 0);
  dim3 grid(count, B * H);
  quant_qk_kernel<DT, D><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(q),
                                              static_cast<const uint16_t*>(k), k_mean, N, nqb,
                                              nkb, first, isd, q_i8, k_i8, q_scale, k_scale);
  return hipGetLastError();
}

hipError_t launch_quant_qk(const void* q, const void* k, const float* k_mean, int dtype, int B,
                           int H, int N, int d, int8_t* q_i8, int8_t* k_i8, float* q_scale,
                           float* k_scale, hipStream_t s) {
  if (!q && !k) return hipSuccess;
  if (dtype == 0 && d == 64) return quant_qk_dispatch<0, 64>(q, k, k_mean, B, H, N, q_i8, k_i8, q_scale, k_scale, s);
  if (dtype == 0 && d == 128) return quant_qk_dispatch<0, 128>(q, k, k_mean, B, H, N, q_i8, k_i8, q_scale, k_scale, s);
  if (dtype == 1 && d == 64) return quant_qk_dispatch<1, 64>(q, k, k_mean, B, H, N, q_i8, k_i8, q_scale, k_scale, s);
  if (dtype == 1 && d == 128) return quant_qk_dispatch<1, 128>(q, k, k_mean, B, H, N, q_i8, k_i8, q_scale, k_scale, s);
  return hipErrorInvalidValue;
}

template <int DT, int D, int PV>
static hipError_t prep_v_dispatch(const void* v, const float* v_recip, int B, int H, int N,
                                  uint8_t* v_out, hipStream_t s) {
  const int nt = ceil_div(N, kKvTile);
  dim3 grid(nt, B * H);
  prep_v_kernel<DT, D, PV><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(v), v_recip, N, nt,
                                                v_out);
  return hipGetLastError();
}

hipError_t launch_prep_v(const void* v, const float* v_recip, int dtype, int B, int H, int N,
                         int d, int pv_mode, uint8_t* v_out, hipStream_t s) {
#define SAGE_PV_CASE(DT, D, PV)                                              \
  if (dtype == DT && d == D && pv_mode == PV)                                \
    return prep_v_dispatch<DT, D, PV>(v, v_recip, B, H, N, v_out, s);
  SAGE_PV_CASE(0, 64, 0) SAGE_PV_CASE(0, 64, 1) SAGE_PV_CASE(0, 128, 0) SAGE_PV_CASE(0, 128, 1)
  SAGE_PV_CASE(1, 64, 0) SAGE_PV_CASE(1, 64, 1) SAGE_PV_CASE(1, 128, 0) SAGE_PV_CASE(1, 128, 1)
#undef SAGE_PV_CASE
  return hipErrorInvalidValue;
}

}  // namespace sage
