// prepass.hip -- the HBM-bound stages before the attention kernel:
//   smoothing of K ("SageAttention: Accurate 8-Bit Attention ..." detail page,
//   §4 Eq. 6: subtract the per-channel token mean), per-block INT8 quantisation
//   of Q/sqrt(d) and of the smoothed K (§3 Algorithm 1; the SageAttention2++
//   review page, section 三 core formulas: delta = max|X|/127), and the
//   preparation of V: fp16, or E4M3 with delta_V = colmax|V|/448 (same
//   section of the SageAttention2++ review page), or INT8 with delta_V =
//   colmax|V|/127 for the all-INT8 kernel variant (SageAttention detail page,
//   §3 Figure 5).
//
// Every quantisation decision is taken in float32 in a fixed order so that the
// codes and scales are reproducible bit for bit: no FP contraction (this file
// is built with -ffp-contract=off), IEEE division, round-to-nearest-even.
#include "sage_common.h"
#include "sage_launch.h"

namespace sage {

// ---------------------------------------------------------------------------
// Rotate-half RoPE of one channel pair (x_i, x_{i+d/2}) with c = cos, s = sin:
// (x_i c - x_{i+d/2} s, x_{i+d/2} c + x_i s), every product and sum rounded
// to float32 (this file is compiled without FP contraction).
__device__ __forceinline__ void rope_pair(float lo, float hi, float c, float s, float& rlo,
                                          float& rhi) {
  rlo = lo * c - hi * s;
  rhi = hi * c + lo * s;
}

// Column statistics.  Without RoPE one thread owns a pair of channels of one
// 256-token chunk of one (b, h) and adds the tokens in increasing order from
// 0.0f; with RoPE it owns the two channel pairs (c, c+1) and (c+d/2, c+1+d/2)
// and adds the rotated values.  Workgroups of 256 threads cover several
// chunks.
template <int D, bool ROPE>
struct ColstatsShape {
  static constexpr int P = ROPE ? D / 4 : D / 2;   // threads per 256-token chunk
};

template <int DT, int D, bool DO_K, bool DO_V, bool ROPE, int UNR = 16>
__device__ __forceinline__ void colstats_chunk(const uint16_t* __restrict__ k,
                                               const uint16_t* __restrict__ v, int N, int H,
                                               int nhd, int nchunks,
                                               const float* __restrict__ rope_cos,
                                               const float* __restrict__ rope_sin,
                                               float* __restrict__ part_sum,
                                               float* __restrict__ part_max, int bh, int chunk,
                                               int p) {
  constexpr int HD = D / 2;
  const int t0 = chunk * kMeanChunk;
  const int cnt = min(kMeanChunk, N - t0);
  const size_t ts = nhd ? (size_t)H * D : (size_t)D;   // token stride (elements)
  const size_t base = row_off<D>(bh, t0, H, N, nhd) + 2 * p;
  const size_t out = ((size_t)bh * nchunks + chunk) * D + 2 * p;
  // Loads are issued in batches of UNR tokens before the batch is added in
  // token order (the chunk's 256 tokens in two batches: each batch costs a
  // full memory round trip, and a chunk is walked by one thread per channel
  // pair).
  if constexpr (!ROPE) {
    if constexpr (DO_K) {
      const uint16_t* kp = k + base;
      float s0 = 0.f, s1 = 0.f;
      for (int t0 = 0; t0 < cnt; t0 += UNR) {
        uint32_t w[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u)   // (past the end: the last token again, not added)
          w[u] = *reinterpret_cast<const uint32_t*>(kp + min(t0 + u, cnt - 1) * ts);
        if (t0 + UNR <= cnt) {   // a whole batch (every batch but a ragged last one)
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            s0 += in_to_f32<DT>((uint16_t)(w[u] & 0xffffu));
            s1 += in_to_f32<DT>((uint16_t)(w[u] >> 16));
          }
        } else {
#pragma unroll
          for (int u = 0; u < UNR; ++u)
            if (t0 + u < cnt) {
              s0 += in_to_f32<DT>((uint16_t)(w[u] & 0xffffu));
              s1 += in_to_f32<DT>((uint16_t)(w[u] >> 16));
            }
        }
      }
      *reinterpret_cast<v2f*>(part_sum + out) = v2f{s0, s1};
    }
    if constexpr (DO_V) {
      const uint16_t* vp = v + base;
      float m0 = 0.f, m1 = 0.f;
      for (int t0 = 0; t0 < cnt; t0 += UNR) {
        uint32_t w[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u)   // (past the end: the last token again, same maximum)
          w[u] = *reinterpret_cast<const uint32_t*>(vp + min(t0 + u, cnt - 1) * ts);
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          m0 = fmaxf(m0, fabsf(in_to_f32<DT>((uint16_t)(w[u] & 0xffffu))));
          m1 = fmaxf(m1, fabsf(in_to_f32<DT>((uint16_t)(w[u] >> 16))));
        }
      }
      *reinterpret_cast<v2f*>(part_max + out) = v2f{m0, m1};
    }
  } else {
    if constexpr (DO_K) {
      const uint16_t* kp = k + base;
      const float* cp = rope_cos + (size_t)t0 * HD + 2 * p;
      const float* sp = rope_sin + (size_t)t0 * HD + 2 * p;
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
      constexpr int RB = 8;   // tokens per batch of loads (four loads each)
      for (int t0 = 0; t0 < cnt; t0 += RB) {
        uint32_t lo[RB], hi[RB];
        v2f c[RB], sn[RB];
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const int t = min(t0 + u, cnt - 1);   // a skipped token re-reads the last one
          lo[u] = *reinterpret_cast<const uint32_t*>(kp + t * ts);
          hi[u] = *reinterpret_cast<const uint32_t*>(kp + t * ts + HD);
          c[u] = *reinterpret_cast<const v2f*>(cp + (size_t)t * HD);
          sn[u] = *reinterpret_cast<const v2f*>(sp + (size_t)t * HD);
        }
#pragma unroll
        for (int u = 0; u < RB; ++u)
          if (t0 + u < cnt) {
            float r0, r1, r2, r3;
            rope_pair(in_to_f32<DT>((uint16_t)(lo[u] & 0xffffu)),
                      in_to_f32<DT>((uint16_t)(hi[u] & 0xffffu)), c[u][0], sn[u][0], r0, r2);
            rope_pair(in_to_f32<DT>((uint16_t)(lo[u] >> 16)), in_to_f32<DT>((uint16_t)(hi[u] >> 16)),
                      c[u][1], sn[u][1], r1, r3);
            s0 += r0;
            s1 += r1;
            s2 += r2;
            s3 += r3;
          }
      }
      *reinterpret_cast<v2f*>(part_sum + out) = v2f{s0, s1};
      *reinterpret_cast<v2f*>(part_sum + out + HD) = v2f{s2, s3};
    }
    if constexpr (DO_V) {
      const uint16_t* vp = v + base;
      float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f;
#pragma unroll 8
      for (int t = 0; t < cnt; ++t) {
        const uint32_t lo = *reinterpret_cast<const uint32_t*>(vp + t * ts);
        const uint32_t hi = *reinterpret_cast<const uint32_t*>(vp + t * ts + HD);
        m0 = fmaxf(m0, fabsf(in_to_f32<DT>((uint16_t)(lo & 0xffffu))));
        m1 = fmaxf(m1, fabsf(in_to_f32<DT>((uint16_t)(lo >> 16))));
        m2 = fmaxf(m2, fabsf(in_to_f32<DT>((uint16_t)(hi & 0xffffu))));
        m3 = fmaxf(m3, fabsf(in_to_f32<DT>((uint16_t)(hi >> 16))));
      }
      *reinterpret_cast<v2f*>(part_max + out) = v2f{m0, m1};
      *reinterpret_cast<v2f*>(part_max + out + HD) = v2f{m2, m3};
    }
  }
}

template <int DT, int D, bool DO_K, bool DO_V, bool ROPE>
__global__ __launch_bounds__(256) void colstats_kernel(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, int N,
                                                       int H, int nhd, int nchunks,
                                                       const float* __restrict__ rope_cos,
                                                       const float* __restrict__ rope_sin,
                                                       float* __restrict__ part_sum,
                                                       float* __restrict__ part_max) {
  constexpr int P = ColstatsShape<D, ROPE>::P;
  constexpr int CPW = 256 / P;
  int chunk = blockIdx.x * CPW + threadIdx.x / P;
  // a chunk per wavefront (P = 64): uniform, so its bounds are scalar
  if constexpr (P % 64 == 0) chunk = __builtin_amdgcn_readfirstlane(chunk);
  if (chunk >= nchunks) return;
  colstats_chunk<DT, D, DO_K, DO_V, ROPE, 128>(k, v, N, H, nhd, nchunks, rope_cos, rope_sin, part_sum,
                                          part_max, blockIdx.y, chunk, threadIdx.x % P);
}

// Finalise: mean = (sequential sum of the chunk partials) / N; for quantised
// V, colmax = max of the partial maxima, delta_V = colmax/vr, r = vr/colmax
// with vr the code range (FP8 448, INT8 127).
template <int D, bool DO_K, bool DO_V>
__device__ __forceinline__ void finalize_channel(const float* __restrict__ part_sum,
                                                 const float* __restrict__ part_max, int N,
                                                 int nchunks, float* __restrict__ k_mean,
                                                 float* __restrict__ v_scale,
                                                 float* __restrict__ v_recip, float vr, int bh,
                                                 int c) {
  {
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
      v_scale[(size_t)bh * D + c] = cm / vr;
      v_recip[(size_t)bh * D + c] = cm > 0.f ? vr / cm : 0.f;
    }
  }
}

template <int D, bool DO_K, bool DO_V>
__global__ __launch_bounds__(128) void finalize_kernel(const float* __restrict__ part_sum,
                                                       const float* __restrict__ part_max, int N,
                                                       int nchunks, float* __restrict__ k_mean,
                                                       float* __restrict__ v_scale,
                                                       float* __restrict__ v_recip, float vr) {
  for (int c = threadIdx.x; c < D; c += blockDim.x)
    finalize_channel<D, DO_K, DO_V>(part_sum, part_max, N, nchunks, k_mean, v_scale, v_recip,
                                    vr, blockIdx.x, c);
}

// ---------------------------------------------------------------------------
// INT8 block quantisation.  One workgroup per block (Q: 128 tokens, K: 64
// tokens) of one (b, h); a block is a contiguous run of ntok*d elements read
// as 16-byte chunks.  Values stay in registers between the absmax reduction
// and the encoding.
template <int DT, int D, bool ROPE>
__device__ __forceinline__ void quant_block(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ mean, int N, int H, int nhd, int nqb, int nkb, float inv_sqrt_d,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin,
    int8_t* __restrict__ q_i8, int8_t* __restrict__ k_i8, float* __restrict__ q_scale,
    float* __restrict__ k_scale, int bh, int bx, float* red) {
  constexpr int MAXC = kQBlock * D / 8 / 256;   // 16-byte chunks per thread (Q block)
  const bool isq = bx < nqb;
  const int blk = isq ? bx : bx - nqb;
  const int btok = isq ? kQBlock : kKBlock;
  const int tok0 = blk * btok;
  const int ntok = min(btok, N - tok0);
  const int nchunk = ntok * (D / 8);
  const size_t base = ((size_t)bh * N + tok0) * D;   // of the INT8 output ([B,H,N,d])
  const uint16_t* src = isq ? q : k;   // (mean: head bh's K mean, read by K blocks only)
  constexpr int CPR = D / 8;   // chunks per token row

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
  // With RoPE every chunk also needs the chunk d/2 channels away in the same
  // row (its rotation partner) and 8 entries of the cos/sin tables.
  constexpr int HD = D / 2;
  const int pch = (ch0 + HD) % D;
  uint4 raw[MAXC], par[MAXC];
  v4f cs[MAXC][2], sn[MAXC][2];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + i * 256;
    const int tok = tok0 + c / CPR;
    const uint16_t* row = src + row_off<D>(bh, tok, H, N, nhd);
    raw[i] = c < nchunk ? *reinterpret_cast<const uint4*>(row + ch0) : uint4{0u, 0u, 0u, 0u};
    if constexpr (ROPE) {
      par[i] = c < nchunk ? *reinterpret_cast<const uint4*>(row + pch) : uint4{0u, 0u, 0u, 0u};
      const size_t toff = (size_t)(c < nchunk ? tok : tok0) * HD + (ch0 % HD);
      cs[i][0] = *reinterpret_cast<const v4f*>(rope_cos + toff);
      cs[i][1] = *reinterpret_cast<const v4f*>(rope_cos + toff + 4);
      sn[i][0] = *reinterpret_cast<const v4f*>(rope_sin + toff);
      sn[i][1] = *reinterpret_cast<const v4f*>(rope_sin + toff + 4);
    }
  }
  float x[MAXC][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const uint32_t ww[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    const uint32_t pp[4] = {par[i].x, par[i].y, par[i].z, par[i].w};
    const bool live = threadIdx.x + i * 256 < nchunk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float f = in_to_f32<DT>((uint16_t)(ww[e >> 1] >> ((e & 1) * 16)));
      if constexpr (ROPE) {
        const float g = in_to_f32<DT>((uint16_t)(pp[e >> 1] >> ((e & 1) * 16)));
        const float c = cs[i][e >> 2][e & 3], sv = sn[i][e >> 2][e & 3];
        const bool low = ch0 < HD;   // own channel in the low half of the pair
        float rl, rh;
        rope_pair(low ? f : g, low ? g : f, c, sv, rl, rh);
        f = low ? rl : rh;
      }
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

template <int DT, int D, bool ROPE>
__global__ __launch_bounds__(256) void quant_qk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ k_mean, int N, int H, int nhd, int nqb, int nkb, int first_blk,
    float inv_sqrt_d, const float* __restrict__ rope_cos, const float* __restrict__ rope_sin,
    int8_t* __restrict__ q_i8, int8_t* __restrict__ k_i8, float* __restrict__ q_scale,
    float* __restrict__ k_scale) {
  __shared__ float red[4];
  quant_block<DT, D, ROPE>(q, k, k_mean ? k_mean + (size_t)blockIdx.y * D : nullptr, N, H, nhd,
                           nqb, nkb, inv_sqrt_d, rope_cos, rope_sin, q_i8, k_i8, q_scale,
                           k_scale, blockIdx.y, blockIdx.x + first_blk, red);
}

// ---------------------------------------------------------------------------
// V preparation.  One workgroup per 64-key tile of one (b, h): the tile is
// staged in LDS as raw 16-bit values, then every thread gathers the keys of
// one output 16-byte chunk (layout documented in sage_attn.h) and converts.
template <int D>
struct PrepVTile {
  static constexpr int LD = D + 8;   // halves per LDS row (16-byte aligned, rotated banks)
  static constexpr int HALVES = kKvTile * LD;
};

template <int DT, int D, int PV>
__device__ __forceinline__ void prep_v_tile(const uint16_t* __restrict__ v,
                                            const float* __restrict__ v_recip, int N, int H,
                                            int nhd, int ntiles, uint8_t* __restrict__ v_out,
                                            int bh, int t, uint16_t* tile) {
  constexpr int LD = PrepVTile<D>::LD;
  const int key0 = t * kKvTile;
  constexpr int NCH = kKvTile * D / 8;
  for (int c = threadIdx.x; c < NCH; c += 256) {
    const int key = c / (D / 8);
    const int col = (c % (D / 8)) * 8;
    uint4 w = {0u, 0u, 0u, 0u};
    if (key0 + key < N)
      w = *reinterpret_cast<const uint4*>(v + row_off<D>(bh, key0 + key, H, N, nhd) + col);
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
    const float* rc = v_recip;   // this head's range/colmax, d entries
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
        w[e >> 2] = PV == kPvFp8 ? pack_fp8x4(f[0], f[1], f[2], f[3])
                                 : pack_i8x4_sym(f[0], f[1], f[2], f[3]);
      }
      *reinterpret_cast<uint4*>(out + (size_t)g * 16) = uint4{w[0], w[1], w[2], w[3]};
    }
  }
}

template <int DT, int D, int PV>
__global__ __launch_bounds__(256) void prep_v_kernel(const uint16_t* __restrict__ v,
                                                     const float* __restrict__ v_recip, int N,
                                                     int H, int nhd, int ntiles,
                                                     uint8_t* __restrict__ v_out) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[PrepVTile<D>::HALVES];
  prep_v_tile<DT, D, PV>(v, PV != kPvFp16 ? v_recip + (size_t)blockIdx.y * D : nullptr, N, H,
                         nhd, ntiles, v_out, blockIdx.y, blockIdx.x, tile);
}

// ---------------------------------------------------------------------------
// Two-launch prepass for short sequences.  The first launch's workgroups take
// roles, ordered so that the longest ones start first:
//   roles 0 .. nch-1     the column sums of one 256-token chunk of K each
//                        (the chunk staged in LDS, 128 tokens at a time,
//                        then every channel summed in token order);
//   next nqb roles       one Q^ block each (no statistics needed);
//   then ntiles roles    one V tile each (FP8, INT8: the tile's workgroup
//                        takes the head's column maxima itself).
// The second launch has one wavefront per K^ block: the head's mean from the
// chunk sums (chunks in order, one IEEE division), then the block.  A head of
// one chunk (N <= 256) needs no second launch: the chunk's workgroup forms
// the mean from its own sums and its four wavefronts quantise the K^ blocks.  Every
// value is computed by the same expressions, in the same order, as in the
// multi-kernel path above (a maximum does not depend on order), so the
// results are identical bit for bit.
constexpr int kStageTok = 128;

// Column sums of chunk `chunk` of head bh into part_sum (as colstats_chunk),
// by the whole workgroup: the chunk's rows are staged in `tile` (kStageTok * D
// halves) and thread c < D adds channel c over the tokens in order.
// Returns thread c's sum (channel c; 0 for c >= D).
template <int DT, int D, bool ROPE>
__device__ __forceinline__ float colstats_chunk_staged(
    const uint16_t* __restrict__ k, int N, int H, int nhd, int nchunks,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin,
    float* __restrict__ part_sum, int bh, int chunk, uint16_t* tile) {
  constexpr int HD = D / 2;
  constexpr int CPR = D / 8;
  const int t0 = chunk * kMeanChunk;
  const int cnt = min(kMeanChunk, N - t0);
  const int c = threadIdx.x;
  float acc = 0.f;
  for (int s0 = 0; s0 < cnt; s0 += kStageTok) {
    const int ns = min(kStageTok, cnt - s0);
    for (int x = threadIdx.x; x < ns * CPR; x += 256)
      *reinterpret_cast<uint4*>(&tile[x * 8]) = *reinterpret_cast<const uint4*>(
          k + row_off<D>(bh, t0 + s0 + x / CPR, H, N, nhd) + (x % CPR) * 8);
    __syncthreads();
    if (c < D) {
      if constexpr (!ROPE) {
#pragma unroll 8
        for (int t = 0; t < ns; ++t) acc += in_to_f32<DT>(tile[t * D + c]);
      } else {
        // rope_pair's arithmetic: the low channel of a pair takes x c - y s,
        // the high one y c + x s (x low, y high), each rounded to float32
        const bool low = c < HD;
        const int pc = low ? c + HD : c - HD;
        const size_t tb = (size_t)(t0 + s0) * HD + (low ? c : pc);
#pragma unroll 8
        for (int t = 0; t < ns; ++t) {
          const float f = in_to_f32<DT>(tile[t * D + c]);
          const float g = in_to_f32<DT>(tile[t * D + pc]);
          const float cs = rope_cos[tb + (size_t)t * HD], sn = rope_sin[tb + (size_t)t * HD];
          float rl, rh;
          rope_pair(low ? f : g, low ? g : f, cs, sn, rl, rh);
          acc += low ? rl : rh;
        }
      }
    }
    __syncthreads();
  }
  if (c < D) part_sum[((size_t)bh * nchunks + chunk) * D + c] = acc;
  return acc;
}

template <int DT, int D, bool ROPE>
__device__ __forceinline__ void kblock_x8(const uint16_t* __restrict__ k, int bh, int tok, int N,
                                          int H, int nhd, int ch0, const float (&mu)[8],
                                          const float* __restrict__ rope_cos,
                                          const float* __restrict__ rope_sin, float (&x)[8]) {
  constexpr int HD = D / 2;
  const uint16_t* row = k + row_off<D>(bh, tok, H, N, nhd);
  const uint4 raw = *reinterpret_cast<const uint4*>(row + ch0);
  const uint32_t ww[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t pp[4] = {0u, 0u, 0u, 0u};
  v4f cs[2], sn[2];
  if constexpr (ROPE) {
    const uint4 par = *reinterpret_cast<const uint4*>(row + (ch0 + HD) % D);
    pp[0] = par.x; pp[1] = par.y; pp[2] = par.z; pp[3] = par.w;
    const size_t toff = (size_t)tok * HD + (ch0 % HD);
    cs[0] = *reinterpret_cast<const v4f*>(rope_cos + toff);
    cs[1] = *reinterpret_cast<const v4f*>(rope_cos + toff + 4);
    sn[0] = *reinterpret_cast<const v4f*>(rope_sin + toff);
    sn[1] = *reinterpret_cast<const v4f*>(rope_sin + toff + 4);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float f = in_to_f32<DT>((uint16_t)(ww[e >> 1] >> ((e & 1) * 16)));
    if constexpr (ROPE) {
      const float g = in_to_f32<DT>((uint16_t)(pp[e >> 1] >> ((e & 1) * 16)));
      const float c = cs[e >> 2][e & 3], sv = sn[e >> 2][e & 3];
      const bool low = ch0 < HD;
      float rl, rh;
      rope_pair(low ? f : g, low ? g : f, c, sv, rl, rh);
      f = low ? rl : rh;
    }
    x[e] = f * 1.0f - mu[e];   // as the block quantiser: scale 1 for K, one rounding
  }
}

// K^ block blk of head bh by one wavefront; mean: the head's d channel means.
template <int DT, int D, bool ROPE>
__device__ __forceinline__ void quant_kblock_wave(
    const uint16_t* __restrict__ k, const float* mean, int N, int H, int nhd,
    int nkb, const float* __restrict__ rope_cos, const float* __restrict__ rope_sin,
    int8_t* __restrict__ k_i8, float* __restrict__ k_scale, int bh, int blk, int lane) {
  constexpr int CPR = D / 8;                  // chunks per token row
  constexpr int CPL = kKBlock * CPR / 64;     // chunks per lane
  const int tok0 = blk * kKBlock;
  const int ntok = min(kKBlock, N - tok0);
  const int ch0 = (lane * 8) % D;
  float mu[8];
  {
    const v4f m0 = *reinterpret_cast<const v4f*>(mean + ch0);
    const v4f m1 = *reinterpret_cast<const v4f*>(mean + ch0 + 4);
    mu[0] = m0[0]; mu[1] = m0[1]; mu[2] = m0[2]; mu[3] = m0[3];
    mu[4] = m1[0]; mu[5] = m1[1]; mu[6] = m1[2]; mu[7] = m1[3];
  }
  float amax = 0.f;
#pragma unroll 4
  for (int i = 0; i < CPL; ++i) {
    const int r = (lane + 64 * i) / CPR;
    if (r < ntok) {
      float x[8];
      kblock_x8<DT, D, ROPE>(k, bh, tok0 + r, N, H, nhd, ch0, mu, rope_cos, rope_sin, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
    }
  }
  const float a = wave_max(amax);
  const float rcp = a > 0.f ? 127.f / a : 0.f;
  int8_t* dst = k_i8 + ((size_t)bh * N + tok0) * D;
#pragma unroll 4
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    const int r = c / CPR;
    if (r < ntok) {
      float x[8];
      kblock_x8<DT, D, ROPE>(k, bh, tok0 + r, N, H, nhd, ch0, mu, rope_cos, rope_sin, x);
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t = __builtin_rintf(x[e] * rcp);
        t = fminf(fmaxf(t, -127.f), 127.f);
        packed[e >> 2] |= ((uint32_t)(uint8_t)(int8_t)(int)t) << ((e & 3) * 8);
      }
      *reinterpret_cast<uint2*>(dst + (size_t)c * 8) = uint2{packed[0], packed[1]};
    }
  }
  if (lane == 0) k_scale[(size_t)bh * nkb + blk] = a / 127.f;
}

// Column maxima |V| of head bh over all N tokens, by the whole workgroup, into
// vmax[D] (LDS); part[4][D] is LDS scratch.
template <int DT, int D>
__device__ __forceinline__ void head_colmax(const uint16_t* __restrict__ v, int bh, int N, int H,
                                            int nhd, float* part, float* vmax) {
  constexpr int CPR = D / 8;
  constexpr int RPP = 256 / CPR;   // token rows per pass of the workgroup
  const int tid = threadIdx.x;
  const int cc = tid % CPR, r0 = tid / CPR;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int t = r0; t < N; t += RPP) {
    const uint4 raw = *reinterpret_cast<const uint4*>(v + row_off<D>(bh, t, H, N, nhd) + cc * 8);
    const uint32_t ww[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      m[e] = fmaxf(m[e], fabsf(in_to_f32<DT>((uint16_t)(ww[e >> 1] >> ((e & 1) * 16)))));
  }
  // lanes l and l + CPR*j of a wavefront hold the same channels
#pragma unroll
  for (int e = 0; e < 8; ++e)
    for (int off = CPR; off < 64; off <<= 1) m[e] = fmaxf(m[e], __shfl_xor(m[e], off, 64));
  const int wave = tid >> 6, lane = tid & 63;
  if (lane < CPR)
#pragma unroll
    for (int e = 0; e < 8; ++e) part[wave * D + lane * 8 + e] = m[e];
  __syncthreads();
  for (int c = tid; c < D; c += 256)
    vmax[c] = fmaxf(fmaxf(part[c], part[D + c]), fmaxf(part[2 * D + c], part[3 * D + c]));
  __syncthreads();
}

template <int DT, int D, int PV, bool ROPE, bool DO_QK, bool DO_V>
__global__ __launch_bounds__(256) void prepass_roles_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int N, int H, int BH, int nhd,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, float inv_sqrt_d,
    float* __restrict__ part_sum, float* __restrict__ k_mean, float* __restrict__ v_scale,
    int8_t* __restrict__ q_i8, int8_t* __restrict__ k_i8, float* __restrict__ q_scale,
    float* __restrict__ k_scale, uint8_t* __restrict__ v_out) {
  constexpr int TILE = PrepVTile<D>::HALVES > kStageTok * D ? PrepVTile<D>::HALVES
                                                            : kStageTok * D;
  __shared__ __attribute__((aligned(16))) uint16_t tile[TILE];
  __shared__ float red[4];
  const int bh = blockIdx.x % BH;
  int role = blockIdx.x / BH;
  const int nch = (N + kMeanChunk - 1) / kMeanChunk;
  const int nqb = (N + kQBlock - 1) / kQBlock, nkb = (N + kKBlock - 1) / kKBlock;
  const int ntiles = (N + kKvTile - 1) / kKvTile;
  if constexpr (DO_QK) {
    if (role < nch) {   // K column sums of one chunk
      const float acc = colstats_chunk_staged<DT, D, ROPE>(k, N, H, nhd, nch, rope_cos,
                                                           rope_sin, part_sum, bh, role, tile);
      if (nch == 1) {
        // the whole head: its mean is this chunk's sum over N (0.0f + sum in
        // the chunk order of finalize_channel is the sum itself), then the
        // K^ blocks, one wavefront each
        __shared__ __attribute__((aligned(16))) float mean[D];
        if (threadIdx.x < D) {
          mean[threadIdx.x] = acc / (float)N;
          k_mean[(size_t)bh * D + threadIdx.x] = mean[threadIdx.x];
        }
        __syncthreads();
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        for (int blk = wave; blk < nkb; blk += 4)
          quant_kblock_wave<DT, D, ROPE>(k, mean, N, H, nhd, nkb, rope_cos, rope_sin, k_i8,
                                         k_scale, bh, blk, lane);
      }
      return;
    }
    role -= nch;
    if (role < nqb) {   // a Q block: quant_block's index bx < nqb selects Q
      quant_block<DT, D, ROPE>(q, k, k_mean + (size_t)bh * D, N, H, nhd, nqb, nkb, inv_sqrt_d,
                               rope_cos, rope_sin, q_i8, k_i8, q_scale, k_scale, bh, role, red);
      return;
    }
    role -= nqb;
  }
  if constexpr (DO_V) {
    if (role >= ntiles) return;
    if constexpr (PV != kPvFp16) {
      constexpr float VR = PV == kPvInt8 ? 127.f : 448.f;
      __shared__ float part[4 * D], vrc[D];
      head_colmax<DT, D>(v, bh, N, H, nhd, part, vrc);
      // the same expressions as the finalisation of the multi-kernel path
      for (int c = threadIdx.x; c < D; c += 256) {
        const float cm = vrc[c];
        if (role == 0) v_scale[(size_t)bh * D + c] = cm / VR;
        vrc[c] = cm > 0.f ? VR / cm : 0.f;
      }
      __syncthreads();
      prep_v_tile<DT, D, PV>(v, vrc, N, H, nhd, ntiles, v_out, bh, role, tile);
    } else {
      prep_v_tile<DT, D, PV>(v, nullptr, N, H, nhd, ntiles, v_out, bh, role, tile);
    }
  }
}

// Second launch of the short-sequence prepass: one wavefront per (K^ block,
// head).  The head's mean, as finalize_channel forms it (chunk sums in order
// from 0.0f, one IEEE division by N), into LDS (block 0 also stores it), then
// the block.
template <int DT, int D, bool ROPE>
__global__ __launch_bounds__(64) void prepass_kblocks_kernel(
    const uint16_t* __restrict__ k, int N, int H, int nhd, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, const float* __restrict__ part_sum,
    float* __restrict__ k_mean, int8_t* __restrict__ k_i8, float* __restrict__ k_scale) {
  __shared__ __attribute__((aligned(16))) float mean[D];
  const int blk = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const int nch = (N + kMeanChunk - 1) / kMeanChunk;
  const int nkb = (N + kKBlock - 1) / kKBlock;
  for (int c = lane; c < D; c += 64) {
    float tot = 0.f;
    for (int j = 0; j < nch; ++j) tot += part_sum[((size_t)bh * nch + j) * D + c];
    mean[c] = tot / (float)N;
    if (blk == 0) k_mean[(size_t)bh * D + c] = mean[c];
  }
  __syncthreads();
  quant_kblock_wave<DT, D, ROPE>(k, mean, N, H, nhd, nkb, rope_cos, rope_sin, k_i8, k_scale, bh,
                                 blk, lane);
}

// ---------------------------------------------------------------------------
// Launchers.
template <int DT, int D, bool ROPE>
static hipError_t colstats_dispatch(const void* k, const void* v, int B, int H, int N, float vr,
                                    const InLayout& in, float* part_sum, float* part_max,
                                    float* k_mean, float* v_scale, float* v_recip,
                                    bool finalize, hipStream_t s) {
  const int nch = ceil_div(N, kMeanChunk);
  const int cpw = 256 / (ROPE ? D / 4 : D / 2);
  dim3 grid(ceil_div(nch, cpw), B * H);
  const bool dk = k != nullptr, dv = v != nullptr;
  auto kp = static_cast<const uint16_t*>(k);
  auto vp = static_cast<const uint16_t*>(v);
#define SAGE_COLSTATS(DK, DV)                                                                 \
  colstats_kernel<DT, D, DK, DV, ROPE><<<grid, 256, 0, s>>>(kp, vp, N, H, in.nhd, nch,         \
                                                            in.rope_cos, in.rope_sin, part_sum, \
                                                            part_max);                          \
  if (finalize)                                                                               \
    finalize_kernel<D, DK, DV><<<B * H, 128, 0, s>>>(part_sum, part_max, N, nch, k_mean,       \
                                                     v_scale, v_recip, vr);
  if (dk && dv) {
    SAGE_COLSTATS(true, true)
  } else if (dk) {
    SAGE_COLSTATS(true, false)
  } else if (dv) {
    SAGE_COLSTATS(false, true)
  }
#undef SAGE_COLSTATS
  return hipGetLastError();
}

hipError_t launch_colstats(const void* k, const void* v, int dtype, int B, int H, int N, int d,
                           int pv_mode, const InLayout& in, float* part_sum, float* part_max,
                           float* k_mean, float* v_scale, float* v_recip, hipStream_t s,
                           bool finalize) {
  // RoPE rotates K only; V statistics never see it
  const bool rope = in.rope_cos != nullptr && k != nullptr;
  const float vr = pv_mode == kPvInt8 ? 127.f : 448.f;
#define SAGE_CS(DT, D)                                                                        \
  if (dtype == DT && d == D)                                                                  \
    return rope ? colstats_dispatch<DT, D, true>(k, v, B, H, N, vr, in, part_sum, part_max,     \
                                                 k_mean, v_scale, v_recip, finalize, s)          \
                : colstats_dispatch<DT, D, false>(k, v, B, H, N, vr, in, part_sum, part_max,    \
                                                  k_mean, v_scale, v_recip, finalize, s);
  SAGE_CS(0, 64) SAGE_CS(0, 128) SAGE_CS(1, 64) SAGE_CS(1, 128)
#undef SAGE_CS
  return hipErrorInvalidValue;
}

template <int DT, int D, bool ROPE>
static hipError_t quant_qk_dispatch(const void* q, const void* k, const float* k_mean, int B,
                                    int H, int N, const InLayout& in, int8_t* q_i8, int8_t* k_i8,
                                    float* q_scale, float* k_scale, hipStream_t s) {
  const int nqb = ceil_div(N, kQBlock), nkb = ceil_div(N, kKBlock);
  const float isd = (float)(1.0 / __builtin_sqrt((double)D));
  const int first = q ? 0 : nqb;
  const int count = (q ? nqb : 0) + (k ? nkb : 0);
  dim3 grid(count, B * H);
  quant_qk_kernel<DT, D, ROPE><<<grid, 256, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), k_mean, N, H, in.nhd, nqb,
      nkb, first, isd, in.rope_cos, in.rope_sin, q_i8, k_i8, q_scale, k_scale);
  return hipGetLastError();
}

hipError_t launch_quant_qk(const void* q, const void* k, const float* k_mean, int dtype, int B,
                           int H, int N, int d, const InLayout& in, int8_t* q_i8, int8_t* k_i8,
                           float* q_scale, float* k_scale, hipStream_t s) {
  if (!q && !k) return hipSuccess;
  const bool rope = in.rope_cos != nullptr;
#define SAGE_QQ(DT, D)                                                                      \
  if (dtype == DT && d == D)                                                                \
    return rope ? quant_qk_dispatch<DT, D, true>(q, k, k_mean, B, H, N, in, q_i8, k_i8,      \
                                                 q_scale, k_scale, s)                        \
                : quant_qk_dispatch<DT, D, false>(q, k, k_mean, B, H, N, in, q_i8, k_i8,     \
                                                  q_scale, k_scale, s);
  SAGE_QQ(0, 64) SAGE_QQ(0, 128) SAGE_QQ(1, 64) SAGE_QQ(1, 128)
#undef SAGE_QQ
  return hipErrorInvalidValue;
}

template <int DT, int D, int PV>
static hipError_t prep_v_dispatch(const void* v, const float* v_recip, int B, int H, int N,
                                  int nhd, uint8_t* v_out, hipStream_t s) {
  const int nt = ceil_div(N, kKvTile);
  dim3 grid(nt, B * H);
  prep_v_kernel<DT, D, PV><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(v), v_recip, N, H,
                                                nhd, nt, v_out);
  return hipGetLastError();
}

hipError_t launch_prep_v(const void* v, const float* v_recip, int dtype, int B, int H, int N,
                         int d, int pv_mode, int nhd, uint8_t* v_out, hipStream_t s) {
#define SAGE_PV_CASE(DT, D, PV)                                              \
  if (dtype == DT && d == D && pv_mode == PV)                                \
    return prep_v_dispatch<DT, D, PV>(v, v_recip, B, H, N, nhd, v_out, s);
  SAGE_PV_CASE(0, 64, 0) SAGE_PV_CASE(0, 64, 1) SAGE_PV_CASE(0, 64, 2)
  SAGE_PV_CASE(0, 128, 0) SAGE_PV_CASE(0, 128, 1) SAGE_PV_CASE(0, 128, 2)
  SAGE_PV_CASE(1, 64, 0) SAGE_PV_CASE(1, 64, 1) SAGE_PV_CASE(1, 64, 2)
  SAGE_PV_CASE(1, 128, 0) SAGE_PV_CASE(1, 128, 1) SAGE_PV_CASE(1, 128, 2)
#undef SAGE_PV_CASE
  return hipErrorInvalidValue;
}

// Q^ and K^ blocks and V tiles in one launch (after the column statistics):
// workgroups [0, nqk) take quant_block's blocks first_blk + x (Q^ blocks,
// then K^ blocks), the rest one V tile each, as quant_qk_kernel and
// prep_v_kernel do in two launches.  FOLD (heads of at most kFoldMaxChunks
// 256-token chunks): no finalize_kernel launch before this one; each K^
// workgroup forms its head's mean from the chunk partials, and each V
// workgroup (FP8, INT8) its head's 1/delta_V, with finalize_channel's
// expressions, into LDS; the head's first K^ block and first V tile also
// store them, as finalize_kernel would.
constexpr int kFoldMaxChunks = 16;
template <int DT, int D, int PV, bool ROPE, bool FOLD>
__global__ __launch_bounds__(256) void quant_qkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ k_mean, float* __restrict__ v_recip,
    int N, int H, int nhd, int nqb, int nkb, int first_blk, int nqk, int ntiles,
    float inv_sqrt_d, const float* __restrict__ rope_cos, const float* __restrict__ rope_sin,
    int8_t* __restrict__ q_i8, int8_t* __restrict__ k_i8, float* __restrict__ q_scale,
    float* __restrict__ k_scale, uint8_t* __restrict__ v_out, const float* __restrict__ part_sum,
    const float* __restrict__ part_max, int nch, float* __restrict__ v_scale) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint16_t tile[PrepVTile<D>::HALVES];
  __shared__ __attribute__((aligned(16))) float stat[FOLD ? D : 4];
  const int bh = blockIdx.y, bx = blockIdx.x;
  if constexpr (FOLD) {
    const bool kblk = bx < nqk && bx + first_blk >= nqb;
    if (kblk) {
      for (int c = threadIdx.x; c < D; c += 256) {
        // the (at most 16) partials loaded at once, then added in chunk order
        float pv[kFoldMaxChunks];
#pragma unroll
        for (int j = 0; j < kFoldMaxChunks; ++j)
          pv[j] = part_sum[((size_t)bh * nch + min(j, nch - 1)) * D + c];
        float tot = 0.f;
#pragma unroll
        for (int j = 0; j < kFoldMaxChunks; ++j)
          if (j < nch) tot += pv[j];
        stat[c] = tot / (float)N;
        if (bx + first_blk == nqb) k_mean[(size_t)bh * D + c] = stat[c];
      }
    } else if (PV != kPvFp16 && bx >= nqk) {
      constexpr float VR = PV == kPvInt8 ? 127.f : 448.f;
      for (int c = threadIdx.x; c < D; c += 256) {
        float cm = 0.f;   // (the last partial re-read past nch: the same maximum)
#pragma unroll
        for (int j = 0; j < kFoldMaxChunks; ++j)
          cm = fmaxf(cm, part_max[((size_t)bh * nch + min(j, nch - 1)) * D + c]);
        stat[c] = cm > 0.f ? VR / cm : 0.f;
        if (bx == nqk) {
          v_scale[(size_t)bh * D + c] = cm / VR;
          v_recip[(size_t)bh * D + c] = stat[c];
        }
      }
    }
    __syncthreads();
  }
  if (bx < nqk) {
    quant_block<DT, D, ROPE>(q, k, FOLD ? stat : k_mean + (size_t)bh * D, N, H, nhd, nqb, nkb,
                             inv_sqrt_d, rope_cos, rope_sin, q_i8, k_i8, q_scale, k_scale, bh,
                             bx + first_blk, red);
  } else {
    const float* rc = PV == kPvFp16 ? nullptr : FOLD ? stat : v_recip + (size_t)bh * D;
    prep_v_tile<DT, D, PV>(v, rc, N, H, nhd, ntiles, v_out, bh, bx - nqk, tile);
  }
}

template <int DT, int D, int PV, bool ROPE>
static hipError_t quant_qkv_dispatch(const void* q, const void* k, const void* v,
                                     float* k_mean, float* v_recip, int B, int H, int N,
                                     const InLayout& in, int8_t* q_i8, int8_t* k_i8,
                                     float* q_scale, float* k_scale, uint8_t* v_out,
                                     const float* part_sum, const float* part_max,
                                     float* v_scale, bool fold, hipStream_t s) {
  const int nqb = ceil_div(N, kQBlock), nkb = ceil_div(N, kKBlock);
  const int nt = ceil_div(N, kKvTile), nch = ceil_div(N, kMeanChunk);
  const float isd = (float)(1.0 / __builtin_sqrt((double)D));
  const int first = q ? 0 : nqb;
  const int nqk = (q ? nqb : 0) + nkb;
  dim3 grid(nqk + nt, B * H);
  auto qp = static_cast<const uint16_t*>(q);
  auto kp = static_cast<const uint16_t*>(k);
  auto vp = static_cast<const uint16_t*>(v);
  if (fold)
    quant_qkv_kernel<DT, D, PV, ROPE, true><<<grid, 256, 0, s>>>(
        qp, kp, vp, k_mean, v_recip, N, H, in.nhd, nqb, nkb, first, nqk, nt, isd, in.rope_cos,
        in.rope_sin, q_i8, k_i8, q_scale, k_scale, v_out, part_sum, part_max, nch, v_scale);
  else
    quant_qkv_kernel<DT, D, PV, ROPE, false><<<grid, 256, 0, s>>>(
        qp, kp, vp, k_mean, v_recip, N, H, in.nhd, nqb, nkb, first, nqk, nt, isd, in.rope_cos,
        in.rope_sin, q_i8, k_i8, q_scale, k_scale, v_out, part_sum, part_max, nch, v_scale);
  return hipGetLastError();
}

bool quant_qkv_folds(int N) { return ceil_div(N, kMeanChunk) <= kFoldMaxChunks; }

hipError_t launch_quant_qkv(const void* q, const void* k, const void* v, float* k_mean,
                            float* v_recip, int dtype, int B, int H, int N, int d, int pv_mode,
                            const InLayout& in, int8_t* q_i8, int8_t* k_i8, float* q_scale,
                            float* k_scale, uint8_t* v_out, const float* part_sum,
                            const float* part_max, float* v_scale, hipStream_t s) {
  if (!k || !v) return hipErrorInvalidValue;
  const bool rope = in.rope_cos != nullptr;
  const bool fold = quant_qkv_folds(N);
#define SAGE_QKV(DT, D, PV)                                                                   \
  if (dtype == DT && d == D && pv_mode == PV)                                                 \
    return rope ? quant_qkv_dispatch<DT, D, PV, true>(q, k, v, k_mean, v_recip, B, H, N, in,   \
                                                      q_i8, k_i8, q_scale, k_scale, v_out,    \
                                                      part_sum, part_max, v_scale, fold, s)   \
                : quant_qkv_dispatch<DT, D, PV, false>(q, k, v, k_mean, v_recip, B, H, N, in,  \
                                                       q_i8, k_i8, q_scale, k_scale, v_out,   \
                                                       part_sum, part_max, v_scale, fold, s);
  SAGE_QKV(0, 64, 0) SAGE_QKV(0, 64, 1) SAGE_QKV(0, 64, 2)
  SAGE_QKV(0, 128, 0) SAGE_QKV(0, 128, 1) SAGE_QKV(0, 128, 2)
  SAGE_QKV(1, 64, 0) SAGE_QKV(1, 64, 1) SAGE_QKV(1, 64, 2)
  SAGE_QKV(1, 128, 0) SAGE_QKV(1, 128, 1) SAGE_QKV(1, 128, 2)
#undef SAGE_QKV
  return hipErrorInvalidValue;
}

template <int DT, int D, int PV>
static hipError_t prepass_head_dispatch(const void* q, const void* k, const void* v, int B,
                                        int H, int N, const InLayout& in, const PrepassOut& o,
                                        hipStream_t s) {
  const float isd = (float)(1.0 / __builtin_sqrt((double)D));
  const bool qk = q != nullptr, dv = v != nullptr, rope = in.rope_cos != nullptr;
  const int BH = B * H;
  const int roles = (qk ? ceil_div(N, kMeanChunk) + ceil_div(N, kQBlock) : 0) +
                    (dv ? ceil_div(N, kKvTile) : 0);
  const long long grid = (long long)BH * roles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  auto qp = static_cast<const uint16_t*>(q);
  auto kp = static_cast<const uint16_t*>(k);
  auto vp = static_cast<const uint16_t*>(v);
#define SAGE_HEAD(ROPE, QK, DV)                                                                \
  prepass_roles_kernel<DT, D, PV, ROPE, QK, DV><<<dim3((unsigned)grid), 256, 0, s>>>(          \
      qp, kp, vp, N, H, BH, in.nhd, in.rope_cos, in.rope_sin, isd, o.part_sum, o.k_mean,       \
      o.v_scale, o.q_i8, o.k_i8, o.q_scale, o.k_scale, o.v_out);
  if (qk && dv) {
    if (rope) { SAGE_HEAD(true, true, true) } else { SAGE_HEAD(false, true, true) }
  } else if (qk) {
    if (rope) { SAGE_HEAD(true, true, false) } else { SAGE_HEAD(false, true, false) }
  } else if (dv) {
    SAGE_HEAD(false, false, true)
  }
#undef SAGE_HEAD
  if (qk && N > kMeanChunk) {   // heads of one chunk finished their K^ above
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 g2(ceil_div(N, kKBlock), BH);
    if (rope)
      prepass_kblocks_kernel<DT, D, true><<<g2, 64, 0, s>>>(kp, N, H, in.nhd, in.rope_cos,
                                                           in.rope_sin, o.part_sum, o.k_mean,
                                                           o.k_i8, o.k_scale);
    else
      prepass_kblocks_kernel<DT, D, false><<<g2, 64, 0, s>>>(kp, N, H, in.nhd, nullptr, nullptr,
                                                            o.part_sum, o.k_mean, o.k_i8,
                                                            o.k_scale);
  }
  return hipGetLastError();
}

hipError_t launch_prepass_head(const void* q, const void* k, const void* v, int dtype, int B,
                               int H, int N, int d, int pv_mode, const InLayout& in,
                               const PrepassOut& o, hipStream_t s) {
#define SAGE_PH(DT, D, PV)                                                     \
  if (dtype == DT && d == D && pv_mode == PV)                                  \
    return prepass_head_dispatch<DT, D, PV>(q, k, v, B, H, N, in, o, s);
  SAGE_PH(0, 64, 0) SAGE_PH(0, 64, 1) SAGE_PH(0, 64, 2)
  SAGE_PH(0, 128, 0) SAGE_PH(0, 128, 1) SAGE_PH(0, 128, 2)
  SAGE_PH(1, 64, 0) SAGE_PH(1, 64, 1) SAGE_PH(1, 64, 2)
  SAGE_PH(1, 128, 0) SAGE_PH(1, 128, 1) SAGE_PH(1, 128, 2)
#undef SAGE_PH
  return hipErrorInvalidValue;
}

}  // namespace sage
