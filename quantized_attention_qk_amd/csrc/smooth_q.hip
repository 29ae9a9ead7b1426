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

  {
    // all of this thread's loads in flight at once, then the LDS stores
    // (token rows tok0 + t at a fixed stride in either layout)
    const uint16_t* q0 = q + row_off<D>(bh, tok0, H, N, nhd);
    const size_t rstride = nhd ? (size_t)H * D : (size_t)D;
    uint4 w[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = tid + i * 256;
      w[i] = uint4{0u, 0u, 0u, 0u};
      if (c < nchunk)
        w[i] = *reinterpret_cast<const uint4*>(q0 + (c / CPR) * rstride + (c % CPR) * 8);
    }
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
      *reinterpret_cast<uint4*>(&tile[(tid + i * 256) * 8]) = w[i];
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

  // every chunk of this thread covers channels ch0..ch0+7 (256 chunks of 8
  // channels span a whole number of rows); the values are re-derived from the
  // staged rows where they are needed instead of being kept in registers
  const int ch0 = (tid * 8) % D;
  float qb8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qb8[e] = qbar[ch0 + e];
  auto chunk = [&](int c, float (&f)[8]) __attribute__((always_inline)) {
    const uint4 raw = *reinterpret_cast<const uint4*>(&tile[c * 8]);
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      f[e] = in_to_f32<DT>((uint16_t)(wd[e >> 1] >> (16 * (e & 1)))) * inv_sqrt_d;
  };
  // the block's largest |value| with (s) and without (p) the mean taken
  // out; the second only where the block is left unsmoothed.  The smoothed
  // values stay in registers for the quantisation below.
  float xs[MAXC][8];
  auto block_amax = [&](bool smoothed, float* red) __attribute__((always_inline)) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = tid + i * 256;
      float f[8];
      chunk(c < nchunk ? c : 0, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = c < nchunk ? (smoothed ? f[e] - qb8[e] : f[e]) : 0.f;
        if (smoothed) xs[i][e] = x;
        m = fmaxf(m, fabsf(x));
      }
    }
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  };
  const float a_s = block_amax(true, red_s);
  const float r_s = a_s > 0.f ? 127.f / a_s : 0.f;
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
  const bool ok = a_s > 0.f && 127.0 * sum_w <= kSqLimit;   // uniform in the block
  float a_p = a_s, r_p = r_s;
  if (!ok) {
    a_p = block_amax(false, red_p);
    r_p = a_p > 0.f ? 127.f / a_p : 0.f;
  }

  const float r = ok ? r_s : r_p;
  int8_t* dst = q_i8 + ((size_t)bh * N + tok0) * D;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + i * 256;
    if (c < nchunk) {
      float f[8];
      if (ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = xs[i][e];
      } else {
        chunk(c, f);
      }
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t = __builtin_rintf(f[e] * r);
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
// is split into three signed base-256 digits, the low two in [-128, 127]
// (|w| <= 2^29/127 < 2^22 leaves the top one in [-64, 64]), each digit plane
// multiplied with K^ (v_mfma_i32_32x32x32_i8, A = 32 keys of K^, B = 32
// blocks' digits; a plane's sums stay below 2^21), and the planes combined
// with weights 1, 2^8, 2^16 in wrapping 32-bit arithmetic, which is exact
// because |w . K^| <= 2^29.
//
// Workgroup = one (b, h), a group of 32 Q blocks and a chunk of kSqChunk
// keys.  Its threads first split the group's w into the digit operands once,
// into LDS (thread (kt, lane) the 16 channels that lane holds in d-step kt);
// each of the four wavefronts then walks a quarter of the chunk in 64-key
// steps, two 32-key MFMA tiles per step.  A step's 32 x 64 values go through
// a per-wavefront LDS tile so that each global store writes four rows of 256
// contiguous bytes (the MFMA layout would give 32 rows of 32 bytes).  All of
// a wavefront's K^ loads are issued before its first store: the vector
// memory counter retires in order, so a load issued after a store could not
// be waited for without waiting for the store too.
constexpr int kSqChunk = 512;
constexpr int kSqGroup = 32;
constexpr int kSqStageLd = 64 + 4;   // staging row: 64 keys + padding (words)
// Blocks [qb0, qb0 + nqr) of the nqb of each head; comp holds nqr rows of ld
// values per head.
template <int D, bool VEC>
__global__ __launch_bounds__(256) void sq_comp_kernel(const int8_t* k_i8, const int32_t* q_w, int N,
                                                      int nqb, int qb0, int nqr, int ld, int bias,
                                                      int nchunk, int ngroup, int nunit,
                                                      int32_t* __restrict__ comp) {
  constexpr int KT = D / 32;
  constexpr int NP = 3;   // digit planes
  __shared__ v4i dig_s[NP][KT][64];
  __shared__ __attribute__((aligned(16))) int32_t stage_s[4][kSqGroup][kSqStageLd];
  // workgroup -> (group, key chunk, b*h): the groups of one (chunk, b*h)
  // unit get workgroup ids 8 apart, which the dispatcher hands to the same
  // XCD one after another, so after the first group the unit's K^ tiles
  // come from that XCD's L2
  const int id = blockIdx.x, k = id / 8;
  const int unit = (k / ngroup) * 8 + id % 8;
  if (unit >= nunit) return;   // (the whole workgroup, before any barrier)
  const int bh = unit / nchunk;
  const int g0 = (k % ngroup) * kSqGroup;   // first of the group's block rows
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int n = lane & 31, hh = lane >> 5;

  // w of this thread's digit slot (d-step kt = wave, the 16 channels lane n,
  // hh holds, block row g0 + n), loaded first; rows past the blocks are
  // clamped loads and get digits 0.  These loads, then the first K^ tiles'
  // are issued here in that order (the inputs are not restrict-qualified, so
  // the barrier keeps the K^ loads above it): the wait for w then leaves
  // the K^ tiles in flight during the digit build.
  const int kt_w = min(wave, KT - 1), qr_w = g0 + n;
  const int32_t* wrow =
      q_w + ((size_t)bh * nqb + qb0 + min(qr_w, nqr - 1)) * D + 32 * kt_w + 16 * hh;
  v4i xs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) xs[j] = *reinterpret_cast<const v4i*>(wrow + 4 * j);
  __builtin_amdgcn_sched_barrier(0);

  // A operand (this lane's key row of K^) of the 32-key tile at t: a row
  // clamped into the head, so the loads need no branch; rows past N are
  // cleared afterwards (only in a head's last tile)
  auto load_a = [&](int t, v4i (&a)[KT]) __attribute__((always_inline)) {
    const int key = min(t + n, N - 1);
    const int8_t* krow = k_i8 + ((size_t)bh * N + key) * D + 16 * hh;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) a[kt] = *reinterpret_cast<const v4i*>(krow + 32 * kt);
  };
  constexpr int NTW = kSqChunk / 4 / 32;   // 32-key tiles per wavefront
  const int c0 = (unit % nchunk) * kSqChunk + wave * (kSqChunk / 4);
  const int c1 = min(c0 + kSqChunk / 4, ld);
  // the wavefront's K^ tiles, all in flight while the digits are built
  // (tiles past the range are loaded too, from clamped rows: unconditional
  // loads let the waits count them exactly)
  v4i abuf[NTW][KT];
#pragma unroll
  for (int i = 0; i < NTW; ++i) load_a(c0 + 32 * i, abuf[i]);
  __builtin_amdgcn_sched_barrier(0);

  // (every thread holds a slot at d = 128; at d = 64 the first two
  // wavefronts do)
  if (KT * 64 >= 256 || tid < KT * 64) {
    uint32_t dd[NP][4] = {};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4i x = qr_w < nqr ? xs[j] : v4i{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int v = x[u];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int dp = p < NP - 1 ? ((v + 128) & 255) - 128 : v;
          v = (v - dp) >> 8;
          dd[p][j] |= ((uint32_t)(uint8_t)(int8_t)dp) << (8 * u);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p)
      dig_s[p][kt_w][lane] = v4i{(int)dd[p][0], (int)dd[p][1], (int)dd[p][2], (int)dd[p][3]};
  }
  __syncthreads();
  v4i dig[NP][KT];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) dig[p][kt] = dig_s[p][kt][lane];

  int32_t(*st)[kSqStageLd] = stage_s[wave];
  // the group's rows of comp as one buffer (32 ld 4 < 2^31 bytes): a store
  // past its valid rows, or at an offset of kOob, is dropped by the
  // hardware, so every flush issues the same stores with no branch (which
  // keeps the load waits above exact)
  constexpr uint32_t kOob = 0x80000000u;
  const int nrow = min(nqr - g0, kSqGroup);
  const uint64_t cb = reinterpret_cast<uint64_t>(comp + ((size_t)bh * nqr + g0) * ld);
  const uint32_t cb_lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)cb);
  const uint32_t cb_hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(cb >> 32));
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<int32_t*>(((uint64_t)cb_hi << 32) | cb_lo), 0,
      __builtin_amdgcn_readfirstlane((int)((uint32_t)nrow * (uint32_t)ld * 4u)), 0x00020000);
  if (c0 >= c1) return;
  // one 64-key step from the staging tile back in row order: lanes 16 k ..
  // 16 k + 15 hold 64 consecutive keys of one block row (keys of a half not
  // computed lie at or past ld and are not stored)
  auto flush = [&](int32_t(*stg)[kSqStageLd], __amdgpu_buffer_rsrc_t rs, int t0)
      __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kSqGroup / 4; ++k) {
      const int row = 4 * k + (lane >> 4);
      const int tk = t0 + 4 * (lane & 15);
      const v4i x = *reinterpret_cast<const v4i*>(&stg[row][4 * (lane & 15)]);
      const uint32_t base = ((uint32_t)row * (uint32_t)ld + (uint32_t)tk) * 4u;
      if constexpr (VEC) {
        __builtin_amdgcn_raw_buffer_store_b128(x, rs, (int)(tk < ld ? base : kOob), 0, 0);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          __builtin_amdgcn_raw_buffer_store_b32(x[u], rs, (int)(tk + u < ld ? base + 4u * u : kOob),
                                                0, 0);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int t = c0 + 32 * i;
    if (t >= c1) break;
    v4i(&a)[KT] = abuf[i];
    if (t + 32 > N) {
      const bool live = t + n < N;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) a[kt] = live ? a[kt] : v4i{0, 0, 0, 0};
    }
    v16i acc[NP] = {};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int p = 0; p < NP; ++p)
        acc[p] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[kt], dig[p][kt], acc[p], 0, 0, 0);
    // register r holds key t + 8 (r/4) + 4 hh + r%4, block row n
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int cv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // copy the elements to scalars first (clang mis-lowers some
        // ext_vector element uses)
        const int r = 4 * j + u;
        const uint32_t p0 = (uint32_t)acc[0][r], p1 = (uint32_t)acc[1][r];
        const uint32_t p2 = (uint32_t)acc[2][r];
        const int P = (int)(p0 + (p1 << 8) + (p2 << 16));
        // P / 2^8 rounded to nearest, ties to even (no overflow: |P| <= 2^29)
        constexpr int kHalf = 1 << (kSqFracBits - 1);
        cv[u] = ((P + (kHalf - 1) + ((P >> kSqFracBits) & 1)) >> kSqFracBits) + bias;
      }
      *reinterpret_cast<v4i*>(&st[n][32 * (i & 1) + 8 * j + 4 * hh]) =
          v4i{cv[0], cv[1], cv[2], cv[3]};
    }
    if (i & 1) flush(st, crs, c0 + 64 * (i / 2));
  }
  // an odd tile count (only at the end of a ragged ld) leaves half a step
  if (((c1 - c0 + 31) / 32) & 1) flush(st, crs, c0 + 64 * ((c1 - c0 - 1) / 64));
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
  const int nchunk = ceil_div(ld, kSqChunk), ngroup = ceil_div(nqr, kSqGroup);
  const long long nunit = (long long)nchunk * B * H;
  const long long nwg = (nunit + 7) / 8 * 8 * ngroup;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg);
  // rows of ld values 16-byte aligned: 16-byte stores
  const bool vec = (ld & 3) == 0;
#define SAGE_SQC(D_, V_)                                                                  \
  if (d == D_ && vec == V_) {                                                             \
    sq_comp_kernel<D_, V_><<<grid, 256, 0, s>>>(k_i8, q_w, N, nqb, qb0, nqr, ld, bias,    \
                                                nchunk, ngroup, (int)nunit, comp);        \
    return hipGetLastError();                                                             \
  }
  SAGE_SQC(64, true) SAGE_SQC(64, false) SAGE_SQC(128, true) SAGE_SQC(128, false)
#undef SAGE_SQC
  return hipErrorInvalidValue;
}

}  // namespace sage
