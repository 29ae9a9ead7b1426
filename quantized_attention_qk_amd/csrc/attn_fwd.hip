// attn_fwd.hip -- the tiled SageAttention kernel for gfx950.
//
// "SageAttention: Accurate 8-Bit Attention for Plug-and-Play Inference
// Acceleration" (paper detail page), §3 Algorithm 1 (SAGEAttn-B) and §4
// Eq. 4-5: for each query block, walk the KV tiles in ascending order,
// S = INT8 Q^ K^T (INT32) * delta_Q * delta_K, online softmax (running max m,
// running sum l, output rescaled by exp(m_old - m_new)), then P~V in FP16 --
// or in FP8 E4M3 with a static delta_P = 1/448 and a per-channel delta_V, as in
// the "8+8" variant of the "SageAttention2++ ..." review page (section 三) --
// accumulated in FP32 (gfx950 has no FP16-accumulator MFMA), and finally
// O = O / l.
//
// MI355X mapping
// * Workgroup = 4 wavefronts = 128 query rows = one delta_Q block of one (b, h).
//   Each wavefront owns 32 query rows for the whole KV walk.
// * Scores are computed transposed, S^T = K^ Q^T, with v_mfma_i32_32x32x32_i8:
//   in the 32x32 accumulator lane l holds query l%32 and keys
//   8*(r/4) + 4*(l/32) + r%4 (r = register 0..15).  That is exactly the B
//   operand layout of O^T = V^T P~^T (v_mfma_f32_32x32x16_f16, or
//   v_mfma_scale_f32_32x32x64_f8f6f4 for FP8), so P~ goes from the softmax to
//   the second MFMA without leaving registers; V is stored pre-permuted (see
//   sage_quant_v) so that its A operand is one 16-byte LDS read per lane.
// * Row reductions (max over keys) are in-lane over 32 values plus one
//   v_permlane32_swap between lanes l and l^32.  The max runs on the INT32
//   scores (exact, and monotone under the positive scale).
// * The dequantisation scale and log2(e) are folded into one scalar per KV
//   tile: P~ = exp2(s * c_j - m) with c_j = delta_Q delta_K[j] log2(e).  For
//   FP8, log2(448) is folded into the same subtraction so the MFMA operand is
//   448 P~ directly, and l is kept in the same units.
// * K^ and prepared-V tiles are staged through LDS (double buffered, XOR
//   swizzled rows); global loads for tile j+1 are in flight during tile j.
// * The output rescale by alpha is skipped when no row of the wavefront has a
//   new maximum (alpha == 1 exactly), which is bit-identical.
#include "sage_common.h"
#include "sage_launch.h"

namespace sage {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448)

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

// One 32-key x 32-query block of S^T (INT32) from the K^ tile in LDS.
template <int D>
__device__ __forceinline__ v16i qk_block(const v4i (&qf)[D / 32], const uint8_t* kb, int blk,
                                         int n, int hh) {
  v16i acc = {};
  const int row = 32 * blk + n;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const v4i a = *reinterpret_cast<const v4i*>(kb + KTile<D>::lds_off(row, 2 * t + hh));
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[t], acc, 0, 0, 0);
  }
  return acc;
}

// Global -> register staging of one K^ tile, then register -> LDS with the
// row swizzle.  Keys >= N are staged as zeros.
template <int D, int NT>
struct KStage {
  static constexpr int PER = KTile<D>::CHUNKS / NT;
  static_assert(PER * NT == KTile<D>::CHUNKS, "threads must tile the K^ tile");
  uint4 r[PER];
  __device__ __forceinline__ void load(const int8_t* __restrict__ k_bh, int key0, int N, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = tid + i * NT;
      const int key = g / KTile<D>::CPR;
      const int kc = g % KTile<D>::CPR;
      r[i] = (key0 + key < N)
                 ? *reinterpret_cast<const uint4*>(k_bh + (size_t)(key0 + key) * D + kc * 16)
                 : uint4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint8_t* kb, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = tid + i * NT;
      const int key = g / KTile<D>::CPR;
      const int kc = g % KTile<D>::CPR;
      *reinterpret_cast<uint4*>(kb + KTile<D>::lds_off(key, kc)) = r[i];
    }
  }
};

// Prepared-V tiles are stored pre-swizzled, so staging is a linear copy.
template <int D, int PV, int NT>
struct VStage {
  static constexpr int PER = VTile<D, PV>::CHUNKS / NT;
  static_assert(PER * NT == VTile<D, PV>::CHUNKS, "threads must tile the V tile");
  uint4 r[PER];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ vtile, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      r[i] = *reinterpret_cast<const uint4*>(vtile + (size_t)(tid + i * NT) * 16);
  }
  __device__ __forceinline__ void store(uint8_t* vb, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) *reinterpret_cast<uint4*>(vb + (tid + i * NT) * 16) = r[i];
  }
};

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

template <int D, int PV, int OUT, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const int8_t* __restrict__ q_i8, const int8_t* __restrict__ k_i8,
                     const uint8_t* __restrict__ v_t, const float* __restrict__ q_scale,
                     const float* __restrict__ k_scale, const float* __restrict__ v_scale,
                     int BH, int N, int nqb, int ntiles, int xcd_remap, void* __restrict__ out) {
  constexpr int KB = KTile<D>::BYTES;
  constexpr int VB = VTile<D, PV>::BYTES;
  constexpr int NCB = D / 32;   // 32-channel blocks of the output
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][KB + VB];

  // Workgroup -> (b*h, query block).
  int wg = blockIdx.x;
  if (xcd_remap) {
    // Consecutive workgroups are dispatched round-robin over the 8 XCDs; give
    // each XCD a contiguous range of (head, block) ids so that the K/V tiles
    // of a head are shared in that XCD's L2.
    const int g8 = gridDim.x & ~7;
    if (wg < g8) wg = (wg & 7) * (g8 >> 3) + (wg >> 3);
  }
  int bh, qb;
  if constexpr (CAUSAL) {   // heaviest query blocks first
    qb = nqb - 1 - wg / BH;
    bh = wg % BH;
  } else {
    bh = wg / nqb;
    qb = wg % nqb;
  }

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int qw0 = qb * kBlockQ + wave * kWaveQ;   // first query row of this wavefront
  const int qrow = qw0 + n;                        // this lane's query row

  const int8_t* q_bh = q_i8 + (size_t)bh * N * D;
  const int8_t* k_bh = k_i8 + (size_t)bh * N * D;
  const uint8_t* v_bh = v_t + (size_t)bh * ntiles * VB;
  const int nkb = ntiles;   // delta_K blocks == KV tiles
  const float* ks_bh = k_scale + (size_t)bh * nkb;

  v4i qf[D / 32];
  load_q_frag<D>(qf, q_bh, qrow, N, hh);
  const float cq = q_scale[(size_t)bh * nqb + qb] * kLog2e;

  const int kv_end = CAUSAL ? min(N, (qb + 1) * kBlockQ) : N;
  const int nt = (kv_end + kKvTile - 1) / kKvTile;

  KStage<D, 256> kst;
  VStage<D, PV, 256> vst;
  kst.load(k_bh, 0, N, tid);
  vst.load(v_bh, tid);
  kst.store(smem[0], tid);
  vst.store(smem[0] + KB, tid);
  __syncthreads();

  float m_run = -__builtin_inff();
  float l_run = 0.f;
  v16f o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = v16f{};

  for (int j = 0; j < nt; ++j) {
    const int key0 = j * kKvTile;
    const bool has_next = j + 1 < nt;
    if (has_next) {
      kst.load(k_bh, key0 + kKvTile, N, tid);
      vst.load(v_bh + (size_t)(j + 1) * VB, tid);
    }
    const uint8_t* kb = smem[j & 1];
    const uint8_t* vb = kb + KB;
    const bool active = !CAUSAL || key0 <= qw0 + (kWaveQ - 1);
    if (active) {
      const float cj = cq * ks_bh[j];
      v16i s[2];
      s[0] = qk_block<D>(qf, kb, 0, n, hh);
      s[1] = qk_block<D>(qf, kb, 1, n, hh);

      // Mask keys past N and, when causal, keys after the query.
      const bool need_mask = (CAUSAL && key0 + kKvTile - 1 > qw0) || (key0 + kKvTile > N);
      uint32_t keep = 0xffffffffu;   // bit 16*blk + r
      if (need_mask) {
        keep = 0u;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * blk + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = key < N && (!CAUSAL || key <= qrow);
            keep |= (uint32_t)ok << (16 * blk + r);
            if (!ok) s[blk][r] = INT32_MIN;
          }
      }
      int mx = INT32_MIN;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = max(mx, max(s[blk][r], s[blk][r + 1]));
      mx = pair_max_i32(mx);
      const float m_new = fmaxf(m_run, (float)mx * cj);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      const float negm = PV == kPvFp8 ? kLog2_448 - m_new : -m_new;

      float p[2][16];
      float lsum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[blk][r], cj, negm));
          if (need_mask && !((keep >> (16 * blk + r)) & 1u)) e = 0.f;
          p[blk][r] = e;
          lsum += e;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;

      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
      }

      if constexpr (PV == kPvFp16) {
        // B operand of step S (16 keys): registers 8*(S%2) .. +7 of block S/2.
#pragma unroll
        for (int S = 0; S < 4; ++S) {
          const int blk = S >> 1, r0 = 8 * (S & 1);
          const v4i pw = {(int)pack_f16x2(p[blk][r0 + 0], p[blk][r0 + 1]),
                          (int)pack_f16x2(p[blk][r0 + 2], p[blk][r0 + 3]),
                          (int)pack_f16x2(p[blk][r0 + 4], p[blk][r0 + 5]),
                          (int)pack_f16x2(p[blk][r0 + 6], p[blk][r0 + 7])};
          const v8h pb = __builtin_bit_cast(v8h, pw);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const int row = 32 * cb + n;
            const v4i a = *reinterpret_cast<const v4i*>(
                vb + row * 128 + (((2 * S + hh) ^ row_swizzle<128>(row)) << 4));
            o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), pb, o[cb],
                                                           0, 0, 0);
          }
        }
      } else {
        // B operand: 32 E4M3 codes, byte 16*blk + r <-> register r of block blk.
        v8i pb;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int blk = w >> 2, r0 = 4 * (w & 3);
          pb[w] = (int)pack_fp8x4(p[blk][r0], p[blk][r0 + 1], p[blk][r0 + 2], p[blk][r0 + 3]);
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int row = 32 * cb + n;
          const int sw = row_swizzle<64>(row);
          const v4i a0 = *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh) ^ sw) << 4));
          const v4i a1 =
              *reinterpret_cast<const v4i*>(vb + row * 64 + (((2 * hh + 1) ^ sw) << 4));
          const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          // scale operands 127 = E8M0 exponent of 1.0 (no block scaling)
          o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, o[cb], 0, 0, 0, 127, 0,
                                                                  127);
        }
      }
    }
    if (has_next) {
      uint8_t* nb = smem[(j + 1) & 1];
      kst.store(nb, tid);
      vst.store(nb + KB, tid);
    }
    __syncthreads();
  }

  // Epilogue: O = O / l (FP8: l is in units of 448 P~, and delta_V per channel).
  const float l_tot = pair_sum_f32(l_run);
  const float inv = 1.0f / l_tot;
  if (qrow < N) {
    const size_t orow = ((size_t)bh * N + qrow) * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int c0 = 32 * cb + 8 * j4 + 4 * hh;
        float y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          y[u] = o[cb][4 * j4 + u] * inv;
          if constexpr (PV == kPvFp8) y[u] *= v_scale[(size_t)bh * D + c0 + u];
        }
        store4<OUT>(out, orow + c0, y[0], y[1], y[2], y[3]);
      }
  }
}

// ---------------------------------------------------------------------------
// Debug kernel: one wavefront per 32-query x 64-key block, using the same
// Q^ fragment load, K^ staging/LDS layout and INT8 MFMA block as above.
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
  KStage<D, 64> kst;
  kst.load(k_bh, kbase, N, lane);
  kst.store(kb, lane);
  __syncthreads();
  const int query = qbase + n;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const v16i s = qk_block<D>(qf, kb, blk, n, hh);
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

// ---------------------------------------------------------------------------
template <int D, int PV, int OUT, bool CAUSAL>
static hipError_t attn_dispatch(const int8_t* q_i8, const int8_t* k_i8, const uint8_t* v_t,
                                const float* q_scale, const float* k_scale,
                                const float* v_scale, int B, int H, int N, void* out,
                                hipStream_t s) {
  const int nqb = ceil_div(N, kBlockQ);
  const int ntiles = ceil_div(N, kKvTile);
  const int BH = B * H;
  const long long grid = (long long)BH * nqb;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  attn_fwd_kernel<D, PV, OUT, CAUSAL><<<dim3((unsigned)grid), 256, 0, s>>>(
      q_i8, k_i8, v_t, q_scale, k_scale, v_scale, BH, N, nqb, ntiles, CAUSAL ? 0 : 1, out);
  return hipGetLastError();
}

template <int D, int PV, int OUT>
static hipError_t attn_dispatch_c(int causal, const int8_t* q_i8, const int8_t* k_i8,
                                  const uint8_t* v_t, const float* q_scale, const float* k_scale,
                                  const float* v_scale, int B, int H, int N, void* out,
                                  hipStream_t s) {
  return causal ? attn_dispatch<D, PV, OUT, true>(q_i8, k_i8, v_t, q_scale, k_scale, v_scale, B,
                                                  H, N, out, s)
                : attn_dispatch<D, PV, OUT, false>(q_i8, k_i8, v_t, q_scale, k_scale, v_scale,
                                                   B, H, N, out, s);
}

hipError_t launch_attn(const int8_t* q_i8, const int8_t* k_i8, const uint8_t* v_t,
                       const float* q_scale, const float* k_scale, const float* v_scale, int B,
                       int H, int N, int d, int causal, int pv_mode, int out_kind, void* out,
                       hipStream_t s) {
#define SAGE_ATTN_CASE(D, PV, OUT)                                                          \
  if (d == D && pv_mode == PV && out_kind == OUT)                                          \
    return attn_dispatch_c<D, PV, OUT>(causal, q_i8, k_i8, v_t, q_scale, k_scale, v_scale, \
                                       B, H, N, out, s);
  SAGE_ATTN_CASE(64, 0, 0) SAGE_ATTN_CASE(64, 0, 1) SAGE_ATTN_CASE(64, 0, 2)
  SAGE_ATTN_CASE(64, 1, 0) SAGE_ATTN_CASE(64, 1, 1) SAGE_ATTN_CASE(64, 1, 2)
  SAGE_ATTN_CASE(128, 0, 0) SAGE_ATTN_CASE(128, 0, 1) SAGE_ATTN_CASE(128, 0, 2)
  SAGE_ATTN_CASE(128, 1, 0) SAGE_ATTN_CASE(128, 1, 1) SAGE_ATTN_CASE(128, 1, 2)
#undef SAGE_ATTN_CASE
  return hipErrorInvalidValue;
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
