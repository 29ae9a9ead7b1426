// ref_rows.hip -- full-precision (float32) softmax attention on selected
// query rows, the reference against which the per-layer P~V precision is
// chosen ("SageAttention ..." detail page, §2 Q2 item 3 and §5: each layer's
// quantised output is compared with full precision by cosine similarity).
//
// One workgroup per (b*h, selected row): each of the 256 threads runs an
// online softmax over keys t, t+256, ...; the partial (max, sum, output)
// states are then merged through LDS.
#include "sage_common.h"
#include "sage_launch.h"

namespace sage {

template <int DT, int D>
__global__ __launch_bounds__(256) void ref_rows_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, int N,
                                                       int causal, const int32_t* __restrict__ rows,
                                                       int nrows, float* __restrict__ out) {
  __shared__ float red_m[256], red_l[256];
  __shared__ float red_o[32][257];
  __shared__ float qs[D];
  const int bh = blockIdx.y;
  const int ri = blockIdx.x;
  const int tid = threadIdx.x;
  const int row = rows[ri];
  float* o_out = out + ((size_t)bh * nrows + ri) * D;
  if (row < 0 || row >= N) {   // invalid row index: NaN output, no access
    for (int c = tid; c < D; c += 256) o_out[c] = __builtin_nanf("");
    return;
  }
  const float scale = 1.0f / sqrtf((float)D);
  const uint16_t* qp = q + ((size_t)bh * N + row) * D;
  for (int c = tid; c < D; c += 256) qs[c] = in_to_f32<DT>(qp[c]) * scale;
  __syncthreads();
  float m = -__builtin_inff(), l = 0.f;
  float o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  const int kend = causal ? row + 1 : N;
  for (int key = tid; key < kend; key += 256) {
    const uint16_t* kp = k + ((size_t)bh * N + key) * D;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) s = __builtin_fmaf(qs[c], in_to_f32<DT>(kp[c]), s);
    const float m_new = fmaxf(m, s);
    const float a = expf(m - m_new);
    const float p = expf(s - m_new);
    l = l * a + p;
    const uint16_t* vp = v + ((size_t)bh * N + key) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(p, in_to_f32<DT>(vp[c]), o[c] * a);
    m = m_new;
  }
  // merge the 256 partial states
  red_m[tid] = m;
  __syncthreads();
  float mall = -__builtin_inff();
  for (int i = 0; i < 256; ++i) mall = fmaxf(mall, red_m[i]);
  const float w = m == -__builtin_inff() ? 0.f : expf(m - mall);
  red_l[tid] = l * w;
  __syncthreads();
  float lall = 0.f;
  for (int i = 0; i < 256; ++i) lall += red_l[i];
  for (int c0 = 0; c0 < D; c0 += 32) {
#pragma unroll
    for (int c = 0; c < 32; ++c) red_o[c][tid] = o[c0 + c] * w;
    __syncthreads();
    if (tid < 32) {
      float acc = 0.f;
      for (int i = 0; i < 256; ++i) acc += red_o[tid][i];
      o_out[c0 + tid] = acc / lall;
    }
    __syncthreads();
  }
}

hipError_t launch_ref_rows(const void* q, const void* k, const void* v, int dtype, int B, int H,
                           int N, int d, int causal, const int32_t* rows, int nrows, float* out,
                           hipStream_t s) {
  dim3 grid(nrows, B * H);
  auto qp = static_cast<const uint16_t*>(q);
  auto kp = static_cast<const uint16_t*>(k);
  auto vp = static_cast<const uint16_t*>(v);
  if (dtype == 0 && d == 64) ref_rows_kernel<0, 64><<<grid, 256, 0, s>>>(qp, kp, vp, N, causal, rows, nrows, out);
  else if (dtype == 0 && d == 128) ref_rows_kernel<0, 128><<<grid, 256, 0, s>>>(qp, kp, vp, N, causal, rows, nrows, out);
  else if (dtype == 1 && d == 64) ref_rows_kernel<1, 64><<<grid, 256, 0, s>>>(qp, kp, vp, N, causal, rows, nrows, out);
  else if (dtype == 1 && d == 128) ref_rows_kernel<1, 128><<<grid, 256, 0, s>>>(qp, kp, vp, N, causal, rows, nrows, out);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sage
