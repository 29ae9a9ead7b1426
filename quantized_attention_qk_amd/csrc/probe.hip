// probe.hip -- micro-benchmarks of the gfx950 units the attention kernel
// leans on: the sustained rate of the three MFMA shapes it issues, the issue
// cost of v_exp_f32 next to v_fma_f32, how VALU work overlaps a stream of
// MFMAs with one or two wavefronts per SIMD, and the LDS read bandwidth alone
// and next to MFMAs.  Every wavefront also stamps its
// loop with the shader clock (s_memtime) and the constant-rate real-time
// counter (s_memrealtime), so the host can derive the clock the chip ran at.
//
// These are measurement tools behind include/sage_probe.h (bench.py
// --mfma-probe); the attention path does not use them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sage_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// LDS bytes a workgroup claims so that at most WPS workgroups of four
// wavefronts (one per SIMD) fit on a CU of 160 KiB: WPS wavefronts per SIMD.
template <int WPS>
constexpr int kLdsClaim = WPS == 1 ? 100000 : 70000;

constexpr int kChains = 4;   // independent accumulators per wavefront

// One MFMA of kind K on accumulator `acc` (operands from registers).
template <int K>
__device__ __forceinline__ v16f mfma(const v8i& a, const v8i& b, v16f acc) {
  if constexpr (K == SAGE_PROBE_MFMA_I8) {
    const v4i a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(
        v16f, __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, __builtin_bit_cast(v16i, acc), 0, 0, 0));
  } else if constexpr (K == SAGE_PROBE_MFMA_F16) {
    const v4i a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a4),
                                                  __builtin_bit_cast(v8h, b4), acc, 0, 0, 0);
  } else {
    // FP8 E4M3 x E4M3, unit block scales (E8M0 exponent 127 = 1.0)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
  }
}

// Every wavefront runs `iters` groups.  A group issues one MFMA of kind K
// (K < 0: none), rotating over kChains accumulators, then NV independent
// v_fma_f32 and NE independent v_exp_f32; scheduling barriers keep the groups
// apart so the wavefront's instruction stream is exactly this pattern.
template <int K, int NV, int NE, int WPS>
__global__ __launch_bounds__(256) void probe_kernel(int iters, int seed,
                                                   long long* __restrict__ stamps,
                                                   float* __restrict__ sink) {
  __shared__ float claim[kLdsClaim<WPS> / 4];
  const int tid = threadIdx.x;
  claim[tid] = (float)seed;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ (seed + i + tid);   // small E4M3 / fp16 / int8 values
    b[i] = 0x30303030 ^ (seed - i + tid);
  }
  v16f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v16f{};
  float x[NV > 0 ? NV : 1], e[NE > 0 ? NE : 1];
#pragma unroll
  for (int i = 0; i < NV; ++i) x[i] = 1.0f + 0.001f * (i + tid);
#pragma unroll
  for (int i = 0; i < NE; ++i) e[i] = -1.0f - 0.01f * (i + tid);
  const float fa = 0.999f, fb = 0.0001f * seed;
  __syncthreads();

  const long long c0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += kChains) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (K >= 0) acc[c] = mfma<K>(a, b, acc[c]);
#pragma unroll
      for (int i = 0; i < NV; ++i) x[i] = __builtin_fmaf(x[i], fa, fb);
#pragma unroll
      for (int i = 0; i < NE; ++i) e[i] = __builtin_amdgcn_exp2f(e[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const long long c1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();

  float s = claim[(tid + 1) & 255];
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][tid & 15];
#pragma unroll
  for (int i = 0; i < NV; ++i) s += x[i];
#pragma unroll
  for (int i = 0; i < NE; ++i) s += e[i];
  sink[blockIdx.x * 256 + tid] = s;
  if ((tid & 63) == 0) {
    const size_t w = (size_t)blockIdx.x * 4 + (tid >> 6);
    stamps[4 * w + 0] = c0;
    stamps[4 * w + 1] = c1;
    stamps[4 * w + 2] = r0;
    stamps[4 * w + 3] = r1;
  }
}

template <int K, int NV, int NE, int WPS>
hipError_t launch(int ncu, int iters, int seed, long long* stamps, float* sink, hipStream_t s) {
  probe_kernel<K, NV, NE, WPS><<<dim3(ncu * WPS), 256, 0, s>>>(iters, seed, stamps, sink);
  return hipGetLastError();
}

template <int K, int NV, int NE>
hipError_t launch_w(int wps, int ncu, int iters, int seed, long long* stamps, float* sink,
                    hipStream_t s) {
  return wps == 1 ? launch<K, NV, NE, 1>(ncu, iters, seed, stamps, sink, s)
                  : launch<K, NV, NE, 2>(ncu, iters, seed, stamps, sink, s);
}

// (NV, NE) pairs instantiated for the mixed and VALU-only probes.
template <int K>
hipError_t launch_mix(int nv, int ne, int wps, int ncu, int iters, int seed, long long* stamps,
                      float* sink, hipStream_t s) {
#define SAGE_PROBE_CASE(V, E) \
  if (nv == V && ne == E) return launch_w<K, V, E>(wps, ncu, iters, seed, stamps, sink, s);
  SAGE_PROBE_CASE(0, 0) SAGE_PROBE_CASE(4, 0) SAGE_PROBE_CASE(6, 0) SAGE_PROBE_CASE(8, 0)
  SAGE_PROBE_CASE(12, 0) SAGE_PROBE_CASE(16, 0) SAGE_PROBE_CASE(0, 2) SAGE_PROBE_CASE(0, 4)
  SAGE_PROBE_CASE(4, 2) SAGE_PROBE_CASE(4, 4) SAGE_PROBE_CASE(2, 2) SAGE_PROBE_CASE(6, 2)
#undef SAGE_PROBE_CASE
  return hipErrorInvalidValue;
}

// LDS read bandwidth next to MFMAs: every wavefront runs `iters` groups of
// [one MFMA of kind K (K < 0: none), NL independent ds_read_b128], each read
// moving 1 KiB (64 lanes x 16 bytes, consecutive addresses, no bank
// conflicts) from the workgroup's LDS claim.  A group consumes the reads
// issued four groups earlier, so each read has four groups' time to land.
template <int K, int NL, int WPS>
__global__ __launch_bounds__(256) void probe_lds_kernel(int iters, int seed,
                                                       long long* __restrict__ stamps,
                                                       float* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) float claim[kLdsClaim<WPS> / 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  for (int i = tid; i < kLdsClaim<WPS> / 4; i += 256) claim[i] = (float)(seed + i);
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ (seed + i + tid);
    b[i] = 0x30303030 ^ (seed - i + tid);
  }
  v16f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v16f{};
  v4i r[kChains][NL];
#pragma unroll
  for (int h = 0; h < kChains; ++h)
#pragma unroll
    for (int i = 0; i < NL; ++i) r[h][i] = v4i{};
  const char* lds = reinterpret_cast<const char*>(claim);
  __syncthreads();

  const long long c0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += kChains) {
    // a 32 KiB window that moves every trip; the groups' reads sit at fixed
    // offsets from it (at most 16 KiB further), inside the 64 KiB claim
    const int base = (lane * 16 + it * (NL * 1024)) & 0x7fff;
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (K >= 0) acc[c] = mfma<K>(a, b, acc[c]);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        asm volatile("" ::"v"(r[c][i]));
        r[c][i] = *reinterpret_cast<const v4i*>(lds + base + (c * NL + i) * 1024);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const long long c1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();

  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][tid & 15];
#pragma unroll
  for (int h = 0; h < kChains; ++h)
#pragma unroll
    for (int i = 0; i < NL; ++i) s += (float)(r[h][i][0] ^ r[h][i][3]);
  sink[blockIdx.x * 256 + tid] = s;
  if ((tid & 63) == 0) {
    const size_t w = (size_t)blockIdx.x * 4 + (tid >> 6);
    stamps[4 * w + 0] = c0;
    stamps[4 * w + 1] = c1;
    stamps[4 * w + 2] = r0;
    stamps[4 * w + 3] = r1;
  }
}

template <int K, int NL>
hipError_t launch_lds(int wps, int ncu, int iters, int seed, long long* stamps, float* sink,
                      hipStream_t s) {
  if (wps == 1)
    probe_lds_kernel<K, NL, 1><<<dim3(ncu), 256, 0, s>>>(iters, seed, stamps, sink);
  else
    probe_lds_kernel<K, NL, 2><<<dim3(ncu * 2), 256, 0, s>>>(iters, seed, stamps, sink);
  return hipGetLastError();
}

template <int K>
hipError_t launch_lds_n(int nl, int wps, int ncu, int iters, int seed, long long* stamps,
                        float* sink, hipStream_t s) {
  if (nl == 1) return launch_lds<K, 1>(wps, ncu, iters, seed, stamps, sink, s);
  if (nl == 2) return launch_lds<K, 2>(wps, ncu, iters, seed, stamps, sink, s);
  if (nl == 4) return launch_lds<K, 4>(wps, ncu, iters, seed, stamps, sink, s);
  return hipErrorInvalidValue;
}

}  // namespace

extern "C" {

int sage_probe_wallclock_khz(int* khz) {
  if (!khz) return 1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 4;
  return hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess ? 0 : 4;
}

int sage_probe_cu_count(int* ncu) {
  if (!ncu) return 1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 4;
  return hipDeviceGetAttribute(ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? 0
                                                                                               : 4;
}

int sage_probe_run(int mfma_kind, int nv, int ne, int waves_per_simd, int ncu, int iters,
                   long long* stamps, float* sink, void* stream) {
  if (waves_per_simd != 1 && waves_per_simd != 2) return 1;
  if (ncu < 1 || ncu > 4096 || iters < kChains || iters % kChains) return 1;
  if (!stamps || !sink) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (mfma_kind) {
    case SAGE_PROBE_NONE: e = launch_mix<-1>(nv, ne, waves_per_simd, ncu, iters, 1, stamps, sink, s); break;
    case SAGE_PROBE_MFMA_I8: e = launch_mix<SAGE_PROBE_MFMA_I8>(nv, ne, waves_per_simd, ncu, iters, 1, stamps, sink, s); break;
    case SAGE_PROBE_MFMA_F16: e = launch_mix<SAGE_PROBE_MFMA_F16>(nv, ne, waves_per_simd, ncu, iters, 1, stamps, sink, s); break;
    case SAGE_PROBE_MFMA_F8: e = launch_mix<SAGE_PROBE_MFMA_F8>(nv, ne, waves_per_simd, ncu, iters, 1, stamps, sink, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : (e == hipErrorInvalidValue ? 2 : 4);
}

int sage_probe_run_lds(int mfma_kind, int nl, int waves_per_simd, int ncu, int iters,
                       long long* stamps, float* sink, void* stream) {
  if (waves_per_simd != 1 && waves_per_simd != 2) return 1;
  if (ncu < 1 || ncu > 4096 || iters < kChains || iters % kChains) return 1;
  if (!stamps || !sink) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (mfma_kind) {
    case SAGE_PROBE_NONE: e = launch_lds_n<-1>(nl, waves_per_simd, ncu, iters, 1, stamps, sink, s); break;
    case SAGE_PROBE_MFMA_I8: e = launch_lds_n<SAGE_PROBE_MFMA_I8>(nl, waves_per_simd, ncu, iters, 1, stamps, sink, s); break;
    case SAGE_PROBE_MFMA_F16: e = launch_lds_n<SAGE_PROBE_MFMA_F16>(nl, waves_per_simd, ncu, iters, 1, stamps, sink, s); break;
    case SAGE_PROBE_MFMA_F8: e = launch_lds_n<SAGE_PROBE_MFMA_F8>(nl, waves_per_simd, ncu, iters, 1, stamps, sink, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : (e == hipErrorInvalidValue ? 2 : 4);
}

}  // extern "C"
