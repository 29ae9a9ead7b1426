// sage_common.h -- device-side types, constants and helpers shared by the
// prepass and attention kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sage_launch.h"

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// 16-bit input element -> exact float32.
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
template <int DT>
__device__ __forceinline__ float in_to_f32(uint16_t b) {
  return DT == 0 ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
}

// Element offset of token t of head bh = b*H + h in a [B,H,N,d] tensor
// (nhd = 0) or a token-major [B,N,H,d] tensor (nhd = 1).
template <int D>
__device__ __forceinline__ size_t row_off(int bh, int t, int H, int N, int nhd) {
  if (!nhd) return ((size_t)bh * N + t) * D;
  const int b = bh / H, h = bh - b * H;
  return (((size_t)b * N + t) * H + h) * D;
}

// Two floats -> packed fp16 pair (v_cvt_pk_f16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  v2f x = {a, b};
  v2h h = __builtin_convertvector(x, v2h);
  return __builtin_bit_cast(uint32_t, h);
}
// Two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  v2f x = {a, b};
  v2bf h = __builtin_convertvector(x, v2bf);
  return __builtin_bit_cast(uint32_t, h);
}
// Four floats -> four OCP E4M3 codes (v_cvt_pk_fp8_f32, round to nearest even).
// The first conversion writes the low half of a register whose high half
// the second one overwrites, so that register may be a's own (no clearing
// or copying instruction).
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Four floats -> four symmetric INT8 codes, clamp(rne(x), -127, 127), packed
// little-endian (first value in the low byte).
__device__ __forceinline__ uint32_t pack_i8x4_sym(float a, float b, float c, float d) {
  const float x[4] = {a, b, c, d};
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = (int)fminf(fmaxf(__builtin_rintf(x[i]), -127.f), 127.f);
    w |= ((uint32_t)q & 0xffu) << (8 * i);
  }
  return w;
}

// LDS swizzles.  gfx950's LDS serves a ds_read_b128 sixteen lanes at a time
// (256 bytes = all 64 banks).  The 16-byte chunk `k` of row `r` is stored at
// chunk k ^ swz(r): for 128-byte rows, rows r and r+1 share a 256-byte bank
// window, so swz(r) = (r / 2) % 8 makes the 16 lanes of a group (16
// consecutive rows, same logical chunk) hit 16 distinct 16-byte bank groups;
// for 64-byte rows, four rows share a window and swz(r) = (r / 4) % 4.
template <int ROW_BYTES>
__device__ __forceinline__ int row_swizzle(int r) {
  if constexpr (ROW_BYTES >= 128) return (r >> 1) & 7;
  else if constexpr (ROW_BYTES == 64) return (r >> 2) & 3;
  else return 0;
}

// Wave-wide max / sum helpers.
__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Reductions over the lane pair (l, l^32).  v_permlane32_swap with the same
// register as both operands leaves {value of lane l%32, value of lane l%32+32}
// in the two results on every lane, so both lanes of a pair compute the same
// combination in the same operand order.
__device__ __forceinline__ int pair_max_i32(int v) {
  auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float pair_sum_f32(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

}  // namespace sage
