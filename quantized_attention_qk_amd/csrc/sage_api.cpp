// sage_api.cpp -- the C ABI declared in include/sage_attn.h.
//
// Every entry point validates all arguments before it enqueues anything, then
// checks for a gfx950 device, then launches the kernels of prepass.hip and
// attn_fwd.hip on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "sage_attn.h"
#include "sage_launch.h"

namespace {

using sage::ceil_div;

using sage::kMaxN;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool shape_ok(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return false;
  if (d != 64 && d != 128) return false;
  // B*H*nqb workgroups must fit a 1-D grid; B*H must fit an int.
  const long long bh = (long long)B * H;
  if (bh > 0x7fffffffLL) return false;
  if (bh * ceil_div(N, sage::kQBlock) > 0x7fffffffLL) return false;
  if (bh > 65535) return false;   // grid.y of the prepass kernels
  return true;
}

// The smoothed-Q compensation values of one pass take at most this many bytes
// of workspace; longer sequences compute them, and run the attention kernel,
// in chunks of query blocks.
constexpr size_t kSqCompMaxBytes = size_t(256) << 20;

// 128-row query blocks per chunk of the smoothed-Q pass: all of them when the
// whole table fits, else a multiple of 2 (the widest attention workgroup
// covers 256 rows).
int sq_chunk_blocks(int B, int H, int N) {
  const size_t nq128 = ceil_div(N, sage::kQBlock), nt = ceil_div(N, sage::kKvTile);
  const size_t per_block = (size_t)B * H * nt * sage::kKvTile * 4;
  if (per_block * nq128 <= kSqCompMaxBytes) return (int)nq128;
  const size_t c = (kSqCompMaxBytes / per_block) & ~size_t(1);
  return (int)(c < 2 ? 2 : c);
}

// Workspace carve-up of sage_attn_fwd (private layout); with smoothed Q also
// the block means, the integer means w and the compensation values (of one
// chunk of query blocks).
struct Layout {
  size_t q_i8, k_i8, v_t, q_scale, k_scale, k_mean, v_scale, v_recip, part_sum, part_max;
  size_t q_mean, q_w, comp, total;
};

Layout make_layout(int B, int H, int N, int d, int pv_mode, bool sq = false) {
  const size_t bh = (size_t)B * H;
  const size_t nqb = ceil_div(N, sage::kQBlock), nkb = ceil_div(N, sage::kKBlock);
  const size_t nt = ceil_div(N, sage::kKvTile), nch = ceil_div(N, sage::kMeanChunk);
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  L.q_i8 = take(bh * N * d);
  L.k_i8 = take(bh * N * d);
  L.v_t = take(bh * nt * sage::v_tile_bytes(d, pv_mode));
  L.q_scale = take(bh * nqb * 4);
  L.k_scale = take(bh * nkb * 4);
  L.k_mean = take(bh * d * 4);
  L.v_scale = take(bh * d * 4);
  L.v_recip = take(bh * d * 4);
  L.part_sum = take(bh * nch * d * 4);
  L.part_max = take(sage::v_quantised(pv_mode) ? bh * nch * d * 4 : 0);
  L.q_mean = take(sq ? bh * nqb * d * 4 : 0);
  L.q_w = take(sq ? bh * nqb * d * 4 : 0);
  L.comp = take(sq ? bh * (size_t)sq_chunk_blocks(B, H, N) * nt * sage::kKvTile * 4 : 0);
  L.total = off;
  return L;
}

// 0 = ok, else a sage_status.  The gfx950 check is cached per device.
int device_check() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
    (void)hipGetLastError();
    return SAGE_ERR_NO_DEVICE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAGE_ERR_HIP;
  static std::atomic<int> cache[64];   // 0 unknown, 1 gfx950, 2 other
  if (dev < 0 || dev >= 64) return SAGE_ERR_UNSUPPORTED;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SAGE_ERR_HIP;
    c = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c == 1 ? SAGE_OK : SAGE_ERR_UNSUPPORTED;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP; }

// The attention kernel alone on prepared operands (q_seed: null, or the
// smoothed-Q accumulator seeds); defined with the stage entry points.
int fwd_quantized(const int8_t* q_i8, const int8_t* k_i8, const void* v_prep,
                  const float* q_scale, const float* k_scale, const float* v_scale,
                  const int32_t* q_seed, void* o, int B, int H, int N, int d, int causal,
                  int pv_mode, int out_dtype, void* stream);

// Layout flag and RoPE tables: both tables or neither, 16-byte aligned.
int validate_in(int layout, const float* rope_cos, const float* rope_sin) {
  if (layout != SAGE_LAYOUT_HND && layout != SAGE_LAYOUT_NHD) return SAGE_ERR_INVALID_ARG;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return SAGE_ERR_INVALID_ARG;
  if (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) return SAGE_ERR_INVALID_ARG;
  return SAGE_OK;
}

// need_o = false: the prepass alone (sage_attn_prepare), o is not used.
int validate_fwd(const void* q, const void* k, const void* v, const void* o, int B, int H, int N,
                 int d, int causal, int pv_mode, int dtype, const void* ws, size_t ws_bytes,
                 bool sq = false, bool need_o = true) {
  if (!q || !k || !v || (need_o && !o) || !ws) return SAGE_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (need_o && !aligned16(o)))
    return SAGE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return SAGE_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
  if (!sage::pv_valid(pv_mode)) return SAGE_ERR_INVALID_ARG;
  if (dtype != SAGE_DT_F16 && dtype != SAGE_DT_BF16) return SAGE_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SAGE_ERR_UNSUPPORTED;
  if (!shape_ok(B, H, N, d)) return SAGE_ERR_UNSUPPORTED;
  if (need_o && (o == q || o == k || o == v)) return SAGE_ERR_INVALID_ARG;
  if (ws_bytes < make_layout(B, H, N, d, pv_mode, sq).total) return SAGE_ERR_WORKSPACE;
  return SAGE_OK;
}

// out_kind < 0: the prepass alone (the workspace's operands, no attention).
int run_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
            int causal, int pv_mode, int dtype, int layout, const float* rope_cos,
            const float* rope_sin, void* ws, size_t ws_bytes, void* stream, int out_kind) {
  int st = validate_fwd(q, k, v, o, B, H, N, d, causal, pv_mode, dtype, ws, ws_bytes, false,
                        out_kind >= 0);
  if (st != SAGE_OK) return st;
  if ((st = validate_in(layout, rope_cos, rope_sin)) != SAGE_OK) return st;
  const sage::InLayout in{layout, rope_cos, rope_sin};
  if ((st = device_check()) != SAGE_OK) return st;
  const Layout L = make_layout(B, H, N, d, pv_mode);
  uint8_t* w = static_cast<uint8_t*>(ws);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  int8_t* q_i8 = reinterpret_cast<int8_t*>(w + L.q_i8);
  int8_t* k_i8 = reinterpret_cast<int8_t*>(w + L.k_i8);
  uint8_t* v_t = w + L.v_t;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool qv = sage::v_quantised(pv_mode);
  hipError_t e;
  if (N <= sage::kHeadPrepassMaxN) {
    const sage::PrepassOut po{F(L.part_sum), F(L.k_mean), F(L.v_scale), q_i8, k_i8,
                              F(L.q_scale), F(L.k_scale), v_t};
    e = sage::launch_prepass_head(q, k, v, dtype, B, H, N, d, pv_mode, in, po, s);
    if (e != hipSuccess) return SAGE_ERR_HIP;
  } else {
    e = sage::launch_colstats(k, qv ? v : nullptr, dtype, B, H, N, d, pv_mode, in,
                              F(L.part_sum), qv ? F(L.part_max) : nullptr, F(L.k_mean),
                              F(L.v_scale), F(L.v_recip), s, !sage::quant_qkv_folds(N));
    if (e != hipSuccess) return SAGE_ERR_HIP;
    e = sage::launch_quant_qkv(q, k, v, F(L.k_mean), F(L.v_recip), dtype, B, H, N, d, pv_mode,
                               in, q_i8, k_i8, F(L.q_scale), F(L.k_scale), v_t, F(L.part_sum),
                               qv ? F(L.part_max) : nullptr, F(L.v_scale), s);
    if (e != hipSuccess) return SAGE_ERR_HIP;
  }
  if (out_kind < 0) return SAGE_OK;
  e = sage::launch_attn(q_i8, k_i8, v_t, F(L.q_scale), F(L.k_scale), F(L.v_scale), nullptr, B,
                        H, N, d, causal, pv_mode, out_kind, layout, o, s);
  return hip_status(e);
}

// The pass with Q smoothed per block: K statistics and K^, V, then the
// smoothed Q^ with its integer means, the compensation values (with FP16
// mode's accumulator bias), and the attention kernel seeded with them.
int run_fwd_sq(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
               int causal, int pv_mode, int dtype, int layout, void* ws, size_t ws_bytes,
               void* stream, int out_kind) {
  int st = validate_fwd(q, k, v, o, B, H, N, d, causal, pv_mode, dtype, ws, ws_bytes, true);
  if (st != SAGE_OK) return st;
  if ((st = validate_in(layout, nullptr, nullptr)) != SAGE_OK) return st;
  const sage::InLayout in{layout, nullptr, nullptr};
  if ((st = device_check()) != SAGE_OK) return st;
  const Layout L = make_layout(B, H, N, d, pv_mode, true);
  uint8_t* w = static_cast<uint8_t*>(ws);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  int8_t* q_i8 = reinterpret_cast<int8_t*>(w + L.q_i8);
  int8_t* k_i8 = reinterpret_cast<int8_t*>(w + L.k_i8);
  int32_t* q_w = reinterpret_cast<int32_t*>(w + L.q_w);
  int32_t* comp = reinterpret_cast<int32_t*>(w + L.comp);
  uint8_t* v_t = w + L.v_t;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool qv = sage::v_quantised(pv_mode);
  hipError_t e = sage::launch_colstats(k, qv ? v : nullptr, dtype, B, H, N, d, pv_mode, in,
                                       F(L.part_sum), qv ? F(L.part_max) : nullptr, F(L.k_mean),
                                       F(L.v_scale), F(L.v_recip), s,
                                       !sage::quant_qkv_folds(N));
  if (e != hipSuccess) return SAGE_ERR_HIP;
  e = sage::launch_quant_qkv(nullptr, k, v, F(L.k_mean), F(L.v_recip), dtype, B, H, N, d,
                             pv_mode, in, nullptr, k_i8, nullptr, F(L.k_scale), v_t,
                             F(L.part_sum), qv ? F(L.part_max) : nullptr, F(L.v_scale), s);
  if (e != hipSuccess) return SAGE_ERR_HIP;
  e = sage::launch_smooth_q(q, dtype, B, H, N, d, layout, q_i8, F(L.q_scale), F(L.q_mean), q_w,
                            s);
  if (e != hipSuccess) return SAGE_ERR_HIP;
  // the compensation values and the attention kernel, one chunk of query
  // blocks at a time (one chunk unless the table passes kSqCompMaxBytes)
  const int nq128 = ceil_div(N, sage::kQBlock), chunk = sq_chunk_blocks(B, H, N);
  for (int q0 = 0; q0 < nq128; q0 += chunk) {
    const int cnt = nq128 - q0 < chunk ? nq128 - q0 : chunk;
    e = sage::launch_sq_comp(k_i8, q_w, B, H, N, d, ceil_div(N, sage::kKvTile) * sage::kKvTile,
                             pv_mode == SAGE_PV_FP16 ? sage::kSqBiasFp16 : 0, comp, s, q0, cnt);
    if (e != hipSuccess) return SAGE_ERR_HIP;
    e = sage::launch_attn(q_i8, k_i8, v_t, F(L.q_scale), F(L.k_scale), F(L.v_scale), comp, B, H,
                          N, d, causal, pv_mode, out_kind, layout, o, s, q0,
                          q0 + cnt >= nq128 ? 0 : cnt);
    if (e != hipSuccess) return SAGE_ERR_HIP;
  }
  return SAGE_OK;
}

}  // namespace

extern "C" {

const char* sage_status_str(int status) {
  switch (status) {
    case SAGE_OK: return "SAGE_OK";
    case SAGE_ERR_INVALID_ARG: return "SAGE_ERR_INVALID_ARG: invalid pointer, size, flag or alignment";
    case SAGE_ERR_UNSUPPORTED: return "SAGE_ERR_UNSUPPORTED: request not supported by this library (d, size or device)";
    case SAGE_ERR_WORKSPACE: return "SAGE_ERR_WORKSPACE: workspace or scratch too small";
    case SAGE_ERR_HIP: return "SAGE_ERR_HIP: the HIP runtime reported an error";
    case SAGE_ERR_NO_DEVICE: return "SAGE_ERR_NO_DEVICE: no HIP device visible";
    default: return "SAGE_ERR_UNKNOWN";
  }
}

int sage_attn_get_tiling(int d, int causal, int pv_mode, int* q_block, int* k_block,
                         int* kv_tile, int* mean_chunk) {
  (void)causal;
  if (d != 64 && d != 128) return SAGE_ERR_UNSUPPORTED;
  if (!sage::pv_valid(pv_mode)) return SAGE_ERR_UNSUPPORTED;
  if (q_block) *q_block = sage::kQBlock;
  if (k_block) *k_block = sage::kKBlock;
  if (kv_tile) *kv_tile = sage::kKvTile;
  if (mean_chunk) *mean_chunk = sage::kMeanChunk;
  return SAGE_OK;
}

size_t sage_attn_workspace_bytes(int B, int H, int N, int d, int pv_mode) {
  if (!shape_ok(B, H, N, d)) return 0;
  if (!sage::pv_valid(pv_mode)) return 0;
  return make_layout(B, H, N, d, pv_mode).total;
}

int sage_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                  int d, int causal, int pv_mode, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return run_fwd(q, k, v, o, B, H, N, d, causal, pv_mode, dtype, SAGE_LAYOUT_HND, nullptr,
                 nullptr, workspace, workspace_bytes, stream, dtype == SAGE_DT_BF16 ? 1 : 0);
}

int sage_attn_prepare(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                      int pv_mode, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return run_fwd(q, k, v, nullptr, B, H, N, d, 0, pv_mode, dtype, SAGE_LAYOUT_HND, nullptr,
                 nullptr, workspace, workspace_bytes, stream, -1);
}

int sage_attn_attend(const void* workspace, size_t workspace_bytes, void* o, int B, int H,
                     int N, int d, int causal, int pv_mode, int out_dtype, void* stream) {
  if (!workspace || !o) return SAGE_ERR_INVALID_ARG;
  if (!aligned16(o) || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return SAGE_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
  if (!sage::pv_valid(pv_mode)) return SAGE_ERR_INVALID_ARG;
  if (out_dtype != SAGE_DT_F16 && out_dtype != SAGE_DT_BF16 && out_dtype != SAGE_OUT_F32)
    return SAGE_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SAGE_ERR_UNSUPPORTED;
  if (!shape_ok(B, H, N, d)) return SAGE_ERR_UNSUPPORTED;
  const Layout L = make_layout(B, H, N, d, pv_mode);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE;
  int st = device_check();
  if (st != SAGE_OK) return st;
  // the same launch as the end of run_fwd, on the operands its prepass left
  uint8_t* w = static_cast<uint8_t*>(const_cast<void*>(workspace));
  auto F = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  return hip_status(sage::launch_attn(reinterpret_cast<int8_t*>(w + L.q_i8),
                                      reinterpret_cast<int8_t*>(w + L.k_i8), w + L.v_t,
                                      F(L.q_scale), F(L.k_scale), F(L.v_scale), nullptr, B, H,
                                      N, d, causal, pv_mode, out_dtype, SAGE_LAYOUT_HND, o,
                                      static_cast<hipStream_t>(stream)));
}

int sage_attn_fwd_f32out(const void* q, const void* k, const void* v, float* o, int B, int H,
                         int N, int d, int causal, int pv_mode, int dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return run_fwd(q, k, v, o, B, H, N, d, causal, pv_mode, dtype, SAGE_LAYOUT_HND, nullptr,
                 nullptr, workspace, workspace_bytes, stream, 2);
}

int sage_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                     int d, int causal, int pv_mode, int dtype, int layout,
                     const float* rope_cos, const float* rope_sin, int out_f32, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (out_f32 != 0 && out_f32 != 1) return SAGE_ERR_INVALID_ARG;
  return run_fwd(q, k, v, o, B, H, N, d, causal, pv_mode, dtype, layout, rope_cos, rope_sin,
                 workspace, workspace_bytes, stream,
                 out_f32 ? 2 : (dtype == SAGE_DT_BF16 ? 1 : 0));
}

size_t sage_attn_sq_workspace_bytes(int B, int H, int N, int d, int pv_mode) {
  if (!shape_ok(B, H, N, d)) return 0;
  if (!sage::pv_valid(pv_mode)) return 0;
  return make_layout(B, H, N, d, pv_mode, true).total;
}

int sage_attn_fwd_sq(const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                     int d, int causal, int pv_mode, int dtype, int layout, int out_f32,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (out_f32 != 0 && out_f32 != 1) return SAGE_ERR_INVALID_ARG;
  return run_fwd_sq(q, k, v, o, B, H, N, d, causal, pv_mode, dtype, layout, workspace,
                    workspace_bytes, stream, out_f32 ? 2 : (dtype == SAGE_DT_BF16 ? 1 : 0));
}

int sage_smooth_q(const void* q, const int8_t* k_i8, int dtype, int B, int H, int N, int d,
                  int seed_pv_mode, int8_t* q_i8, float* q_scale, float* q_mean, int32_t* q_w,
                  int32_t* q_comp, void* stream) {
  if (!q || !k_i8 || !q_i8 || !q_scale || !q_mean || !q_w || !q_comp) return SAGE_ERR_INVALID_ARG;
  if (seed_pv_mode != -1 && !sage::pv_valid(seed_pv_mode)) return SAGE_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_i8) || !aligned16(q_i8) || !aligned16(q_w) ||
      !aligned16(q_comp) || (reinterpret_cast<uintptr_t>(q_scale) & 3u) ||
      (reinterpret_cast<uintptr_t>(q_mean) & 3u))
    return SAGE_ERR_INVALID_ARG;
  if (dtype != SAGE_DT_F16 && dtype != SAGE_DT_BF16) return SAGE_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID_ARG;
  if (!shape_ok(B, H, N, d)) return SAGE_ERR_UNSUPPORTED;
  int st = device_check();
  if (st != SAGE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = sage::launch_smooth_q(q, dtype, B, H, N, d, SAGE_LAYOUT_HND, q_i8, q_scale,
                                       q_mean, q_w, s);
  if (e != hipSuccess) return SAGE_ERR_HIP;
  const int ld = seed_pv_mode < 0 ? N : ceil_div(N, sage::kKvTile) * sage::kKvTile;
  const int bias = seed_pv_mode == SAGE_PV_FP16 ? sage::kSqBiasFp16 : 0;
  return hip_status(sage::launch_sq_comp(k_i8, q_w, B, H, N, d, ld, bias, q_comp, s));
}

int sage_attn_fwd_quantized_sq(const int8_t* q_i8, const int8_t* k_i8, const void* v_prep,
                               const float* q_scale, const float* k_scale, const float* v_scale,
                               const int32_t* q_seed, void* o, int B, int H, int N, int d,
                               int causal, int pv_mode, int out_dtype, void* stream) {
  if (!q_seed || (reinterpret_cast<uintptr_t>(q_seed) & 15u)) return SAGE_ERR_INVALID_ARG;
  return fwd_quantized(q_i8, k_i8, v_prep, q_scale, k_scale, v_scale, q_seed, o, B, H, N, d,
                       causal, pv_mode, out_dtype, stream);
}

size_t sage_smooth_quant_qk_scratch_bytes(int B, int H, int N, int d) {
  if (!shape_ok(B, H, N, d)) return 0;
  return (size_t)B * H * ceil_div(N, sage::kMeanChunk) * d * 4;
}

int sage_smooth_quant_qk(const void* q, const void* k, int dtype, int B, int H, int N, int d,
                         int8_t* q_i8, int8_t* k_i8, float* q_scale, float* k_scale,
                         float* k_mean, void* scratch, size_t scratch_bytes, void* stream) {
  return sage_smooth_quant_qk_ex(q, k, dtype, SAGE_LAYOUT_HND, nullptr, nullptr, B, H, N, d, q_i8,
                                 k_i8, q_scale, k_scale, k_mean, scratch, scratch_bytes, stream);
}

int sage_smooth_quant_qk_ex(const void* q, const void* k, int dtype, int layout,
                            const float* rope_cos, const float* rope_sin, int B, int H, int N,
                            int d, int8_t* q_i8, int8_t* k_i8, float* q_scale, float* k_scale,
                            float* k_mean, void* scratch, size_t scratch_bytes, void* stream) {
  if (!q || !k || !q_i8 || !k_i8 || !q_scale || !k_scale || !k_mean || !scratch)
    return SAGE_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_i8) || !aligned16(k_i8) ||
      !aligned16(scratch) || (reinterpret_cast<uintptr_t>(k_mean) & 7u) ||
      (reinterpret_cast<uintptr_t>(q_scale) & 3u) || (reinterpret_cast<uintptr_t>(k_scale) & 3u))
    return SAGE_ERR_INVALID_ARG;
  if (dtype != SAGE_DT_F16 && dtype != SAGE_DT_BF16) return SAGE_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID_ARG;
  if (!shape_ok(B, H, N, d)) return SAGE_ERR_UNSUPPORTED;
  int st = validate_in(layout, rope_cos, rope_sin);
  if (st != SAGE_OK) return st;
  if (scratch_bytes < sage_smooth_quant_qk_scratch_bytes(B, H, N, d)) return SAGE_ERR_WORKSPACE;
  if ((st = device_check()) != SAGE_OK) return st;
  const sage::InLayout in{layout, rope_cos, rope_sin};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N <= sage::kHeadPrepassMaxN) {
    const sage::PrepassOut po{static_cast<float*>(scratch), k_mean, nullptr, q_i8, k_i8,
                              q_scale, k_scale, nullptr};
    return hip_status(sage::launch_prepass_head(q, k, nullptr, dtype, B, H, N, d, SAGE_PV_FP16,
                                                in, po, s));
  }
  hipError_t e = sage::launch_colstats(k, nullptr, dtype, B, H, N, d, SAGE_PV_FP16, in,
                                       static_cast<float*>(scratch), nullptr, k_mean, nullptr,
                                       nullptr, s);
  if (e != hipSuccess) return SAGE_ERR_HIP;
  e = sage::launch_quant_qk(q, k, k_mean, dtype, B, H, N, d, in, q_i8, k_i8, q_scale, k_scale, s);
  return hip_status(e);
}

size_t sage_quant_v_bytes(int B, int H, int N, int d, int pv_mode) {
  if (!shape_ok(B, H, N, d)) return 0;
  if (!sage::pv_valid(pv_mode)) return 0;
  return (size_t)B * H * ceil_div(N, sage::kKvTile) * sage::v_tile_bytes(d, pv_mode);
}

size_t sage_quant_v_scratch_bytes(int B, int H, int N, int d, int pv_mode) {
  if (!shape_ok(B, H, N, d)) return 0;
  if (!sage::v_quantised(pv_mode)) return 0;
  // partial maxima + reciprocal scales
  return align_up((size_t)B * H * ceil_div(N, sage::kMeanChunk) * d * 4) + (size_t)B * H * d * 4;
}

int sage_quant_v(const void* v, int dtype, int B, int H, int N, int d, int pv_mode, void* v_out,
                 float* v_scale, void* scratch, size_t scratch_bytes, void* stream) {
  return sage_quant_v_ex(v, dtype, SAGE_LAYOUT_HND, B, H, N, d, pv_mode, v_out, v_scale, scratch,
                         scratch_bytes, stream);
}

int sage_quant_v_ex(const void* v, int dtype, int layout, int B, int H, int N, int d,
                    int pv_mode, void* v_out, float* v_scale, void* scratch,
                    size_t scratch_bytes, void* stream) {
  if (layout != SAGE_LAYOUT_HND && layout != SAGE_LAYOUT_NHD) return SAGE_ERR_INVALID_ARG;
  if (!v || !v_out) return SAGE_ERR_INVALID_ARG;
  if (!aligned16(v) || !aligned16(v_out)) return SAGE_ERR_INVALID_ARG;
  if (dtype != SAGE_DT_F16 && dtype != SAGE_DT_BF16) return SAGE_ERR_INVALID_ARG;
  if (!sage::pv_valid(pv_mode)) return SAGE_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID_ARG;
  if (!shape_ok(B, H, N, d)) return SAGE_ERR_UNSUPPORTED;
  const bool qv = sage::v_quantised(pv_mode);
  if (qv && (!v_scale || !scratch || !aligned16(scratch) ||
              (reinterpret_cast<uintptr_t>(v_scale) & 7u)))
    return SAGE_ERR_INVALID_ARG;
  if (scratch_bytes < sage_quant_v_scratch_bytes(B, H, N, d, pv_mode)) return SAGE_ERR_WORKSPACE;
  int st = device_check();
  if (st != SAGE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* v_recip = nullptr;
  float* part_max = nullptr;
  if (qv) {
    part_max = static_cast<float*>(scratch);
    v_recip = reinterpret_cast<float*>(
        static_cast<uint8_t*>(scratch) +
        align_up((size_t)B * H * ceil_div(N, sage::kMeanChunk) * d * 4));
  }
  if (N <= sage::kHeadPrepassMaxN) {
    const sage::PrepassOut po{nullptr, nullptr, v_scale, nullptr, nullptr, nullptr, nullptr,
                              static_cast<uint8_t*>(v_out)};
    const sage::InLayout in{layout, nullptr, nullptr};
    return hip_status(sage::launch_prepass_head(nullptr, nullptr, v, dtype, B, H, N, d, pv_mode,
                                                in, po, s));
  }
  if (qv) {
    const sage::InLayout in{layout, nullptr, nullptr};
    hipError_t e = sage::launch_colstats(nullptr, v, dtype, B, H, N, d, pv_mode, in, nullptr,
                                         part_max, nullptr, v_scale, v_recip, s);
    if (e != hipSuccess) return SAGE_ERR_HIP;
  }
  return hip_status(sage::launch_prep_v(v, v_recip, dtype, B, H, N, d, pv_mode, layout,
                                        static_cast<uint8_t*>(v_out), s));
}

int sage_attn_fwd_quantized(const int8_t* q_i8, const int8_t* k_i8, const void* v_prep,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            void* o, int B, int H, int N, int d, int causal, int pv_mode,
                            int out_dtype, void* stream) {
  return fwd_quantized(q_i8, k_i8, v_prep, q_scale, k_scale, v_scale, nullptr, o, B, H, N, d,
                       causal, pv_mode, out_dtype, stream);
}

}  // extern "C"

namespace {

int fwd_quantized(const int8_t* q_i8, const int8_t* k_i8, const void* v_prep,
                  const float* q_scale, const float* k_scale, const float* v_scale,
                  const int32_t* q_seed, void* o, int B, int H, int N, int d, int causal,
                  int pv_mode, int out_dtype, void* stream) {
  if (!q_i8 || !k_i8 || !v_prep || !q_scale || !k_scale || !o) return SAGE_ERR_INVALID_ARG;
  if (!aligned16(q_i8) || !aligned16(k_i8) || !aligned16(v_prep) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(q_scale) & 3u) || (reinterpret_cast<uintptr_t>(k_scale) & 3u))
    return SAGE_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
  if (!sage::pv_valid(pv_mode)) return SAGE_ERR_INVALID_ARG;
  if (out_dtype != SAGE_DT_F16 && out_dtype != SAGE_DT_BF16 && out_dtype != SAGE_OUT_F32)
    return SAGE_ERR_INVALID_ARG;
  if (sage::v_quantised(pv_mode) && (!v_scale || (reinterpret_cast<uintptr_t>(v_scale) & 3u)))
    return SAGE_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID_ARG;
  if (!shape_ok(B, H, N, d)) return SAGE_ERR_UNSUPPORTED;
  int st = device_check();
  if (st != SAGE_OK) return st;
  return hip_status(sage::launch_attn(q_i8, k_i8, static_cast<const uint8_t*>(v_prep), q_scale,
                                      k_scale, v_scale, q_seed, B, H, N, d, causal, pv_mode,
                                      out_dtype, SAGE_LAYOUT_HND, o,
                                      static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int sage_attn_ref_rows_f32(const void* q, const void* k, const void* v, int dtype, int B, int H,
                           int N, int d, int causal, const int32_t* rows, int nrows, float* o,
                           void* stream) {
  if (!q || !k || !v || !rows || !o) return SAGE_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (reinterpret_cast<uintptr_t>(rows) & 3u) ||
      (reinterpret_cast<uintptr_t>(o) & 3u))
    return SAGE_ERR_INVALID_ARG;
  if (dtype != SAGE_DT_F16 && dtype != SAGE_DT_BF16) return SAGE_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || nrows < 1) return SAGE_ERR_INVALID_ARG;
  if (!shape_ok(B, H, N, d)) return SAGE_ERR_UNSUPPORTED;
  int st = device_check();
  if (st != SAGE_OK) return st;
  return hip_status(sage::launch_ref_rows(q, k, v, dtype, B, H, N, d, causal, rows, nrows, o,
                                          static_cast<hipStream_t>(stream)));
}

int sage_attn_debug_s_i32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d,
                          int b, int h, int q0, int nq, int k0, int nk, int32_t* s_out,
                          void* stream) {
  if (!q_i8 || !k_i8 || !s_out) return SAGE_ERR_INVALID_ARG;
  if (!aligned16(q_i8) || !aligned16(k_i8) || (reinterpret_cast<uintptr_t>(s_out) & 3u))
    return SAGE_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID_ARG;
  if (!shape_ok(B, H, N, d)) return SAGE_ERR_UNSUPPORTED;
  if (b < 0 || b >= B || h < 0 || h >= H) return SAGE_ERR_INVALID_ARG;
  const int n32 = ceil_div(N, 32) * 32;
  if (q0 < 0 || k0 < 0 || nq < 32 || nk < 32 || (q0 | k0 | nq | nk) % 32 != 0 ||
      (long long)q0 + nq > n32 || (long long)k0 + nk > n32)
    return SAGE_ERR_INVALID_ARG;
  int st = device_check();
  if (st != SAGE_OK) return st;
  return hip_status(sage::launch_debug_s(q_i8, k_i8, B, H, N, d, b, h, q0, nq, k0, nk, s_out,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" {

int sage_attn_debug_s_fwd(const void* workspace, size_t workspace_bytes, int B, int H, int N,
                          int d, int causal, int pv_mode, int smooth_q, int b, int h, int q0,
                          int nq, int k0, int nk, int32_t* s_out, float* o_rows, void* stream) {
  if (!workspace || !s_out || !o_rows) return SAGE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0 ||
      (reinterpret_cast<uintptr_t>(s_out) & 3u) || (reinterpret_cast<uintptr_t>(o_rows) & 15u))
    return SAGE_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
  if (smooth_q != 0 && smooth_q != 1) return SAGE_ERR_INVALID_ARG;
  if (!sage::pv_valid(pv_mode)) return SAGE_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID_ARG;
  if (!shape_ok(B, H, N, d)) return SAGE_ERR_UNSUPPORTED;
  if (b < 0 || b >= B || h < 0 || h >= H) return SAGE_ERR_INVALID_ARG;
  if (q0 < 0 || q0 >= N || nq < 1 || nq > N - q0 || k0 < 0 || k0 >= N || nk < 1 || nk > N - k0)
    return SAGE_ERR_INVALID_ARG;
  const Layout L = make_layout(B, H, N, d, pv_mode, smooth_q == 1);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE;
  // with Q smoothed the workspace holds the compensation values of the last
  // chunk only: the whole table must have fit in one
  if (smooth_q && sq_chunk_blocks(B, H, N) < ceil_div(N, sage::kQBlock)) return SAGE_ERR_UNSUPPORTED;
  int st = device_check();
  if (st != SAGE_OK) return st;
  const uint8_t* w = static_cast<const uint8_t*>(workspace);
  auto F = [&](size_t off) { return reinterpret_cast<const float*>(w + off); };
  return hip_status(sage::launch_attn_dump(
      reinterpret_cast<const int8_t*>(w + L.q_i8), reinterpret_cast<const int8_t*>(w + L.k_i8),
      w + L.v_t, F(L.q_scale), F(L.k_scale), sage::v_quantised(pv_mode) ? F(L.v_scale) : nullptr,
      smooth_q ? reinterpret_cast<const int32_t*>(w + L.comp) : nullptr, B, H, N, d, causal,
      pv_mode, b, h, q0, nq, k0, nk, s_out, o_rows, static_cast<hipStream_t>(stream)));
}

int sage_attn_debug_fwd_f32(const void* q, const void* k, const void* v, float* o, int B, int H,
                            int N, int d, int causal, int pv_mode, int dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return sage_attn_fwd_f32out(q, k, v, o, B, H, N, d, causal, pv_mode, dtype, workspace,
                              workspace_bytes, stream);
}

}  // extern "C"
