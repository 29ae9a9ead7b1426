/*
 * sage_probe.h -- micro-benchmarks of the gfx950 units behind the attention
 * kernel's roofline (libsage_probe.so; used by bench.py --mfma-probe).  Not
 * part of the attention path.
 *
 * The kernel launches ncu * waves_per_simd workgroups of 256 threads (four
 * wavefronts, one per SIMD), each claiming enough LDS that at most
 * waves_per_simd of them share a CU; with ncu = the device's CU count every
 * SIMD runs waves_per_simd wavefronts.  Each wavefront issues `iters` groups
 * of
 *     one MFMA of `mfma_kind` (none for SAGE_PROBE_NONE), rotating over four
 *     independent accumulators, then nv independent v_fma_f32 and ne
 *     independent v_exp_f32,
 * with operands in registers.  Supported (nv, ne): (0,0) (4,0) (6,0) (8,0)
 * (12,0) (16,0) (0,2) (0,4) (2,2) (4,2) (4,4) (6,2).
 *
 * stamps: device int64 [4 * 4 * ncu * waves_per_simd]; per wavefront w:
 *   stamps[4w + 0], [4w + 1]  shader-clock counter (s_memtime) before / after
 *   stamps[4w + 2], [4w + 3]  real-time counter (s_memrealtime) before / after
 * The clock the wavefront ran at is (c1 - c0) / (r1 - r0) times the real-time
 * counter's rate (sage_probe_wallclock_khz).
 * sink: device float [256 * ncu * waves_per_simd], written with the results
 * so nothing is optimised away.
 * Returns 0, 1 for an invalid argument, 2 for an unsupported (nv, ne), 4 for
 * a HIP error.  Asynchronous on `stream` (a hipStream_t).
 *
 * MFMA shapes (operations = 2 x multiply-accumulates):
 *   SAGE_PROBE_MFMA_I8   v_mfma_i32_32x32x32_i8            65536 ops
 *   SAGE_PROBE_MFMA_F16  v_mfma_f32_32x32x16_f16           32768 ops
 *   SAGE_PROBE_MFMA_F8   v_mfma_scale_f32_32x32x64_f8f6f4  131072 ops (E4M3)
 */
#ifndef SAGE_PROBE_H
#define SAGE_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

enum { SAGE_PROBE_NONE = -1, SAGE_PROBE_MFMA_I8 = 0, SAGE_PROBE_MFMA_F16 = 1,
       SAGE_PROBE_MFMA_F8 = 2 };

int sage_probe_run(int mfma_kind, int nv, int ne, int waves_per_simd, int ncu, int iters,
                   long long* stamps, float* sink, void* stream);

/*
 * LDS read bandwidth next to MFMAs: the same launch, stamps and sink, but
 * each group issues one MFMA of `mfma_kind` (none for SAGE_PROBE_NONE) and
 * nl (1, 2 or 4) independent ds_read_b128, each moving 1 KiB per wavefront
 * (consecutive 16-byte lanes, no bank conflicts) from the workgroup's LDS; a
 * group consumes the reads issued four groups earlier.  Returns as
 * sage_probe_run (2 for an unsupported nl).
 */
int sage_probe_run_lds(int mfma_kind, int nl, int waves_per_simd, int ncu, int iters,
                       long long* stamps, float* sink, void* stream);

/* Rate of the s_memrealtime counter in kHz; the device's CU count. */
int sage_probe_wallclock_khz(int* khz);
int sage_probe_cu_count(int* ncu);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_PROBE_H */
