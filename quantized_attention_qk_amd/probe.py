"""Micro-benchmarks of the gfx950 units behind the attention kernel's roofline
(ctypes over libsage_probe.so, include/sage_probe.h).

mfma_rates(): sustained INT8, FP16 and FP8 MFMA rates with every SIMD busy,
              and the clock the chip ran at meanwhile.
issue_table(): cycles per group of [one MFMA + nv v_fma_f32 + ne v_exp_f32]
              per SIMD, with one or two wavefronts per SIMD -- how much VALU
              work hides under a stream of MFMAs.
lds_table():  LDS read bandwidth (16-byte reads per lane) alone and next to a
              stream of MFMAs.
"""
from __future__ import annotations

import ctypes
import os

import torch

PROBE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsage_probe.so")

NONE, I8, F16, F8 = -1, 0, 1, 2
OPS_PER_MFMA = {I8: 2 * 32 * 32 * 32, F16: 2 * 32 * 32 * 16, F8: 2 * 32 * 32 * 64}
NAMES = {NONE: "none", I8: "i8_32x32x32", F16: "f16_32x32x16", F8: "fp8_32x32x64"}

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError(f"{PROBE_PATH} is missing: build with "
                               "`python -m quantized_attention_qk_amd.build`")
        h = ctypes.CDLL(PROBE_PATH)
        h.sage_probe_run.restype = ctypes.c_int
        h.sage_probe_run.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p] * 3
        h.sage_probe_run_lds.restype = ctypes.c_int
        h.sage_probe_run_lds.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 3
        for name in ("sage_probe_wallclock_khz", "sage_probe_cu_count"):
            getattr(h, name).restype = ctypes.c_int
            getattr(h, name).argtypes = [ctypes.POINTER(ctypes.c_int)]
        _lib = h
    return _lib


def _query(name: str) -> int:
    v = ctypes.c_int()
    rc = getattr(lib(), name)(ctypes.byref(v))
    if rc != 0:
        raise RuntimeError(f"{name} failed ({rc})")
    return v.value


def run(kind: int, nv: int = 0, ne: int = 0, wps: int = 2, iters: int = 16384,
        repeats: int = 3, nl: int = 0) -> dict:
    """One probe configuration on every CU; the last of `repeats` launches is
    measured.  Returns the wall time, the clock and per-SIMD cycle counts.
    nl > 0: the LDS probe (nl 16-byte reads per lane and group, nv = ne = 0)."""
    if nl and (nv or ne):
        raise ValueError("the LDS probe runs no VALU groups")
    ncu = _query("sage_probe_cu_count")
    rt_khz = _query("sage_probe_wallclock_khz")
    nwaves = 4 * ncu * wps
    stamps = torch.zeros(4 * nwaves, dtype=torch.int64, device="cuda")
    sink = torch.empty(256 * ncu * wps, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for r in range(repeats):
        if r == repeats - 1:
            e0.record(stream)
        if nl:
            rc = lib().sage_probe_run_lds(kind, nl, wps, ncu, iters, stamps.data_ptr(),
                                          sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
        else:
            rc = lib().sage_probe_run(kind, nv, ne, wps, ncu, iters, stamps.data_ptr(),
                                      sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"probe ({kind}, nv={nv}, ne={ne}, nl={nl}, {wps}) failed ({rc})")
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    st = stamps.view(nwaves, 4).cpu().double()
    cyc = (st[:, 1] - st[:, 0])
    rtt = (st[:, 3] - st[:, 2])
    clock_ghz = float((cyc / rtt).median()) * rt_khz * 1e3 / 1e9
    res = {"mfma": NAMES[kind], "nv": nv, "ne": ne, "nl": nl, "waves_per_simd": wps, "iters": iters,
           "cus": ncu, "ms": round(ms, 4), "clock_ghz": round(clock_ghz, 3),
           # one SIMD runs wps wavefronts of `iters` groups each
           "cycles_per_group_per_simd": round(float(cyc.median()) / (iters * wps), 2)}
    if nl:
        # 1 KiB per read and wavefront; per CU and shader clock
        res["lds_bytes_per_clk_per_cu"] = round(
            1024.0 * nl * iters * 4 * wps / float(cyc.median()), 1)
    if kind != NONE:
        ops = OPS_PER_MFMA[kind] * iters * nwaves
        res["tops"] = round(ops / (ms * 1e-3) / 1e12, 1)
    return res


def mfma_rates() -> dict:
    """Sustained rate of each MFMA shape (two wavefronts per SIMD, operands
    in registers, four independent accumulators per wavefront)."""
    out = {}
    for kind in (I8, F16, F8):
        r = run(kind, wps=2, iters=32768 if kind != F8 else 16384)
        out[NAMES[kind]] = {"tops": r["tops"], "clock_ghz": r["clock_ghz"],
                            "cycles_per_mfma_per_simd": r["cycles_per_group_per_simd"]}
    return out


ISSUE_CASES = [(0, 0), (4, 0), (6, 0), (8, 0), (12, 0), (16, 0), (0, 2), (0, 4), (2, 2),
               (4, 2), (6, 2), (4, 4)]


def issue_table(kinds=(NONE, F16, I8), wps_list=(1, 2)) -> list[dict]:
    rows = []
    for kind in kinds:
        for wps in wps_list:
            for nv, ne in ISSUE_CASES:
                if kind == NONE and nv == 0 and ne == 0:
                    continue
                rows.append(run(kind, nv, ne, wps=wps, iters=8192, repeats=2))
    return rows


def lds_table(kinds=(NONE, F16, I8), nls=(1, 2, 4), wps_list=(1, 2)) -> list[dict]:
    """LDS read bandwidth alone (kind NONE) and with one MFMA per group."""
    rows = []
    for kind in kinds:
        for wps in wps_list:
            for nl in nls:
                rows.append(run(kind, wps=wps, iters=8192, repeats=2, nl=nl))
    return rows
