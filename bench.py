"""Benchmark of the SageAttention forward pass on one MI355X.

One step = one full forward pass (smooth/quantise prepass + attention kernel)
over one batch of seeded synthetic inputs already resident in HBM.  Default
workload: B=1, H=24, N=16384, d=128, non-causal, bf16, FP16 P~V.

Prints ONE JSON line: attention TOPS (4 B H N^2 d / t, halved when causal),
the attention kernel's roofline position (timed live with HIP events on the
launch stream), and the CPU oracle's throughput on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload c3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA (published)
FP8_PEAK_TFLOPS = 5000.0
FP16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_fwd_counters.json")
KERNEL_SRC = os.path.join(ROOT, "quantized_attention_qk_amd", "csrc", "attn_fwd.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed whole passes for at least this long before the warm-up "
                         "steps, so that the GPU's clock has settled (power-limited part)")
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle sample")
    ap.add_argument("--layout", default="HND", choices=["HND", "NHD"],
                    help="q, k, v, o layout: [B,H,N,d] or token-major [B,N,H,d]")
    ap.add_argument("--rope", action="store_true",
                    help="apply rotary embeddings to Q and K inside the quantisation prepass")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only run the micro-benchmarks of libsage_probe.so: sustained INT8, "
                         "FP16 and FP8 MFMA rates with the clock they ran at, and the issue "
                         "cost of VALU work and the LDS read bandwidth next to a stream of MFMAs")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a device-to-device copy of BYTES (3 launches), to calibrate "
                         "the HBM byte counters against a known traffic")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only time torch's own streaming kernels (a device copy, a "
                         "float32-accumulated sum of bf16 data and a fill, 128 MiB and 1 GiB): "
                         "the HBM rates plain copy, read and write kernels reach on this GPU")
    return ap.parse_args()


def stream_probe():
    """HBM rates of torch's own streaming kernels, the yardstick for the
    prepass kernels: a device copy (bytes read + written), a full sum of a
    bf16 tensor with float32 accumulation (bytes read) and a fill (bytes
    written), averaged over 20 launches after 3 untimed ones, at 128 MiB
    (one 16-bit tensor of c2) and 1 GiB."""
    import torch
    res = {}
    for mib in (128, 1024):
        n = mib * 1024 * 1024 // 2
        x = torch.randn(n, dtype=torch.bfloat16, device="cuda")
        y = torch.empty_like(x)
        for name, fn, nbytes in (("copy", lambda: y.copy_(x), 4 * n),
                                 ("sum", lambda: torch.sum(x, dtype=torch.float32), 2 * n),
                                 ("fill", lambda: y.fill_(1.0), 2 * n)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(20):
                fn()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / 20
            res[f"{name}_{mib}MiB"] = {"ms": round(ms, 4), "TB_per_s": round(nbytes / ms / 1e9, 2)}
        del x, y
    print(json.dumps({"stream_probe": res}), flush=True)


def copy_probe(nbytes: int):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter readings
    give the factor between those counters and true HBM bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": src.numel() * 4, "launches": 3}), flush=True)


def kernel_src_hash() -> str:
    """Hash of the attention kernel's sources (the dispatcher, the kernel
    templates, the per-mode translation units and the shared headers)."""
    csrc = os.path.join(ROOT, "quantized_attention_qk_amd", "csrc")
    files = ["attn_fwd.hip", "attn_fwd_kernel.h", "sage_common.h", "sage_launch.h"]
    files += sorted(f for f in os.listdir(csrc) if f.startswith("attn_fwd_d"))
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 counter summary, or None when absent or the kernel changed."""
    try:
        data = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("kernel_src_hash") != kernel_src_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def clock_from_profiles(workload: str):
    """The shader clock during the attention kernel, from the committed
    rocprofv3 counter run (GRBM_GUI_ACTIVE cycles per dispatch over the
    dispatch duration, per XCD), or None when absent or the kernel changed."""
    try:
        data = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("kernel_src_hash") != kernel_src_hash():
        return None
    return entry.get("clock_ghz")


def measured_mfma_peak(pv_mode: str):
    """Sustained MFMA rates on this GPU right now (libsage_probe.so, two
    wavefronts per SIMD on every CU, ~25 ms of back-to-back launches so the
    power-limited clock settles): the INT8 rate, and the mixed rate of the
    kernel's P~V mode (half the operations INT8, half FP16 / FP8 / INT8)."""
    from quantized_attention_qk_amd import probe
    i8 = probe.run(probe.I8, wps=2, iters=32768, repeats=10)["tops"]
    other = {"fp16": probe.F16, "fp8": probe.F8, "int8": probe.I8}[pv_mode]
    pv = i8 if other == probe.I8 else \
        probe.run(other, wps=2, iters=32768 if other == probe.F16 else 16384, repeats=10)["tops"]
    return i8, 1.0 / (0.5 / i8 + 0.5 / pv)


def cpu_baseline(wl, min_seconds: float):
    """Time the CPU oracle (as it stands) on whole heads of the workload until
    at least `min_seconds` have elapsed (at most 4 heads)."""
    import numpy as np

    import oracle
    from workloads import make_inputs
    threads = os.environ.get("OMP_NUM_THREADS") or str(os.cpu_count())
    one = wl.with_(B=1, H=1)
    done, t_total, ops = 0, 0.0, 0.0
    while done < 4 and (t_total < min_seconds or done == 0):
        inp = make_inputs(one.with_(seed=wl.seed + 1000 + done))
        t0 = time.perf_counter()
        pq = oracle.smooth_quant_qk(inp.qf, inp.kf, smooth_q=wl.smooth_q)
        oracle.sage_attention(inp.qf, inp.kf, inp.vf, causal=wl.causal, pv_mode=wl.pv_mode,
                              prep=pq)
        t_total += time.perf_counter() - t0
        ops += one.ops
        done += 1
    return {"value": ops / t_total / 1e12, "unit": "TOPS", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} whole head(s) (B=1,H=1,N={wl.N},d={wl.d}, all query rows, "
                      f"prepass included) of workload {wl.name}; {t_total:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.stream_probe:
        stream_probe()
        return
    if args.mfma_probe:
        from quantized_attention_qk_amd import probe
        print(json.dumps({"mfma_rates": probe.mfma_rates()}), flush=True)
        for row in probe.issue_table():
            print(json.dumps(row), flush=True)
        for row in probe.lds_table():
            print(json.dumps(row), flush=True)
        return

    import torch

    import quantized_attention_qk_amd as qa
    from workloads import make_inputs, named

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    wl = named(args.workload)
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    if args.layout == "NHD":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    rope = None
    if args.rope:
        from workloads import rope_tables
        rope = tuple(torch.from_numpy(t).cuda() for t in rope_tables(N, d))
    out = torch.empty_like(q)
    ws = torch.empty(qa.workspace_bytes(B, H, N, d, wl.pv_mode, wl.smooth_q), dtype=torch.uint8,
                     device="cuda")

    # A step is the whole pass.  On [B,H,N,d] inputs without RoPE or smoothed Q
    # it is issued as its two halves, sage_attn_prepare then sage_attn_attend
    # (the same launches as sage_attn, bit for bit), so that HIP events around
    # the attention launch time the kernel inside the timed passes.
    split = args.layout == "HND" and rope is None and not wl.smooth_q
    stream = torch.cuda.current_stream()
    kev = []

    def step(record=False, whole=False):
        if whole or not split:
            qa.sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out=out, workspace=ws,
                         layout=args.layout, rope=rope, smooth_q=wl.smooth_q)
            return
        qa.prepare(q, k, v, wl.pv_mode, ws)
        if record:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
        qa.attend(ws, B, H, N, d, wl.causal, wl.pv_mode, out_dtype=q.dtype, out=out)
        if record:
            b.record(stream)
            kev.append((a, b))

    # The part runs at a power-limited clock that takes a few hundred
    # milliseconds of load to settle; the first passes after idle run at a
    # different speed (c2's attention kernel: 15% apart).  Passes until
    # --settle-ms have elapsed come before the W warm-up steps.
    n_settle, t_settle = 0, time.perf_counter()
    while args.settle_ms > 0:
        step(whole=True)
        n_settle += 1
        if n_settle % 8 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t_settle) * 1e3 >= args.settle_ms or n_settle >= 4000:
                break
    # Passes shorter than 0.1 ms keep the single call: two calls and two
    # events per pass would make the host, not the GPU, set the pace.
    if split:
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(8):
            step(whole=True)
        s1.record(stream)
        torch.cuda.synchronize()
        n_settle += 8
        split = s0.elapsed_time(s1) / 8 >= 0.1
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step(record=True)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    tops = wl.ops / (ms * 1e-3) / 1e12

    # The attention kernel alone, on prepared operands, on the same stream.
    qk = qa.smooth_quant_qk(q, k, layout=args.layout, rope=rope)
    vp, vs = qa.quant_v(v, wl.pv_mode, layout=args.layout)
    seed = None
    if wl.smooth_q:   # smoothed Q^ and the accumulator seeds (HND layout)
        sq = qa.smooth_q(q, qk["k_i8"], seed_pv_mode=wl.pv_mode)
        qk = dict(qk, q_i8=sq["q_i8"], q_scale=sq["q_scale"])
        seed = sq["q_comp"]
    out2 = torch.empty((B, H, N, d), dtype=q.dtype, device="cuda")

    def kernel_only():
        qa.sage_attn_quantized(qk, vp, vs, causal=wl.causal, pv_mode=wl.pv_mode,
                               out_dtype=q.dtype, out=out2, q_seed=seed)

    for _ in range(max(2, args.warmup)):
        kernel_only()
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(args.steps):
        kernel_only()
    k1.record(stream)
    torch.cuda.synchronize()
    kms_b2b = k0.elapsed_time(k1) / args.steps
    o_hnd = out.transpose(1, 2) if args.layout == "NHD" else out
    assert torch.equal(o_hnd, out2), "attention-only path must reproduce the full pass"
    if split:
        # the attention kernel as it ran inside the timed passes
        kms = sum(a.elapsed_time(b) for a, b in kev) / len(kev)
        ref = qa.sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode)
        assert torch.equal(out, ref), "prepare + attend must reproduce sage_attn"
    else:
        kms = kms_b2b
    ktops = wl.ops / (kms * 1e-3) / 1e12

    traffic = traffic_from_profiles(wl.name)
    clock = clock_from_profiles(wl.name)
    i8_meas, mixed_meas = measured_mfma_peak(wl.pv_mode)
    # FP8 and INT8 P~V run at the INT8 MFMA rate; FP16 P~V at half of it
    mixed_peak = INT8_PEAK_TOPS if wl.pv_mode in ("fp8", "int8") else \
        1.0 / (0.5 / INT8_PEAK_TOPS + 0.5 / FP16_PEAK_TFLOPS)
    res = {
        "metric": "attention TOPS at N=16K,d=128 (1 MI355X) and % of INT8 MFMA peak",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp16": "i8+f16", "fp8": "i8+fp8e4m3", "int8": "i8"}[wl.pv_mode],
        "data": "synthetic (seeded numpy draws, see workloads/)",
        "config": {"workload": f"{wl.name}: B={B},H={H},N={N},d={d} "
                               f"{'causal' if wl.causal else 'non-causal'} {wl.dtype}, "
                               f"INT8 QK^T + {wl.pv_mode.upper()} P~V"
                               f"{', Q smoothed' if wl.smooth_q else ''}",
                   "B": B, "H": H, "N": N, "d": d, "causal": wl.causal,
                   "pv_mode": wl.pv_mode, "in_dtype": wl.dtype, "layout": args.layout,
                   "rope": bool(args.rope), "smooth_q": wl.smooth_q},
        "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2),
        "roofline": {"kernel": "attn_fwd_kernel", "bound": "mfma",
                     "achieved": round(ktops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(ktops / INT8_PEAK_TOPS, 4), "traffic": traffic,
                     "kernel_ms": round(kms, 4),
                     # how kernel_ms was taken: "in_pass" = HIP events around
                     # the attention launch of every timed pass; "back_to_back"
                     # = the kernel alone, launched repeatedly after the passes
                     "kernel_ms_source": "in_pass" if split else "back_to_back",
                     "kernel_ms_back_to_back": round(kms_b2b, 4),
                     "ops_per_launch": wl.ops,
                     "mixed_mfma_peak": round(mixed_peak, 1),
                     "frac_of_mixed_peak": round(ktops / mixed_peak, 4),
                     # the same ratios against rates measured on this GPU
                     # just now (bench.py --mfma-probe kernels)
                     "measured_int8_peak": round(i8_meas, 1),
                     "frac_of_measured_int8_peak": round(ktops / i8_meas, 4),
                     "measured_mixed_peak": round(mixed_meas, 1),
                     "frac_of_measured_mixed_peak": round(ktops / mixed_meas, 4),
                     "clock_ghz": clock,
                     "hbm_gbps": None if traffic is None else round(traffic / (kms * 1e-3) / 1e9, 1)},
        "prepass_ms": round(ms - kms, 4),
        "settle_passes": n_settle,
        "wall_s_timed": round(t_wall, 3),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
