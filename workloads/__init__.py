"""Seeded synthetic inputs for the SageAttention forward pass.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds no step of the method: it only draws random numbers and
rounds them to the 16-bit input type, so that both sides of every parity check
see bit-identical inputs.

Shapes and value distributions follow the workloads on the pages:

* "SageAttention: Accurate 8-Bit Attention for Plug-and-Play Inference
  Acceleration" (paper detail page), §3, Figure 4: K carries large
  channel-wise outliers that are a bias shared by all tokens, Q has milder
  outliers, V is benign.
* Same page, §5, Table 7: real-model shapes (B, H, N, d), including the ragged
  token counts 17776, 1105 and 197 used here as ragged-tail cases.

The pages measure on real model activations, which are not available here;
these seeded draws stand in for them.

Generation recipe: ``numpy.random.default_rng(seed)``; float32
``standard_normal`` drawn in the order Q, K, V, then the extras of the
workload; then each tensor is rounded to its 16-bit type with
round-to-nearest-even.  All tensors are contiguous [B, H, N, d].
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "TABLE7", "SHARDS", "PV_INT8", "SMOOTH_Q", "named", "make_inputs", "round_to_bf16_bits",
           "round_to_fp16", "bf16_bits_to_f32", "Inputs", "rope_tables", "to_nhd"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "fp16" or "bf16": element type of q, k, v and o
    causal: bool
    pv_mode: str        # "fp16", "fp8" or "int8"
    seed: int
    extras: str         # which outlier recipe to apply (see _apply_extras)
    note: str = ""
    smooth_q: bool = False   # also smooth Q per block (the SageAttention2 step)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def ops(self) -> float:
        """Attention operation count 4*B*H*N^2*d, halved when causal."""
        o = 4.0 * self.B * self.H * float(self.N) ** 2 * self.d
        return o / 2 if self.causal else o


# The five workloads of the build.  c3 is the headline throughput shape.
WORKLOADS = {
    "c1": Workload("c1", 1, 2, 1024, 64, "fp16", False, "fp16", 0, "kbias4",
                   "small case: K plus a per-channel bias ~ N(0, 4^2)"),
    "c2": Workload("c2", 4, 32, 4096, 128, "bf16", True, "fp16", 1, "kchan20",
                   "LLM prefill: 4 K channels biased by +-20 for all tokens"),
    "c3": Workload("c3", 1, 24, 16384, 128, "bf16", False, "fp16", 2, "q8_kbias5",
                   "video DiT: 2 Q outlier channels x8, K bias ~ N(0, 5^2)"),
    "c4": Workload("c4", 8, 16, 8192, 64, "fp16", False, "fp8", 3, "kbias4",
                   "8+8 mode: FP8 P~V with per-channel V scales"),
    "c5": Workload("c5", 1, 32, 32768, 128, "bf16", True, "fp8", 4, "kbias4",
                   "long context, causal, FP8 P~V"),
}


# The real-model shapes of "SageAttention ..." detail page, §5 Table 7
# (B, H, N, d), with seeded synthetic activations of the Figure-4 kind (K with
# a per-channel bias shared by all tokens).  The LLM shape runs causal.
TABLE7 = {
    "t7_cogvideox": Workload("t7_cogvideox", 2, 30, 17776, 64, "fp16", False, "fp16", 21,
                             "kbias4", "CogVideoX shape, ragged N"),
    "t7_unidiffuser": Workload("t7_unidiffuser", 2, 24, 1105, 64, "fp16", False, "fp16", 22,
                               "kbias4", "Unidiffuser shape, ragged N"),
    "t7_ultrapixel": Workload("t7_ultrapixel", 8, 30, 4096, 64, "fp16", False, "fp16", 23,
                              "kbias4", "UltraPixel shape"),
    "t7_llama2": Workload("t7_llama2", 1, 32, 4096, 128, "fp16", True, "fp16", 24, "kchan20",
                          "Llama2 prefill shape, causal"),
    "t7_timm": Workload("t7_timm", 12, 64, 197, 64, "fp16", False, "fp16", 25, "kbias4",
                        "TIMM shape, 197 tokens"),
}


# One GPU's share of a workload sharded by heads over 8 GPUs (heads are
# independent, so each GPU runs the same kernel on H/8 heads at full N).
SHARDS = {
    "c3_shard8": Workload("c3_shard8", 1, 3, 16384, 128, "bf16", False, "fp16", 2, "q8_kbias5",
                          "c3 split by heads over 8 GPUs: 3 heads per GPU"),
}


# The all-INT8 variant (INT8 P~V) of "SageAttention ..." detail page, §3
# Figure 5, on the headline shape and on the FP8 workload's shape (same
# inputs as c3 and c4, only the P~V precision differs).
PV_INT8 = {
    "c3i8": WORKLOADS["c3"].with_(name="c3i8", pv_mode="int8",
                                  note="c3 with INT8 P~V (static delta_P = 1/127)"),
    "c4i8": WORKLOADS["c4"].with_(name="c4i8", pv_mode="int8",
                                  note="c4 with INT8 P~V (static delta_P = 1/127)"),
}


# Q smoothed per block as well as K: on the headline shape, and on inputs whose
# Q carries a per-channel bias shared by all tokens (the case it is for).
SMOOTH_Q = {
    "c3sq": WORKLOADS["c3"].with_(name="c3sq", smooth_q=True,
                                  note="c3 with Q smoothed per 128-token block"),
    "qb_sq": Workload("qb_sq", 2, 16, 4096, 128, "bf16", False, "fp16", 5, "qbias4_kbias4",
                      "Q and K with per-channel biases ~ N(0, 4^2), Q smoothed", True),
    "qb_plain": Workload("qb_plain", 2, 16, 4096, 128, "bf16", False, "fp16", 5, "qbias4_kbias4",
                         "the inputs of qb_sq without smoothing Q"),
}


def named(name: str) -> Workload:
    """A workload of WORKLOADS, TABLE7, SHARDS, PV_INT8 or SMOOTH_Q by name."""
    for table in (WORKLOADS, TABLE7, SHARDS, PV_INT8, SMOOTH_Q):
        if name in table:
            return table[name]
    raise KeyError(name)


def round_to_fp16(x: np.ndarray) -> np.ndarray:
    """float32 -> float16 with round-to-nearest-even (numpy's cast)."""
    return x.astype(np.float16)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    Inputs are finite by construction, so no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    """One draw: 16-bit storage (``*_bits`` as uint16) and the exact float32 values."""
    wl: Workload
    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    qf: np.ndarray
    kf: np.ndarray
    vf: np.ndarray

    def torch_tensors(self, device="cpu"):
        """q, k, v as torch tensors of the 16-bit dtype (imports torch lazily)."""
        import torch
        dt = torch.float16 if self.wl.dtype == "fp16" else torch.bfloat16
        out = []
        for bits in (self.q_bits, self.k_bits, self.v_bits):
            t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt)
            out.append(t.to(device))
        return tuple(out)


def _apply_extras(wl: Workload, rng, q, k, v):
    B, H, d = wl.B, wl.H, wl.d
    e = wl.extras
    if e == "none":
        pass
    elif e.startswith("kbias"):
        std = float(e[len("kbias"):])
        k += (rng.standard_normal((B, H, 1, d), dtype=np.float32) * np.float32(std))
    elif e == "kchan20":
        chans = rng.choice(d, 4, replace=False)
        k[..., chans] += np.float32(20.0) * np.array([1, -1, 1, -1], np.float32)
    elif e == "q8_kbias5":
        qch = rng.choice(d, 2, replace=False)
        q[..., qch] *= np.float32(8.0)
        k += (rng.standard_normal((B, H, 1, d), dtype=np.float32) * np.float32(5.0))
    elif e.startswith("qbias"):
        # "qbiasA_kbiasB": Q and K each carry a per-channel bias shared by all
        # tokens, ~ N(0, A^2) and N(0, B^2) (the case that smoothing Q, on top
        # of smoothing K, is for)
        qa_, kb_ = e[len("qbias"):].split("_kbias")
        q += (rng.standard_normal((B, H, 1, d), dtype=np.float32) * np.float32(float(qa_)))
        k += (rng.standard_normal((B, H, 1, d), dtype=np.float32) * np.float32(float(kb_)))
    elif e == "vout":
        # one V token per (b, h) with value 6e4 in every channel, which queries
        # avoid (a shared query-channel bias against a large negative key
        # component): the per-channel FP8 V scale then pushes every other V
        # value into E4M3's coarse subnormal range.
        N = v.shape[2]
        c0 = int(rng.integers(0, d))
        t0 = int(rng.integers(0, N))
        q[..., c0] += np.float32(5.0)
        k[..., t0, c0] -= np.float32(60.0)
        v[..., t0, :] = np.float32(6.0e4)
    elif e == "ramp":
        # scores that climb along the keys: one channel of K grows linearly
        # with the token index (to 15*sqrt(d)) and Q carries +4 in that
        # channel, so the logits rise by about 60 (natural units) from the
        # first key to the last.  Later tiles then lie far above the running
        # maximum of earlier ones (a recompute case of the attention kernel).
        N = k.shape[2]
        c0 = int(rng.integers(0, d))
        q[..., c0] += np.float32(4.0)
        ramp = np.arange(N, dtype=np.float32) / np.float32(max(N - 1, 1))
        k[..., c0] += ramp * np.float32(15.0 * np.sqrt(d))
    else:
        raise ValueError(f"unknown extras recipe {e!r}")


def make_inputs(wl: Workload | str, **overrides) -> Inputs:
    """Draw q, k, v for a workload (or a named one with fields overridden)."""
    if isinstance(wl, str):
        wl = named(wl)
    if overrides:
        wl = wl.with_(**overrides)
    shape = (wl.B, wl.H, wl.N, wl.d)
    rng = np.random.default_rng(wl.seed)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    _apply_extras(wl, rng, q, k, v)
    if wl.dtype == "fp16":
        qh, kh, vh = (round_to_fp16(t) for t in (q, k, v))
        return Inputs(wl, qh.view(np.uint16), kh.view(np.uint16), vh.view(np.uint16),
                      qh.astype(np.float32), kh.astype(np.float32), vh.astype(np.float32))
    if wl.dtype == "bf16":
        qb, kb, vb = (round_to_bf16_bits(t) for t in (q, k, v))
        return Inputs(wl, qb, kb, vb, bf16_bits_to_f32(qb), bf16_bits_to_f32(kb),
                      bf16_bits_to_f32(vb))
    raise ValueError(f"dtype {wl.dtype!r}")


def make_inputs_uniform(wl: Workload, scale: float = 2.0, q_spans=None) -> Inputs:
    """As make_inputs, but q, k, v uniform in [-scale, scale) (float32 draws in
    the order Q, K, V, then the extras, then the 16-bit rounding): for heads of
    millions of tokens, where normal draws alone would take minutes.
    q_spans: optional [(t0, count), ...]; Q is then drawn on those token spans
    only (in that order) and zero elsewhere."""
    shape = (wl.B, wl.H, wl.N, wl.d)
    rng = np.random.default_rng(wl.seed)

    def draw(shp):
        x = rng.random(shp, dtype=np.float32)
        x *= np.float32(2.0 * scale)
        x -= np.float32(scale)
        return x
    if q_spans is None:
        q = draw(shape)
    else:
        q = np.zeros(shape, np.float32)
        for (t0, cnt) in q_spans:
            q[:, :, t0:t0 + cnt] = draw((wl.B, wl.H, cnt, wl.d))
    k, v = draw(shape), draw(shape)
    _apply_extras(wl, rng, q, k, v)
    if wl.dtype == "fp16":
        qh, kh, vh = (round_to_fp16(t) for t in (q, k, v))
        del q, k, v
        return Inputs(wl, qh.view(np.uint16), kh.view(np.uint16), vh.view(np.uint16),
                      qh.astype(np.float32), kh.astype(np.float32), vh.astype(np.float32))
    if wl.dtype == "bf16":
        qb, kb, vb = (round_to_bf16_bits(t) for t in (q, k, v))
        del q, k, v
        return Inputs(wl, qb, kb, vb, bf16_bits_to_f32(qb), bf16_bits_to_f32(kb),
                      bf16_bits_to_f32(vb))
    raise ValueError(f"dtype {wl.dtype!r}")


def small(name="t", B=1, H=2, N=200, d=64, dtype="fp16", causal=False, pv_mode="fp16",
          seed=11, extras="kbias4") -> Workload:
    """A small ad-hoc workload for tests."""
    return Workload(name, B, H, N, d, dtype, causal, pv_mode, seed, extras)


def rope_tables(N: int, d: int, base: float = 10000.0, offset: int = 0):
    """Rotary tables as a model would pass them: angle(t, i) = (t + offset) *
    base^(-2i/d) for token t and pair i < d/2, evaluated in float64 and
    rounded to float32.  Returns (cos, sin), each float32 [N, d/2]."""
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / d)
    ang = (np.arange(N, dtype=np.float64) + offset)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def to_nhd(x: np.ndarray) -> np.ndarray:
    """[B, H, N, d] -> contiguous [B, N, H, d] (the token-major layout)."""
    return np.ascontiguousarray(np.swapaxes(x, 1, 2))
