"""Per-layer choice of the P~V precision by cosine similarity.

"SageAttention: Accurate 8-Bit Attention ..." detail page, §2 Q2 item 3 (and
§4 check 6, §6 step 4): each layer is profiled once against full precision;
layers whose cosine similarity stays above 99.8% use the faster kernel, the
others fall back to the more precise one.  The page's faster kernel is the
all-INT8 one (INT8 P~V), its precise one keeps P~V in FP16; candidates=
("int8",) reproduces that choice.  On gfx950 the default fast candidate is
FP8 E4M3 P~V: the FP8 MFMA runs at the INT8 rate with a float32 accumulator,
whose rescale at a new row max is one multiply per value, against three
instructions per value for the INT32 sum of INT8 P~V; FP8 is the faster of
the two at both head sizes.  Several candidates are tried in the order given
(fastest first).

Every number is computed on the GPU: the candidate kernel's float32 output
and a float32 full-precision reference (sage_attn_ref_rows_f32) on a seeded
subsample of query rows; only the cosine of the two is formed here (torch
reductions on device tensors).
"""
from __future__ import annotations

import json

import torch

from .api import ref_rows, sage_attn

DEFAULT_THRESHOLD = 0.998   # 99.8%, the threshold on the page


def sample_rows(N: int, rows: int, seed: int) -> torch.Tensor:
    """Seeded subsample of query rows (always includes the first and last)."""
    g = torch.Generator().manual_seed(seed)
    n = min(rows, N)
    pick = torch.randperm(N, generator=g)[:n]
    pick[0] = 0
    if n > 1:
        pick[1] = N - 1
    return torch.unique(pick).to(torch.int32)


def layer_cosine(q, k, v, causal: bool = False, pv_mode: str = "fp8", rows: int = 512,
                 seed: int = 0) -> float:
    """Cosine similarity between the quantised output (pv_mode) and the
    float32 reference, over a seeded subsample of query rows of all heads.
    An all-zero output (INT8 V can quantise every value of a channel whose
    range one outlier token sets to 0) counts as cosine 0 against a nonzero
    reference, and two all-zero outputs as 1."""
    N = q.shape[2]
    idx = sample_rows(N, rows, seed)
    out = sage_attn(q, k, v, causal=causal, pv_mode=pv_mode, out_f32=True)
    ref = ref_rows(q, k, v, idx.to(q.device), causal=causal)
    got = out[:, :, idx.to(q.device).long()].double().flatten()
    ref = ref.double().flatten()
    ng, nr = float(got.norm()), float(ref.norm())
    if ng == 0.0 or nr == 0.0:
        return 1.0 if ng == nr else 0.0
    return float((got @ ref) / (ng * nr))


FAST_MODES = ("fp8", "int8")


def choose_mode(cos_fast, threshold: float = DEFAULT_THRESHOLD, candidates=("fp8",)) -> str:
    """The first candidate whose cosine (a float, or a dict mode -> cosine)
    reaches the threshold, else FP16."""
    for mode in candidates:
        if mode not in FAST_MODES:
            raise ValueError(f"not a fast P~V mode: {mode!r}")
        c = cos_fast[mode] if isinstance(cos_fast, dict) else cos_fast
        if c >= threshold:
            return mode
    return "fp16"


def select_pv_modes(layers, threshold: float = DEFAULT_THRESHOLD, rows: int = 512,
                    seed: int = 0, candidates=("fp8",)) -> dict:
    """layers: mapping name -> (q, k, v) or (q, k, v, causal), device tensors.

    Returns {name: {"pv_mode": one of candidates or "fp16", "cos_<mode>":
    float for each candidate}}, the table the pages build once per model and
    then reuse.
    """
    table = {}
    for name, spec in layers.items():
        q, k, v = spec[:3]
        causal = bool(spec[3]) if len(spec) > 3 else False
        cos = {m: layer_cosine(q, k, v, causal=causal, pv_mode=m, rows=rows, seed=seed)
               for m in candidates}
        entry = {"pv_mode": choose_mode(cos, threshold, candidates)}
        entry.update({f"cos_{m}": c for m, c in cos.items()})
        table[name] = entry
    return table


def save_modes(table: dict, path: str) -> None:
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)


def load_modes(path: str) -> dict:
    with open(path) as f:
        table = json.load(f)
    for name, e in table.items():
        if e.get("pv_mode") not in ("fp16",) + FAST_MODES:
            raise ValueError(f"layer {name!r}: bad pv_mode {e.get('pv_mode')!r}")
    return table
