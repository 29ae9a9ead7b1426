"""GPU parity over a seeded random sample of the option space of the forward
pass ("SageAttention ..." detail page, §3 Algorithm 1; P~V in FP16, FP8 as in
the "SageAttention2++ ..." review page, section 三, or INT8 as in the detail
page's Figure 5; RoPE fused into the quantisation as in its §7 item 1; Q
smoothed per block as in the SageAttention2 abstract).

Each case draws B, H, N (tile boundaries and arbitrary lengths up to 700),
d, the input dtype, causal or not, the P~V mode, the layout, RoPE or smoothed
Q (or neither) and an input recipe, and compares the whole float32 O of the
library's forward call element by element with the oracle on the same
inputs.  Bar: max |O - O_oracle| <= 2e-3 and cosine >= 0.9999; with FP8 or
INT8 P~V each element may exceed 2e-3 by the oracle's bound for P^ values
that lie, to float32 accuracy, on a rounding boundary of their codes
(reading C-s).  O in the 16-bit input dtype is within that plus one ulp of
the dtype.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import make_inputs, rope_tables, small

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-3
O_COS = 0.9999
N_EDGE = [1, 2, 31, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257, 383, 511, 513, 640]
RECIPES = ["none", "kbias4", "kchan20", "q8_kbias5", "qbias4_kbias4", "ramp"]


def _draw_cases(n=48, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        N = int(rng.choice(N_EDGE)) if i % 2 == 0 else int(rng.integers(1, 701))
        variant = str(rng.choice(["plain", "rope", "smooth_q"]))
        cfg = dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), N=N,
                   d=int(rng.choice([64, 128])), dtype=str(rng.choice(["fp16", "bf16"])),
                   causal=bool(rng.integers(0, 2)), pv_mode=str(rng.choice(["fp16", "fp8", "int8"])),
                   layout=str(rng.choice(["HND", "NHD"])), variant=variant,
                   extras=str(rng.choice(RECIPES)), seed=int(rng.integers(100, 10000)))
        cfg["name"] = (f"rc{i:02d}_B{cfg['B']}H{cfg['H']}N{N}d{cfg['d']}_{cfg['dtype']}"
                       f"{'_causal' if cfg['causal'] else ''}_{cfg['pv_mode']}_{cfg['layout']}"
                       f"_{variant}_{cfg['extras']}")
        cases.append(cfg)
    return cases


CASES = _draw_cases()


def note(msg):
    print(f"[gpu-random] {msg}", flush=True)
    sys.stdout.flush()


def ulp16(x, dtype):
    x = np.abs(x)
    if dtype == "fp16":
        e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
        return 2.0 ** (e - 10)
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c["name"])
def test_random_config_parity(cfg):
    import quantized_attention_qk_amd as qa
    note(f"case {cfg['name']} seed {cfg['seed']}")
    wl = small(cfg["name"], B=cfg["B"], H=cfg["H"], N=cfg["N"], d=cfg["d"], dtype=cfg["dtype"],
               causal=cfg["causal"], pv_mode=cfg["pv_mode"], seed=cfg["seed"],
               extras=cfg["extras"])
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cpu")
    nhd = cfg["layout"] == "NHD"
    if nhd:
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    qf, kf = inp.qf, inp.kf
    rope = None
    if cfg["variant"] == "rope":
        c, s = rope_tables(wl.N, wl.d, offset=cfg["seed"] % 97)
        rope = (torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda())
        qf, kf = oracle.rope_rotate_half(qf, c, s), oracle.rope_rotate_half(kf, c, s)
    sq = cfg["variant"] == "smooth_q"
    kw = dict(causal=wl.causal, pv_mode=wl.pv_mode, layout=cfg["layout"], rope=rope,
              smooth_q=sq)
    o32 = qa.sage_attn(q, k, v, out_f32=True, **kw)
    o16 = qa.sage_attn(q, k, v, **kw).float()
    torch.cuda.synchronize()
    o32, o16 = o32.cpu().numpy(), o16.cpu().numpy()
    if nhd:
        o32, o16 = np.swapaxes(o32, 1, 2), np.swapaxes(o16, 1, 2)
    quantised_p = wl.pv_mode in ("fp8", "int8")
    res = oracle.sage_attention(qf, kf, inp.vf, causal=wl.causal, pv_mode=wl.pv_mode,
                                smooth_q=sq, p_flip=quantised_p)
    ref, allow = res if quantised_p else (res, 0.0)
    err = np.abs(o32.astype(np.float64) - ref)
    cos = oracle.cos_sim(o32, ref)
    note(f"{cfg['name']}: max|dO| = {err.max():.3e}  cos = {cos:.7f}  "
         f"beyond 2e-3: {int((err > O_MAX_ABS).sum())}")
    assert np.all(err <= O_MAX_ABS + allow), float((err - O_MAX_ABS - allow).max())
    assert cos >= O_COS, cos
    lim16 = O_MAX_ABS + ulp16(ref, wl.dtype) + allow
    assert np.all(np.abs(o16 - ref) <= lim16), "16-bit O"
