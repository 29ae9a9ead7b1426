"""Bit-exact INT32 scores of the timed attention kernel on the five workloads.

"SageAttention: Accurate 8-Bit Attention ..." (paper detail page), §3
Algorithm 1: S = Q^ K^^T is an INT32 product of the INT8 codes.  The debug
entry sage_attn_debug_s_fwd re-runs the attention kernel's own debug
instantiation (same source, schedule, LDS staging, and the accumulator start
values the timed kernel uses: FP16 mode's 1.5 * 2^23 bias, the smoothed-Q
compensation seeds) on the operands a forward pass left in its workspace, and
stores every score it computes with the start bias removed.  Here those
scores must equal the oracle's INT32 product of the oracle's own codes
(S + C with Q smoothed), every element, and the O rows of that same launch
must equal the forward pass's float32 O bit for bit.

Windows: all of c1; for the other workloads whole query blocks (every key
tile of the row block: first, last, the causal diagonal and everything
between) -- the first and last block and two seeded ones, on the first, last
and a seeded head.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import make_inputs, make_inputs_uniform, named, small

pytestmark = pytest.mark.gpu

QROWS = 128   # rows per checked window (one delta_Q block)


def note(msg):
    print(f"[gpu-s-exact] {msg}", flush=True)
    sys.stdout.flush()


def qa():
    import quantized_attention_qk_amd as m
    return m


def rows_per_workgroup(wl):
    # 8 wavefronts of 32 rows for FP16 P~V at d = 128 without a mask, else 4
    return 256 if (wl.pv_mode == "fp16" and wl.d == 128 and not wl.causal) else 128


def check_window(wl, inp, ws, pq, b, h, q0, nq, k0, nk, o_full):
    """pq: the oracle's prepass of head (b, h) alone (arrays [1, 1, ...])."""
    s, o = qa().debug_s_fwd(ws, wl.B, wl.H, wl.N, wl.d, wl.causal, wl.pv_mode, wl.smooth_q,
                            b, h, q0, nq, k0, nk)
    torch.cuda.synchronize()
    s, o = s.cpu().numpy(), o.cpu().numpy()
    ref = oracle.s_int32_tile(pq["q_i8"], pq["k_i8"], 0, 0, q0, nq, k0, nk).astype(np.int64)
    if wl.smooth_q:
        ref = ref + pq["q_comp"][0, 0][np.arange(q0, q0 + nq) // 128][:, k0:k0 + nk]
    # the scores the kernel computes: every key < N; with the causal mask the
    # tiles up to the end of the row's query block
    keys = np.arange(k0, k0 + nk)[None, :]
    rows = np.arange(q0, q0 + nq)[:, None]
    want = np.broadcast_to(keys < wl.N, (nq, nk))
    if wl.causal:
        bq = rows_per_workgroup(wl)
        want = want & (keys < ((rows // bq) + 1) * bq)
    got = s != qa().api.S_NOT_COMPUTED
    assert np.array_equal(got, want), \
        f"computed set differs: {int((got != want).sum())} entries (b={b},h={h},q0={q0},k0={k0})"
    bad = (s.astype(np.int64) != ref) & want
    assert not bad.any(), (f"S differs at {int(bad.sum())} entries (b={b},h={h},q0={q0},k0={k0}), "
                           f"first {np.argwhere(bad)[:3].tolist()}")
    # the dump launch computed the same O rows as the forward pass, bit for bit
    of = o_full[b, h, q0:q0 + nq].cpu().numpy()
    assert np.array_equal(o.view(np.uint32), of.view(np.uint32)), "dump launch O != forward O"
    return int(want.sum())


def run_workload(wl, heads, qstarts, kwin=None):
    note(f"{wl.name}: {wl}")
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    ws = torch.empty(qa().workspace_bytes(B, H, N, d, wl.pv_mode, wl.smooth_q), dtype=torch.uint8,
                     device="cuda")
    o_full = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True,
                            workspace=ws, smooth_q=wl.smooth_q)
    torch.cuda.synchronize()
    total = 0
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        pq = oracle.smooth_quant_qk(inp.qf[sl], inp.kf[sl], smooth_q=wl.smooth_q)
        for q0 in qstarts:
            nq = min(QROWS, N - q0)
            k0, nk = (0, N) if kwin is None else kwin
            note(f"  head (b={b},h={h}) rows [{q0},{q0 + nq}) keys [{k0},{k0 + nk})")
            total += check_window(wl, inp, ws, pq, b, h, q0, nq, k0, nk, o_full)
    note(f"{wl.name}: {total} scores bit-exact")


def seeded_heads(wl, n=1):
    rng = np.random.default_rng(wl.seed + 7)
    hs = {(0, 0), (wl.B - 1, wl.H - 1)}
    hs |= {(int(rng.integers(0, wl.B)), int(rng.integers(0, wl.H))) for _ in range(n)}
    return sorted(hs)


def seeded_blocks(wl, n=2):
    rng = np.random.default_rng(wl.seed + 11)
    nb = -(-wl.N // QROWS)
    bl = {0, nb - 1} | {int(x) for x in rng.integers(0, nb, n)}
    return sorted(QROWS * x for x in bl)


def test_s_exact_c1_all_tiles():
    wl = named("c1")
    run_workload(wl, [(0, h) for h in range(wl.H)], [q0 for q0 in range(0, wl.N, QROWS)])


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5", "c3i8", "c4i8", "c3sq", "qb_sq"])
def test_s_exact_workload(name):
    wl = named(name)
    run_workload(wl, seeded_heads(wl), seeded_blocks(wl))


# ragged token counts, both d, every P~V mode, causal and not, Q smoothed
SMALL = [
    small("sx300c", N=300, d=128, causal=True, dtype="bf16"),
    small("sx1105", N=1105, d=64, H=1, extras="kchan20"),
    small("sx197f8", N=197, d=64, pv_mode="fp8"),
    small("sx2177c", N=2177, d=128, H=1, causal=True, pv_mode="fp8", dtype="bf16"),
    small("sx640i8", B=2, H=3, N=640, d=128, dtype="bf16", pv_mode="int8", extras="q8_kbias5"),
    small("sx1000r", N=1000, d=64, extras="ramp"),
    small("sx700sq", N=700, d=128, dtype="bf16", extras="qbias4_kbias4").with_(smooth_q=True),
    small("sx333sqc8", N=333, d=64, causal=True, pv_mode="fp8",
          extras="qbias4_kbias4").with_(smooth_q=True),
    small("sx260sqi8", N=260, d=128, pv_mode="int8", extras="qbias4_kbias4").with_(smooth_q=True),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_s_exact_small(wl):
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    run_workload(wl, heads, list(range(0, wl.N, QROWS)))


def test_s_exact_unaligned_window():
    # a window that starts and ends inside query blocks and key tiles
    wl = small("sxwin", N=1000, d=128, dtype="bf16", causal=True)
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    ws = torch.empty(qa().workspace_bytes(1, 2, 1000, 128, "fp16"), dtype=torch.uint8,
                     device="cuda")
    o_full = qa().sage_attn(q, k, v, causal=True, out_f32=True, workspace=ws)
    pq = oracle.smooth_quant_qk(inp.qf[:, 1:2], inp.kf[:, 1:2])
    n = check_window(wl, inp, ws, pq, 0, 1, 77, 301, 33, 555, o_full)
    note(f"unaligned window: {n} scores bit-exact")


def test_s_exact_long_head():
    # one head of 2^20 + 37 tokens (K^ tile index up to 16384): the first and
    # last query block against the first and last 4096 keys
    wl = small("sxlong", B=1, H=1, N=(1 << 20) + 37, d=128, dtype="bf16", seed=31)
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    N = wl.N
    ws = torch.empty(qa().workspace_bytes(1, 1, N, 128, "fp16"), dtype=torch.uint8,
                     device="cuda")
    o_full = qa().sage_attn(q, k, v, out_f32=True, workspace=ws)
    pq = oracle.smooth_quant_qk(inp.qf, inp.kf)
    for q0 in (0, N - 100):
        for (k0, nk) in ((0, 4096), (N - 4096, 4096)):
            note(f"  rows from {q0}, keys [{k0},{k0 + nk})")
            check_window(wl, inp, ws, pq, 0, 0, q0, min(QROWS, N - q0), k0, nk, o_full)


def test_s_exact_max_length():
    """One head of 2^24 tokens, the longest the library takes (d = 128, FP16
    P~V: K^ spans 2^31 bytes, V' 4 GiB).  Q is drawn on its first and last
    128-token blocks and zero elsewhere.  The prepass alone fills the workspace
    (sage_attn_prepare; the whole attention would take minutes), then the timed
    kernel's debug launch runs the first and the last query block over all
    2^24 keys: its INT32 scores on the first and last 4096 keys equal the
    oracle's, and O of sampled rows of those blocks is within the 2e-3 bar of
    the oracle's attention over all keys."""
    N = 1 << 24
    wl = small("sxmax", B=1, H=1, N=N, d=128, dtype="fp16", seed=37)
    spans = [(0, QROWS), (N - QROWS, QROWS)]
    note(f"max length: drawing inputs {wl} (uniform in [-2, 2), Q on two blocks)")
    inp = make_inputs_uniform(wl, q_spans=spans)
    q, k, v = inp.torch_tensors("cuda")
    ws = torch.empty(qa().workspace_bytes(1, 1, N, 128, "fp16"), dtype=torch.uint8, device="cuda")
    note("max length: prepass on the GPU")
    qa().prepare(q, k, v, "fp16", ws)
    torch.cuda.synchronize()
    del q, k, v
    # the oracle's prepass of K (all tokens) and of the two Q blocks (a Q
    # block's codes and scale depend on that block alone)
    note("max length: oracle prepass")
    q_sub = np.concatenate([inp.qf[:, :, t0:t0 + c] for (t0, c) in spans], axis=2)
    pq = oracle.smooth_quant_qk(q_sub, inp.kf)
    o_rows = {}
    for i, (q0, _) in enumerate(spans):
        for (k0, nk) in ((0, 4096), (N - 4096, 4096)):
            note(f"  rows [{q0},{q0 + QROWS}) keys [{k0},{k0 + nk})")
            s, o = qa().debug_s_fwd(ws, 1, 1, N, 128, False, "fp16", False, 0, 0, q0, QROWS, k0, nk)
            torch.cuda.synchronize()
            s = s.cpu().numpy()
            ref = oracle.s_int32_tile(pq["q_i8"], pq["k_i8"], 0, 0, i * QROWS, QROWS, k0, nk)
            assert np.array_equal(s.astype(np.int64), ref.astype(np.int64)), \
                f"S differs at {int((s != ref).sum())} entries (q0={q0}, k0={k0})"
            o = o.cpu().numpy()
            if q0 in o_rows:   # the same rows from another launch: the same bits
                assert np.array_equal(o.view(np.uint32), o_rows[q0].view(np.uint32))
            o_rows[q0] = o
    # O of sampled rows: the oracle's tiled attention over all keys, on the
    # operands of its prepass (as oracle.sage_attention assembles them)
    note("max length: oracle O of sampled rows over all keys")
    sub = np.array([0, 1, 77, 127, 128, 196, 254, 255])          # rows of q_sub
    rows = np.where(sub < QROWS, sub, sub - QROWS + N - QROWS)     # rows of the head
    vvals, _, _ = oracle.prep_v(inp.vf, "fp16")
    ref = oracle.attention(pq["q_i8"][0, 0, sub].astype(np.float64),
                           pq["q_scale"][0, 0, sub // QROWS],
                           pq["k_i8"][0, 0].astype(np.float64),
                           pq["k_scale"][0, 0, np.arange(N) // 64], vvals[0, 0], np.ones(128),
                           causal=False, p_round=oracle.fp16_round, rows=rows)
    got = np.stack([o_rows[0][r] if r < QROWS else o_rows[N - QROWS][r - (N - QROWS)]
                    for r in rows])
    err = np.abs(got.astype(np.float64) - ref)
    note(f"max length: max|dO| = {err.max():.3e}")
    assert err.max() <= 2e-3 and oracle.cos_sim(got, ref) >= 0.9999
