"""Streams and graph capture of the forward pass (needs an MI355X).

The C ABI promises stream-ordered work with no allocation and no state shared
between calls, so (1) two calls on two streams may run at once, and (2) a
whole pass can be captured into a HIP graph and replayed (callers that batch
short sequences do this to save launch time).  Graph replays are checked
several times, with the program's own eager work and new input data between
them, each against an eager run.  Streams keep the default priority.
"""
import sys

import pytest
import torch

from workloads import make_inputs, small

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[gpu-streams] {msg}", flush=True)
    sys.stdout.flush()


def qa():
    import quantized_attention_qk_amd as m
    return m


CASES = [small("g16", B=2, H=3, N=700, d=128, dtype="bf16", causal=True, seed=41),
         small("g8", B=1, H=4, N=2500, d=64, pv_mode="fp8", seed=42)]
# the INT8 P~V pass with Q smoothed (six kernels, seeds in the workspace)
GRAPH_CASES = CASES + [small("gi8sq", B=1, H=3, N=1300, d=128, pv_mode="int8", seed=43,
                             extras="qbias4_kbias4").with_(smooth_q=True)]


def test_two_streams_at_once():
    a, b = (make_inputs(w) for w in CASES)
    ta, tb = a.torch_tensors("cuda"), b.torch_tensors("cuda")
    wa, wb = CASES
    ref_a = qa().sage_attn(*ta, causal=wa.causal, pv_mode=wa.pv_mode, out_f32=True)
    ref_b = qa().sage_attn(*tb, causal=wb.causal, pv_mode=wb.pv_mode, out_f32=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa = qa().sage_attn(*ta, causal=wa.causal, pv_mode=wa.pv_mode, out_f32=True)
        with torch.cuda.stream(s2):
            ob = qa().sage_attn(*tb, causal=wb.causal, pv_mode=wb.pv_mode, out_f32=True)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa.view(torch.int32), ref_a.view(torch.int32))
        assert torch.equal(ob.view(torch.int32), ref_b.view(torch.int32))
    note("two streams: 3 concurrent pairs bitwise equal to sequential runs")


@pytest.mark.parametrize("wl", GRAPH_CASES, ids=lambda w: w.name)
def test_graph_capture_and_replay(wl):
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    ws = torch.empty(qa().workspace_bytes(B, H, N, d, wl.pv_mode, wl.smooth_q),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    # eager warm-up on a side stream, as graph capture wants
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out=out, workspace=ws,
                       out_f32=True, smooth_q=wl.smooth_q)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out=out, workspace=ws,
                       out_f32=True, smooth_q=wl.smooth_q)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    for rep in range(4):
        if rep >= 2:   # new inputs in the captured buffers: the replay must follow them
            for t in (q, k, v):
                t.copy_(torch.randn(t.shape, generator=gen, device="cuda").to(t.dtype))
        # the program's own eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True,
                             smooth_q=wl.smooth_q)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {rep}"
        del junk
    note(f"{wl.name}: 4 graph replays bitwise equal to eager runs")


@pytest.mark.parametrize("wl", [small("pa300", N=300, d=64, seed=44),
                                small("pa3000c8", B=1, H=2, N=3000, d=128, dtype="bf16",
                                      causal=True, pv_mode="fp8", seed=45),
                                small("pa5000i8", B=1, H=2, N=5000, d=64, pv_mode="int8",
                                      seed=46)],
                         ids=lambda w: w.name)
def test_prepare_then_attend_is_the_forward_pass(wl):
    """sage_attn_prepare followed by sage_attn_attend on one workspace gives
    the forward pass's output bit for bit (16-bit and float32 outputs), for
    the short, folded-statistics and long prepass paths."""
    q, k, v = make_inputs(wl).torch_tensors("cuda")
    B, H, N, d = q.shape
    ref16 = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode)
    ref32 = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True)
    ws = torch.empty(qa().workspace_bytes(B, H, N, d, wl.pv_mode), dtype=torch.uint8,
                     device="cuda")
    qa().prepare(q, k, v, wl.pv_mode, ws)
    o16 = qa().attend(ws, B, H, N, d, wl.causal, wl.pv_mode, out_dtype=q.dtype)
    o32 = qa().attend(ws, B, H, N, d, wl.causal, wl.pv_mode, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o16.view(torch.int16), ref16.view(torch.int16))
    assert torch.equal(o32.view(torch.int32), ref32.view(torch.int32))
    note(f"{wl.name}: prepare + attend bitwise equal to sage_attn")
