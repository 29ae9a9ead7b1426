"""sage_attn_fwd_noalloc: the forward pass with the library's own fixed
device workspace, for callers that cannot allocate.  Its output must equal
sage_attn_fwd's (same kernels, caller-owned workspace) bit for bit, on two
calls in a row, the second with a smaller input; sizes past the fixed
workspace are refused.
"""
import ctypes

import pytest
import torch

from workloads import make_inputs, small

pytestmark = pytest.mark.gpu

WORKSPACE_ERR = 3


def lib():
    from quantized_attention_qk_amd._lib import lib as _l
    return _l()


def run_noalloc(q, k, v, o, causal, pv):
    B, H, N, d = q.shape
    dt = 0 if q.dtype == torch.float16 else 1
    return lib().sage_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       B, H, N, d, int(causal), pv, dt,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def reference(q, k, v, causal, pv):
    B, H, N, d = q.shape
    dt = 0 if q.dtype == torch.float16 else 1
    need = lib().sage_attn_workspace_bytes(B, H, N, d, pv)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    rc = lib().sage_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, d,
                             int(causal), pv, dt, ws.data_ptr(), need,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    return o


@pytest.mark.parametrize("pv", [0, 1, 2], ids=["fp16", "fp8", "int8"])
def test_noalloc_matches_fwd_twice(pv):
    mode = ["fp16", "fp8", "int8"][pv]
    # the second call is smaller and causal: stale contents of the fixed
    # workspace from the first call must not leak into it
    cases = [small("na_big", B=2, H=4, N=3000, d=128, dtype="bf16", pv_mode=mode, seed=41,
                   extras="kbias4"),
             small("na_small", B=1, H=3, N=333, d=64, dtype="fp16", causal=True, pv_mode=mode,
                   seed=42, extras="kbias4")]
    for wl in cases:
        inp = make_inputs(wl)
        q, k, v = inp.torch_tensors("cuda")
        o = torch.full_like(q, float("nan"))
        assert run_noalloc(q, k, v, o, wl.causal, pv) == 0
        ref = reference(q, k, v, wl.causal, pv)
        torch.cuda.synchronize()
        print(f"[no-alloc] {wl.name} {mode}: max |d| = "
              f"{(o.float() - ref.float()).abs().max().item():.3e}", flush=True)
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), wl.name


def test_noalloc_refuses_beyond_fixed_size():
    # c3's shape needs about 200 MB of workspace, more than the fixed array
    assert lib().sage_attn_workspace_bytes(1, 24, 16384, 128, 0) > (128 << 20)
    p = 1 << 20
    assert lib().sage_attn_fwd_noalloc(p, p, p, p + 4096, 1, 24, 16384, 128, 0, 0, 1,
                                       None) == WORKSPACE_ERR
