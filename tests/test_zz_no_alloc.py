"""lh_attention_backward_noalloc (the dense attention backward with its scratch
in the library's fixed array) against lh_attention_backward with a
caller-provided workspace: the same kernels, so bit-identical gradients.  Two
calls in a row, the second on a smaller input (the array keeps the first call's
contents), in bf16 (MFMA path) and fp32 (vector-ALU path)."""
import numpy as np
import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _inputs(torch, BH, S, d, io, seed):
    g = torch.Generator().manual_seed(seed)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    q, k, v, do = (torch.randn((BH, S, d), generator=g).to(dt).cuda() for _ in range(4))
    return q, k, v, do


def _both(lh, torch, BH, S, d, io, seed):
    say(f"case noalloc BH={BH} S={S} d={d} io={io}")
    q, k, v, do = _inputs(torch, BH, S, d, io, seed)
    o = torch.empty((BH, S, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((BH, S), dtype=torch.float32, device="cuda")
    assert lh.lh_attention_forward(q, k, v, o, lse, BH, S, d, io) == 0, lh.lh_last_error()
    ref = [torch.empty((BH, S, d), dtype=torch.float32, device="cuda") for _ in range(3)]
    got = [torch.full((BH, S, d), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    nb = lh.attention_backward_ws_bytes(BH, S, io)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    assert lh.lh_attention_backward(q, k, v, o, lse, do, *ref, BH, S, d, io, ws, nb) == 0, lh.lh_last_error()
    assert lh.lh_attention_backward_noalloc(q, k, v, o, lse, do, *got, BH, S, d, io) == 0, lh.lh_last_error()
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(a).all(), name
        assert torch.equal(a, b), f"{name}: max diff {float((a - b).abs().max()):.3e}"


@pytest.mark.parametrize("io,d", [("bf16", 128), ("f32", 64)])
def test_noalloc_equals_workspace_variant_twice(lh, io, d):
    import torch
    _both(lh, torch, 4, 2048, d, io, 1)   # first call: 8192 rows of scratch
    _both(lh, torch, 2, 640, d, io, 2)    # second, smaller: the array still holds the first call's rows


def test_noalloc_refuses_beyond_its_array(lh):
    import torch
    q = torch.zeros(16, dtype=torch.uint8, device="cuda")
    p = q.data_ptr()
    st = lh.lh_attention_backward_noalloc(p, p, p, p, p, p, p, p, p, 8, (1 << 19) + 64, 128, "bf16")
    assert st == 4 and "scratch" in lh.lh_last_error()
