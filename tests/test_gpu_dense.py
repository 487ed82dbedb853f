"""GPU parity of the dense causal attention entry points, lh_attention_forward
and lh_attention_backward (the attention of stage iii on given [BH, S, d]
tensors: the dense baseline at S = N, and its backward), against the oracle's
fp64 attention (``attend``) and its adjoint (``attend_adjoint``) on exactly the
same input values.

Bars (the stage bars of the layer tests):
  O     fp32 1e-4 max-abs; bf16 2^-8 max|V| + 1e-4 (P is rounded to bf16 for P V)
  LSE   fp32 1e-4; bf16 1e-3
  dQ, dK, dV, relative to each gradient's largest magnitude: fp32 1e-5; bf16
        3 * 2^-8 (P and dS are rounded to bf16, and delta uses the forward's O,
        which carries the bf16 rounding of P).
"""
import numpy as np
import pytest

import oracle as orc
from gpu_helpers import say, to_dev
from hierarchical_sparse_attention_mean_amd import synth

pytestmark = pytest.mark.gpu

GRAD_TOL = {"f32": 1e-5, "bf16": 3 * 2.0 ** -8}
LSE_TOL = {"f32": 1e-4, "bf16": 1e-3}

CASES = [                                 # dense: S = N
    ("tiny", dict(N=1000)),               # fp32, d=64, S not a multiple of 64
    ("tiny", dict(N=768, d=128)),         # fp32, d=128
    ("bwd8k", dict(N=2048, H=2)),         # bf16, d=128
    ("bwd8k", dict(N=1024, H=2, d=64)),   # bf16, d=64
]


@pytest.mark.parametrize("name,over", CASES)
def test_dense_attention_forward_backward(lh, name, over):
    import torch
    cfg = synth.config(name, **over)
    dt, S, d = cfg["dtype"], cfg["N"], cfg["d"]
    BH = cfg["B"] * cfg["H"]
    say(f"case dense S={S} BH={BH} d={d} io={dt}")
    inp = synth.make_inputs(cfg, with_do=True)
    host = {n: inp[n].reshape(BH, S, d) for n in ("q", "k", "v", "do")}
    q, k, v, do = (to_dev(host[n], dt) for n in ("q", "k", "v", "do"))
    o = torch.empty((BH, S, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((BH, S), dtype=torch.float32, device="cuda")
    assert lh.lh_attention_forward(q, k, v, o, lse, BH, S, d, dt) == 0, lh.lh_last_error()
    dq, dk, dv = (torch.empty((BH, S, d), dtype=torch.float32, device="cuda") for _ in range(3))
    nb = lh.attention_backward_ws_bytes(BH, S, dt)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    assert lh.lh_attention_backward(q, k, v, o, lse, do, dq, dk, dv, BH, S, d, dt, ws, nb) == 0, lh.lh_last_error()
    torch.cuda.synchronize()
    o_g, lse_g = o.cpu().numpy(), lse.cpu().numpy()
    grads_g = [g.cpu().numpy() for g in (dq, dk, dv)]
    for h in range(BH):
        x = [synth.as_f64(host[n][h], dt) for n in ("q", "k", "v", "do")]
        ot_ref, lse_ref = orc.attend(x[0], x[1], x[2])
        e_o = float(np.max(np.abs(o_g[h] - ot_ref)))
        e_l = float(np.max(np.abs(lse_g[h] - lse_ref)))
        bar_o = 1e-4 if dt == "f32" else 2.0 ** -8 * float(np.max(np.abs(x[2]))) + 1e-4
        refs = orc.attend_adjoint(x[0], x[1], x[2], x[3])
        rel = [float(np.max(np.abs(g[h] - r)) / np.max(np.abs(r))) for g, r in zip(grads_g, refs)]
        say(f"  head {h}: |O - oracle| {e_o:.3e}, |LSE - oracle| {e_l:.3e}, "
            f"gradient errors (relative to max) dQ {rel[0]:.3e} dK {rel[1]:.3e} dV {rel[2]:.3e}")
        assert e_o <= bar_o and e_l <= LSE_TOL[dt]
        assert max(rel) <= GRAD_TOL[dt]
