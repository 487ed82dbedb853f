"""GPU parity of the projection-inclusive layer (lh_layer_forward /
lh_layer_backward: W_Q, W_K, W_V, the Lighthouse attention of every head, W_O,
and the backward with the selection frozen) against the fp64 oracle
``oracle.layer_ref`` on the same input values.

The oracle mirrors the layer's storage roundings in bf16 mode (Q, K, V, O, dO,
dQ, dK, dV rounded to bf16 once).  The selection is an integer decision taken
on scores of the GPU's own projections; where the oracle's fp64 projections
select differently (near-ties at the boundary), the oracle is re-run with the
GPU's selection injected, as in the forward tests.

Bars:
  Q, K, V  fp32: 1e-5 relative to the largest |Q|; bf16: every element within
           one bf16 ulp of the oracle plus the worst-case error of an fp32 dot
           product of length d_model, d_model 2^-24 sum_k |x_k w_k| (the GPU
           rounds an fp32 sum to bf16, the oracle the exact one)
  Y        fp32: 1e-4 relative to max|Y|; bf16: 2e-2 relative to max|Y|
  dX, dW   relative to each gradient's largest magnitude: fp32 1e-4; bf16
           3 * 2^-8 (the attention backward rounds P and dS to bf16)
"""
import numpy as np
import pytest

import oracle as orc
from gpu_helpers import bf16_tensor_to_f64, say, to_dev
from hierarchical_sparse_attention_mean_amd import synth

pytestmark = pytest.mark.gpu

Y_TOL = {"f32": 1e-4, "bf16": 2e-2}
GRAD_TOL = {"f32": 1e-4, "bf16": 3 * 2.0 ** -8}

CASES = [
    ("tiny", {}),                                                         # fp32, d_model 128
    ("tiny", dict(B=2, H=3, d=64, d_model=192, N=1040, k=32)),           # fp32, ragged tiles, K tail, batch 2
    ("bwd8k", dict(H=2, N=2048, d_model=256)),                            # bf16, d 128
    ("bwd8k", dict(B=2, H=3, d=64, d_model=192, N=1040, k=32)),          # bf16, ragged, batch 2, d 64
    ("bwd8k", dict(N=4096, k=32)),                                        # bf16, the pages' d_model 1024, 8 x 128
]


def _f64(t, dt):
    return bf16_tensor_to_f64(t) if dt == "bf16" else t.double().cpu().numpy()


def _ulp_bf16(x):
    """Spacing of bf16 numbers at |x| (2^(e-7) for 2^e <= |x| < 2^(e+1))."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _proj_bar(x64, w64, ref):
    """One bf16 ulp plus the fp32 dot-product error bound K u sum |x w|, u = 2^-24."""
    K = x64.shape[-1]
    return _ulp_bf16(ref) * (1 + 1e-9) + K * 2.0 ** -24 * (np.abs(x64) @ np.abs(w64))


def run_layer(lh, cfg, with_backward=True):
    import torch
    dt = cfg["dtype"]
    inp = synth.layer_inputs(cfg, with_dy=with_backward)
    dev = {n: to_dev(a, dt) for n, a in inp.items()}
    y, saved, plan = lh.layer_forward(dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wo"], cfg["H"], cfg["L"],
                                      cfg["p"], cfg["k"], y_dtype=torch.float32)
    out = dict(inp=inp, dev=dev, y=y, saved=saved, plan=plan)
    if with_backward:
        out["grads"] = lh.layer_backward(dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wo"], dev["dy"], saved,
                                         plan, dx_dtype=torch.float32)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,over", CASES)
def test_layer_forward_backward(lh, name, over):
    cfg = synth.config(name, **over)
    dt, B, H, N, d = cfg["dtype"], cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    say(f"case layer B={B} H={H} N={N} d_model={cfg['d_model']} d={d} L={cfg['L']} p={cfg['p']} k={cfg['k']} io={dt}")
    r = run_layer(lh, cfg)
    plan, saved, inp = r["plan"], r["saved"], r["inp"]
    store = "bf16" if dt == "bf16" else None
    w64 = [synth.as_f64(inp[n], dt) for n in ("wq", "wk", "wv", "wo")]
    gflags = lh.saved_view(plan.view(saved, "inner"), plan.inner, "flags").cpu().numpy().astype(bool).reshape(B, H, -1)
    grads = [g.double().cpu().numpy() for g in r["grads"]]
    ref_grads = {n: 0.0 for n in ("dwq", "dwk", "dwv", "dwo")}
    for b in range(B):
        x64 = synth.as_f64(inp["x"][b], dt)
        fw = orc.layer_forward(x64, *w64, H, cfg["L"], cfg["p"], cfg["k"], store=store)
        # projections
        for n in ("q", "k", "v"):
            g = _f64(plan.view(saved, n)[b], dt)
            if dt == "bf16":
                w = w64[("q", "k", "v").index(n)]
                bar = orc.heads_of(_proj_bar(x64, w, orc.concat_heads(fw[n])), H)
                bad = np.abs(g - fw[n]) > bar
                assert not bad.any(), f"{n}: {int(bad.sum())} elements beyond the bar"
            else:
                err = np.abs(g - fw[n]).max() / np.abs(fw[n]).max()
                assert err < 1e-5, f"{n}: {err}"
        # selection: the oracle's own, else the GPU's injected
        nd = int(np.sum(fw["flags"] != gflags[b]))
        if nd:
            say(f"  batch {b}: oracle selection differs in {nd} entries; injecting the GPU's")
            fw = orc.layer_forward(x64, *w64, H, cfg["L"], cfg["p"], cfg["k"], flags=gflags[b], store=store)
        y = r["y"][b].double().cpu().numpy()
        yerr = np.abs(y - fw["y"]).max() / np.abs(fw["y"]).max()
        say(f"  batch {b}: max|Y - oracle| / max|Y| = {yerr:.3g}")
        assert yerr < Y_TOL[dt]
        # backward with the GPU's selection frozen
        bw = orc.layer_backward(x64, *w64, synth.as_f64(inp["dy"][b], dt), H, cfg["L"], cfg["p"], gflags[b],
                                store=store)
        gerr = np.abs(grads[0][b] - bw["dx"]).max() / np.abs(bw["dx"]).max()
        say(f"  batch {b}: dX rel err {gerr:.3g}")
        assert gerr < GRAD_TOL[dt]
        for n in ref_grads:
            ref_grads[n] = ref_grads[n] + bw[n]
    for g, n in zip(grads[1:], ("dwq", "dwk", "dwv", "dwo")):
        err = np.abs(g - ref_grads[n]).max() / np.abs(ref_grads[n]).max()
        say(f"  {n} rel err {err:.3g}")
        assert err < GRAD_TOL[dt], n


def test_layer_deterministic_and_timed(lh):
    """Two runs give bit-equal outputs and gradients; stage timing brackets the
    four projection stages and leaves the results unchanged."""
    import torch
    cfg = synth.config("bwd8k", B=2, H=3, d=64, d_model=192, N=1040, k=32)
    a = run_layer(lh, cfg)
    assert lh.lh_timing_begin() == 0
    b = run_layer(lh, cfg)
    st, stages = lh.lh_timing_end()
    assert st == 0
    for nm in ("proj", "out_proj", "out_proj_bwd", "proj_bwd", "attn_fwd", "attn_bwd_dkdv"):
        ms, spans = stages[nm]
        say(f"  stage {nm}: {spans} spans, {ms:.3f} ms")
        assert spans >= 1 and ms > 0
    assert torch.equal(a["y"], b["y"])
    for ga, gb in zip(a["grads"], b["grads"]):
        assert torch.equal(ga, gb)
    pa, pb = a["plan"], b["plan"]
    for n in ("q", "k", "v", "o"):
        assert torch.equal(pa.view(a["saved"], n), pb.view(b["saved"], n)), n
    ia, ib = pa.view(a["saved"], "inner"), pb.view(b["saved"], "inner")
    for n in ("scores", "flags", "slot", "coords", "qt", "kt", "vt", "ot", "lse"):
        assert torch.equal(lh.saved_view(ia, pa.inner, n), lh.saved_view(ib, pb.inner, n)), n


def test_layer_fullsize_512k_sampled(lh):
    """The layer at its benchmark shape (N = 524,288, d_model 1024, 8 heads of
    128, bf16), checked where the host's fp64 arithmetic is cheap: the projections
    of sampled tokens, Y rows of sampled tokens from the stored O, columns of
    dW_O = O^T dY, and two adjoint identities that tie dX to the weight
    gradients: <dX, X> = sum over Q, K, V of <dW, W>, and <dW_O, W_O> = <dY, Y>."""
    cfg = synth.config("512k")
    say("case layer 512k full size")
    r = run_layer(lh, cfg)
    plan, saved, inp = r["plan"], r["saved"], r["inp"]
    H, N, d, dm = cfg["H"], cfg["N"], cfg["d"], cfg["d_model"]
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(N, size=64, replace=False))
    x64 = synth.as_f64(inp["x"][0][rows], "bf16")
    w64 = {n: synth.as_f64(inp[n], "bf16") for n in ("wq", "wk", "wv", "wo")}
    for n in ("q", "k", "v"):
        ref = orc.round_bf16(x64 @ w64["w" + n])                       # [rows, H d], bf16 storage
        g = bf16_tensor_to_f64(plan.view(saved, n)[0][:, rows]).transpose(1, 0, 2).reshape(len(rows), H * d)
        bad = np.abs(g - ref) > _proj_bar(x64, w64["w" + n], ref)
        assert not bad.any(), f"{n}: {int(bad.sum())} elements beyond the bar"
    o = plan.view(saved, "o")[0]                                        # [H, N, d] bf16
    orows = bf16_tensor_to_f64(o[:, rows]).transpose(1, 0, 2).reshape(len(rows), H * d)
    y = r["y"][0][rows].double().cpu().numpy()
    ref = orows @ w64["wo"]
    err = np.abs(y - ref).max() / np.abs(ref).max()
    say(f"  Y rows: rel err {err:.3g}")
    assert err < 1e-4
    # dW_O columns: O^T dY over all 524,288 tokens, fp64 on the host in chunks
    dwq, dwk, dwv, dwo = (g.double().cpu().numpy() for g in r["grads"][1:])
    cols = np.sort(rng.choice(dm, size=8, replace=False))
    dy_bits = inp["dy"][0]
    acc = np.zeros((H * d, len(cols)))
    for t0 in range(0, N, 65536):
        oc = bf16_tensor_to_f64(o[:, t0:t0 + 65536]).transpose(1, 0, 2).reshape(-1, H * d)
        acc += oc.T @ synth.as_f64(dy_bits[t0:t0 + 65536][:, cols], "bf16")
    err = np.abs(dwo[:, cols] - acc).max() / np.abs(acc).max()
    say(f"  dW_O columns: rel err {err:.3g}")
    assert err < 1e-3
    # adjoint identities: fp64 inner products on the host, in chunks of tokens
    dx = r["grads"][0][0]
    y = r["y"][0]
    lhs_x = lhs_y = 0.0
    for t0 in range(0, N, 65536):
        xs = synth.as_f64(inp["x"][0][t0:t0 + 65536], "bf16")
        lhs_x += float(np.sum(dx[t0:t0 + 65536].double().cpu().numpy() * xs))
        dys = synth.as_f64(dy_bits[t0:t0 + 65536], "bf16")
        lhs_y += float(np.sum(y[t0:t0 + 65536].double().cpu().numpy() * dys))
    rhs_x = sum(float(np.sum(g * w)) for g, w in ((dwq, w64["wq"]), (dwk, w64["wk"]), (dwv, w64["wv"])))
    rhs_y = float(np.sum(dwo * w64["wo"]))
    say(f"  <dX, X> = {lhs_x:.6g}, sum <dW, W> = {rhs_x:.6g};  <dY, Y> = {lhs_y:.6g}, <dW_O, W_O> = {rhs_y:.6g}")
    assert abs(lhs_x - rhs_x) <= 1e-3 * (abs(lhs_x) + abs(rhs_x))
    assert abs(lhs_y - rhs_y) <= 1e-3 * (abs(lhs_y) + abs(rhs_y))
