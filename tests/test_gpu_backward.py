"""GPU parity of the backward (selection frozen, indices carry no gradient).

Two references, both the fp64 oracle with the GPU's selection injected:
  * stage-consistent: the oracle's adjoints (scatter, attention, gather, pool)
    evaluated on the GPU's own gathered rows, so only the kernels' arithmetic
    differs -- bar (relative to the gradient's largest magnitude) 1e-5 in fp32
    mode (fp32 accumulation over <= S terms) and 3 * 2^-8 in bf16 mode: the
    bf16 MFMA backward takes three operands rounded to bf16 (P, dS and dO~, each
    within the bf16 unit roundoff 2^-8, relative), and consumes the forward's O~
    and LSE, computed from bf16-rounded probabilities;
  * end to end: the oracle's own pyramid and backward -- bar 2e-2 of the
    gradient's largest magnitude, the forward's bf16 bar applied to the
    gradients' scale.  In bf16 mode the oracle differentiates its bf16-mode
    forward (pooled levels stored in bf16, store="bf16"), the forward whose
    output the forward tests compare; the error against the pure-fp64 pyramid
    is printed as well.
At full size, properties that hold at any size: exact scaling by 2,
run-to-run bit equality, finite values.
"""
import numpy as np
import pytest

import oracle as orc
from gpu_helpers import bf16_tensor_to_f64, gpu_head, head_inputs_f64, run_forward, say, to_dev
from hierarchical_sparse_attention_mean_amd import synth

pytestmark = pytest.mark.gpu

STAGE_TOL = {"f32": 1e-5, "bf16": 3 * 2.0 ** -8}
E2E_TOL = 2e-2


def _grads_stage_consistent(g, do64, N, L, p):
    """Oracle adjoints on the GPU's own gathered rows."""
    sf = g["coords"]
    dot = orc.scatter_adjoint(do64, sf, N, L, p)
    dqt, dkt, dvt = orc.attend_adjoint(g["qt"], g["kt"], g["vt"], dot)
    lev, pos = orc.coords_of_flat(sf, N, L, p)
    sizes = orc.level_sizes(N, L, p)
    out = []
    for dt in (dqt, dkt, dvt):
        dl = [np.zeros((n, dt.shape[1])) for n in sizes]
        for m in range(len(sf)):
            dl[lev[m]][pos[m]] = dt[m]
        out.append(orc.pool_adjoint(dl, N, p))
    return out


def _run_bwd(lh, cfg, heads, grad_dtype="f32", pure=True):
    import torch
    say(f"case bwd N={cfg['N']} H={cfg['H']} d={cfg['d']} L={cfg['L']} p={cfg['p']} k={cfg['k']} io={cfg['dtype']}")
    inp = synth.make_inputs(cfg, with_do=True)
    run = run_forward(lh, cfg, inp)
    dout = to_dev(inp["do"], cfg["dtype"])
    gdt = torch.float32 if grad_dtype == "f32" else torch.bfloat16
    dq, dk, dv = lh.backward(run["q"], run["k"], run["v"], dout, run["saved"], run["plan"], grad_dtype=gdt)
    torch.cuda.synchronize()
    N, L, p, H = cfg["N"], cfg["L"], cfg["p"], cfg["H"]
    for h in heads:
        b, hh = divmod(h, H)
        g = gpu_head(lh, run, h)
        q64, k64, v64 = head_inputs_f64(cfg, inp, h)
        do64 = synth.as_f64(inp["do"][b, hh], cfg["dtype"])
        got = [bf16_tensor_to_f64(x[b, hh]) for x in (dq, dk, dv)]
        ref_s = _grads_stage_consistent(g, do64, N, L, p)
        store = "bf16" if cfg["dtype"] == "bf16" else None
        ref_e = orc.backward_head(q64, k64, v64, do64, L, p, g["flags"], store=store)
        ref_p = orc.backward_head(q64, k64, v64, do64, L, p, g["flags"]) if store and pure else None
        for i, (name, a, rs, re) in enumerate(zip(("dq", "dk", "dv"), got, ref_s, ref_e)):
            scale = np.max(np.abs(re))
            es = np.max(np.abs(a - rs)) / scale
            ee = np.max(np.abs(a - re)) / scale
            msg = f"  head {h} {name}: max|g|={scale:.3e} stage err={es:.3e} end-to-end err={ee:.3e}"
            if ref_p is not None:
                msg += f" (pure-fp64 pyramid: {np.max(np.abs(a - ref_p[i])) / scale:.3e})"
            say(msg)
            extra = 2.0 ** -8 if grad_dtype == "bf16" else 0.0
            assert es <= STAGE_TOL[cfg["dtype"]] + extra
            assert ee <= E2E_TOL + extra
    return run, dq, dk, dv


def test_backward_tiny_fp32(lh):
    _run_bwd(lh, synth.config("tiny"), heads=[0, 1])


def test_backward_8k_bf16(lh):
    _run_bwd(lh, synth.config("bwd8k"), heads=[0, 5])


def test_backward_8k_select_all(lh):
    """k = 4096 at N = 8192: every entry selected (S = |P|)."""
    _run_bwd(lh, synth.config("bwd8k", k=4096, H=2), heads=[1])


def test_backward_shapes(lh):
    _run_bwd(lh, synth.config("tiny", N=2048, L=4, p=2, k=13, B=2, H=1, d=128), heads=[0, 1])
    _run_bwd(lh, synth.config("tiny", N=1552, L=3, p=4, k=40, H=1), heads=[0], grad_dtype="bf16")
    _run_bwd(lh, synth.config("tiny", N=1944, L=3, p=3, k=20, H=1), heads=[0])   # p not a power of two
    # ranges of 64 rows (level 3): the long-range pass of the scatter adjoint, fp32 path
    _run_bwd(lh, synth.config("tiny", N=4096, L=4, p=4, k=16, H=1), heads=[0])


def test_backward_degenerate_shapes(lh):
    """Smallest shapes: one coarsest window (N = 16, S = 9), three heads of
    N = 6 at p = 2 (S = 5), and a bf16 sub-sequence shorter than one 32-row
    attention tile (N = 64, S = 28, rows padded to Sv = 64)."""
    _run_bwd(lh, synth.config("tiny", N=16, L=3, p=4, k=1, H=1), heads=[0])
    _run_bwd(lh, synth.config("tiny", N=6, L=2, p=2, k=1, H=3), heads=[0, 2])
    _run_bwd(lh, synth.config("bwd8k", N=64, L=3, p=4, k=3, H=1), heads=[0])


@pytest.mark.parametrize("over", [
    dict(N=2048, H=2, d=64),                  # bf16 MFMA backward at d = 64
    dict(N=2048, L=4, p=2, k=16, H=1, d=64),  # p = 2: the one-position-per-thread scatter and pool adjoints
    dict(N=2048, L=5, p=4, k=8, H=1),         # five levels
    dict(N=2048, L=6, p=4, k=2, H=1),         # six levels (the widest level template)
], ids=["d64", "p2-L4", "L5", "L6"])
def test_backward_shapes_bf16(lh, over):
    _run_bwd(lh, synth.config("bwd8k", **over), heads=[0])


@pytest.mark.parametrize("L,p,k", [(3, 2, 1536), (5, 4, 1536), (4, 4, 1536)],
                         ids=["L3-p2-k1536", "L5-p4-k1536", "L4-p4-k1536"])
def test_backward_ablation_grid_98k(lh, L, p, k):
    """Backward parity at cells of the pages' ablation grid at the training shape
    N = 98,304 (one head, d = 128, bf16; S = 30,720, 24,960 and 19,968): the
    whole head's dQ, dK, dV against the oracle with the GPU's selection injected,
    stage-consistent and end to end."""
    _run_bwd(lh, synth.config("98k", H=1, L=L, p=p, k=k), heads=[0], pure=False)


def test_backward_properties_scale_and_determinism(lh):
    import torch
    cfg = synth.config("bwd8k", N=65536, H=2)
    inp = synth.make_inputs(cfg, with_do=True)
    run = run_forward(lh, cfg, inp)
    dout = to_dev(inp["do"], cfg["dtype"])
    g1 = lh.backward(run["q"], run["k"], run["v"], dout, run["saved"], run["plan"], grad_dtype=torch.float32)
    g2 = lh.backward(run["q"], run["k"], run["v"], dout * 2, run["saved"], run["plan"], grad_dtype=torch.float32)
    g3 = lh.backward(run["q"], run["k"], run["v"], dout, run["saved"], run["plan"], grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for a, b, c in zip(g1, g2, g3):
        assert torch.isfinite(a).all()
        assert torch.equal(a, c)
        assert torch.equal(2 * a, b)


def test_stage_timing_leaves_results_unchanged(lh):
    """Stage timing (events around each stage's launches) changes no output
    bit, and records every stage of the forward and the backward."""
    import torch
    cfg = synth.config("bwd8k", N=65536, H=2)
    inp = synth.make_inputs(cfg, with_do=True)
    run = run_forward(lh, cfg, inp)
    dout = to_dev(inp["do"], cfg["dtype"])
    g1 = lh.backward(run["q"], run["k"], run["v"], dout, run["saved"], run["plan"], grad_dtype=torch.float32)
    o1 = run["o"].clone()
    torch.cuda.synchronize()
    assert lh.lh_timing_begin() == 0
    run2 = run_forward(lh, cfg, inp)
    g2 = lh.backward(run2["q"], run2["k"], run2["v"], dout, run2["saved"], run2["plan"], grad_dtype=torch.float32)
    st, stages = lh.lh_timing_end()
    assert st == 0, lh.lh_last_error()
    torch.cuda.synchronize()
    assert torch.equal(o1, run2["o"])
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    layer_stages = {"proj", "out_proj", "out_proj_bwd", "proj_bwd"}   # only the projection-inclusive layer runs these
    for name, (ms, spans) in stages.items():
        say(f"  stage {name}: {spans} spans, {ms:.3f} ms")
        if name in layer_stages:
            assert spans == 0, name
        else:
            assert spans == 1 and ms > 0, name
    # switched off again: a further call records nothing
    lh.lh_timing_begin()
    st, stages = lh.lh_timing_end()
    assert st == 0 and all(s == 0 for _, s in stages.values())


def test_concurrent_streams(lh):
    """Forward and backward in flight on two streams at once, each call with its
    own buffers: the library keeps no shared mutable state, so both streams'
    outputs and gradients equal those of a lone run bit for bit."""
    import torch
    cfg = synth.config("bwd8k", N=16384, H=2)
    inp = synth.make_inputs(cfg, with_do=True)
    ref = run_forward(lh, cfg, inp, out_dtype="bf16")
    q, k, v = ref["q"], ref["k"], ref["v"]
    dout = to_dev(inp["do"], cfg["dtype"])
    g_ref = lh.backward(q, k, v, dout, ref["saved"], ref["plan"], grad_dtype=torch.float32)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    runs = []
    for st in streams:
        with torch.cuda.stream(st):
            o, saved, plan = lh.forward(q, k, v, cfg["L"], cfg["p"], cfg["k"], out_dtype=torch.bfloat16)
            g = lh.backward(q, k, v, dout, saved, plan, grad_dtype=torch.float32)
            runs.append((o, g))
    torch.cuda.synchronize()
    for o, g in runs:
        assert torch.equal(o.view(torch.int16), ref["o"].view(torch.int16))
        for a, b in zip(g, g_ref):
            assert torch.equal(a, b)


def test_autograd_transposed_inputs(lh):
    """LighthouseAttention through torch.autograd on [B, N, H, d] tensors viewed
    as [B, H, N, d] (non-contiguous), with a non-contiguous upstream gradient
    too: the output and the gradients equal those of lh.forward / lh.backward on
    contiguous copies, bit for bit (the kernels are deterministic)."""
    import torch
    cfg = synth.config("bwd8k", N=4096, H=2)
    inp = synth.make_inputs(cfg, with_do=True)
    q, k, v, do = (to_dev(inp[n], cfg["dtype"]) for n in ("q", "k", "v", "do"))
    L, p, topk = cfg["L"], cfg["p"], cfg["k"]
    o_ref, saved, plan = lh.forward(q, k, v, L, p, topk)
    g_ref = lh.backward(q, k, v, do, saved, plan)
    # leaves stored as [B, N, H, d]; the layer sees their [B, H, N, d] transposes
    base = [x.transpose(1, 2).contiguous().requires_grad_(True) for x in (q, k, v)]
    views = [b.transpose(1, 2) for b in base]
    assert not any(x.is_contiguous() for x in views)
    o = lh.LighthouseAttention.apply(*views, L, p, topk)
    do_view = do.transpose(1, 2).contiguous().transpose(1, 2)
    assert not do_view.is_contiguous()
    o.backward(do_view)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    for b, ref in zip(base, g_ref):
        assert b.grad.shape == b.shape
        assert torch.equal(b.grad.transpose(1, 2).contiguous().view(torch.int16), ref.view(torch.int16))
