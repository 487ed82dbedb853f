"""GPU parity of the forward: the HIP path (through the C ABI) against the fp64
oracle, stage by stage and end to end.

Bars (from the method's acceptance criteria and the arithmetic):
  scores               <= 1e-5 relative to the fp64 norms of the same inputs
  top-k flags          bit-exact when the oracle selects on the GPU's own scores
  order / slot map     bit-exact (integer work)
  gathered rows        level 0 bit-exact; pooled rows within one rounding of the
                       storage dtype (bf16: 2^-8 relative, fp32: 2e-6) of the fp64 mean
  O~, LSE              fp32 mode 1e-4 (the end-to-end fp32 bar: with rows scaled
                       x4 the logits reach |z| ~ 30, so fp32 logits carry ~1e-5
                       relative error into the softmax weights); bf16 mode
                       2^-8 max|V~| + 1e-4 (the P.V product takes P rounded to
                       bf16: each weight off by at most the bf16 unit roundoff
                       2^-8, relative, so |dO~| <= 2^-8 sum_j P_j |V~_j| <=
                       2^-8 max|V~|), against the oracle run on the GPU's own
                       gathered rows
  scatter              bit-exact against the oracle's fixed-point scatter of the
                       GPU's own O~
  O end to end         1e-4 max-abs (fp32) / 2e-2 max-abs (bf16) against the oracle
                       on the same inputs; in bf16 mode the oracle stores the
                       pooled levels in bf16 like the benchmarked bf16 layer
                       (store="bf16"), and the pure-fp64 error is printed too; if
                       fp64 and fp32 scores order a near-tie differently the
                       oracle is re-run with the GPU's selection injected (the
                       size of the difference is printed)
"""
import numpy as np
import pytest

import oracle as orc
from gpu_helpers import gpu_head, head_inputs_f64, run_forward, say, split_levels, to_dev
from hierarchical_sparse_attention_mean_amd import synth

pytestmark = pytest.mark.gpu

def stage_ot_tol(dt, vt):
    return 1e-4 if dt == "f32" else 2.0 ** -8 * float(np.max(np.abs(vt))) + 1e-4


LSE_TOL = {"f32": 1e-4, "bf16": 1e-3}
E2E_TOL = {"f32": 1e-4, "bf16": 2e-2}


def check_head(cfg, inp, g, h, L, p, topk, out_dtype="f32", full_attention=True, sample_rows=256, e2e=True,
               pure=True):
    N, dt = cfg["N"], cfg["dtype"]
    q64, k64, v64 = head_inputs_f64(cfg, inp, h)
    # ---- scores
    qk_o, kq_o = orc.scores(q64, k64, L, p)
    qk_g, kq_g = split_levels(g["qk_flat"], N, L, p), split_levels(g["kq_flat"], N, L, p)
    for a, b in zip(qk_o + kq_o, qk_g + kq_g):
        assert np.max(np.abs(a - b) / np.maximum(np.abs(a), 1e-30)) <= 1e-5
    # ---- selection on the GPU's own scores: bit-exact
    fl = orc.select(qk_g, kq_g, p, topk)
    assert np.array_equal(fl, g["flags"]), "top-k flags differ"
    # ---- order, slot map
    sf = orc.order(g["flags"], N, L, p)
    assert np.array_equal(sf, g["coords"]), "topological order differs"
    S = len(sf)
    assert np.array_equal(g["slot"][sf], np.arange(S))
    assert np.all(g["slot"][~g["flags"]] == -1)
    # ---- gathered rows
    lev, pos = orc.coords_of_flat(sf, N, L, p)
    rows = np.arange(S)
    for name, x in (("qt", q64), ("kt", k64), ("vt", v64)):
        ref = orc.gather(orc.pyramid(x, L, p), sf, N, L, p)
        got = g[name]
        base = lev == 0
        assert np.array_equal(got[base], ref[base]), f"{name}: level-0 rows not bit-exact"
        rel = 2.0 ** -8 if dt == "bf16" else 2e-6
        assert np.all(np.abs(got[~base] - ref[~base]) <= rel * np.abs(ref[~base]) + 1e-6), f"{name} pooled rows"
    for n in ("qt", "kt", "vt"):
        assert not np.any(g[n + "_pad"]), f"{n}: padding rows not zero"
    # ---- attention on the GPU's own gathered rows
    if full_attention:
        ot_ref, lse_ref = orc.attend(g["qt"], g["kt"], g["vt"])
    else:
        rng = np.random.default_rng(h)
        rows = np.unique(np.concatenate([[0, 1, S - 1], rng.integers(0, S, sample_rows)]))
        ot_ref, lse_ref = orc.attend_rows(g["qt"], g["kt"], g["vt"], rows)
    err_ot = np.max(np.abs(g["ot32"][rows].astype(np.float64) - ot_ref))
    err_lse = np.max(np.abs(g["lse"][rows] - lse_ref))
    say(f"  head {h}: S={S} |O~ - oracle(O~)|={err_ot:.3e} |LSE - oracle|={err_lse:.3e}")
    assert err_ot <= stage_ot_tol(dt, g["vt"])
    assert err_lse <= LSE_TOL[dt]
    # ---- scatter: bit-exact on the GPU's own O~
    o_fx = orc.scatter_fixed(g["ot32"].astype(np.float64), sf, N, L, p, out_dtype)
    assert np.array_equal(o_fx, g["o"]), "scatter not bit-exact"
    # ---- end to end
    if e2e:
        store = "bf16" if dt == "bf16" else None
        res = orc.forward_head(q64, k64, v64, L, p, topk, store=store)
        nd = int(np.sum(res["flags"] != g["flags"]))
        say(f"  head {h}: the oracle's own fp64-score selection differs from the GPU's in {nd} entries")
        if nd:
            res = orc.forward_head(q64, k64, v64, L, p, topk, flags=g["flags"], store=store)
        err = np.max(np.abs(res["o"] - g["o"]))
        msg = f"  head {h}: end-to-end |O - oracle O| = {err:.3e}"
        if store and pure:
            ref = orc.forward_head(q64, k64, v64, L, p, topk, flags=g["flags"])
            msg += f" (pure-fp64 pyramid: {np.max(np.abs(ref['o'] - g['o'])):.3e})"
        say(msg)
        assert err <= E2E_TOL[dt] + (2.0 ** -8 * np.max(np.abs(res["o"])) if out_dtype == "bf16" else 0.0)
    return S


def _run(lh, cfg, topk=None, L=None, p=None, out_dtype="f32", heads=None, **kw):
    L = cfg["L"] if L is None else L
    p = cfg["p"] if p is None else p
    topk = cfg["k"] if topk is None else topk
    say(f"case N={cfg['N']} H={cfg['H']} d={cfg['d']} L={L} p={p} k={topk} io={cfg['dtype']} out={out_dtype}")
    inp = synth.make_inputs(cfg)
    run = run_forward(lh, cfg, inp, out_dtype=out_dtype, topk=topk, L=L, p=p)
    BH = cfg["B"] * cfg["H"]
    for h in (range(BH) if heads is None else heads):
        g = gpu_head(lh, run, h)
        check_head(cfg, inp, g, h, L, p, topk, out_dtype=out_dtype, **kw)
    return run


def test_tiny_fp32(lh):
    run = _run(lh, synth.config("tiny"))
    assert run["plan"].S == 576


def test_tiny_fp32_bf16_output(lh):
    _run(lh, synth.config("tiny"), out_dtype="bf16")


def test_tiny_select_everything(lh):
    """k = N: every pyramid entry is selected, S = |P|."""
    run = _run(lh, synth.config("tiny"), topk=1024)
    assert run["plan"].S == 1344


def test_tiny_L1_dense(lh):
    """L = 1: the layer is dense causal attention over all N rows."""
    run = _run(lh, synth.config("tiny"), L=1)
    assert run["plan"].S == 1024


@pytest.mark.parametrize("N,L,p,k,B,H", [
    (1552, 3, 4, 40, 1, 2),     # 97 coarsest windows: ragged against every work-group tile
    (2048, 4, 2, 13, 2, 1),     # p = 2, four levels, B = 2
    (3072, 2, 4, 5, 1, 3),      # two levels
    (512, 3, 2, 0, 1, 1),       # k = 0: only the coarsest level
    (4096, 5, 2, 200, 1, 1),    # five levels
    (3328, 5, 4, 16, 1, 2),     # five levels, p = 4: coarsest windows split over row-groups, ragged last work-group
    (3240, 5, 3, 10, 1, 1),     # five levels, p = 3: coarsest windows walked whole
    (4096, 5, 8, 4, 1, 1),      # five levels, p = 8: one coarsest window walked by eight row-groups
    (1944, 3, 3, 20, 1, 2),     # p = 3: a pooling factor that is not a power of two
    (4096, 3, 8, 12, 1, 1),     # p = 8: both coarser levels shared by eight positions in the scatter
    (16, 3, 4, 1, 1, 1),        # one coarsest window (S = 9)
    (4, 2, 4, 0, 1, 1),         # N = p and k = 0: the single coarsest entry (S = 1)
    (6, 2, 2, 1, 1, 3),         # N = 6, p = 2, three heads (B*H not a multiple of 8)
])
def test_shapes_fp32(lh, N, L, p, k, B, H):
    cfg = synth.config("tiny", N=N, L=L, p=p, k=k, B=B, H=H, recipe="mod97x4")
    _run(lh, cfg)


@pytest.mark.parametrize("N,L,p,k,d", [
    (2048, 2, 4, 64, 64),    # two levels
    (4096, 5, 4, 8, 128),    # five levels, p = 4 (groups of four positions in the scatter)
    (2048, 6, 4, 4, 128),    # six levels: the widest level templates
    (1024, 8, 2, 4, 64),     # eight levels, p = 2
    (64, 3, 4, 3, 128),      # S = 28: less than one 32-row attention tile, rows padded to Sv = 64
])
def test_shapes_bf16(lh, N, L, p, k, d):
    """bf16 storage at the level counts the bf16 workloads do not reach, stage by stage."""
    _run(lh, synth.config("bwd8k", N=N, L=L, p=p, k=k, H=1, d=d))


@pytest.mark.parametrize("d", [64, 128])
def test_small_bf16(lh, d):
    cfg = synth.config("bwd8k", N=4096, H=2, d=d)
    _run(lh, cfg)


def test_ties_everywhere(lh):
    """Constant inputs: every score ties, the selection is decided by the
    lowest-stream-index rule alone."""
    cfg = synth.config("tiny", H=1)
    inp = synth.make_inputs(cfg)
    for n in ("q", "k"):
        inp[n][:] = 0.5
    run = run_forward(lh, cfg, inp)
    g = gpu_head(lh, run, 0)
    check_head(cfg, inp, g, 0, cfg["L"], cfg["p"], cfg["k"])
    E = orc.budget(cfg["N"], cfg["L"], cfg["p"], cfg["k"])
    assert np.array_equal(np.nonzero(g["flags"][:cfg["N"] + cfg["N"] // 4])[0], np.arange(E))


def _boundary_candidates(qk_flat, kq_flat, N, L, p, topk):
    """Keys in the top-k's boundary histogram bin, from the GPU's own scores:
    the same 12-bit digit of the score bits over the per-head [min, max]
    range that the kernels use (coverage probe for the refine paths)."""
    n = [N // p ** l for l in range(L)]
    E = sum(n[:-1])
    bsel = min((L - 1) * p * topk, E)
    hi = np.maximum(qk_flat[:E], kq_flat[:E]).astype(np.float32).view(np.uint32).astype(np.int64)
    umin, umax = int(hi.min()), int(hi.max())
    sh = 0
    while ((umax - umin) >> sh) >= 4096:
        sh += 1
    hist = np.bincount((hi - umin) >> sh, minlength=4096)
    above = np.cumsum(hist[::-1])[::-1] - hist   # keys in higher bins
    b = int(np.nonzero((above < bsel) & (above + hist >= bsel))[0][0])
    return int(hist[b])


@pytest.mark.parametrize("N,frac,topk,lo,hi", [
    (16384, 0.01, 16, 1, 1024),
    (16384, 0.05, 128, 1025, 2048),
    (16384, 0.10, 256, 2049, 4096),
    (16384, 0.20, 256, 4097, 8192),
    (16384, 0.50, 256, 8193, 16384),        # up to the most candidates ranked in LDS
    (65536, 0.50, 256, 16385, 1 << 30),     # more than LDS holds: radix passes over the list
])
def test_topk_dense_boundary_bin(lh, N, frac, topk, lo, hi):
    """Scores with two values only: Q_t = c_t u with c_t in {1, 2} (a seeded
    fraction `frac` of rows get 2), K_t = u / 4, so every key's score is |u| or
    2|u| exactly and the boundary bin holds every entry scoring 2|u|.  Its size
    (checked from the GPU's scores) steers the refine through candidate lists
    of every size its LDS ranking takes, and past them into the radix path; the
    selection must still be bit-exact."""
    cfg = synth.config("tiny", N=N, H=1, k=topk)
    inp = synth.make_inputs(cfg)
    u = (np.linspace(0.5, 1.5, cfg["d"]) / 8).astype(np.float32)
    c = np.where(np.random.default_rng(7).random(cfg["N"]) < frac, 2.0, 1.0).astype(np.float32)
    inp["q"][0, 0] = c[:, None] * u[None, :]
    inp["k"][0, 0] = u[None, :] / 4
    run = run_forward(lh, cfg, inp)
    g = gpu_head(lh, run, 0)
    C = _boundary_candidates(g["qk_flat"], g["kq_flat"], cfg["N"], cfg["L"], cfg["p"], topk)
    say(f"  boundary bin: {C} candidates")
    assert lo <= C <= hi
    check_head(cfg, inp, g, 0, cfg["L"], cfg["p"], topk, full_attention=False, sample_rows=128)


def test_98k_bf16(lh):
    """98K training shape (all 8 heads run; three checked): selection, order and
    scatter exact, attention on sampled rows, and the whole output of each
    checked head end to end against the oracle's fp64 forward (2e-2 bar), with
    the size of the oracle's own selection difference printed."""
    cfg = synth.config("98k")
    _run(lh, cfg, full_attention=False, sample_rows=192, e2e=True, heads=[0, 3, 7])


@pytest.mark.parametrize("L,p,k,e2e", [
    (3, 2, 1536, True),    # p = 2: pooling fan-in 2, up to 3 contributors per position (S = 30,720)
    (5, 2, 2048, True),    # five levels (S = 22,528)
    (4, 4, 3072, False),   # S = 38,400
    (3, 4, 6144, False),   # the largest k of the pages' grid (S = 55,296)
])
def test_ablation_grid_98k_bf16(lh, L, p, k, e2e):
    """Shapes of the pages' ablation grid at N = 98,304 (one head): selection,
    order and scatter exact; attention on sampled rows; the whole output end to
    end where the oracle's forward fits the test's time (S <= 30,720)."""
    cfg = synth.config("98k", H=1, L=L, p=p, k=k)
    _run(lh, cfg, full_attention=False, sample_rows=128, e2e=e2e, pure=False)


def test_deterministic(lh):
    import torch
    cfg = synth.config("bwd8k", N=16384)
    inp = synth.make_inputs(cfg)
    a = run_forward(lh, cfg, inp, out_dtype="bf16")
    b = run_forward(lh, cfg, inp, out_dtype="bf16")
    assert torch.equal(a["o"].view(torch.int16), b["o"].view(torch.int16))
    for n in ("scores", "flags", "slot", "coords", "qt", "kt", "vt", "ot", "lse"):
        x = lh.saved_view(a["saved"], a["plan"], n)
        y = lh.saved_view(b["saved"], b["plan"], n)
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), n


@pytest.mark.parametrize("N,L,p,k", [(1024, 3, 4, 64), (1024, 3, 4, 8), (1024, 3, 8, 4), (1944, 3, 3, 64),
                                     (1024, 4, 2, 64)])
def test_scatter_large_values(lh, N, L, p, k):
    """Sub-sequence outputs of magnitude >= 2^18 make the scatter form its
    fixed-point sums in int64 instead of fp64; the result stays bit-exact.
    V is scaled by 2^20 on half of the positions, so both forms occur.  p = 4,
    p = 2 and p = 3 take the scatter's thread layouts (groups of four positions
    sharing their coarser entries, the same with one level-1 entry per pair,
    one position per thread).  At p >= 4 a budget >= N / 4 (k = 64) takes the
    one-pass kernel and a smaller one the two passes, whose coarse pass has a
    per-group level at p = 4 and none at p = 8; p = 2 always takes one pass."""
    cfg = synth.config("tiny", N=N, L=L, p=p, k=k)
    inp = synth.make_inputs(cfg)
    N, L, p = cfg["N"], cfg["L"], cfg["p"]
    inp["v"] = inp["v"].copy()
    inp["v"][..., N // 2:, :] *= 2.0 ** 20
    run = run_forward(lh, cfg, inp)
    for h in range(cfg["B"] * cfg["H"]):
        g = gpu_head(lh, run, h)
        big = np.abs(g["ot32"]) >= 2.0 ** 18
        assert big.any() and (~big).any()
        o_fx = orc.scatter_fixed(g["ot32"].astype(np.float64), g["coords"], N, L, p, "f32")
        assert np.array_equal(o_fx, g["o"]), "scatter not bit-exact"


def test_binding_refuses_mismatched_operands(lh):
    """Operands the kernels would misread are refused by the binding: another
    dtype or shape than q, a plan made for another problem, host buffers."""
    import torch
    cfg = synth.config("bwd8k", N=2048, H=2)
    inp = synth.make_inputs(cfg, with_do=True)
    run = run_forward(lh, cfg, inp)
    q, k, v = run["q"], run["k"], run["v"]
    L, p, topk = cfg["L"], cfg["p"], cfg["k"]
    with pytest.raises(ValueError, match="dtype"):
        lh.forward(q, k.float(), v, L, p, topk)
    with pytest.raises(ValueError, match="shape"):
        lh.forward(q, k, v[:, :1].contiguous(), L, p, topk)
    other = lh.Plan(cfg["B"], cfg["H"], 4096, cfg["d"], L, p, topk, q.dtype)
    with pytest.raises(ValueError, match="plan"):
        lh.forward(q, k, v, L, p, topk, plan=other)
    dout = to_dev(inp["do"], cfg["dtype"])
    with pytest.raises(ValueError, match="device"):
        lh.backward(q, k, v, dout.cpu(), run["saved"], run["plan"])
    with pytest.raises(ValueError, match="device"):
        lh.backward(q, k, v, dout, run["saved"].cpu(), run["plan"])
    with pytest.raises(ValueError, match="plan"):
        lh.backward(q, k, v, dout, run["saved"], other)
