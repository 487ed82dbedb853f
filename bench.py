"""Benchmark of the Lighthouse attention layer on one MI355X.

One step = the whole layer: forward (pool+score, top-k, compaction+gather,
sub-sequence attention, scatter) and backward (scatter adjoint, attention
backward, gather+pool adjoint) for one batch of seeded synthetic bf16 inputs
already resident in HBM.  Default workload: B=1, H=8, d=128, N=524,288, L=3,
p=4, k=4,096 (S=65,536).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 512k] [--no-dense] [--layer]
    python bench.py --ablation [--steps K] [--warmup W]     (the ablation grid at N = 98,304)

Prints one JSON line (rank 0).  Besides the contract fields it carries:
  roofline      the dominant kernel of the step (by time): its algorithmic FLOPs
                per launch / its mean launch time, from the library's stage
                timing (HIP events recorded around each launch on the stream it
                runs on, over the timed steps); `traffic` is the kernel's HBM
                bytes per launch from hardware counters (profiles/), or null
                when the kernel's sources changed since the counters were taken
  cpu_baseline  the fp64 oracle on one head of the same workload (fwd + bwd),
                on this host's cores, scaled to the layer's tokens/s
  extra         per-stage times (with algorithmic bytes and achieved GB/s for the
                memory-bound stages), forward-only time, the attention backward's
                algorithmic rate (its 5 products over the dQ and dK/dV kernels'
                time, which execute 7), the dense causal
                attention kernels at S = N (one forward and one backward; skipped
                with --no-dense), and (with --layer) the
                projection-inclusive layer (X -> W_Q, W_K, W_V -> Lighthouse ->
                W_O, forward and backward) at d_model = 1024 with the TFLOP/s of
                its four product stages
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_flops(S: int, d: int, BH: int, products: int = 2) -> float:
    """Algorithmic FLOPs of causal attention over S rows: `products` d-long
    multiply-add contractions per causal (query, key) pair, S (S+1) / 2 pairs
    per head, 2 FLOPs per multiply-add.  Forward: Q.K^T and P.V (2); dQ~:
    S, dP, dS.K (3); dK~/dV~: S, dP, P^T.dO, dS^T.Q (4)."""
    return 2.0 * products * (S * (S + 1) / 2.0) * d * BH


# stage -> (matmul products per causal pair, kernel sources) for the MFMA stages
ATTN_STAGES = {
    "attn_fwd": (2, ["k_attn_mfma.hip", "attn_tiles.h"]),
    "attn_bwd_dq": (3, ["k_attn_mfma_bwd.hip", "attn_tiles.h"]),
    "attn_bwd_dkdv": (4, ["k_attn_mfma_bwd.hip", "attn_tiles.h"]),
}


def hbm_stage_bytes(cfg: dict, S: int) -> dict:
    """Algorithmic HBM bytes of the memory-bound stages for one step: what each
    stage must read and write once (bf16 or fp32 storage of Q, K, V, O and the
    gradients as the workload has it; O~, dQ~, dK~, dV~ in fp32; scores fp32,
    read by the top-k's histogram and filter passes; flags 1 byte; slot map and
    coordinates 4 bytes)."""
    B, H, N, d, L, p = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["L"], cfg["p"]
    BH = B * H
    io = 2 if cfg["dtype"] == "bf16" else 4
    n = [N // p ** l for l in range(L)]
    P, E = sum(n), sum(n[:-1])
    Sv = (S + 63) // 64 * 64
    r16, r32 = d * io, d * 4
    return {
        "pool_score": BH * (3 * N * r16 + 3 * sum(n[1:]) * r16 + 2 * P * 4),
        "topk": BH * (2 * E * 2 * 4 + P),
        "gather": BH * (2 * P + P * 4 + S * 4 + 2 * 3 * S * r16),
        "scatter": BH * (S * r32 + P * 4 + N * r16),
        "scatter_bwd": BH * (N * r16 + S * r32 + 2 * S * 4 + Sv * r16 + Sv * 8),
        "pool_bwd": BH * (3 * S * r32 + P * 4 + 3 * N * r16),
    }


def sources_sha256(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "hierarchical_sparse_attention_mean_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(stage: str, config: str):
    """HBM bytes per launch of a stage's kernel from its committed counter
    summary (profiles/<stage>_<config>_pmc.md), or None if there is none or the
    kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{config}_pmc.md")
    if stage not in ATTN_STAGES or not os.path.exists(path):
        return None
    text = open(path).read()
    m = {k: re.search(rf"^{k}:\s*(\S+)", text, re.M) for k in ("source_sha256", "fetch_bytes_per_launch",
                                                               "write_bytes_per_launch")}
    if not all(m.values()) or m["source_sha256"].group(1) != sources_sha256(ATTN_STAGES[stage][1]):
        return None
    return float(m["fetch_bytes_per_launch"].group(1)) + float(m["write_bytes_per_launch"].group(1))


def time_lighthouse(lh, torch, x, cfg: dict, steps: int, warmup: int, copy_mib: int = 0) -> dict:
    """Times the layer (forward + backward) of workload `cfg` on the resident
    inputs x = (q, k, v, dO): `warmup` untimed steps, then `steps` timed ones
    with the library's stage timing on, then `steps` forward-only ones.
    Returns S, ms per step, forward-only ms and the per-stage records (ms per
    step and per launch; TFLOP/s of the MFMA stages; algorithmic bytes, GB/s
    and fraction of the HBM peak of the memory-bound stages).  `copy_mib` runs
    one plain device copy of that size before the timed steps (a known-size
    reference dispatch for hardware byte counters)."""
    q, kk, v, do = x
    B, H, N, d, L, p, k = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["L"], cfg["p"], cfg["k"]
    BH, io, dev = B * H, q.dtype, q.device
    plan = lh.Plan(B, H, N, d, L, p, k, io)
    S = plan.S
    o = torch.empty((B, H, N, d), dtype=io, device=dev)
    dq, dk, dv = (torch.empty((B, H, N, d), dtype=io, device=dev) for _ in range(3))
    saved = torch.empty(plan.saved_bytes, dtype=torch.uint8, device=dev)
    fws = torch.empty(plan.fwd_ws_bytes, dtype=torch.uint8, device=dev)
    bws = torch.empty(plan.bwd_ws_bytes, dtype=torch.uint8, device=dev)
    a7 = plan.args()

    def fwd():
        st = lh.lh_forward(q, kk, v, o, io, *a7[:7], a7[7], saved, saved.numel(), fws, fws.numel())
        if st:
            raise lh.LighthouseError(st, "lh_forward")

    def bwd():
        st = lh.lh_backward(q, kk, v, do, io, saved, saved.numel(), dq, dk, dv, io, *a7[:7], a7[7], bws,
                            bws.numel())
        if st:
            raise lh.LighthouseError(st, "lh_backward")

    for i in range(warmup):
        fwd()
        bwd()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{warmup} done")
    if copy_mib:
        src = torch.ones(copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy: {copy_mib} MiB read, {copy_mib} MiB written")
        del src, dst
    torch.cuda.synchronize()
    lh.lh_timing_begin()   # events around each stage's launches, on their stream
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
        bwd()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st, stages = lh.lh_timing_end()
    if st:
        raise lh.LighthouseError(st, "lh_timing_end")
    ms = (t1 - t0) * 1e3 / steps
    log(f"[bench] {steps} steps: {ms:.3f} ms/step")
    stage_ms = {n: {"ms_per_step": t / steps, "ms_per_launch": t / c if c else None, "launches_per_step": c / steps}
                for n, (t, c) in stages.items()}
    for n, rec in stage_ms.items():
        log(f"[bench]   {n:14s} {rec['ms_per_step']:8.3f} ms/step")

    # forward alone
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    ms_fwd = (time.perf_counter() - t0) * 1e3 / steps
    log(f"[bench] forward only: {ms_fwd:.3f} ms")

    for n in ATTN_STAGES:
        rec = stage_ms[n]
        if rec["ms_per_launch"]:
            rec["tflops"] = attention_flops(S, d, BH, ATTN_STAGES[n][0]) / (rec["ms_per_launch"] * 1e-3) / 1e12
    for n, nbytes in hbm_stage_bytes(cfg, S).items():
        rec = stage_ms[n]
        if rec["ms_per_step"] > 0:
            rec["algorithmic_bytes"] = nbytes
            rec["gbs"] = nbytes / (rec["ms_per_step"] * 1e-3) / 1e9
            rec["frac_of_hbm_peak"] = rec["gbs"] / PEAK_HBM_GBS
            log(f"[bench]   {n:14s} {rec['gbs']:8.0f} GB/s ({rec['frac_of_hbm_peak']:.0%} of {PEAK_HBM_GBS:.0f})")
    return {"S": S, "ms": ms, "ms_fwd": ms_fwd, "stages": stage_ms}


def resident_inputs(torch, np, synth, cfg: dict, name: str, dev):
    """The workload's seeded q, k, v, dO as device tensors (bf16 or fp32)."""
    log(f"[bench] generating {name} inputs (B={cfg['B']} H={cfg['H']} N={cfg['N']} d={cfg['d']})")
    t0 = time.perf_counter()
    inp = synth.make_inputs(cfg, with_do=True)
    out = []
    for n in ("q", "k", "v", "do"):
        a = inp.pop(n)
        if cfg["dtype"] == "bf16":
            out.append(torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev))
        else:
            out.append(torch.from_numpy(a).to(dev))
        del a
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")
    return tuple(out)


# The pages' ablation axes -- budget k, pooling factor p, levels L -- each varied
# on its own around one default cell (L = 3, p = 4, k = 1536), at the training
# shape N = 98,304, B = 1, H = 8, d = 128, bf16.  The p = 2 axis is taken at both
# budgets the pages name for it (1536 and 4096).
ABLATION_GRID = [
    (3, 4, 1536), (3, 4, 2048), (3, 4, 3072), (3, 4, 4096), (3, 4, 6144),
    (3, 2, 1536), (3, 2, 4096),
    (4, 4, 1536), (5, 4, 1536),
]


def run_ablation(args, torch, np, lh, synth) -> int:
    """Forward + backward over ABLATION_GRID on the same resident inputs; one
    JSON line whose value is the default cell's tokens/s and whose extra.grid
    holds every cell (S, ms per step, forward ms, tokens/s, TFLOP/s of the
    attention kernels, fraction of the HBM peak of the memory-bound stages)."""
    base = synth.config("98k")
    B, N = base["B"], base["N"]
    x = resident_inputs(torch, np, synth, base, "98k", torch.device("cuda:0"))
    grid = []
    for L, p, k in ABLATION_GRID:
        cfg = synth.config("98k", L=L, p=p, k=k)
        log(f"[bench] ablation cell L={L} p={p} k={k}")
        r = time_lighthouse(lh, torch, x, cfg, args.steps, args.warmup)
        st = r["stages"]
        grid.append({"L": L, "p": p, "k": k, "S": r["S"], "ms_per_step": r["ms"], "ms_forward": r["ms_fwd"],
                     "tokens_per_s": B * N / (r["ms"] * 1e-3),
                     "attn_tflops": {n: st[n].get("tflops") for n in ATTN_STAGES},
                     "hbm_frac_of_peak": {n: st[n].get("frac_of_hbm_peak") for n in hbm_stage_bytes(cfg, r["S"])}})
    d0 = grid[0]
    line = {
        "metric": "Lighthouse fwd+bwd tokens/s over the ablation grid at N=98,304, H=8, d=128",
        "value": d0["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": d0["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Lighthouse layer fwd+bwd over the ablation grid (L, p, k) at B=1 H=8 d=128 "
                               "N=98304; value at L=3 p=4 k=1536", "B": B, "H": base["H"], "d": base["d"], "N": N},
        "roofline": None,
        "cpu_baseline": None,
        "extra": {"grid": grid},
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline(cfg: dict) -> dict:
    """The oracle as it stands, on head 0 of the workload, forward + backward."""
    import numpy as np

    import oracle as orc
    from hierarchical_sparse_attention_mean_amd import synth

    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    cores = blas or affinity   # the BLAS products are the oracle's only multi-threaded work
    one = synth.make_inputs(cfg, with_do=True, heads=[0])
    q, k, v, do = (synth.as_f64(one[n][0], cfg["dtype"]) for n in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    res = orc.forward_head(q, k, v, cfg["L"], cfg["p"], cfg["k"])
    t1 = time.perf_counter()
    orc.backward_head(q, k, v, do, cfg["L"], cfg["p"], res["flags"])
    t2 = time.perf_counter()
    per_head = t2 - t0
    layer_s = per_head * cfg["B"] * cfg["H"]
    return {"value": cfg["B"] * cfg["N"] / layer_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_count": os.cpu_count(), "affinity_cores": affinity, "blas_threads": blas,
            "sample": f"head 0 of {cfg['B'] * cfg['H']}, full forward ({t1 - t0:.1f} s) + backward ({t2 - t1:.1f} s) "
                      f"in fp64 numpy; layer time = per-head time x {cfg['B'] * cfg['H']} heads",
            "ms_per_step": layer_s * 1e3}


def layer_flops(N: int, dm: int, Hd: int) -> dict:
    """Algorithmic FLOPs of the layer's product stages (2 per multiply-add):
    proj [Q K V] = X W (N x d_model x 3 H d); out_proj Y = O W_O (N x H d x
    d_model); out_proj_bwd dO = dY W_O^T and dW_O = O^T dY; proj_bwd dX =
    [dQ dK dV] W^T and dW = X^T [dQ dK dV]."""
    return {"proj": 2.0 * N * dm * 3 * Hd, "out_proj": 2.0 * N * Hd * dm,
            "out_proj_bwd": 2 * 2.0 * N * Hd * dm, "proj_bwd": 2 * 2.0 * N * dm * 3 * Hd}


def time_layer(lh, synth, cfg: dict, args, dev) -> dict:
    """Forward + backward of the projection-inclusive layer on the same workload
    (bf16 x, weights, y, dy, dx; fp32 weight gradients)."""
    import numpy as np
    import torch
    B, H, N, d, dm = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["d_model"]
    t0 = time.perf_counter()
    inp = synth.layer_inputs(cfg, with_dy=True)
    bf = cfg["dtype"] == "bf16"
    io = torch.bfloat16 if bf else torch.float32
    t = {n: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if bf else torch.from_numpy(a)).to(dev)
         for n, a in inp.items()}
    del inp
    log(f"[bench] layer inputs resident in HBM (d_model={dm}, {time.perf_counter() - t0:.1f} s)")
    plan = lh.LayerPlan(B, H, N, dm, d, cfg["L"], cfg["p"], cfg["k"], io)
    y = torch.empty((B, N, dm), dtype=io, device=dev)
    dx = torch.empty((B, N, dm), dtype=io, device=dev)
    dws = [torch.empty(w.shape, dtype=torch.float32, device=dev) for w in (t["wq"], t["wk"], t["wv"], t["wo"])]
    saved = torch.empty(plan.saved_bytes, dtype=torch.uint8, device=dev)
    fws = torch.empty(plan.fwd_ws_bytes, dtype=torch.uint8, device=dev)
    bws = torch.empty(plan.bwd_ws_bytes, dtype=torch.uint8, device=dev)
    w = (t["x"], t["wq"], t["wk"], t["wv"], t["wo"])

    def fwd():
        st = lh.lh_layer_forward(*w, y, io, *plan.args(), saved, saved.numel(), fws, fws.numel())
        if st:
            raise lh.LighthouseError(st, "lh_layer_forward")

    def bwd():
        st = lh.lh_layer_backward(*w, t["dy"], saved, saved.numel(), dx, io, *dws, *plan.args(), bws, bws.numel())
        if st:
            raise lh.LighthouseError(st, "lh_layer_backward")

    for i in range(max(1, args.warmup)):
        fwd()
        bwd()
        torch.cuda.synchronize()
    log("[bench] layer warmup done")
    lh.lh_timing_begin()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    st, stages = lh.lh_timing_end()
    if st:
        raise lh.LighthouseError(st, "lh_timing_end")
    fl = layer_flops(B * N, dm, H * d)
    out = {"ms_per_step": ms, "tokens_per_s": B * N / (ms * 1e-3), "d_model": dm, "stages": {}}
    for n, (tm, c) in stages.items():
        rec = {"ms_per_step": tm / args.steps}
        if n in fl and tm > 0:
            rec["tflops"] = fl[n] / (tm / args.steps * 1e-3) / 1e12
        out["stages"][n] = rec
        log(f"[bench]   layer {n:14s} {rec['ms_per_step']:8.3f} ms/step" +
            (f"  {rec['tflops']:7.1f} TFLOP/s" if "tflops" in rec else ""))
    log(f"[bench] layer fwd+bwd: {ms:.3f} ms/step, {out['tokens_per_s']:.4g} tokens/s")
    del saved, fws, bws, y, dx, dws, t
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="512k")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip timing the dense causal attention kernels at S = N (one forward and one backward)")
    ap.add_argument("--layer", action="store_true",
                    help="also time the projection-inclusive layer (W_Q, W_K, W_V, W_O around the attention)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ablation", action="store_true",
                    help="time forward + backward over the ablation grid at N = 98,304 instead (one JSON line)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the timed steps (a known-size "
                         "reference dispatch for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the library has no "
              f"multi-GPU path: heads or sequence shards would have to be split across GPUs)", file=sys.stderr)
        return 2

    import numpy as np  # noqa: F401
    import torch

    from hierarchical_sparse_attention_mean_amd import lighthouse as lh
    from hierarchical_sparse_attention_mean_amd import synth

    if args.ablation:
        return run_ablation(args, torch, np, lh, synth)

    cfg = synth.config(args.config)
    B, H, N, d, L, p, k = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["L"], cfg["p"], cfg["k"]
    BH = B * H
    dev = torch.device("cuda:0")
    q, kk, v, do = resident_inputs(torch, np, synth, cfg, args.config, dev)
    io = q.dtype
    run = time_lighthouse(lh, torch, (q, kk, v, do), cfg, args.steps, args.warmup, args.copy_mib)
    S, ms, ms_fwd, stage_ms = run["S"], run["ms"], run["ms_fwd"], run["stages"]

    # dominant kernel: the MFMA attention stage with the most time per step
    dom = max(ATTN_STAGES, key=lambda n: stage_ms[n]["ms_per_step"])
    dom_ms = stage_ms[dom]["ms_per_launch"]
    dom_flops = attention_flops(S, d, BH, ATTN_STAGES[dom][0])
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    traffic = counter_traffic(dom, args.config)
    log(f"[bench] dominant kernel {dom}: {dom_ms:.3f} ms/launch, {achieved:.1f} TFLOP/s")

    # the backward's algorithmic products (5: S, dP, P^T dO, dS^T Q, dS K) over the time of both kernels that
    # run them (7 executed: the dQ kernel recomputes S and dP so that no kernel needs floating-point atomics)
    bwd_ms = stage_ms["attn_bwd_dq"]["ms_per_step"] + stage_ms["attn_bwd_dkdv"]["ms_per_step"]
    bwd_alg = attention_flops(S, d, BH, 5) / (bwd_ms * 1e-3) / 1e12
    extra = {"ms_forward": ms_fwd, "ms_backward": ms - ms_fwd, "stages": stage_ms,
             "tokens_per_s_forward": B * N / (ms_fwd * 1e-3),
             "attn_bwd_algorithmic_tflops": bwd_alg, "attn_bwd_algorithmic_frac": bwd_alg / PEAK_BF16_TFLOPS}
    stream = torch.cuda.current_stream()
    if not args.no_dense:
        # the same attention kernels on the full sequence (S = N): dense causal attention forward and backward
        q3, k3, v3, do3 = (x.reshape(BH, N, d) for x in (q, kk, v, do))
        od = torch.empty((BH, N, d), dtype=torch.float32, device=dev)
        lsed = torch.empty((BH, N), dtype=torch.float32, device=dev)
        grads = [torch.empty((BH, N, d), dtype=torch.float32, device=dev) for _ in range(3)]
        nb = lh.attention_backward_ws_bytes(BH, N, io)
        wsd = torch.empty(nb, dtype=torch.uint8, device=dev)
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        lh.lh_timing_begin()
        e0.record(stream)
        st = lh.lh_attention_forward(q3, k3, v3, od, lsed, BH, N, d, io)
        e1.record(stream)
        st2 = lh.lh_attention_backward(q3, k3, v3, od, lsed, do3, *grads, BH, N, d, io, wsd, nb)
        e2.record(stream)
        torch.cuda.synchronize()
        st3, dstages = lh.lh_timing_end()
        if st or st2 or st3:
            raise lh.LighthouseError(st or st2 or st3, "dense attention")
        fms, bms = e0.elapsed_time(e1), e1.elapsed_time(e2)
        extra["dense_attn_fwd_ms_at_S_eq_N"] = fms
        extra["dense_attn_fwd_tflops"] = attention_flops(N, d, BH) / (fms * 1e-3) / 1e12
        extra["dense_attn_bwd_ms_at_S_eq_N"] = bms
        extra["dense_attn_bwd_tflops_executed"] = attention_flops(N, d, BH, 7) / (bms * 1e-3) / 1e12
        extra["dense_attn_bwd_stage_ms"] = {n: dstages[n][0] for n in ("scatter_bwd", "attn_bwd_dq", "attn_bwd_dkdv")}
        extra["lighthouse_fwd_speedup_vs_dense"] = fms / ms_fwd
        extra["lighthouse_step_speedup_vs_dense"] = (fms + bms) / ms
        log(f"[bench] dense causal attention at S=N: forward {fms:.1f} ms, backward {bms:.1f} ms")
        del od, lsed, grads, wsd

    if args.layer:
        extra["layer"] = time_layer(lh, synth, cfg, args, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on one head (cpu_baseline)")
        cpu = cpu_baseline(cfg)
        log(f"[bench] oracle: {cpu['ms_per_step'] / 1e3:.1f} s per layer step")

    line = {
        "metric": "Lighthouse fwd+bwd tokens/s (ms/layer) at N=512K, H=8, d=128",
        "value": B * N / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if io == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"Lighthouse layer fwd+bwd, {args.config}: B={B} H={H} d={d} N={N} L={L} p={p} "
                               f"k={k} (S={S})", "B": B, "H": H, "d": d, "N": N, "L": L, "p": p, "k": k, "S": S},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "flops_per_launch": dom_flops, "ms_per_launch": dom_ms},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
