"""Benchmark of the Lighthouse attention layer on one MI355X.

One step = the whole layer: forward (pool+score, top-k, compaction+gather,
sub-sequence attention, scatter) and backward (scatter adjoint, attention
backward, gather+pool adjoint) for one batch of seeded synthetic bf16 inputs
already resident in HBM.  Default workload: B=1, H=8, d=128, N=524,288, L=3,
p=4, k=4,096 (S=65,536).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 512k] [--dense]

Prints one JSON line (rank 0).  Besides the contract fields it carries:
  roofline      dominant kernel (the sub-sequence attention), algorithmic FLOPs
                per launch / its mean launch time from HIP events on its stream
  cpu_baseline  the fp64 oracle on one head of the same workload (fwd + bwd),
                on this host's cores, scaled to the layer's tokens/s
  extra         forward-only time, attention fwd/bwd kernel times, and (with
                --dense) the dense causal attention kernel at S = N
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_flops(S: int, d: int, BH: int) -> float:
    """Algorithmic FLOPs of causal attention over S rows: Q.K^T and P.V over
    the S^2/2 causal pairs, 2 FLOPs per multiply-add."""
    return 2.0 * 2.0 * (S * S / 2.0) * d * BH


def cpu_baseline(cfg: dict) -> dict:
    """The oracle as it stands, on head 0 of the workload, forward + backward."""
    import numpy as np

    import oracle as orc
    from hierarchical_sparse_attention_mean_amd import synth

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
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
            "sample": f"head 0 of {cfg['B'] * cfg['H']}, full forward ({t1 - t0:.1f} s) + backward ({t2 - t1:.1f} s) "
                      f"in fp64 numpy; layer time = per-head time x {cfg['B'] * cfg['H']} heads",
            "ms_per_step": layer_s * 1e3}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="512k")
    ap.add_argument("--dense", action="store_true", help="also time dense causal attention at S = N")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (heads or sequence shards "
              f"would be split across GPUs; see the design notes)", file=sys.stderr)
        return 2

    import numpy as np  # noqa: F401
    import torch

    from hierarchical_sparse_attention_mean_amd import lighthouse as lh
    from hierarchical_sparse_attention_mean_amd import synth

    cfg = synth.config(args.config)
    B, H, N, d, L, p, k = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["L"], cfg["p"], cfg["k"]
    BH = B * H
    dev = torch.device("cuda:0")
    log(f"[bench] generating {args.config} inputs (B={B} H={H} N={N} d={d})")
    t0 = time.perf_counter()
    inp = synth.make_inputs(cfg, with_do=True)
    tens = {}
    for n in ("q", "k", "v", "do"):
        a = inp.pop(n)
        if cfg["dtype"] == "bf16":
            tens[n] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            tens[n] = torch.from_numpy(a).to(dev)
        del a
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")
    q, kk, v, do = tens["q"], tens["k"], tens["v"], tens["do"]
    io = q.dtype
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

    def step():
        fwd()
        bwd()

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/step")

    # forward alone
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    ms_fwd = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"[bench] forward only: {ms_fwd:.3f} ms")

    # dominant kernel: the sub-sequence attention, launched exactly as inside
    # lh_forward (same kernel, grid and operands), timed with HIP events on the
    # stream it runs on
    qt = lh.saved_view(saved, plan, "qt")
    kt = lh.saved_view(saved, plan, "kt")
    vop = lh.saved_view(saved, plan, "vtt" if io == torch.bfloat16 else "vt")
    ot = torch.empty((BH, S, d), dtype=torch.float32, device=dev)
    lse = torch.empty((BH, S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        st = lh.lh_attention_forward(qt, kt, vop, ot, lse, BH, S, d, io)
        b.record(stream)
        if st:
            raise lh.LighthouseError(st, "lh_attention_forward")
    torch.cuda.synchronize()
    attn_ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    flops = attention_flops(S, d, BH)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    log(f"[bench] attention forward kernel: {attn_ms:.3f} ms, {achieved:.1f} TFLOP/s")

    extra = {"ms_forward": ms_fwd, "ms_backward": ms - ms_fwd, "attn_fwd_kernel_ms": attn_ms,
             "attn_fwd_flops": flops, "tokens_per_s_forward": B * N / (ms_fwd * 1e-3)}
    if args.dense:
        if io == torch.bfloat16:   # V^T, columns in the kernel's order (bits 2 and 3 of the index swapped)
            col = torch.arange(N, device=dev)
            perm = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1)
            vt_dense = v.reshape(BH, N, d).transpose(1, 2)[:, :, perm].contiguous()
        else:
            vt_dense = v.reshape(BH, N, d)
        od = torch.empty((BH, N, d), dtype=torch.float32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lh.lh_attention_forward(q.reshape(BH, N, d), kk.reshape(BH, N, d), vt_dense, od, None, BH, N, d, io)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1)
        extra["dense_attn_fwd_ms_at_S_eq_N"] = dms
        extra["dense_attn_fwd_tflops"] = attention_flops(N, d, BH) / (dms * 1e-3) / 1e12
        extra["lighthouse_fwd_speedup_vs_dense"] = dms / ms_fwd
        log(f"[bench] dense causal attention at S=N: {dms:.1f} ms")
        del od, vt_dense

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
        "roofline": {"bound": "mfma", "kernel": "sub-sequence causal attention forward", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": None},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
