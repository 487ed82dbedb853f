"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and read its intermediates back; build the oracle's view of the same head."""
from __future__ import annotations

import sys

import numpy as np

import oracle as orc
from hierarchical_sparse_attention_mean_amd import synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        u = t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        return synth.bf16_bits_to_f32(u).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def run_forward(lh, cfg: dict, inp: dict, out_dtype: str = "f32", topk: int | None = None, L: int | None = None,
                p: int | None = None):
    import torch
    dt = cfg["dtype"]
    q, k, v = (to_dev(inp[n], dt) for n in ("q", "k", "v"))
    L = cfg["L"] if L is None else L
    p = cfg["p"] if p is None else p
    topk = cfg["k"] if topk is None else topk
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o, saved, plan = lh.forward(q, k, v, L, p, topk, out_dtype=odt)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, o=o, saved=saved, plan=plan)


def gpu_head(lh, run: dict, h: int) -> dict:
    """Intermediates of head h as numpy (float64 for floating arrays)."""
    plan, saved = run["plan"], run["saved"]
    P = plan.layout["P"]
    out = {}
    sc = lh.saved_view(saved, plan, "scores")[h].cpu().numpy()
    out["qk_flat"], out["kq_flat"] = sc[0].astype(np.float64), sc[1].astype(np.float64)
    out["flags"] = lh.saved_view(saved, plan, "flags")[h].cpu().numpy().astype(bool)
    out["slot"] = lh.saved_view(saved, plan, "slot")[h].cpu().numpy()
    out["coords"] = lh.saved_view(saved, plan, "coords")[h].cpu().numpy().astype(np.int64)
    S = plan.layout["S"]
    for n in ("qt", "kt", "vt"):   # rows S..Sv-1 are padding (zero)
        full = bf16_tensor_to_f64(lh.saved_view(saved, plan, n)[h])
        out[n], out[n + "_pad"] = full[:S], full[S:]
    out["ot32"] = lh.saved_view(saved, plan, "ot")[h].cpu().numpy()
    out["lse"] = lh.saved_view(saved, plan, "lse")[h].cpu().numpy().astype(np.float64)
    o = run["o"]
    b, hh = divmod(h, plan.H)
    out["o"] = bf16_tensor_to_f64(o[b, hh])
    assert len(out["flags"]) == P
    return out


def split_levels(flat: np.ndarray, N: int, L: int, p: int):
    sizes = orc.level_sizes(N, L, p)
    off = orc.flat_offsets(N, L, p)
    return [flat[off[l]:off[l] + sizes[l]] for l in range(L)]


def head_inputs_f64(cfg: dict, inp: dict, h: int):
    B, H = cfg["B"], cfg["H"]
    b, hh = divmod(h, H)
    return tuple(synth.as_f64(inp[n][b, hh], cfg["dtype"]) for n in ("q", "k", "v"))
