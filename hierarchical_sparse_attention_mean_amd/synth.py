"""Seeded synthetic inputs for the Lighthouse attention layer.

This module only draws random numbers and converts them to the storage format
(fp32, or bf16 bit patterns by round-to-nearest-even); it holds none of the
method's arithmetic.  Tests, the benchmark and the oracle's timing leg all take
their inputs from here, so every side sees identical values.

Workloads (all B = 1, causal):
  tiny   fp32, H=2,  d=64,  N=1,024,     L=3, p=4, k=64     rows t = 0 mod 97 get Q, K x4
  98k    bf16, H=8,  d=128, N=98,304,    L=3, p=4, k=768    round(1% N) distinct rows get Q, K x3
  512k   bf16, H=8,  d=128, N=524,288,   L=3, p=4, k=4,096  same recipe as 98k
  1m     bf16, H=8,  d=128, N=1,048,576, L=4, p=4, k=4,096  per-row multiplier m_t drawn from a Zipf(1.2)
                                                            law truncated to {1..16}, applied to Q, K
  bwd8k  bf16, H=8,  d=128, N=8,192,     L=3, p=4, k=64     98k recipe; dO ~ N(0,1)
Q, K, V (and dO) are iid N(0,1) before the multipliers; V is never scaled.

Random streams: tensor s (0=Q, 1=K, 2=V, 4=dO) of head j (= b*H + h) uses
SeedSequence(seed, spawn_key=(s, j)); the row positions / multipliers, shared by
all heads, use spawn_key=(3,).  Any single head can therefore be regenerated on
its own.

Projection-inclusive layer (``layer_inputs``): d_model = 1024 for the bf16
workloads (the pages' 530M decoder: d_model 1024, 8 heads of 128), 128 for tiny.
X [B, N, d_model] and dY are iid N(0,1), X rows scaled by the same per-row
multipliers as Q and K above; W_Q, W_K, W_V [d_model, H d] are iid
N(0, 1/d_model) and W_O [H d, d_model] iid N(0, 1/(H d)), so that the
projections have unit variance.  Streams: spawn_key=(10 + i, b) for X (i=0) and
dY (i=1) of batch element b, spawn_key=(20 + i,) for W_Q, W_K, W_V, W_O.
"""
from __future__ import annotations

import numpy as np

CONFIGS = {
    "tiny":  dict(index=0, B=1, H=2, d=64, N=1024, L=3, p=4, k=64, dtype="f32", recipe="mod97x4", d_model=128),
    "98k":   dict(index=1, B=1, H=8, d=128, N=98304, L=3, p=4, k=768, dtype="bf16", recipe="pct1x3", d_model=1024),
    "512k":  dict(index=2, B=1, H=8, d=128, N=524288, L=3, p=4, k=4096, dtype="bf16", recipe="pct1x3",
                  d_model=1024),
    "1m":    dict(index=3, B=1, H=8, d=128, N=1048576, L=4, p=4, k=4096, dtype="bf16", recipe="zipf",
                  d_model=1024),
    "bwd8k": dict(index=4, B=1, H=8, d=128, N=8192, L=3, p=4, k=64, dtype="bf16", recipe="pct1x3", d_model=1024),
}

SEED_BASE = 20260


def config(name: str, **over) -> dict:
    c = dict(CONFIGS[name])
    c.update(over)
    c.setdefault("seed", SEED_BASE + c["index"])
    return c


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=tuple(key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> the exact fp32 value."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def row_multipliers(cfg: dict) -> np.ndarray:
    """Per-row multiplier m_t (fp32, length N) applied to Q_t and K_t."""
    N = cfg["N"]
    m = np.ones(N, dtype=np.float32)
    rec = cfg["recipe"]
    if rec == "mod97x4":
        m[np.arange(0, N, 97)] = 4.0
    elif rec == "pct1x3":
        n = int(round(0.01 * N))
        pos = _rng(cfg["seed"], 3).choice(N, size=n, replace=False)
        m[pos] = 3.0
    elif rec == "zipf":
        alpha, top = 1.2, 16
        w = np.arange(1, top + 1, dtype=np.float64) ** -alpha
        cdf = np.cumsum(w) / w.sum()
        u = _rng(cfg["seed"], 3).random(N)
        m = (np.searchsorted(cdf, u, side="right") + 1).astype(np.float32)
        m = np.minimum(m, top)
    elif rec == "none":
        pass
    else:
        raise ValueError(rec)
    return m


def head_tensor(cfg: dict, which: str, j: int, mult: np.ndarray | None = None) -> np.ndarray:
    """One head's [N, d] tensor ('q', 'k', 'v' or 'do') in storage format:
    float32 for fp32 workloads, uint16 bf16 bits for bf16 workloads."""
    s = {"q": 0, "k": 1, "v": 2, "do": 4}[which]
    x = _rng(cfg["seed"], s, j).standard_normal((cfg["N"], cfg["d"]), dtype=np.float32)
    if which in ("q", "k"):
        if mult is None:
            mult = row_multipliers(cfg)
        x *= mult[:, None]
    if cfg["dtype"] == "bf16":
        return f32_to_bf16_bits(x)
    return x


def make_inputs(cfg: dict, with_do: bool = False, heads=None) -> dict:
    """Arrays [B, H, N, d] (or [len(heads), N, d] for a head subset) of q, k, v
    (and do), in storage format."""
    mult = row_multipliers(cfg)
    B, H = cfg["B"], cfg["H"]
    js = list(range(B * H)) if heads is None else list(heads)
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    out = {}
    for nm in names:
        arr = np.stack([head_tensor(cfg, nm, j, mult) for j in js])
        out[nm] = arr.reshape(B, H, cfg["N"], cfg["d"]) if heads is None else arr
    return out


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage-format array -> float64 with exactly the stored values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def layer_inputs(cfg: dict, with_dy: bool = False) -> dict:
    """x [B, N, d_model], wq, wk, wv [d_model, H d], wo [H d, d_model] (and dy
    [B, N, d_model]) in storage format (see the module notes)."""
    B, N, H, d, dm = cfg["B"], cfg["N"], cfg["H"], cfg["d"], cfg["d_model"]
    mult = row_multipliers(cfg)
    conv = f32_to_bf16_bits if cfg["dtype"] == "bf16" else (lambda a: a)
    out = {}
    xs = []
    for b in range(B):
        x = _rng(cfg["seed"], 10, b).standard_normal((N, dm), dtype=np.float32)
        x *= mult[:, None]
        xs.append(conv(x))
    out["x"] = np.stack(xs)
    for i, nm in enumerate(("wq", "wk", "wv")):
        w = _rng(cfg["seed"], 20 + i).standard_normal((dm, H * d), dtype=np.float32) / np.float32(np.sqrt(dm))
        out[nm] = conv(w)
    wo = _rng(cfg["seed"], 23).standard_normal((H * d, dm), dtype=np.float32) / np.float32(np.sqrt(H * d))
    out["wo"] = conv(wo)
    if with_dy:
        out["dy"] = np.stack([conv(_rng(cfg["seed"], 11, b).standard_normal((N, dm), dtype=np.float32))
                              for b in range(B)])
    return out
