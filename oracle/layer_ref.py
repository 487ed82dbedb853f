"""Projection-inclusive Lighthouse layer: plain fp64 CPU oracle.  TEST
INFRASTRUCTURE ONLY (same rules as ``lighthouse_ref``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
use it; the product path never does, and nothing here comes from it).

What it computes, for one sequence X [N, d_model] ("Long Context Pre-Training
with Lighthouse Attention"):

  projections   Sec. 3.1: per head h, Q_h = X W_Q[:, h d:(h+1) d], likewise K_h
                and V_h (W_Q, W_K, W_V in R^{d_model x d} per head; the H heads'
                matrices side by side as [d_model, H d]).
  attention     Sec. 3.2: the Lighthouse pipeline on (Q_h, K_h, V_h), one head at
                a time (``lighthouse_ref.forward_head``), giving O_h [N, d].
  output        Y = [O_0 | ... | O_{H-1}] W_O, W_O in R^{H d x d_model}.
  backward      Sec. 3.2: the selection is discrete and frozen; gradients reach
                W_Q, W_K, W_V only through the scatter, the sub-sequence
                attention and the gather (``lighthouse_ref.backward_head``), and
                the chain rule through the two products gives dX and every dW.

Readings taken where the pages leave a step open:
  * W_O is the output projection of the attention block of the Llama-3-style
    decoder the pages train (experiments paragraph: d_model = 1024, 8 heads of
    head dimension 128); the pages define only W_Q, W_K, W_V (Sec. 3.1).
  * No rotary embedding, bias or normalisation: the pages place the pyramid
    directly on the projections (Sec. 3.2).
  * bf16 mode (``store="bf16"``): every tensor the layer stores between its
    steps -- Q, K, V after the projection, O before W_O, dO after dY W_O^T, and
    dQ, dK, dV after the attention backward -- is rounded to bf16 once, and the
    attention's pooled levels are stored in bf16 in the forward and in the
    backward alike (``backward_head(store=...)``); the products themselves are
    exact (fp64) here.

Every function has a pin in ``tests/test_layer_oracle_pins.py``: a textbook
multi-head attention layer (L = 1), a wiring check with permutation weights,
and central finite differences of every gradient with the selection frozen.
"""
from __future__ import annotations

import numpy as np

from .lighthouse_ref import backward_head, forward_head, round_bf16


def _store(x: np.ndarray, store: str | None) -> np.ndarray:
    return round_bf16(x) if store == "bf16" else x


def heads_of(z: np.ndarray, H: int) -> np.ndarray:
    """[N, H d] -> [H, N, d]: the column block h d .. (h+1) d - 1 is head h."""
    N, Hd = z.shape
    return z.reshape(N, H, Hd // H).transpose(1, 0, 2)


def concat_heads(z: np.ndarray) -> np.ndarray:
    """[H, N, d] -> [N, H d] (inverse of ``heads_of``)."""
    H, N, d = z.shape
    return z.transpose(1, 0, 2).reshape(N, H * d)


def layer_forward(x, wq, wk, wv, wo, H: int, L: int, p: int, topk: int, flags=None,
                  store: str | None = None) -> dict:
    """One sequence.  x [N, d_model]; wq, wk, wv [d_model, H d]; wo [H d, d_model].
    ``flags`` ([H, |P|], optional) injects each head's selection.  Returns the
    projected q, k, v [H, N, d], the per-head results of ``forward_head``, the
    concatenated output o [N, H d] and y [N, d_model]."""
    x = np.asarray(x, dtype=np.float64)
    wq, wk, wv, wo = (np.asarray(w, dtype=np.float64) for w in (wq, wk, wv, wo))
    q = heads_of(_store(x @ wq, store), H)
    k = heads_of(_store(x @ wk, store), H)
    v = heads_of(_store(x @ wv, store), H)
    res = []
    for h in range(H):
        fl = None if flags is None else np.asarray(flags[h], dtype=bool)
        res.append(forward_head(q[h], k[h], v[h], L, p, topk, flags=fl, store=store))
    o = _store(concat_heads(np.stack([r["o"] for r in res])), store)
    return dict(q=q, k=k, v=v, heads=res, flags=np.stack([r["flags"] for r in res]), o=o, y=o @ wo)


def layer_backward(x, wq, wk, wv, wo, dy, H: int, L: int, p: int, flags, store: str | None = None) -> dict:
    """Gradients of sum(Y * dY) for one sequence with each head's selection
    ``flags`` [H, |P|] frozen: dx [N, d_model], dwq, dwk, dwv [d_model, H d],
    dwo [H d, d_model], and the intermediate do, dq, dk, dv [H, N, d]."""
    x = np.asarray(x, dtype=np.float64)
    wq, wk, wv, wo = (np.asarray(w, dtype=np.float64) for w in (wq, wk, wv, wo))
    dy = np.asarray(dy, dtype=np.float64)
    fw = layer_forward(x, wq, wk, wv, wo, H, L, p, 0, flags=flags, store=store)
    dwo = fw["o"].T @ dy                              # Y = O W_O
    do = heads_of(_store(dy @ wo.T, store), H)
    g = [backward_head(fw["q"][h], fw["k"][h], fw["v"][h], do[h], L, p, np.asarray(flags[h], dtype=bool), store)
         for h in range(H)]
    dq, dk, dv = (np.stack([_store(gh[i], store) for gh in g]) for i in range(3))
    dqc, dkc, dvc = concat_heads(dq), concat_heads(dk), concat_heads(dv)
    dx = dqc @ wq.T + dkc @ wk.T + dvc @ wv.T         # Q = X W_Q, K = X W_K, V = X W_V
    return dict(dx=dx, dwq=x.T @ dqc, dwk=x.T @ dkc, dwv=x.T @ dvc, dwo=dwo, do=do, dq=dq, dk=dk, dv=dv)
