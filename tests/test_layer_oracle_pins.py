"""Pins of the projection-inclusive layer oracle (``oracle.layer_ref``) against
things other than itself: the textbook multi-head causal attention layer (which
the Lighthouse layer must reduce to when every token is kept), permutation
weights that route known columns to known heads, and central finite differences
of every gradient with the selection frozen."""
import math

import numpy as np
import pytest

import oracle as orc


def _textbook_mha(x, wq, wk, wv, wo, H):
    """Causal multi-head attention written out with loops over heads and query
    rows: y = sum_h softmax_causal(q_h k_h^T / sqrt(d)) v_h W_O[h-block]."""
    N, _ = x.shape
    d = wq.shape[1] // H
    y = np.zeros((N, wo.shape[1]))
    for h in range(H):
        cols = slice(h * d, (h + 1) * d)
        q, k, v = x @ wq[:, cols], x @ wk[:, cols], x @ wv[:, cols]
        o = np.zeros((N, d))
        for i in range(N):
            z = np.array([q[i] @ k[j] for j in range(i + 1)]) / math.sqrt(d)
            e = np.exp(z - z.max())
            o[i] = (e / e.sum()) @ v[:i + 1]
        y += o @ wo[cols, :]
    return y


def _weights(rng, dm, H, d):
    s = 1.0 / math.sqrt(dm)
    return (rng.standard_normal((dm, H * d)) * s, rng.standard_normal((dm, H * d)) * s,
            rng.standard_normal((dm, H * d)) * s, rng.standard_normal((H * d, dm)) / math.sqrt(H * d))


@pytest.mark.parametrize("N,dm,H,d", [(48, 12, 3, 4), (64, 16, 2, 8)])
def test_layer_reduces_to_textbook_mha(N, dm, H, d):
    """L = 1: the pyramid is level 0 alone, which is always kept, so the layer is
    plain causal multi-head attention with input and output projections."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((N, dm))
    wq, wk, wv, wo = _weights(rng, dm, H, d)
    fw = orc.layer_forward(x, wq, wk, wv, wo, H, L=1, p=2, topk=0)
    assert all(r["S"] == N for r in fw["heads"])
    np.testing.assert_allclose(fw["y"], _textbook_mha(x, wq, wk, wv, wo, H), rtol=1e-11, atol=1e-12)


def test_layer_wiring_with_permutation_weights():
    """W_Q, W_K, W_V pick permuted columns of X (d_model = H d), W_O permutes the
    concatenated head outputs: then head h must see exactly X[:, perm[h-block]]
    and Y must be the permuted concatenation of the per-head outputs."""
    rng = np.random.default_rng(5)
    N, H, d, L, p, k = 64, 2, 4, 3, 2, 3
    dm = H * d
    x = rng.standard_normal((N, dm))
    perms = [rng.permutation(dm) for _ in range(4)]
    wq, wk, wv = (np.eye(dm)[:, pm] for pm in perms[:3])     # (X W)[:, c] = X[:, pm[c]]
    wo = np.eye(dm)[perms[3]]                                # (O W_O)[:, perm[r]] = O[:, r]
    fw = orc.layer_forward(x, wq, wk, wv, wo, H, L, p, k)
    for h in range(H):
        cols = slice(h * d, (h + 1) * d)
        ref = orc.forward_head(x[:, perms[0][cols]], x[:, perms[1][cols]], x[:, perms[2][cols]], L, p, k)
        assert np.array_equal(ref["flags"], fw["flags"][h])
        np.testing.assert_allclose(fw["y"][:, perms[3][cols]], ref["o"], rtol=0, atol=1e-14)


def test_layer_selection_does_not_see_wv():
    """The scores use Q and K only (Sec. 3.4): W_V changes neither the selection,
    and Y is linear in W_V."""
    rng = np.random.default_rng(9)
    N, dm, H, d, L, p, k = 64, 8, 2, 4, 3, 2, 2
    x = rng.standard_normal((N, dm))
    wq, wk, wv, wo = _weights(rng, dm, H, d)
    a = orc.layer_forward(x, wq, wk, wv, wo, H, L, p, k)
    b = orc.layer_forward(x, wq, wk, -2.5 * wv, wo, H, L, p, k)
    assert np.array_equal(a["flags"], b["flags"])
    np.testing.assert_allclose(b["y"], -2.5 * a["y"], rtol=1e-12, atol=1e-13)


def test_layer_backward_finite_differences():
    """Every entry of dX, dW_Q, dW_K, dW_V, dW_O against central differences of
    sum(Y * G) with the selection frozen (the layer is then smooth)."""
    rng = np.random.default_rng(3)
    N, dm, H, d, L, p, k = 16, 6, 2, 4, 2, 2, 2
    x = rng.standard_normal((N, dm))
    ws = list(_weights(rng, dm, H, d))
    G = rng.standard_normal((N, dm))
    flags = orc.layer_forward(x, *ws, H, L, p, k)["flags"]
    assert 0 < int(flags.sum()) < flags.size
    bw = orc.layer_backward(x, *ws, G, H, L, p, flags)

    def loss(xx, wl):
        return float(np.sum(orc.layer_forward(xx, *wl, H, L, p, 0, flags=flags)["y"] * G))

    eps = 1e-6
    args = [x] + ws
    names = ["dx", "dwq", "dwk", "dwv", "dwo"]
    for a, nm in enumerate(names):
        fd = np.zeros_like(args[a])
        for idx in np.ndindex(*args[a].shape):
            plus = [t.copy() for t in args]
            minus = [t.copy() for t in args]
            plus[a][idx] += eps
            minus[a][idx] -= eps
            fd[idx] = (loss(plus[0], plus[1:]) - loss(minus[0], minus[1:])) / (2 * eps)
        np.testing.assert_allclose(bw[nm], fd, rtol=1e-6, atol=1e-7, err_msg=nm)


def test_layer_bf16_store_points():
    """bf16 mode rounds the stored tensors and nothing else: the projections are
    the bf16 roundings of the exact products."""
    rng = np.random.default_rng(4)
    N, dm, H, d, L, p, k = 32, 8, 2, 4, 2, 2, 2
    x = orc.round_bf16(rng.standard_normal((N, dm)))
    ws = [orc.round_bf16(w) for w in _weights(rng, dm, H, d)]
    fw = orc.layer_forward(x, *ws, H, L, p, k, store="bf16")
    np.testing.assert_array_equal(orc.concat_heads(fw["q"]), orc.round_bf16(x @ ws[0]))
    np.testing.assert_array_equal(fw["o"], orc.round_bf16(fw["o"]))
    np.testing.assert_allclose(fw["y"], fw["o"] @ ws[3], rtol=1e-15)
