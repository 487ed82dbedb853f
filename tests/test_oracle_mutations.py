"""The oracle's pins catch plausible mistakes: each test plants one mistake in
the fp64 oracle (on the CPU, through monkeypatch, so the oracle's own internal
calls see it too), runs every pin of ``test_oracle_pins.py`` (of
``test_layer_oracle_pins.py`` for the layer oracle), and requires at least one
of them to fail with an AssertionError.

The mistakes are the kind a reader of the pages could make: a flipped tie
order, swapped streams, a dropped factor or scale, an off-by-one window, range
or mask, the wrong pooling or rounding rule, a missing term of an adjoint.
"""
import inspect
import itertools
import math
from dataclasses import dataclass
from typing import Callable

import numpy as np
import pytest

import oracle
import oracle.layer_ref as yr
import oracle.lighthouse_ref as lr
import test_layer_oracle_pins as layer_pins
import test_oracle_pins as pins


def _pin_calls(module=pins):
    """(name, function, kwargs) for every pin of ``module``, parametrized cases expanded."""
    for name, f in inspect.getmembers(module, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = set(inspect.signature(f).parameters)
        grids = []
        for m in getattr(f, "pytestmark", []):
            if m.name != "parametrize":
                continue
            names = [a.strip() for a in m.args[0].split(",")]
            cases = []
            for v in m.args[1]:
                v = v if isinstance(v, tuple) else (v,)
                cases.append(dict(zip(names, v)))
            grids.append(cases)
        for combo in itertools.product(*grids):
            kw = {}
            for c in combo:
                kw.update(c)
            if set(kw) == params:
                yield name, f, kw


# ---- mutated copies (one change each, marked "mistake") ----------------------
def _select_variant(tie_index_desc=False, budget_without_p=False):
    def select(qk, kq, p, k):
        L = len(qk)
        sizes = [len(x) for x in qk]
        P = sum(sizes)
        E = P - sizes[-1]
        B = min((L - 1) * (1 if budget_without_p else p) * k, E)   # mistake if budget_without_p
        flags = np.zeros(P, dtype=bool)
        flags[E:] = True
        if B == 0:
            return flags
        val = np.concatenate([np.concatenate(qk)[:E], np.concatenate(kq)[:E]])
        idx = np.concatenate([np.arange(E), P + np.arange(E)])
        walk = np.lexsort((-idx if tie_index_desc else idx, -val))   # mistake if tie_index_desc
        entry = idx[walk] % P
        first = np.full(E, np.iinfo(np.int64).max, dtype=np.int64)
        np.minimum.at(first, entry, np.arange(len(walk)))
        flags[np.argsort(first, kind="stable")[:B]] = True
        return flags
    return select


def _order_variant(coarser_first=False, by_start=False):
    def order(flags, N, L, p):
        f = np.nonzero(flags)[0].astype(np.int64)
        lev, pos = lr.coords_of_flat(f, N, L, p)
        key = pos * (np.int64(p) ** lev) if by_start else lr.window_end(lev, pos, p)   # mistake if by_start
        return f[np.lexsort((-lev if coarser_first else lev, key))]                  # mistake if coarser_first
    return order


def _attend_variant(mask_extra=0):
    def attend(qt, kt, vt, row_block=1024):
        S, d = qt.shape
        z = (qt @ kt.T) * (1.0 / math.sqrt(d))
        rows, cols = np.arange(S)[:, None], np.arange(S)[None, :]
        z = np.where(cols <= rows + mask_extra, z, -np.inf)   # mistake if mask_extra: later rows visible
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        s = e.sum(axis=1, keepdims=True)
        return (e / s) @ vt, (zmax + np.log(s))[:, 0]
    return attend


def _scatter_range_variant(shifted=True):
    def scatter_range(lev, pos, N, p):
        w = p ** int(lev)
        lo = (int(pos) + 1) * w - 1 if shifted else int(pos) * w   # mistake if not shifted: the window itself
        return lo, min(N - 1, lo + w - 1)
    return scatter_range


def _scatter_adjoint_variant(shifted=True):
    rng_of = _scatter_range_variant(shifted)

    def scatter_adjoint(do, sorted_flat, N, L, p):
        lev, pos = lr.coords_of_flat(sorted_flat, N, L, p)
        out = np.zeros((len(sorted_flat), do.shape[1]))
        for m in range(len(sorted_flat)):
            lo, hi = rng_of(lev[m], pos[m], N, p)   # mistake if not shifted (the forward keeps the shift)
            if lo <= hi:
                out[m] = do[lo:hi + 1].sum(axis=0)
        return out
    return scatter_adjoint


def _attend_adjoint_variant(rowsum=True):
    def attend_adjoint(qt, kt, vt, dot, row_block=1024):
        S, d = qt.shape
        scale = 1.0 / math.sqrt(d)
        z = (qt @ kt.T) * scale
        z = np.where(np.arange(S)[None, :] <= np.arange(S)[:, None], z, -np.inf)
        e = np.exp(z - z.max(axis=1, keepdims=True))
        prob = e / e.sum(axis=1, keepdims=True)
        dp = dot @ vt.T
        # mistake if not rowsum: the softmax Jacobian's rowsum term is missing
        dz = prob * (dp - np.sum(dp * prob, axis=1, keepdims=True)) if rowsum else prob * dp
        return (dz @ kt) * scale, (dz.T @ qt) * scale, prob.T @ dot
    return attend_adjoint


def _pool_adjoint_variant(weight=True):
    def pool_adjoint(dlevels, N, p):
        out = np.zeros((N, dlevels[0].shape[1]))
        for l, dl in enumerate(dlevels):
            out += np.repeat(dl, p ** l, axis=0) / (p ** l if weight else 1)   # mistake if not weight
        return out
    return pool_adjoint


def _to_fixed_variant(rne=True):
    def to_fixed(x):
        y = np.asarray(x, dtype=np.float64) * 2.0 ** lr.FIX_FRAC_BITS
        return (np.rint(y) if rne else np.trunc(y)).astype(np.int64)   # mistake if not rne
    return to_fixed


def _round_bf16_variant(rne=True):
    def round_bf16(x):
        u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
        r = (((u + 0x7FFF + ((u >> 16) & 1)) if rne else u) >> 16) << 16   # mistake if not rne: truncation
        return r.astype(np.uint32).view(np.float32).astype(np.float64)
    return round_bf16


def _gather_variant(level0=False):
    def gather(levels, sorted_flat, N, L, p):
        lev, pos = lr.coords_of_flat(sorted_flat, N, L, p)
        # mistake if level0: the level-0 row at the window start instead of the entry's own row
        return np.stack([levels[0][pos[m] * p ** lev[m]] if level0 else levels[lev[m]][pos[m]]
                         for m in range(len(sorted_flat))])
    return gather


@dataclass
class Mutation:
    name: str
    target: str
    make: Callable   # original function -> mutated function


def _wrap_scores_squared(orig):
    def scores(q, k, L, p):
        qk, kq = orig(q, k, L, p)
        return [x * x for x in qk], [x * x for x in kq]   # mistake: squared norms
    return scores


def _wrap_scores_mean_pool(orig):
    def scores(q, k, L, p):
        qk, kq = orig(q, k, L, p)
        out = []
        for s in (qk, kq):
            out.append([s[0]] + [s[0].reshape(len(s[l]), p ** l).mean(axis=1) for l in range(1, L)])   # mistake
        return out[0], out[1]
    return scores


def _wrap_scores_rescore_pooled(orig):
    def scores(q, k, L, p):
        lq, lk = lr.pyramid(q, L, p), lr.pyramid(k, L, p)
        return ([np.sqrt((x * x).sum(axis=1)) for x in lq],   # mistake: norms of the pooled rows
                [np.sqrt((x * x).sum(axis=1)) for x in lk])
    return scores


def _wrap_pyramid_shifted(orig):
    def pyramid(x, L, p, store=None):
        lev = orig(x, L, p, store)
        shifted = orig(np.roll(np.asarray(x, dtype=np.float64), -1, axis=0), L, p, store)
        return [lev[0]] + shifted[1:]   # mistake: windows start one token late
    return pyramid


def _wrap_pyramid_sum(orig):
    def pyramid(x, L, p, store=None):
        return [lv * p ** l for l, lv in enumerate(orig(x, L, p, store))]   # mistake: sums, not means
    return pyramid


def _wrap_select_streams_swapped(orig):
    return lambda qk, kq, p, k: orig(kq, qk, p, k)   # mistake: KQ takes the lower stream indices


def _wrap_select_drop_coarsest(orig):
    def select(qk, kq, p, k):
        f = orig(qk, kq, p, k).copy()
        f[sum(len(x) for x in qk) - len(qk[-1]):] = False   # mistake: the coarsest level is not kept
        return f
    return select


def _wrap_attend_no_scale(orig):
    return lambda qt, kt, vt, row_block=1024: orig(qt * math.sqrt(qt.shape[1]), kt, vt, row_block)   # mistake


def _wrap_attend_adjoint_dq_unscaled(orig):
    def attend_adjoint(qt, kt, vt, dot, row_block=1024):
        dq, dk, dv = orig(qt, kt, vt, dot, row_block)
        return dq * math.sqrt(qt.shape[1]), dk, dv   # mistake: dQ without 1/sqrt(d)
    return attend_adjoint



def _wrap_backward_ignores_store(orig):
    def backward_head(q, k, v, do, L, p, flags, store=None):
        return orig(q, k, v, do, L, p, flags)   # mistake: adjoint at the unrounded rows in bf16 mode
    return backward_head

MUTATIONS = [
    Mutation("select: ties go to the higher stream index", "select", lambda o: _select_variant(tie_index_desc=True)),
    Mutation("select: budget (L-1) k, factor p dropped", "select", lambda o: _select_variant(budget_without_p=True)),
    Mutation("select: QK and KQ stream offsets swapped", "select", _wrap_select_streams_swapped),
    Mutation("select: coarsest level not kept", "select", _wrap_select_drop_coarsest),
    Mutation("scores: squared norms", "scores", _wrap_scores_squared),
    Mutation("scores: coarser levels mean-pooled", "scores", _wrap_scores_mean_pool),
    Mutation("scores: coarser levels re-scored from pooled rows", "scores", _wrap_scores_rescore_pooled),
    Mutation("pyramid: windows shifted by one token", "pyramid", _wrap_pyramid_shifted),
    Mutation("pyramid: window sums instead of means", "pyramid", _wrap_pyramid_sum),
    Mutation("order: coarser level first at equal window ends", "order", lambda o: _order_variant(coarser_first=True)),
    Mutation("order: by window start", "order", lambda o: _order_variant(by_start=True)),
    Mutation("gather: level-0 row for every entry", "gather", lambda o: _gather_variant(level0=True)),
    Mutation("attend: 1/sqrt(d) dropped", "attend", _wrap_attend_no_scale),
    Mutation("attend: mask admits the next row", "attend", lambda o: _attend_variant(mask_extra=1)),
    Mutation("scatter: unshifted range", "scatter_range", lambda o: _scatter_range_variant(shifted=False)),
    Mutation("scatter adjoint: unshifted range", "scatter_adjoint", lambda o: _scatter_adjoint_variant(shifted=False)),
    Mutation("attention adjoint: rowsum term missing", "attend_adjoint", lambda o: _attend_adjoint_variant(rowsum=False)),
    Mutation("attention adjoint: dQ without 1/sqrt(d)", "attend_adjoint", _wrap_attend_adjoint_dq_unscaled),
    Mutation("pool adjoint: 1/p^l missing", "pool_adjoint", lambda o: _pool_adjoint_variant(weight=False)),
    Mutation("fixed point: truncation on the way in", "to_fixed", lambda o: _to_fixed_variant(rne=False)),
    Mutation("bf16: truncation instead of rounding", "round_bf16", lambda o: _round_bf16_variant(rne=False)),
    Mutation("backward: bf16 storage of the pooled levels ignored", "backward_head", _wrap_backward_ignores_store),
]


def test_copies_without_their_mistake_reproduce_the_oracle():
    """Each mutated copy, with its mistake switched off, equals the oracle's own
    function, so a planted mistake differs from the oracle by its marked line only."""
    rng = np.random.default_rng(5)
    N, L, p, d = 64, 3, 4, 8
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    qk, kq = lr.scores(q, k, L, p)
    qk = [np.round(x, 1) for x in qk]   # ties, so that the tie order matters
    kq = [np.round(x, 1) for x in kq]
    for kk in (1, 3, 100):
        assert np.array_equal(_select_variant()(qk, kq, p, kk), lr.select(qk, kq, p, kk))
    flags = lr.select(qk, kq, p, 3)
    assert np.array_equal(_order_variant()(flags, N, L, p), lr.order(flags, N, L, p))
    sf = lr.order(flags, N, L, p)
    levels = lr.pyramid(q, L, p)
    assert np.array_equal(_gather_variant()(levels, sf, N, L, p), lr.gather(levels, sf, N, L, p))
    qt, kt, vt = (lr.gather(lr.pyramid(x, L, p), sf, N, L, p) for x in (q, k, v))
    for a, b in zip(_attend_variant()(qt, kt, vt), lr.attend(qt, kt, vt)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    for lev in range(L):
        for pos in range(N // p ** lev):
            assert _scatter_range_variant()(lev, pos, N, p) == lr.scatter_range(lev, pos, N, p)
    np.testing.assert_array_equal(_scatter_adjoint_variant()(do, sf, N, L, p), lr.scatter_adjoint(do, sf, N, L, p))
    dot = lr.scatter_adjoint(do, sf, N, L, p)
    for a, b in zip(_attend_adjoint_variant()(qt, kt, vt, dot), lr.attend_adjoint(qt, kt, vt, dot)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    dl = [rng.standard_normal((n, d)) for n in lr.level_sizes(N, L, p)]
    np.testing.assert_array_equal(_pool_adjoint_variant()(dl, N, p), lr.pool_adjoint(dl, N, p))
    x = rng.standard_normal(1000) * 3
    np.testing.assert_array_equal(_to_fixed_variant()(x), lr.to_fixed(x))
    np.testing.assert_array_equal(_round_bf16_variant()(x), lr.round_bf16(x))


def test_pins_pass_unmutated():
    """The harness itself: every expanded pin passes on the oracle as it is."""
    calls = list(_pin_calls())
    assert len(calls) >= 50
    for name, f, kw in calls:
        f(**kw)


@pytest.mark.parametrize("mut", MUTATIONS, ids=[m.name for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(mut, monkeypatch):
    bad = mut.make(getattr(lr, mut.target))
    monkeypatch.setattr(lr, mut.target, bad)        # the oracle's internal calls
    monkeypatch.setattr(oracle, mut.target, bad)    # the pins' calls (orc.<name>)
    caught = None
    with np.errstate(all="ignore"):
        for name, f, kw in _pin_calls():
            try:
                f(**kw)
            except AssertionError:
                caught = name
                break
    assert caught is not None, f"no pin fails with the planted mistake: {mut.name}"


# ---- the projection-inclusive layer (oracle/layer_ref.py) ---------------------
def _heads_interleaved(z, H):
    N, Hd = z.shape
    return z.reshape(N, Hd // H, H).transpose(2, 0, 1)   # mistake: head h = columns h, h + H, ...


def _concat_interleaved(z):
    H, N, d = z.shape
    return z.transpose(1, 2, 0).reshape(N, H * d)   # the inverse of the interleaved split


def _wrap_layer_q_from_wk(orig):
    def layer_forward(x, wq, wk, wv, wo, H, L, p, topk, flags=None, store=None):
        return orig(x, wk, wk, wv, wo, H, L, p, topk, flags=flags, store=store)   # mistake: Q = X W_K
    return layer_forward


def _wrap_layer_dx_without_v(orig):
    def layer_backward(x, wq, wk, wv, wo, dy, H, L, p, flags, store=None):
        g = orig(x, wq, wk, wv, wo, dy, H, L, p, flags, store)
        g["dx"] = g["dx"] - yr.concat_heads(g["dv"]) @ np.asarray(wv, dtype=np.float64).T   # mistake: no V path
        return g
    return layer_backward


def _wrap_layer_dwq_dwk_swapped(orig):
    def layer_backward(x, wq, wk, wv, wo, dy, H, L, p, flags, store=None):
        g = orig(x, wq, wk, wv, wo, dy, H, L, p, flags, store)
        g["dwq"], g["dwk"] = g["dwk"], g["dwq"]   # mistake
        return g
    return layer_backward


def _wrap_layer_no_wo(orig):
    def layer_forward(x, wq, wk, wv, wo, H, L, p, topk, flags=None, store=None):
        r = orig(x, wq, wk, wv, wo, H, L, p, topk, flags=flags, store=store)
        r["y"] = r["o"] @ np.eye(*np.asarray(wo).shape)   # mistake: W_O replaced by a plain truncation
        return r
    return layer_forward


LAYER_MUTATIONS = [
    Mutation("layer: heads interleaved instead of column blocks", "heads_of", lambda o: _heads_interleaved),
    Mutation("layer: head concat interleaved", "concat_heads", lambda o: _concat_interleaved),
    Mutation("layer: Q projected with W_K", "layer_forward", _wrap_layer_q_from_wk),
    Mutation("layer: W_O product dropped", "layer_forward", _wrap_layer_no_wo),
    Mutation("layer backward: dX misses the V path", "layer_backward", _wrap_layer_dx_without_v),
    Mutation("layer backward: dW_Q and dW_K swapped", "layer_backward", _wrap_layer_dwq_dwk_swapped),
]


@pytest.mark.parametrize("mut", LAYER_MUTATIONS, ids=[m.name for m in LAYER_MUTATIONS])
def test_planted_layer_mistake_fails_a_pin(mut, monkeypatch):
    bad = mut.make(getattr(yr, mut.target))
    monkeypatch.setattr(yr, mut.target, bad)
    monkeypatch.setattr(oracle, mut.target, bad)
    caught = None
    with np.errstate(all="ignore"):
        for name, f, kw in _pin_calls(layer_pins):
            try:
                f(**kw)
            except AssertionError:
                caught = name
                break
    assert caught is not None, f"no layer pin fails with the planted mistake: {mut.name}"


def test_layer_pins_pass_unmutated():
    calls = list(_pin_calls(layer_pins))
    assert len(calls) >= 5
    for name, f, kw in calls:
        f(**kw)
