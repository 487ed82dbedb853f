"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a value the
pages print, a closed form, an invariant the pages state, a textbook special
case computed by independent naive loops, or brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# sizes: the worked example of Sec. 3.5 and the pyramid bound of Sec. 3.3
# --------------------------------------------------------------------------
def test_page_example_subsequence_length():
    """N=10^6, L=4, p=4, k=4096: the oracle's own selection + order produce a
    sub-sequence whose length is the value the paper prints (~6.5e4)."""
    g = _load("page_example.json")
    N, L, p, k = g["N"], g["L"], g["p"], g["k"]
    rng = np.random.default_rng(1)
    q = rng.standard_normal((N, 4))
    kk = rng.standard_normal((N, 4))
    qk, kq = orc.scores(q, kk, L, p)
    flags = orc.select(qk, kq, p, k)
    S = len(orc.order(flags, N, L, p))
    assert abs(S - g["S_printed"]) <= g["S_printed_halfwidth"]
    # and it is exactly the closed form of Eq. 8 (budget not exhausted here)
    assert S == N // p ** (L - 1) + (L - 1) * p * k == 64777


def test_pyramid_size_bound():
    for c in _load("pyramid_bound.json")["cases"]:
        N, L, p = c["N"], c["L"], c["p"]
        total = sum(orc.level_sizes(N, L, p))
        assert total <= N * p / (p - 1)
        # geometric series closed form
        assert total == sum(N // p ** l for l in range(L))


def test_divisibility_required():
    with pytest.raises(ValueError):
        orc.level_sizes(1000, 3, 4)        # 16 does not divide 1000
    assert orc.level_sizes(1008, 3, 4) == [1008, 252, 63]


@pytest.mark.parametrize("N,L,p,k,S", [
    (1024, 3, 4, 64, 576), (98304, 3, 4, 768, 12288), (524288, 3, 4, 4096, 65536),
    (1048576, 4, 4, 4096, 65536), (1024, 3, 4, 1024, 1344), (8192, 3, 4, 64, 1024)])
def test_workload_lengths(N, L, p, k, S):
    """S = n_{L-1} + min((L-1)pk, |E|); equals Eq. 8 unless the budget exceeds
    the candidates (then every entry is selected and S = |P|)."""
    sizes = orc.level_sizes(N, L, p)
    assert sizes[-1] + orc.budget(N, L, p, k) == S
    if (L - 1) * p * k <= sum(sizes[:-1]):
        assert S == orc.subsequence_length_eq8(N, L, p, k)
    else:
        assert S == sum(sizes)


# --------------------------------------------------------------------------
# pyramid (Sec. 3.3)
# --------------------------------------------------------------------------
def test_pyramid_direct_equals_recursive():
    """Level l is the mean over the level-0 window; equivalently the mean of
    the p entries of level l-1 it covers (the 'pooling of the previous level')."""
    rng = np.random.default_rng(2)
    N, d, L, p = 4 * 4 * 4 * 3, 5, 4, 4
    x = rng.standard_normal((N, d))
    lv = orc.pyramid(x, L, p)
    for l in range(1, L):
        prev = lv[l - 1]
        rec = np.array([prev[i * p:(i + 1) * p].mean(axis=0) for i in range(len(lv[l]))])
        assert np.max(np.abs(rec - lv[l])) <= 1e-12
    # an explicit loop over the window for one entry
    l, i = 2, 5
    acc = np.zeros(d)
    for t in range(i * p ** l, (i + 1) * p ** l):
        acc += x[t]
    assert np.allclose(acc / p ** l, lv[l][i], rtol=0, atol=1e-13)


def test_pyramid_linear_and_constant():
    rng = np.random.default_rng(3)
    x, y = rng.standard_normal((2, 64, 3))
    a = orc.pyramid(2.0 * x - y, 3, 2)
    b = [2.0 * u - w for u, w in zip(orc.pyramid(x, 3, 2), orc.pyramid(y, 3, 2))]
    for u, w in zip(a, b):
        assert np.max(np.abs(u - w)) < 1e-13
    c = orc.pyramid(np.full((64, 3), 7.25), 3, 2)
    assert all(np.all(u == 7.25) for u in c)


# --------------------------------------------------------------------------
# scores (Sec. 3.4)
# --------------------------------------------------------------------------
def test_scores_are_l2_norms_of_q_and_k():
    N, d = 16, 4
    q = np.zeros((N, d))
    k = np.zeros((N, d))
    q[:, 0], q[:, 1] = 3.0, 4.0          # ||q_t|| = 5
    k[:, 2] = -2.0                       # ||k_t|| = 2
    q[7] = [0, 0, 12, 5]                 # 13
    k[9] = [1, 2, 2, 0]                  # 3
    qk, kq = orc.scores(q, k, 2, 4)
    assert qk[0][7] == 13.0 and qk[0][0] == 5.0
    assert kq[0][9] == 3.0 and kq[0][0] == 2.0
    # coarse = max over the window, not the norm of the pooled row
    assert qk[1][1] == 13.0 and qk[1][0] == 5.0
    assert kq[1][2] == 3.0


def test_max_pool_recursive_exact():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((2, 256, 6))
    qk, kq = orc.scores(q, k, 4, 4)
    for s in (qk, kq):
        for l in range(1, 4):
            rec = s[l - 1].reshape(-1, 4).max(axis=1)
            assert np.array_equal(rec, s[l])      # bit-exact


# --------------------------------------------------------------------------
# select (Sec. 3.4 / 3.5): brute force
# --------------------------------------------------------------------------
def _brute_select(qk, kq, p, k):
    """Independent formulation: rank each candidate by r = max(QK, KQ) with the
    stream index g of the score that attains it (QK wins ties), then sort the
    tuples (-r, g) with Python's sort and keep the first B."""
    L = len(qk)
    sizes = [len(x) for x in qk]
    P = sum(sizes)
    E = P - sizes[-1]
    B = min((L - 1) * p * k, E)
    qf = [float(v) for lev in qk for v in lev]
    kf = [float(v) for lev in kq for v in lev]
    items = []
    for f in range(E):
        if qf[f] >= kf[f]:
            items.append((-qf[f], f, f))
        else:
            items.append((-kf[f], P + f, f))
    items.sort()
    sel = set(f for _, _, f in items[:B]) | set(range(E, P))
    return sel


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("N,L,p,k", [(64, 3, 2, 3), (64, 3, 4, 1), (128, 4, 2, 2), (48, 2, 4, 5), (16, 3, 2, 100)])
def test_select_brute_force_with_ties(seed, N, L, p, k):
    rng = np.random.default_rng(100 + seed)
    d = 3
    # integer-valued rows from a tiny set: many exact ties within and across streams
    q = rng.integers(0, 3, size=(N, d)).astype(np.float64)
    kk = rng.integers(0, 3, size=(N, d)).astype(np.float64)
    qk, kq = orc.scores(q, kk, L, p)
    flags = orc.select(qk, kq, p, k)
    assert set(np.nonzero(flags)[0].tolist()) == _brute_select(qk, kq, p, k)


def test_select_counts_and_coarsest():
    rng = np.random.default_rng(5)
    N, L, p, k = 1024, 3, 4, 64
    q, kk = rng.standard_normal((2, N, 8))
    qk, kq = orc.scores(q, kk, L, p)
    flags = orc.select(qk, kq, p, k)
    sizes = orc.level_sizes(N, L, p)
    E = sum(sizes[:-1])
    assert flags[E:].all()
    assert flags[:E].sum() == (L - 1) * p * k
    # everything when the budget exceeds the candidates
    flags_all = orc.select(qk, kq, p, N)
    assert flags_all.all()


def test_select_kq_entry_enters_whole():
    """An entry picked through its KQ score is selected like any other (one flag
    per entry, not per stream)."""
    N, L, p = 16, 2, 4
    q = np.ones((N, 2))
    kk = np.ones((N, 2))
    kk[5] = [30.0, 40.0]           # KQ of token 5 is the largest score anywhere
    qk, kq = orc.scores(q, kk, L, p)
    flags = orc.select(qk, kq, p, 1)   # budget (L-1) p k = 4
    assert flags[5]
    # the remaining 3 picks are the lowest flat indices among the tied QK=sqrt(2)
    assert np.nonzero(flags[:N])[0].tolist() == [0, 1, 2, 5]


# --------------------------------------------------------------------------
# order + mask (Sec. 3.5): explicit coordinate mask == plain causal mask
# --------------------------------------------------------------------------
def _attend_coordinate_mask(entries, lq, lk, lv, p):
    """Attention over an *unsorted* list of (level, pos) entries where entry e
    sees e' iff (end', level') <= (end, level) lexicographically (base
    positions no greater than its own; finer first at equal ends)."""
    n = len(entries)
    d = lq[0].shape[1]
    out = np.zeros((n, lv[0].shape[1]))
    for a, (la, ia) in enumerate(entries):
        ea = (ia + 1) * p ** la - 1
        logits, vals = [], []
        for (lb, ib) in entries:
            eb = (ib + 1) * p ** lb - 1
            if (eb, lb) <= (ea, la):
                logits.append(float(lq[la][ia] @ lk[lb][ib]) / math.sqrt(d))
                vals.append(lv[lb][ib])
        z = np.array(logits)
        w = np.exp(z - z.max())
        out[a] = (w / w.sum()) @ np.array(vals)
    return out


@pytest.mark.parametrize("N,L,p,k", [(64, 3, 2, 2), (64, 3, 4, 1), (32, 2, 2, 40)])
def test_topological_order_gives_causal_mask(N, L, p, k):
    rng = np.random.default_rng(7)
    d = 4
    q, kk, v = rng.standard_normal((3, N, d))
    res = orc.forward_head(q, kk, v, L, p, k)
    lev, pos = orc.coords_of_flat(res["sorted_flat"], N, L, p)
    entries = list(zip(lev.tolist(), pos.tolist()))
    perm = rng.permutation(len(entries))
    shuffled = [entries[i] for i in perm]
    lq, lk, lv = orc.pyramid(q, L, p), orc.pyramid(kk, L, p), orc.pyramid(v, L, p)
    o_mask = _attend_coordinate_mask(shuffled, lq, lk, lv, p)
    inv = np.argsort(perm)
    assert np.max(np.abs(o_mask[inv] - res["ot"])) < 1e-12


# --------------------------------------------------------------------------
# attention: textbook special cases
# --------------------------------------------------------------------------
def _naive_causal_sdpa(q, k, v):
    """Eq. (1) with a causal mask, by plain loops."""
    N, d = q.shape
    out = np.zeros((N, v.shape[1]))
    for i in range(N):
        zs = []
        for j in range(i + 1):
            s = 0.0
            for c in range(d):
                s += q[i, c] * k[j, c]
            zs.append(s / math.sqrt(d))
        mx = max(zs)
        ws = [math.exp(z - mx) for z in zs]
        tot = sum(ws)
        for j in range(i + 1):
            out[i] += (ws[j] / tot) * v[j]
    return out


def test_L1_is_dense_causal_attention():
    """With one level, S = N, the gather and scatter are the identity and the
    layer is plain causal SDPA."""
    rng = np.random.default_rng(8)
    N, d = 24, 8
    q, kk, v = rng.standard_normal((3, N, d))
    res = orc.forward_head(q, kk, v, 1, 4, 5)
    assert res["S"] == N
    assert np.max(np.abs(res["o"] - _naive_causal_sdpa(q, kk, v))) < 1e-12
    # LSE normalises each row
    z = (q @ kk.T) / math.sqrt(d)
    for i in range(N):
        assert abs(np.exp(z[i, :i + 1] - res["lse"][i]).sum() - 1.0) < 1e-12


def test_select_all_brute_force_forward():
    """k large enough to select every entry: the output equals brute-force
    masked attention over the whole pyramid (entries pooled by explicit loops,
    mask from base positions), scattered with the closed-form index
    i = floor((t+1)/p^l) - 1 of the entry covering t at level l."""
    rng = np.random.default_rng(9)
    N, d, L, p = 64, 4, 3, 4
    q, kk, v = rng.standard_normal((3, N, d))
    res = orc.forward_head(q, kk, v, L, p, N)
    sizes = [N // p ** l for l in range(L)]
    assert res["S"] == sum(sizes)
    pooled = {}
    for l in range(L):
        for i in range(sizes[l]):
            acc = [np.zeros(d), np.zeros(d), np.zeros(d)]
            for t in range(i * p ** l, (i + 1) * p ** l):
                acc[0] += q[t]
                acc[1] += kk[t]
                acc[2] += v[t]
            pooled[(l, i)] = [a / p ** l for a in acc]
    ents = sorted(pooled.keys())
    out_e = {}
    for (la, ia) in ents:
        ea = (ia + 1) * p ** la - 1
        zs, vs = [], []
        for (lb, ib) in ents:
            eb = (ib + 1) * p ** lb - 1
            if eb < ea or (eb == ea and lb <= la):
                zs.append(pooled[(la, ia)][0] @ pooled[(lb, ib)][1] / math.sqrt(d))
                vs.append(pooled[(lb, ib)][2])
        zs = np.array(zs)
        w = np.exp(zs - zs.max())
        out_e[(la, ia)] = (w / w.sum()) @ np.array(vs)
    o = np.zeros((N, d))
    for t in range(N):
        for l in range(L):
            i = (t + 1) // p ** l - 1
            if i >= 0:
                o[t] += out_e[(l, i)]
    assert np.max(np.abs(o - res["o"])) < 1e-12


# --------------------------------------------------------------------------
# scatter (Sec. 3.6)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N,L,p", [(64, 3, 4), (96, 2, 4), (64, 4, 2), (1024, 3, 4)])
def test_scatter_fan_in_disjoint_coverage(N, L, p):
    P = sum(orc.level_sizes(N, L, p))
    flags = np.ones(P, dtype=bool)
    sf = orc.order(flags, N, L, p)
    lev, pos = orc.coords_of_flat(sf, N, L, p)
    fan = np.zeros(N, dtype=int)
    per_level = [np.zeros(N, dtype=int) for _ in range(L)]
    for l, i in zip(lev, pos):
        lo, hi = orc.scatter_range(l, i, N, p)
        fan[lo:hi + 1] += 1
        per_level[l][lo:hi + 1] += 1
    assert fan.max() <= L
    for l in range(L):
        assert per_level[l].max() <= 1                       # disjoint within a level
        assert per_level[l][p ** l - 1:].min() == 1          # covers t >= p^l - 1
        assert per_level[l][:p ** l - 1].sum() == 0
    assert fan[p ** (L - 1) - 1:].min() >= 1


def test_causality_with_frozen_selection():
    """With the index set frozen, O_{<=t0} does not move when Q, K, V change at
    positions > t0: no base position receives a summary of its own future."""
    rng = np.random.default_rng(10)
    N, d, L, p, k = 128, 4, 3, 4, 4
    q, kk, v = rng.standard_normal((3, N, d))
    base = orc.forward_head(q, kk, v, L, p, k)
    for t0 in (0, 3, 14, 15, 16, 63, 100, 126):
        q2, k2, v2 = q.copy(), kk.copy(), v.copy()
        q2[t0 + 1:] += rng.standard_normal((N - t0 - 1, d))
        k2[t0 + 1:] += rng.standard_normal((N - t0 - 1, d))
        v2[t0 + 1:] += rng.standard_normal((N - t0 - 1, d))
        r2 = orc.forward_head(q2, k2, v2, L, p, k, flags=base["flags"])
        assert np.max(np.abs(r2["o"][:t0 + 1] - base["o"][:t0 + 1])) < 1e-12


def test_linear_in_v_with_frozen_selection():
    rng = np.random.default_rng(11)
    N, d, L, p, k = 64, 4, 3, 2, 3
    q, kk, v1, v2 = rng.standard_normal((4, N, d))
    r = orc.forward_head(q, kk, v1, L, p, k)
    fl = r["flags"]
    a = orc.forward_head(q, kk, 2.0 * v1 - 3.0 * v2, L, p, k, flags=fl)["o"]
    b = 2.0 * r["o"] - 3.0 * orc.forward_head(q, kk, v2, L, p, k, flags=fl)["o"]
    assert np.max(np.abs(a - b)) < 1e-12


def test_fixed_point_scatter_close_to_fp64():
    rng = np.random.default_rng(12)
    N, d, L, p, k = 256, 8, 3, 4, 8
    q, kk, v = rng.standard_normal((3, N, d))
    r = orc.forward_head(q, kk, v, L, p, k)
    ot32 = r["ot"].astype(np.float32).astype(np.float64)
    exact = orc.scatter(ot32, r["sorted_flat"], N, L, p)
    fx = orc.scatter_fixed(ot32, r["sorted_flat"], N, L, p, "f32")
    # quantisation <= L * 2^-33, then one fp32 rounding of the result
    assert np.all(np.abs(fx - exact) <= L * 2.0 ** -33 + np.abs(exact) * 2.0 ** -24)
    # integer sum is order-free: a reversed scatter gives the same bits
    rev = r["sorted_flat"][::-1].copy()
    fx_rev = orc.scatter_fixed(ot32[::-1].copy(), rev, N, L, p, "f32")
    assert np.array_equal(fx, fx_rev)


def test_fixed_point_rounding_rules():
    x = np.array([2.0 ** -33, 3 * 2.0 ** -33, -2.0 ** -33, 1.5, -0.75])
    assert orc.to_fixed(x).tolist() == [0, 2, 0, 3 * 2 ** 31, -3 * 2 ** 30]
    acc = np.array([[1], [2 ** 32 + 1], [-(2 ** 32)]], dtype=np.int64)
    out = orc.from_fixed(acc, "f32")[:, 0]
    assert out.tolist() == [np.float32(2.0 ** -32), 1.0, -1.0]
    # bf16 output: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    acc = np.array([[2 ** 32 + 2 ** 24]], dtype=np.int64)
    assert orc.from_fixed(acc, "bf16")[0, 0] == 1.0


# --------------------------------------------------------------------------
# backward (Sec. 3.2): finite differences and the textbook L=1 case
# --------------------------------------------------------------------------
def test_backward_finite_differences():
    rng = np.random.default_rng(13)
    N, d, L, p, k = 32, 4, 3, 2, 2
    q, kk, v, do = rng.standard_normal((4, N, d))
    fl = orc.forward_head(q, kk, v, L, p, k)["flags"]
    dq, dk, dv = orc.backward_head(q, kk, v, do, L, p, fl)

    def loss(a, b, c):
        return float(np.sum(orc.forward_head(a, b, c, L, p, k, flags=fl)["o"] * do))

    eps = 1e-6
    for which, g in ((0, dq), (1, dk), (2, dv)):
        for (t, c) in [(0, 0), (1, 3), (5, 2), (8, 1), (15, 0), (16, 3), (22, 2), (31, 1)]:
            args_p = [q.copy(), kk.copy(), v.copy()]
            args_m = [q.copy(), kk.copy(), v.copy()]
            args_p[which][t, c] += eps
            args_m[which][t, c] -= eps
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[t, c]) < 1e-7 * max(1.0, abs(fd)), (which, t, c, fd, g[t, c])


def test_backward_bf16_store_finite_differences():
    """store="bf16": the gradient of the forward whose pooled levels are the
    exact means plus their bf16 rounding offsets at the base point, held as
    constants (the storage rounding passes the gradient through), by central
    differences of that forward built here from the pinned forward steps.  The
    rounding moves the gradient measurably, so a backward that ignored
    ``store`` fails."""
    rng = np.random.default_rng(17)
    N, d, L, p, k = 32, 4, 3, 2, 2
    q, kk, v, do = rng.standard_normal((4, N, d))
    fl = orc.forward_head(q, kk, v, L, p, k, store="bf16")["flags"]
    dq, dk, dv = orc.backward_head(q, kk, v, do, L, p, fl, store="bf16")
    offs = [[b - a for a, b in zip(orc.pyramid(x, L, p), orc.pyramid(x, L, p, store="bf16"))]
            for x in (q, kk, v)]
    sf = orc.order(fl, N, L, p)

    def loss(*xs):
        rows = [orc.gather([lv + o for lv, o in zip(orc.pyramid(x, L, p), off)], sf, N, L, p)
                for x, off in zip(xs, offs)]
        ot, _ = orc.attend(*rows)
        return float(np.sum(orc.scatter(ot, sf, N, L, p) * do))

    eps = 1e-6
    for which, g in ((0, dq), (1, dk), (2, dv)):
        for (t, c) in [(0, 0), (1, 3), (5, 2), (8, 1), (15, 0), (16, 3), (22, 2), (31, 1)]:
            args_p = [q.copy(), kk.copy(), v.copy()]
            args_m = [q.copy(), kk.copy(), v.copy()]
            args_p[which][t, c] += eps
            args_m[which][t, c] -= eps
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[t, c]) < 1e-7 * max(1.0, abs(fd)), (which, t, c, fd, g[t, c])
    pure = orc.backward_head(q, kk, v, do, L, p, fl)
    assert max(np.max(np.abs(a - b)) for a, b in zip(pure, (dq, dk, dv))) > 1e-5


def test_backward_L1_textbook():
    """L=1: the gradient is the textbook causal-attention gradient, here by
    plain loops over the softmax Jacobian."""
    rng = np.random.default_rng(14)
    N, d = 12, 4
    q, kk, v, do = rng.standard_normal((4, N, d))
    fl = np.ones(N, dtype=bool)
    dq, dk, dv = orc.backward_head(q, kk, v, do, 1, 2, fl)
    s = 1.0 / math.sqrt(d)
    eq, ek, ev = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    for i in range(N):
        z = np.array([q[i] @ kk[j] * s for j in range(i + 1)])
        w = np.exp(z - z.max())
        pr = w / w.sum()
        g = np.array([do[i] @ v[j] for j in range(i + 1)])    # dL/dP_ij
        for j in range(i + 1):
            ev[j] += pr[j] * do[i]
            dz = pr[j] * (g[j] - sum(pr[u] * g[u] for u in range(i + 1)))
            eq[i] += dz * s * kk[j]
            ek[j] += dz * s * q[i]
    for a, b in ((dq, eq), (dk, ek), (dv, ev)):
        assert np.max(np.abs(a - b)) < 1e-12


def test_attend_rows_matches_attend():
    rng = np.random.default_rng(15)
    S, d = 300, 8
    qt, kt, vt = rng.standard_normal((3, S, d))
    o, lse = orc.attend(qt, kt, vt, row_block=64)
    rows = [0, 1, 63, 64, 150, 299]
    o2, lse2 = orc.attend_rows(qt, kt, vt, rows)
    assert np.max(np.abs(o2 - o[rows])) < 1e-13
    assert np.max(np.abs(lse2 - lse[rows])) < 1e-13


def test_round_bf16_cases():
    """bf16 keeps 8 significant bits: 1 + 2^-8 is a tie between 1 and 1 + 2^-7
    (to even: 1); 1 + 3 * 2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6 (to even:
    1 + 2^-6); just above the half-ulp rounds up; sign and powers of two exact."""
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -3.0, 2.0 ** -100, 0.0])
    assert orc.round_bf16(x).tolist() == [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -3.0, 2.0 ** -100, 0.0]


def test_pyramid_bf16_store_rounds_only_pooled_levels():
    rng = np.random.default_rng(16)
    x = orc.round_bf16(rng.standard_normal((64, 5)))
    a = orc.pyramid(x, 3, 4)
    b = orc.pyramid(x, 3, 4, store="bf16")
    assert np.array_equal(a[0], b[0])
    for u, w in zip(a[1:], b[1:]):
        # bf16 keeps 8 significant bits: unit roundoff 2^-8 (after the fp32 rounding)
        assert np.all(np.abs(u - w) <= (2.0 ** -8 + 2.0 ** -23) * np.abs(u))
        assert np.array_equal(orc.round_bf16(w), w)                # already bf16 values
