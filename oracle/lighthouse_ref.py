"""Lighthouse attention: plain fp64 CPU oracle.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The product path (the HIP library
and its Python binding) never does, and this module imports nothing from it.

What it computes, step by step, in the order the method is described, in float64
on whatever input values it is given (bf16 inputs are passed upcast exactly):

  "Paper" = "Long Context Pre-Training with Lighthouse Attention" (HTML mirror of
  arXiv 2605.06554).  Its display equations were lost in extraction; section
  labels follow the paper's own cross-references (Sec. 3.1 ... 3.6).
  "Blog"  = "Lighthouse Attention：让长上下文预训练只在"塔尖"上算注意力" (a
  section-by-section paraphrase of the paper with the same 3.x headings).

  1. pyramid        Paper §3.3 (window W_i^(l) = [i p^l, (i+1) p^l - 1], mean pool
                    of Q, K and V alike; requires p^(L-1) | N).
  2. scores         Paper §3.4 (level 0: per-head l2 norms of Q rows (QK score)
                    and of K rows (KQ score); coarser levels max-pool the level-0
                    scores over the window instead of re-scoring pooled rows).
  3. select         Paper §3.4 (one selection jointly over the concatenated QK and
                    KQ streams across levels; coarsest level always kept) and
                    §3.5 (budget: each non-coarsest level adds at most p*k, so the
                    gathered length obeys Eq. 8).
  4. order          Paper §3.5 (gather sorted topologically by pyramid coordinate
                    so that the mask of Eq. 9 is the plain S x S causal mask).
  5. gather         Paper §3.5.
  6. attend         Paper §3.1 Eq. (1) / §3.5 Eq. (9): softmax(Q K^T / sqrt(d) +
                    causal mask) V over the gathered sub-sequence.
  7. scatter        Paper §3.6 (output of entry (l, i) written to the window
                    shifted by p^l - 1, i.e. starting at its last summarised
                    token; contributions of different levels summed; the
                    integer-atomic kernel's fixed-point arithmetic is modelled
                    exactly by ``scatter_fixed``).
  backward          Paper §3.2: indices are discrete and carry no gradient; the
                    gradient flows through scatter, attention, gather and pool.

Readings taken where the pages leave a step open:
  * attention scale 1/sqrt(d) for every entry, pooled or not;
  * scores are l2 norms, not squared norms;
  * selection budget B = min((L-1) p k, |E|) *distinct* entries over the
    non-coarsest levels E, ranked by walking the concatenated QK||KQ stream in
    (value descending, stream index ascending) order; the stream index of the QK
    score of flat entry f is f and of its KQ score |P| + f, where the flat index
    runs level-major, finest level first;
  * topological order: by window end (i+1) p^l - 1 ascending, finer level first
    among equal ends;
  * the scatter range [end, end + p^l - 1] is clipped at N - 1; positions with no
    selected contributor receive 0;
  * fixed point: int64 with 32 fractional bits, round-half-even in and out;
  * bf16 mode (``store="bf16"``): the paper benchmarks the layer in bf16 and
    hands the gathered sub-sequence to stock FlashAttention as bf16 tensors
    (§3.5; experiments paragraph on Fig. 3), so the pooled levels l >= 1 are
    rounded to bf16 (round to nearest even) once, right after their exact
    mean; every other step stays fp64.  Level 0 is the bf16 input itself.

Every function here has a pin in tests/ against something other than itself
(closed forms, a textbook special case, brute force, finite differences).
"""
from __future__ import annotations

import math

import numpy as np

FIX_FRAC_BITS = 32


# ----------------------------------------------------------------------------
# sizes (Paper §3.3 pyramid size; §3.5 Eq. 8)
# ----------------------------------------------------------------------------
def level_sizes(N: int, L: int, p: int) -> list[int]:
    """n_l = N / p^l for l = 0..L-1.  Paper §3.3 requires p^(L-1) | N."""
    if L < 1 or p < 2:
        raise ValueError("need L >= 1 and p >= 2")
    if N % (p ** (L - 1)) != 0:
        raise ValueError("p^(L-1) must divide N")
    return [N // p ** l for l in range(L)]


def flat_offsets(N: int, L: int, p: int) -> list[int]:
    """Offset of level l in the flat pyramid index (level-major, finest first)."""
    off, acc = [], 0
    for n in level_sizes(N, L, p):
        off.append(acc)
        acc += n
    return off


def budget(N: int, L: int, p: int, k: int) -> int:
    """Number of non-coarsest entries selected: min((L-1) p k, |E|)."""
    sizes = level_sizes(N, L, p)
    n_cand = sum(sizes[:-1])
    return min((L - 1) * p * k, n_cand)


def subsequence_length_eq8(N: int, L: int, p: int, k: int) -> int:
    """Paper §3.5 Eq. 8: S = N / p^(L-1) + (L-1) p k (an upper bound)."""
    return N // p ** (L - 1) + (L - 1) * p * k


# ----------------------------------------------------------------------------
# 1. pyramid (Paper §3.3)
# ----------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), returned as float64:
    keep the top 16 bits of the fp32 pattern after adding half an ulp of bf16
    (plus one if the kept part is odd).  x must already be an fp32 value or be
    rounded to fp32 first (done here)."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def pyramid(x: np.ndarray, L: int, p: int, store: str | None = None) -> list[np.ndarray]:
    """Levels 0..L-1 of one tensor x [N, d]: X^(l)_i = mean of x over the
    base tokens t in [i p^l, (i+1) p^l - 1] (direct mean from level 0).
    store="bf16" rounds the pooled levels (l >= 1) to bf16 after the mean."""
    x = np.asarray(x, dtype=np.float64)
    N, d = x.shape
    out = []
    for l, n in enumerate(level_sizes(N, L, p)):
        w = p ** l
        lev = x.reshape(n, w, d).mean(axis=1)
        if store == "bf16" and l > 0:
            lev = round_bf16(lev)
        out.append(lev)
    return out


# ----------------------------------------------------------------------------
# 2. scores (Paper §3.4)
# ----------------------------------------------------------------------------
def scores(q: np.ndarray, k: np.ndarray, L: int, p: int):
    """QK and KQ score of every pyramid entry, as two lists of per-level arrays.

    Level 0: QK_t = ||Q_t||_2 and KQ_t = ||K_t||_2.  Level l: the maximum of the
    level-0 score over the window of base tokens the entry summarises."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N = q.shape[0]
    a = np.sqrt(np.sum(q * q, axis=1))
    b = np.sqrt(np.sum(k * k, axis=1))
    qk, kq = [], []
    for l, n in enumerate(level_sizes(N, L, p)):
        w = p ** l
        qk.append(a.reshape(n, w).max(axis=1))
        kq.append(b.reshape(n, w).max(axis=1))
    return qk, kq


# ----------------------------------------------------------------------------
# 3. select (Paper §3.4, §3.5)
# ----------------------------------------------------------------------------
def select(qk: list[np.ndarray], kq: list[np.ndarray], p: int, k: int) -> np.ndarray:
    """Boolean flag per flat pyramid entry: True if the entry is in the index set I.

    The candidates are the entries of levels 0..L-2.  Their QK scores (stream
    index f) and KQ scores (stream index |P| + f) are concatenated into one
    stream; walking it in (score descending, stream index ascending) order, the
    first B distinct entries are kept, B = min((L-1) p k, |E|).  An entry reached
    through its KQ score is selected as a whole (it enters the gather with its
    own Q, K and V).  Every entry of the coarsest level is always in I."""
    L = len(qk)
    sizes = [len(x) for x in qk]
    P = sum(sizes)
    E = P - sizes[-1]
    B = min((L - 1) * p * k, E)
    flags = np.zeros(P, dtype=bool)
    flags[E:] = True
    if B == 0:
        return flags
    qk_flat = np.concatenate(qk)[:E]
    kq_flat = np.concatenate(kq)[:E]
    stream_val = np.concatenate([qk_flat, kq_flat])
    stream_idx = np.concatenate([np.arange(E), P + np.arange(E)])
    walk = np.lexsort((stream_idx, -stream_val))  # value desc, then index asc
    entry_in_walk = stream_idx[walk] % P
    # first position at which each entry appears in the walk
    first_pos = np.full(E, np.iinfo(np.int64).max, dtype=np.int64)
    np.minimum.at(first_pos, entry_in_walk, np.arange(len(walk)))
    kept = np.argsort(first_pos, kind="stable")[:B]
    flags[kept] = True
    return flags


# ----------------------------------------------------------------------------
# 4. order (Paper §3.5)
# ----------------------------------------------------------------------------
def coords_of_flat(f: np.ndarray, N: int, L: int, p: int):
    """(level, position) of flat pyramid indices."""
    off = flat_offsets(N, L, p)
    f = np.asarray(f, dtype=np.int64)
    lev = np.zeros_like(f)
    for l in range(1, L):
        lev += (f >= off[l]).astype(np.int64)
    pos = f - np.asarray(off, dtype=np.int64)[lev]
    return lev, pos


def window_end(lev, pos, p: int):
    """Base position of an entry: the last token of its window, (i+1) p^l - 1."""
    return (np.asarray(pos, dtype=np.int64) + 1) * (np.int64(p) ** np.asarray(lev, dtype=np.int64)) - 1


def order(flags: np.ndarray, N: int, L: int, p: int) -> np.ndarray:
    """Flat indices of the selected entries in topological order: window end
    ascending, finer level first among entries with the same end."""
    f = np.nonzero(flags)[0].astype(np.int64)
    lev, pos = coords_of_flat(f, N, L, p)
    end = window_end(lev, pos, p)
    return f[np.lexsort((lev, end))]


# ----------------------------------------------------------------------------
# 5. gather (Paper §3.5)
# ----------------------------------------------------------------------------
def gather(levels: list[np.ndarray], sorted_flat: np.ndarray, N: int, L: int, p: int) -> np.ndarray:
    lev, pos = coords_of_flat(sorted_flat, N, L, p)
    d = levels[0].shape[1]
    out = np.empty((len(sorted_flat), d), dtype=np.float64)
    for m in range(len(sorted_flat)):
        out[m] = levels[lev[m]][pos[m]]
    return out


# ----------------------------------------------------------------------------
# 6. attend (Paper §3.1 Eq. (1), §3.5 Eq. (9))
# ----------------------------------------------------------------------------
def attend(qt: np.ndarray, kt: np.ndarray, vt: np.ndarray, row_block: int = 1024):
    """Causal softmax attention over the sorted sub-sequence: row m attends to
    rows m' <= m with logits Q_m . K_m' / sqrt(d).  Returns (O, LSE) where LSE
    is the natural-log log-sum-exp of each row's logits.

    Rows are computed in groups of ``row_block`` only to bound memory; each row
    is the exact full-row softmax of its own logits."""
    S, d = qt.shape
    scale = 1.0 / math.sqrt(d)
    o = np.empty((S, vt.shape[1]), dtype=np.float64)
    lse = np.empty(S, dtype=np.float64)
    for r0 in range(0, S, row_block):
        r1 = min(S, r0 + row_block)
        z = (qt[r0:r1] @ kt[:r1].T) * scale
        rows = np.arange(r0, r1)[:, None]
        cols = np.arange(r1)[None, :]
        z = np.where(cols <= rows, z, -np.inf)
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        ssum = e.sum(axis=1, keepdims=True)
        o[r0:r1] = (e / ssum) @ vt[:r1]
        lse[r0:r1] = (zmax + np.log(ssum))[:, 0]
    return o, lse


def attend_rows(qt: np.ndarray, kt: np.ndarray, vt: np.ndarray, rows):
    """The rows ``rows`` of ``attend`` only (same per-row definition), for
    checking sampled outputs of a sub-sequence too long to attend in full."""
    S, d = qt.shape
    scale = 1.0 / math.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((len(rows), vt.shape[1]), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    for n, m in enumerate(rows):
        z = (kt[:m + 1] @ qt[m]) * scale
        zmax = z.max()
        e = np.exp(z - zmax)
        ssum = e.sum()
        o[n] = (e / ssum) @ vt[:m + 1]
        lse[n] = zmax + np.log(ssum)
    return o, lse


# ----------------------------------------------------------------------------
# 7. scatter (Paper §3.6)
# ----------------------------------------------------------------------------
def scatter_range(lev: int, pos: int, N: int, p: int):
    """Base positions [lo, hi] (inclusive) that entry (lev, pos) writes: the
    window shifted by p^lev - 1, clipped at N - 1."""
    w = p ** int(lev)
    lo = (int(pos) + 1) * w - 1
    hi = min(N - 1, lo + w - 1)
    return lo, hi


def scatter(ot: np.ndarray, sorted_flat: np.ndarray, N: int, L: int, p: int) -> np.ndarray:
    """O_t = sum of the outputs of all selected entries whose range holds t (fp64)."""
    lev, pos = coords_of_flat(sorted_flat, N, L, p)
    out = np.zeros((N, ot.shape[1]), dtype=np.float64)
    for m in range(len(sorted_flat)):
        lo, hi = scatter_range(lev[m], pos[m], N, p)
        if lo <= hi:
            out[lo:hi + 1] += ot[m]
    return out


def to_fixed(x: np.ndarray) -> np.ndarray:
    """RNE(x * 2^32) as int64 (x is taken exactly as given, e.g. fp32 values)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.rint(x * float(2 ** FIX_FRAC_BITS))
    if np.any(np.abs(y) >= 2.0 ** 62):
        raise OverflowError("value out of fixed-point range")
    return y.astype(np.int64)


def from_fixed(acc: np.ndarray, out_dtype: str = "f32") -> np.ndarray:
    """int64 fixed point -> fp32 (RNE), optionally then -> bf16 (RNE), returned
    as float64 holding exactly the rounded values."""
    v = acc.astype(np.float64) * 2.0 ** -FIX_FRAC_BITS
    v32 = v.astype(np.float32)
    if out_dtype == "f32":
        return v32.astype(np.float64)
    if out_dtype == "bf16":
        u = v32.view(np.uint32).astype(np.uint64)
        r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
        return r.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(out_dtype)


def scatter_fixed(ot: np.ndarray, sorted_flat: np.ndarray, N: int, L: int, p: int,
                  out_dtype: str = "f32") -> np.ndarray:
    """Scatter with the integer-atomic kernel's arithmetic: each contribution is
    quantised to int64 fixed point, the integers are summed (order-free), and
    the sum is converted back.  Bit-exact model of a deterministic integer
    scatter given the same O~ values."""
    lev, pos = coords_of_flat(sorted_flat, N, L, p)
    q = to_fixed(ot)
    acc = np.zeros((N, ot.shape[1]), dtype=np.int64)
    for m in range(len(sorted_flat)):
        lo, hi = scatter_range(lev[m], pos[m], N, p)
        if lo <= hi:
            acc[lo:hi + 1] += q[m]
    return from_fixed(acc, out_dtype)


# ----------------------------------------------------------------------------
# whole forward for one head (Paper §3.2 four-stage pipeline)
# ----------------------------------------------------------------------------
def forward_head(q, k, v, L: int, p: int, topk: int, flags=None, out_dtype: str | None = None,
                 store: str | None = None):
    """One (b, h) head.  q, k, v: [N, d] arrays (any float dtype, upcast to fp64).

    ``flags`` (optional) injects a selection instead of computing one.  Returns a
    dict with the pyramid scores, the selection, the sorted flat indices, the
    gathered rows, O~, LSE, the fp64 output O, and (if ``out_dtype`` is given)
    the fixed-point output.  ``store="bf16"`` rounds the pooled levels to bf16
    (see the module notes)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    level_sizes(N, L, p)
    qk, kq = scores(q, k, L, p)
    if flags is None:
        flags = select(qk, kq, p, topk)
    sorted_flat = order(flags, N, L, p)
    lq, lk, lv = pyramid(q, L, p, store), pyramid(k, L, p, store), pyramid(v, L, p, store)
    qt = gather(lq, sorted_flat, N, L, p)
    kt = gather(lk, sorted_flat, N, L, p)
    vt = gather(lv, sorted_flat, N, L, p)
    ot, lse = attend(qt, kt, vt)
    res = dict(qk=qk, kq=kq, flags=flags, sorted_flat=sorted_flat, qt=qt, kt=kt, vt=vt,
               ot=ot, lse=lse, o=scatter(ot, sorted_flat, N, L, p), S=len(sorted_flat))
    if out_dtype is not None:
        res["o_fixed"] = scatter_fixed(ot, sorted_flat, N, L, p, out_dtype)
    return res


# ----------------------------------------------------------------------------
# backward for one head, selection frozen (Paper §3.2)
# ----------------------------------------------------------------------------
def scatter_adjoint(do: np.ndarray, sorted_flat: np.ndarray, N: int, L: int, p: int) -> np.ndarray:
    """dO~_m = sum of dO_t over the scatter range of entry m."""
    lev, pos = coords_of_flat(sorted_flat, N, L, p)
    out = np.zeros((len(sorted_flat), do.shape[1]), dtype=np.float64)
    for m in range(len(sorted_flat)):
        lo, hi = scatter_range(lev[m], pos[m], N, p)
        if lo <= hi:
            out[m] = do[lo:hi + 1].sum(axis=0)
    return out


def attend_adjoint(qt, kt, vt, dot, row_block: int = 1024):
    """Adjoint of ``attend``: returns (dQ~, dK~, dV~) for upstream dO~.

    With P the causal softmax matrix and Z the logits:
      dV = P^T dO,  dP = dO V^T,  dZ = P o (dP - rowsum(dP o P)),
      dQ = dZ K / sqrt(d),  dK = dZ^T Q / sqrt(d)."""
    S, d = qt.shape
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(qt)
    dk = np.zeros_like(kt)
    dv = np.zeros_like(vt)
    for r0 in range(0, S, row_block):
        r1 = min(S, r0 + row_block)
        z = (qt[r0:r1] @ kt[:r1].T) * scale
        rows = np.arange(r0, r1)[:, None]
        cols = np.arange(r1)[None, :]
        z = np.where(cols <= rows, z, -np.inf)
        e = np.exp(z - z.max(axis=1, keepdims=True))
        prob = e / e.sum(axis=1, keepdims=True)
        dv[:r1] += prob.T @ dot[r0:r1]
        dp = dot[r0:r1] @ vt[:r1].T
        dz = prob * (dp - np.sum(dp * prob, axis=1, keepdims=True))
        dq[r0:r1] += (dz @ kt[:r1]) * scale
        dk[:r1] += (dz.T @ qt[r0:r1]) * scale
    return dq, dk, dv


def pool_adjoint(dlevels: list[np.ndarray], N: int, p: int) -> np.ndarray:
    """Adjoint of ``pyramid``: dX_t = sum_l dX^(l)_{floor(t / p^l)} / p^l."""
    d = dlevels[0].shape[1]
    out = np.zeros((N, d), dtype=np.float64)
    for l, dl in enumerate(dlevels):
        w = p ** l
        out += np.repeat(dl, w, axis=0) / w
    return out


def backward_head(q, k, v, do, L: int, p: int, flags: np.ndarray, store: str | None = None):
    """(dQ, dK, dV) of sum(O * dO) for one head with the selection ``flags``
    frozen: no gradient reaches the scores.

    ``store="bf16"`` differentiates the bf16-mode forward of ``forward_head``:
    the attention adjoint is taken at the gathered rows as that forward stores
    them (pooled levels rounded to bf16), and the rounding itself passes the
    gradient through unchanged -- it is the gradient of the forward whose
    pooled levels carry their rounding offsets, taken at the base point, as
    constants."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    N, d = q.shape
    sizes = level_sizes(N, L, p)
    sorted_flat = order(flags, N, L, p)
    qt = gather(pyramid(q, L, p, store), sorted_flat, N, L, p)
    kt = gather(pyramid(k, L, p, store), sorted_flat, N, L, p)
    vt = gather(pyramid(v, L, p, store), sorted_flat, N, L, p)
    dot = scatter_adjoint(do, sorted_flat, N, L, p)
    dqt, dkt, dvt = attend_adjoint(qt, kt, vt, dot)
    lev, pos = coords_of_flat(sorted_flat, N, L, p)
    grads = []
    for dt in (dqt, dkt, dvt):
        dl = [np.zeros((n, d), dtype=np.float64) for n in sizes]
        for m in range(len(sorted_flat)):   # gather adjoint: each entry appears once
            dl[lev[m]][pos[m]] = dt[m]
        grads.append(pool_adjoint(dl, N, p))
    return tuple(grads)
