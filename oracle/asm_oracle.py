"""Attention-state memory (ASM): the fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The library's product path never
calls it, and it imports nothing from the library: the two implementations
share no code.  Every function here is plain numpy in float64, written to be
checked against the pages by eye, not to be fast.

Sources (cited by page title and section):

* [TS] "Context Memorization for Efficient Long Context Generation" -- the
  technical summary on gist.science ("Resumen Técnico: Memoria de Estado de
  Atención ...").  Sections used: "Metodología" (the attention state and the
  online-softmax decomposition), its "Fase de Calibración Offline"
  (Recolección, Agrupamiento, Agregación, Eficiencia) and "Fase de Inferencia
  Online" (Recuperación, Fusión, Complejidad).
* [NEWS] "Búsqueda de Memoria Reemplaza Atención Lineal en Prefijos Largos"
  (aiexpert.news), the paragraph on how the method works.
* [ABS] "Запоминание контекста для эффективной генерации длинного контекста"
  (chatpaper abstract, English part).

Conventions (readings where the pages are silent; each is listed in the design
notes with its reason):

* An attention state is a pair (a, lse): a is the softmax-weighted average of
  the values, lse = log Z with Z = sum_j exp(scale * q.k_j) the unshifted
  normaliser ([TS] Metodología names the pair (a, Z)).  The empty state is
  (a = 0, lse = -inf); merging with it is the identity.
* scale is passed in by the caller (the tests use float32(1/sqrt(d))).
* Cosine similarity cos(x, c) = x.c / (|x| |c|); a zero vector has cosine 0
  with everything, so a zero centroid scores 0 and a zero query ties
  everywhere (lowest index wins).
* Ties in the nearest-centroid search go to the lowest index.
* k-means ([TS] Agrupamiento says "e.g. K-means") uses the same cosine metric as
  retrieval ([TS] Recuperación), first-K initialisation, and keeps the previous
  centroid for an empty cluster; the centroid is the arithmetic mean of the
  members' raw queries ([TS] Agregación), rounded once to the table's type.
* Aggregated normaliser: Z_bar = mean of the members' Z, so
  lse_bar = logsumexp(lse_i) - log n_k; a_bar is the Z-weighted mean of the
  members' a_i ([TS] Agregación: merge with the online-softmax rule into a
  lossless average).

* Whitening at retrieval ([TS] Recuperación, optional): x -> W (x - mu) fit
  per head on the calibration queries, W the symmetric inverse square root of
  their ridged population covariance; whitened rows are rounded once to the
  table's type and scored by cosine.

Inputs arrive as float64 arrays.  bf16 data arrive as uint16 bit patterns and
are widened with `bf16_bits_to_f64` (exact); float32 data with `f32_to_f64`
(exact).
"""
from __future__ import annotations

import math

import numpy as np

EMPTY_LSE = -np.inf

# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly: a bf16 value is the upper
    half of the float32 with the same bits."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_f64(x) -> np.ndarray:
    """Widen float32 values to float64 (exact)."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def round_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 with round-to-nearest, ties-to-even, in one
    step (no intermediate float32 rounding).

    bf16 keeps 8 significant bits and float32's exponent range.  For a finite
    nonzero x with binary exponent e (x = m * 2**e, 0.5 <= |m| < 1) the spacing
    of bf16 values around x is 2**(e-8), but never finer than the subnormal
    spacing 2**-133.  x / spacing is exact in float64; np.rint rounds it to
    the nearest integer with ties to even, and the product is the rounded
    value.  Results of magnitude 2**128 or more overflow to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    finite = np.isfinite(flat)
    # non-finite inputs
    nan = np.isnan(flat)
    out[nan] = 0x7FC0
    posinf = np.isposinf(flat)
    neginf = np.isneginf(flat)
    out[posinf] = 0x7F80
    out[neginf] = 0xFF80
    xf = flat[finite]
    _, e = np.frexp(xf)
    quantum_exp = np.maximum(e - 8, -133)
    q = np.ldexp(np.ones_like(xf), quantum_exp)
    r = np.rint(xf / q) * q
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    bits32 = r.astype(np.float32).view(np.uint32)  # exact: r has <= 8 significant bits
    out[finite] = (bits32 >> np.uint32(16)).astype(np.uint16)
    return out.reshape(x.shape)


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round float64 values once to the storage type ("bf16" or "f32") and
    return them widened back to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(round_to_bf16_bits(x))
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# O1 / O2: the attention state and the online-softmax merge
# [TS] Metodología: attention over a block of keys is summarised by its output
# and its normaliser; attention over concatenated blocks decomposes into the
# blocks' states combined by the online-softmax identity.
# --------------------------------------------------------------------------


def state(q, K, V, scale: float):
    """Attention state of one query (q [d]) over one key block (K, V [n, d]).

    Returns (a [d], lse): s_j = scale * q.k_j, a = sum_j softmax(s)_j v_j,
    lse = log sum_j exp(s_j).  An empty block gives the empty state (0, -inf).
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64).reshape(-1, q.shape[-1])
    V = np.asarray(V, np.float64)
    V = V.reshape(K.shape[0], V.shape[-1])
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), EMPTY_LSE
    s = scale * (K @ q)
    m = s.max()
    w = np.exp(s - m)
    z = w.sum()
    a = (w @ V) / z
    return a, m + math.log(z)


def states(Q, K, V, scale: float):
    """`state` for many queries at once: Q [N, d] over one block K, V [n, d].
    Returns A [N, d], LSE [N]."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64).reshape(-1, Q.shape[-1])
    V = np.asarray(V, np.float64)
    V = V.reshape(K.shape[0], V.shape[-1])
    N = Q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((N, V.shape[1])), np.full(N, EMPTY_LSE)
    S = scale * (Q @ K.T)  # [N, n]
    m = S.max(axis=1)
    W = np.exp(S - m[:, None])
    z = W.sum(axis=1)
    A = (W @ V) / z[:, None]
    return A, m + np.log(z)


def merge(a1, l1, a2, l2):
    """Online-softmax merge of two states over disjoint key blocks.

    With Z_i = exp(l_i): a = (Z1 a1 + Z2 a2) / (Z1 + Z2), lse = log(Z1 + Z2),
    evaluated relative to m = max(l1, l2) so nothing overflows.  Merging with
    the empty state (lse = -inf) returns the other state; two empty states
    give the empty state.  Broadcasts over leading axes (a [..., d], l [...]).
    """
    a1 = np.asarray(a1, np.float64)
    a2 = np.asarray(a2, np.float64)
    l1 = np.asarray(l1, np.float64)
    l2 = np.asarray(l2, np.float64)
    m = np.maximum(l1, l2)
    both_empty = np.isneginf(m)
    m_safe = np.where(both_empty, 0.0, m)
    w1 = np.where(np.isneginf(l1), 0.0, np.exp(l1 - m_safe))
    w2 = np.where(np.isneginf(l2), 0.0, np.exp(l2 - m_safe))
    z = w1 + w2
    z_safe = np.where(both_empty, 1.0, z)
    a = (w1[..., None] * a1 + w2[..., None] * a2) / z_safe[..., None]
    a = np.where(both_empty[..., None], 0.0, a)
    lse = np.where(both_empty, EMPTY_LSE, m_safe + np.log(z_safe))
    if np.ndim(lse) == 0:
        return a, float(lse)
    return a, lse


# --------------------------------------------------------------------------
# O3: collection of prefix states, chunk by chunk
# [TS] Recolección: per response query, record the query and its attention
# state over the prefix.  [TS] Eficiencia: a long prefix may be split into
# chunks whose states are computed independently and merged.
# --------------------------------------------------------------------------


def build_states(Q, Kp, Vp, chunk: int, scale: float):
    """Prefix attention states of every query, chunk by chunk.

    Q [Hq, N, d]; Kp, Vp [Hkv, L, d]; query head h reads kv head
    h // (Hq // Hkv).  The prefix is cut into ceil(L / chunk) consecutive
    chunks; each chunk's state is computed on its own and the running state is
    merged with it in chunk order.

    Returns (A_chunks [nc, Hq, N, d], LSE_chunks [nc, Hq, N], A [Hq, N, d],
    LSE [Hq, N]).
    """
    Q = np.asarray(Q, np.float64)
    Kp = np.asarray(Kp, np.float64)
    Vp = np.asarray(Vp, np.float64)
    Hq, N, d = Q.shape
    Hkv, L, _ = Kp.shape
    group = Hq // Hkv
    nc = -(-L // chunk) if L > 0 else 0
    A_chunks = np.zeros((nc, Hq, N, d))
    L_chunks = np.full((nc, Hq, N), EMPTY_LSE)
    A = np.zeros((Hq, N, d))
    LSE = np.full((Hq, N), EMPTY_LSE)
    for h in range(Hq):
        g = h // group
        run_a = np.zeros((N, d))
        run_l = np.full(N, EMPTY_LSE)
        for c in range(nc):
            lo, hi = c * chunk, min(L, (c + 1) * chunk)
            a_c, l_c = states(Q[h], Kp[g, lo:hi], Vp[g, lo:hi], scale)
            A_chunks[c, h], L_chunks[c, h] = a_c, l_c
            run_a, run_l = merge(run_a, run_l, a_c, l_c)
        A[h], LSE[h] = run_a, run_l
    return A_chunks, L_chunks, A, LSE


# --------------------------------------------------------------------------
# O4 / O5: cosine retrieval
# [TS] Recuperación: the nearest memory centroid is the one of highest cosine
# similarity with the incoming query.
# --------------------------------------------------------------------------


def inv_norms(C):
    """1/|c| per row of C [..., K, d]; 0 for a zero row."""
    C = np.asarray(C, np.float64)
    n = np.sqrt((C * C).sum(axis=-1))
    return np.where(n > 0, 1.0 / np.where(n > 0, n, 1.0), 0.0)


def cosine(X, C):
    """cos(x_i, c_k) for X [N, d] and C [K, d] -> [N, K]."""
    X = np.asarray(X, np.float64)
    C = np.asarray(C, np.float64)
    xin = inv_norms(X)
    cin = inv_norms(C)
    return (X @ C.T) * xin[:, None] * cin[None, :]


def assign(X, C):
    """Nearest centroid by cosine, lowest index on ties.

    Returns (idx [N] int, cos [N, K], gap [N]) where gap is the best cosine
    minus the second best (inf when K == 1).
    """
    cs = cosine(X, C)
    idx = np.argmax(cs, axis=1)  # first occurrence of the maximum
    N, K = cs.shape
    top1 = cs[np.arange(N), idx]
    if K > 1:
        rest = cs.copy()
        rest[np.arange(N), idx] = -np.inf
        gap = top1 - rest.max(axis=1)
    else:
        gap = np.full(N, np.inf)
    return idx, cs, gap


def accept_index(idx_other, cos_rows, tol: float = 1e-5):
    """Which of the indices in idx_other [N] are acceptable nearest-centroid
    picks: exactly the oracle's pick, or within tol (cosine units) of the best
    cosine.  cos_rows is the oracle's [N, K] cosine matrix."""
    cs = np.asarray(cos_rows, np.float64)
    idx_other = np.asarray(idx_other).astype(np.int64)
    N = cs.shape[0]
    ok_range = (idx_other >= 0) & (idx_other < cs.shape[1])
    safe = np.where(ok_range, idx_other, 0)
    best = cs.max(axis=1)
    picked = cs[np.arange(N), safe]
    return ok_range & (picked >= best - tol)


# --------------------------------------------------------------------------
# O6: k-means on the collected queries
# [TS] Agrupamiento: the collected query vectors are clustered into K
# centroids.  [TS] Agregación: a centroid's query is the mean of its
# cluster's queries.
# --------------------------------------------------------------------------


def centroid_update(X, idx, C_prev, dtype: str):
    """One mean step: C_k = round(sum_{i: idx_i = k} x_i / n_k) with a float64
    sum and one rounding to `dtype`; an empty cluster keeps C_prev[k].

    Returns (C [K, d] float64 holding `dtype` values, counts [K] int64)."""
    X = np.asarray(X, np.float64)
    C_prev = np.asarray(C_prev, np.float64)
    K = C_prev.shape[0]
    idx = np.asarray(idx).astype(np.int64)
    counts = np.bincount(idx, minlength=K).astype(np.int64)
    sums = np.zeros_like(C_prev)
    np.add.at(sums, idx, X)
    C = C_prev.copy()
    nz = counts > 0
    C[nz] = round_to_dtype(sums[nz] / counts[nz, None], dtype)
    return C, counts


def lloyd(X, K: int, iters: int, dtype: str):
    """k-means with cosine assignment: C^0 = X[:K]; then `iters` rounds of
    (assign, mean step).  Returns (C^T, idx^T, counts^T)."""
    X = np.asarray(X, np.float64)
    C = X[:K].copy()
    idx = np.zeros(X.shape[0], dtype=np.int64)
    counts = np.zeros(K, dtype=np.int64)
    for _ in range(iters):
        idx, _, _ = assign(X, C)
        C, counts = centroid_update(X, idx, C, dtype)
    return C, idx, counts


# --------------------------------------------------------------------------
# O7: attention-aware aggregation of each cluster's states
# [TS] Agregación: the entry's state merges every member's state with the
# online-softmax rule, a lossless average of the cluster's prefix attention.
# --------------------------------------------------------------------------


def aggregate(A, LSE, idx, K: int):
    """Per cluster k with members M_k (n_k = |M_k| > 0):
    a_bar_k = sum_i Z_i a_i / sum_i Z_i and lse_bar_k = log(sum_i Z_i / n_k),
    with Z_i = exp(lse_i) taken relative to the members' largest lse.  An
    empty cluster, or one whose members are all empty states, gives (0, -inf).

    A [N, d], LSE [N], idx [N] -> (A_bar [K, d], LSE_bar [K])."""
    A = np.asarray(A, np.float64)
    LSE = np.asarray(LSE, np.float64)
    idx = np.asarray(idx).astype(np.int64)
    d = A.shape[1]
    Abar = np.zeros((K, d))
    Lbar = np.full(K, EMPTY_LSE)
    order = np.argsort(idx, kind="stable")
    bounds = np.searchsorted(idx[order], np.arange(K + 1))
    for k in range(K):
        mem = order[bounds[k]:bounds[k + 1]]
        n = mem.size
        if n == 0:
            continue
        l = LSE[mem]
        m = l.max()
        if np.isneginf(m):
            continue
        w = np.exp(l - m)
        z = w.sum()
        Abar[k] = (w @ A[mem]) / z
        Lbar[k] = m + math.log(z) - math.log(n)
    return Abar, Lbar


# --------------------------------------------------------------------------
# O8 / O9: one decode step
# [TS] Fusión: the retrieved state is merged, by the online-softmax identity,
# with the query's own attention over the tokens that are not in the prefix;
# prefix tokens are never attended.  [NEWS] describes the same retrieval and
# merge.
# --------------------------------------------------------------------------


def decode_with_idx(q, idx, Abar, LSEbar, K_loc, V_loc, scale: float):
    """Decode with the memory entries already chosen.

    q [B, Hq, d]; idx [B, Hq]; Abar [Hq, K, d]; LSEbar [Hq, K];
    K_loc, V_loc: per sequence b an array [Hkv, n_b, d] (n_b may be 0).
    Query head h reads kv head h // (Hq // Hkv).

    Returns (out [B, Hq, d], out_lse [B, Hq])."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    out_lse = np.full((B, Hq), EMPTY_LSE)
    for b in range(B):
        Kb = np.asarray(K_loc[b], np.float64)
        Vb = np.asarray(V_loc[b], np.float64)
        group = Hq // Kb.shape[0]
        for h in range(Hq):
            g = h // group
            k = int(idx[b, h])
            mem_a, mem_l = Abar[h, k], LSEbar[h, k]
            loc_a, loc_l = state(q[b, h], Kb[g], Vb[g], scale)
            out[b, h], out_lse[b, h] = merge(mem_a, mem_l, loc_a, loc_l)
    return out, out_lse


def decode(q, C, Abar, LSEbar, K_loc, V_loc, scale: float):
    """Full decode step: nearest centroid by cosine per (b, h), gather its
    state, attend the local tokens, merge.

    Returns (out [B, Hq, d], out_lse [B, Hq], idx [B, Hq], cos [B, Hq, K],
    gap [B, Hq])."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    K = C.shape[1]
    idx = np.zeros((B, Hq), dtype=np.int64)
    cs = np.zeros((B, Hq, K))
    gap = np.zeros((B, Hq))
    for h in range(Hq):
        i, c, g = assign(q[:, h, :], C[h])
        idx[:, h], cs[:, h], gap[:, h] = i, c, g
    out, out_lse = decode_with_idx(q, idx, Abar, LSEbar, K_loc, V_loc, scale)
    return out, out_lse, idx, cs, gap


# --------------------------------------------------------------------------
# Hierarchical lookup
# [TS] Complejidad: the lookup cost grows with the logarithm of the memory
# size through a hierarchical index.  The pages say no more; the reading
# taken is a two-level index.  The K entry queries of a head are clustered,
# with the build's own cosine k-means (first-S initialisation, means rounded
# to the table's type), into S super-centroids.  A query scores the S
# supers, probes the p best non-empty ones (lowest index on ties) and takes
# the entry of highest cosine among their members (lowest entry index on
# ties).  Probing every non-empty super is the flat search.
# --------------------------------------------------------------------------


def build_index(C, S: int, iters: int, dtype: str):
    """Super-centroids of the entry queries C [K, d] of one head.

    Returns (SC [S, d], e2s [K] super of every entry, counts [S]): the
    partition is the last assignment, whose means are SC."""
    SC, e2s, counts = lloyd(np.asarray(C, np.float64), S, iters, dtype)
    return SC, e2s, counts


def index_members(e2s, S: int):
    """(offsets [S+1], members [K]): the entries of super s are
    members[offsets[s]:offsets[s+1]], in ascending order."""
    e2s = np.asarray(e2s).astype(np.int64)
    counts = np.bincount(e2s, minlength=S)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    members = np.argsort(e2s, kind="stable").astype(np.int64)
    return offsets, members


def probe_supers(q, SC, counts, p: int):
    """The p non-empty supers of highest cosine with q, best first, lowest
    index on ties.  Returns (probes [<= p], cos [S])."""
    cs = cosine(np.asarray(q, np.float64)[None], SC)[0]
    valid = np.nonzero(np.asarray(counts) > 0)[0]
    order = valid[np.lexsort((valid, -cs[valid]))]
    return order[:p], cs


def lookup_probed(q, C, e2s, probes):
    """The entry of highest cosine with q among the members of the probed
    supers, lowest entry index on ties.  Returns (idx, candidates, their
    cosines)."""
    e2s = np.asarray(e2s).astype(np.int64)
    cand = np.nonzero(np.isin(e2s, np.asarray(probes)))[0]
    ce = cosine(np.asarray(q, np.float64)[None], np.asarray(C, np.float64)[cand])[0]
    j = int(np.argmax(ce))  # first maximum: candidates ascend
    return int(cand[j]), cand, ce


def lookup_hier(q, C, SC, e2s, counts, p: int):
    """Two-level lookup of one query: probe, then search the probed
    members.  Returns (idx, probes)."""
    probes, _ = probe_supers(q, SC, counts, p)
    idx, _, _ = lookup_probed(q, C, e2s, probes)
    return idx, probes


# --------------------------------------------------------------------------
# Whitening at retrieval
# [TS] Recuperación: the nearest centroid is found by cosine similarity,
# optionally after a whitening transform.  The pages say no more; the reading
# taken: the transform is fit per head on that head's calibration queries X
# (the Recolección corpus) as the standard whitening x -> W (x - mu), with mu
# the mean of X, Sigma the population covariance of X plus a small ridge
# eps * I (eps = ridge * trace(Sigma) / d, ridge = 1e-6 by default, so that a
# rank-deficient corpus still has a whitening), and W = Sigma^(-1/2), the
# symmetric inverse square root.  Both the query and the table rows are
# mapped and rounded once to the table's type, then scored by cosine exactly
# as in the plain lookup; the merge uses the raw query.
# --------------------------------------------------------------------------


def whiten_fit(X, ridge: float = 1e-6):
    """(mu [d], W [d, d]) of the calibration queries X [N, d]: mean, ridged
    population covariance, and its symmetric inverse square root from the
    eigendecomposition Sigma = V diag(lam) V^T, W = V diag(lam^-1/2) V^T."""
    X = np.asarray(X, dtype=np.float64)
    N, d = X.shape
    mu = X.mean(axis=0)
    Xc = X - mu
    Sigma = Xc.T @ Xc / N
    Sigma = Sigma + (ridge * np.trace(Sigma) / d) * np.eye(d)
    lam, V = np.linalg.eigh(Sigma)
    W = (V * (1.0 / np.sqrt(lam))) @ V.T
    return mu, W


def whiten_apply(Y, mu, W):
    """W (y - mu) for every row y of Y [..., d], in float64 (no rounding)."""
    Y = np.asarray(Y, dtype=np.float64)
    return (Y - mu) @ np.asarray(W, dtype=np.float64).T


def whiten_rows(Y, mu, W, dtype: str):
    """whiten_apply rounded once to the storage type, widened back to
    float64: the whitened table or query as it is stored and scored."""
    return round_to_dtype(whiten_apply(Y, mu, W), dtype)


def lookup_whitened(q, C, mu, W, dtype: str):
    """Nearest table row of each query row q [M, d] after whitening both
    sides (rounded to dtype): (idx [M], cos [M, K]) as in `assign`."""
    qw = whiten_rows(np.atleast_2d(q), mu, W, dtype)
    Cw = whiten_rows(C, mu, W, dtype)
    idx, cs, _ = assign(qw, Cw)
    return idx, cs
