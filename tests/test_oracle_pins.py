"""Pins for the fp64 oracle: each test ties an oracle function to something
other than itself -- a closed form, a library routine, an invariant the pages
state, brute force on a tiny input, or a hand-worked example under
tests/golden/.  A plausible slip in the oracle (dropped term, wrong sign or
index, transposed operand, wrong tie rule) fails at least one of these."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.spatial.distance
import torch

from oracle import asm_oracle as O

RTOL = 1e-12


def rng(*seed):
    return np.random.default_rng(list(seed))


# ---------------------------------------------------------------- formats

def test_bf16_widen_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x7F80, 0x8000, 0x4049], np.uint16)
    v = O.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == 2.0 ** -133
    assert v[3] == (2 - 2 ** -7) * 2.0 ** 127
    assert np.isposinf(v[4])
    assert v[5] == 0.0 and math.copysign(1, v[5]) < 0
    assert v[6] == 3.140625


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_bits_to_f64(bits)
    fin = np.isfinite(vals)
    return bits[fin], vals[fin]


def test_bf16_rounding_matches_torch_on_float32_inputs():
    r = rng(0, 1)
    x = np.concatenate([
        r.standard_normal(200000).astype(np.float32),
        (r.standard_normal(20000) * 1e-39).astype(np.float32),  # subnormals
        (r.standard_normal(20000) * 3e38).astype(np.float32),   # near overflow
        np.array([0.0, -0.0, 1.00390625, 1.01171875, 3.3895314e38, -3.4e38], np.float32),
    ])
    # bf16 midpoints: add half an ulp to random bf16 values
    b = torch.from_numpy(r.standard_normal(20000).astype(np.float32)).to(torch.bfloat16)
    bb = b.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32) << 16
    mid = (bb | 0x8000).view(np.float32)
    x = np.concatenate([x, mid])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.round_to_bf16_bits(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_rounding_brute_force_float64_inputs():
    """Nearest bf16 by exhaustive search, ties to the even bit pattern; the
    inputs include float64 values just above/below a bf16 midpoint, where a
    detour through float32 would round twice and go wrong."""
    bits, vals = _all_finite_bf16()
    order = np.argsort(vals, kind="stable")
    vals_s, bits_s = vals[order], bits[order]
    # drop -0 (keep +0) so the sorted values are strictly increasing
    keep = ~((vals_s == 0) & (bits_s == 0x8000))
    vals_s, bits_s = vals_s[keep], bits_s[keep]
    r = rng(0, 2)
    base = O.bf16_bits_to_f64(r.integers(0x0080, 0x7F00, 3000).astype(np.uint16))
    base = base * np.where(r.random(3000) < 0.5, -1, 1)
    _, e = np.frexp(base)
    half = np.ldexp(1.0, e - 9)
    xs = np.concatenate([base + half * (1 + 2.0 ** -30), base + half * (1 - 2.0 ** -30),
                         base + half, r.standard_normal(3000) * 10.0 ** r.integers(-30, 30, 3000)])
    got = O.round_to_bf16_bits(xs)
    pos = np.searchsorted(vals_s, xs)
    lo = np.clip(pos - 1, 0, len(vals_s) - 1)
    hi = np.clip(pos, 0, len(vals_s) - 1)
    dlo = np.abs(xs - vals_s[lo])
    dhi = np.abs(vals_s[hi] - xs)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((bits_s[hi] & 1) == 0) & ((bits_s[lo] & 1) == 1))
    ref_vals = np.where(pick_hi, vals_s[hi], vals_s[lo])
    np.testing.assert_array_equal(O.bf16_bits_to_f64(got), ref_vals)
    # and the double-rounding trap really is exercised
    via_f32 = torch.from_numpy(xs.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.any(via_f32.astype(np.float64) != ref_vals)


# ---------------------------------------------------------------- state

def test_state_closed_forms():
    r = rng(1, 0)
    d = 8
    scale = 0.25
    q = r.standard_normal(d)
    k = r.standard_normal((1, d))
    v = r.standard_normal((1, d))
    a, l = O.state(q, k, v, scale)
    np.testing.assert_allclose(a, v[0], rtol=0, atol=0)
    assert abs(l - scale * float(k[0] @ q)) < 1e-14
    # q = 0: uniform weights
    V = r.standard_normal((5, d))
    a, l = O.state(np.zeros(d), r.standard_normal((5, d)), V, scale)
    np.testing.assert_allclose(a, V.mean(0), rtol=RTOL, atol=1e-15)
    assert abs(l - math.log(5)) < 1e-14
    # n identical keys
    kk = np.repeat(k, 7, axis=0)
    V = r.standard_normal((7, d))
    a, l = O.state(q, kk, V, scale)
    np.testing.assert_allclose(a, V.mean(0), rtol=RTOL, atol=1e-14)
    assert abs(l - (scale * float(k[0] @ q) + math.log(7))) < 1e-13
    # empty block
    a, l = O.state(q, np.zeros((0, d)), np.zeros((0, d)), scale)
    assert np.isneginf(l) and np.all(a == 0)


def test_state_hand_worked():
    """d = 4, scale 1/2, q = (2,0,0,0); key 1 = e_1 gives score 1, key 2 = 0
    gives score 0: lse = log(e + 1), a = (e v1 + v2) / (e + 1)."""
    q = np.array([2.0, 0, 0, 0])
    K = np.array([[1.0, 0, 0, 0], [0.0, 0, 0, 0]])
    V = np.array([[1.0, 2, 3, 4], [-1.0, 0, 5, 1]])
    a, l = O.state(q, K, V, 0.5)
    assert abs(l - math.log(math.e + 1)) < 1e-15
    np.testing.assert_allclose(a, (math.e * V[0] + V[1]) / (math.e + 1), rtol=1e-15)


def test_state_against_scipy():
    r = rng(1, 1)
    for n, d in [(1, 4), (3, 16), (257, 64), (1000, 128)]:
        q = r.standard_normal(d) * 3
        K = r.standard_normal((n, d))
        V = r.standard_normal((n, d))
        scale = 1 / math.sqrt(d)
        s = scale * (K @ q)
        a, l = O.state(q, K, V, scale)
        assert abs(l - scipy.special.logsumexp(s)) < 1e-12 * max(1, abs(l))
        np.testing.assert_allclose(a, scipy.special.softmax(s) @ V, rtol=1e-11, atol=1e-13)
        A, L = O.states(np.stack([q, -q]), K, V, scale)
        np.testing.assert_allclose(A[0], a, rtol=1e-12, atol=1e-14)
        assert abs(L[1] - scipy.special.logsumexp(-s)) < 1e-12 * max(1, abs(L[1]))


def test_state_key_shift_and_permutation():
    r = rng(1, 2)
    d, n = 32, 50
    q, K, V = r.standard_normal(d), r.standard_normal((n, d)), r.standard_normal((n, d))
    u = r.standard_normal(d)
    scale = 0.3
    a, l = O.state(q, K, V, scale)
    a2, l2 = O.state(q, K + u, V, scale)
    np.testing.assert_allclose(a2, a, rtol=1e-11, atol=1e-13)
    assert abs(l2 - (l + scale * float(q @ u))) < 1e-11
    p = r.permutation(n)
    a3, l3 = O.state(q, K[p], V[p], scale)
    np.testing.assert_allclose(a3, a, rtol=1e-12, atol=1e-14)
    assert abs(l3 - l) < 1e-12


# ---------------------------------------------------------------- merge

def test_merge_is_the_block_split_identity():
    """Merging the states of two halves equals the state of the whole block
    (the online-softmax decomposition of the Metodología section)."""
    r = rng(2, 0)
    for n, d in [(2, 4), (17, 8), (300, 64)]:
        q = r.standard_normal(d) * 2
        K = r.standard_normal((n, d))
        V = r.standard_normal((n, d))
        scale = 1 / math.sqrt(d)
        whole = O.state(q, K, V, scale)
        for m in [0, 1, n // 3, n - 1, n]:
            s1 = O.state(q, K[:m], V[:m], scale)
            s2 = O.state(q, K[m:], V[m:], scale)
            a, l = O.merge(*s1, *s2)
            np.testing.assert_allclose(a, whole[0], rtol=1e-12, atol=1e-14)
            assert abs(l - whole[1]) < 1e-12


def test_merge_algebra():
    r = rng(2, 1)
    d = 6
    st = [(r.standard_normal(d), float(r.uniform(-5, 20))) for _ in range(3)]
    (a1, l1), (a2, l2), (a3, l3) = st
    # Z-weighted form with Z = exp(l), exactly as the merge rule is written
    Z1, Z2 = math.exp(l1), math.exp(l2)
    a, l = O.merge(a1, l1, a2, l2)
    np.testing.assert_allclose(a, (Z1 * a1 + Z2 * a2) / (Z1 + Z2), rtol=1e-12)
    assert abs(l - np.logaddexp(l1, l2)) < 1e-13
    # commutative and associative
    b, lb = O.merge(a2, l2, a1, l1)
    np.testing.assert_allclose(b, a, rtol=1e-14)
    x = O.merge(*O.merge(a1, l1, a2, l2), a3, l3)
    y = O.merge(a1, l1, *O.merge(a2, l2, a3, l3))
    np.testing.assert_allclose(x[0], y[0], rtol=1e-12)
    assert abs(x[1] - y[1]) < 1e-12
    # identity element and the empty/empty case
    e = (np.zeros(d), -np.inf)
    c, lc = O.merge(a1, l1, *e)
    np.testing.assert_array_equal(c, a1)
    assert lc == l1
    c, lc = O.merge(*e, a1, l1)
    np.testing.assert_array_equal(c, a1)
    c, lc = O.merge(*e, *e)
    assert np.isneginf(lc) and np.all(c == 0) and not np.any(np.isnan(c))
    # large normalisers do not overflow
    c, lc = O.merge(a1, 1000.0, a2, 0.0)
    np.testing.assert_allclose(c, a1, rtol=0, atol=1e-300 + 1e-15 * np.abs(a1 - a2).max())
    assert abs(lc - 1000.0) < 1e-12


def test_merge_vectorised_matches_scalar():
    r = rng(2, 2)
    A1, A2 = r.standard_normal((5, 3, 4)), r.standard_normal((5, 3, 4))
    L1, L2 = r.uniform(-3, 3, (5, 3)), r.uniform(-3, 3, (5, 3))
    L1[0, 0] = -np.inf
    L1[1, 1] = L2[1, 1] = -np.inf
    A, L = O.merge(A1, L1, A2, L2)
    for i in range(5):
        for j in range(3):
            a, l = O.merge(A1[i, j], L1[i, j], A2[i, j], L2[i, j])
            np.testing.assert_allclose(A[i, j], a, rtol=1e-15)
            assert (L[i, j] == l) or abs(L[i, j] - l) < 1e-15


# ---------------------------------------------------------------- build_states

def test_build_states_chunked_equals_monolithic_and_gqa():
    r = rng(3, 0)
    Hq, Hkv, N, d = 4, 2, 5, 16
    for L, chunk in [(64, 16), (70, 16), (10, 64), (1, 1)]:
        Q = r.standard_normal((Hq, N, d)) * 2
        Kp = r.standard_normal((Hkv, L, d))
        Vp = r.standard_normal((Hkv, L, d)) + np.arange(Hkv)[:, None, None] * 10
        Ac, Lc, A, LSE = O.build_states(Q, Kp, Vp, chunk, 1 / math.sqrt(d))
        nc = -(-L // chunk)
        assert Ac.shape == (nc, Hq, N, d)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = (Q[h] @ Kp[g].T) / math.sqrt(d)
            np.testing.assert_allclose(LSE[h], scipy.special.logsumexp(s, axis=1), rtol=1e-12)
            np.testing.assert_allclose(A[h], scipy.special.softmax(s, axis=1) @ Vp[g],
                                       rtol=1e-11, atol=1e-12)
            for c in range(nc):
                sc = s[:, c * chunk:(c + 1) * chunk]
                np.testing.assert_allclose(Lc[c, h], scipy.special.logsumexp(sc, axis=1),
                                           rtol=1e-12)
                # each chunk's own output: softmax over that chunk's keys only,
                # not the running state merged so far
                vc = Vp[g, c * chunk:(c + 1) * chunk]
                np.testing.assert_allclose(Ac[c, h], scipy.special.softmax(sc, axis=1) @ vc,
                                           rtol=1e-11, atol=1e-12)
    # empty prefix
    Ac, Lc, A, LSE = O.build_states(np.ones((2, 3, 4)), np.zeros((1, 0, 4)),
                                    np.zeros((1, 0, 4)), 8, 0.5)
    assert Ac.shape[0] == 0 and np.all(np.isneginf(LSE)) and np.all(A == 0)


# ---------------------------------------------------------------- cosine / assign

def test_cosine_against_scipy_and_brute_force_argmax():
    r = rng(4, 0)
    X = r.standard_normal((20, 5))
    C = r.standard_normal((7, 5))
    cs = O.cosine(X, C)
    for i in range(20):
        for k in range(7):
            ref = 1.0 - scipy.spatial.distance.cosine(X[i], C[k])
            assert abs(cs[i, k] - ref) < 1e-14
    idx, _, gap = O.assign(X, C)
    for i in range(20):
        best = max(range(7), key=lambda k: (cs[i, k], -k))
        assert idx[i] == best
        srt = sorted(cs[i], reverse=True)
        assert abs(gap[i] - (srt[0] - srt[1])) < 1e-15


def test_assign_matches_euclidean_on_unit_sphere():
    """For unit-norm centroids the cosine argmax equals the Euclidean argmin
    (|x - c|^2 = |x|^2 + 1 - 2 x.c): check against scikit-learn."""
    from sklearn.metrics import pairwise_distances_argmin
    r = rng(4, 1)
    X = r.standard_normal((300, 16)) * r.uniform(0.1, 10, (300, 1))
    C = r.standard_normal((40, 16))
    Cn = C / np.linalg.norm(C, axis=1, keepdims=True)
    idx, _, _ = O.assign(X, C)
    np.testing.assert_array_equal(idx, pairwise_distances_argmin(X, Cn))


def test_assign_invariances_and_ties():
    r = rng(4, 2)
    X = r.standard_normal((50, 8))
    C = r.standard_normal((12, 8))
    idx, _, _ = O.assign(X, C)
    # power-of-two scaling of queries and of single centroids changes nothing
    C2 = C.copy()
    C2[3] *= 4.0
    C2[7] *= 0.125
    np.testing.assert_array_equal(O.assign(X * 8.0, C2)[0], idx)
    # a duplicate of centroid i at a higher index never wins
    C3 = np.vstack([C, C[idx[0]][None]])
    np.testing.assert_array_equal(O.assign(X, C3)[0], idx)
    # a zero centroid has cosine 0; all-negative cosines pick it
    C4 = np.vstack([np.zeros((1, 8)), -X[:1]])
    i4, cs4, _ = O.assign(X[:1], C4)
    assert cs4[0, 0] == 0.0 and i4[0] == 0
    # dot product alone would pick the long centroid; cosine does not
    Xs = np.array([[1.0, 0.1]])
    Cs = np.array([[1.0, 0.0], [10.0, 5.0]])
    assert O.assign(Xs, Cs)[0][0] == 0


def test_accept_index():
    cs = np.array([[0.5, 0.5 - 5e-6, 0.1], [0.9, 0.2, 0.8]])
    ok = O.accept_index(np.array([1, 2]), cs)
    assert ok[0] and not ok[1]
    assert not O.accept_index(np.array([3, 0]), cs)[0]


# ---------------------------------------------------------------- k-means

def test_lloyd_hand_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kmeans_2d_hand.json")))
    X = np.array(g["X"], np.float64)
    C = X[:g["K"]].copy()
    for t in range(len(g["idx"])):
        idx, cs, gap = O.assign(X, C)
        np.testing.assert_array_equal(idx, g["idx"][t])
        if t == 1:
            np.testing.assert_allclose(gap, g["gap_iter2"], rtol=1e-15)
        C, counts = O.centroid_update(X, idx, C, "bf16")
        np.testing.assert_array_equal(C, np.array(g["C"][t]))
        np.testing.assert_array_equal(counts, g["counts"][t])
    C_l, idx_l, counts_l = O.lloyd(X, g["K"], len(g["idx"]), "bf16")
    np.testing.assert_array_equal(C_l, np.array(g["C"][-1]))
    np.testing.assert_array_equal(idx_l, g["idx"][-1])


def test_lloyd_special_cases():
    r = rng(5, 0)
    X = O.bf16_bits_to_f64(O.round_to_bf16_bits(r.standard_normal((64, 16))))
    # K = N with distinct directions: identity assignment, X is a fixed point
    C, idx, counts = O.lloyd(X, 64, 3, "bf16")
    np.testing.assert_array_equal(idx, np.arange(64))
    np.testing.assert_array_equal(C, X)
    assert np.all(counts == 1)
    # K = 1: the single centroid is the rounded global mean
    C, idx, counts = O.lloyd(X, 1, 2, "bf16")
    np.testing.assert_array_equal(C[0], O.round_to_dtype(X.mean(0), "bf16"))
    assert counts[0] == 64


def test_centroid_update_against_pandas_groupby():
    import pandas as pd
    r = rng(5, 1)
    X = r.standard_normal((500, 6))
    idx = r.integers(0, 10, 500)
    idx[idx == 7] = 3  # cluster 7 empty
    prev = r.standard_normal((10, 6))
    C, counts = O.centroid_update(X, idx, prev, "f32")
    means = pd.DataFrame(X).groupby(idx).mean()
    for k in range(10):
        if k == 7:
            np.testing.assert_array_equal(C[k], prev[k])
            assert counts[k] == 0
        else:
            ref = means.loc[k].to_numpy().astype(np.float32).astype(np.float64)
            np.testing.assert_array_equal(C[k], ref)
            assert counts[k] == np.sum(idx == k)


# ---------------------------------------------------------------- aggregate

def test_aggregate_properties():
    r = rng(6, 0)
    N, d, K = 200, 5, 12
    A = r.standard_normal((N, d))
    LSE = r.uniform(-2, 6, N)
    idx = r.integers(0, K - 2, N)   # clusters K-2, K-1 empty
    idx[0] = 9                      # make cluster 9 a singleton
    idx[idx == 9] = 8
    idx[0] = 9
    Abar, Lbar = O.aggregate(A, LSE, idx, K)
    # singleton: unchanged
    np.testing.assert_array_equal(Abar[9], A[0])
    assert Lbar[9] == LSE[0]
    # empty: (0, -inf)
    assert np.all(Abar[10:] == 0) and np.all(np.isneginf(Lbar[10:]))
    # lossless sum: n_k Z_bar_k a_bar_k = sum Z_i a_i and n_k Z_bar_k = sum Z_i
    for k in range(K - 2):
        m = idx == k
        n = m.sum()
        Z = np.exp(LSE[m])
        np.testing.assert_allclose(n * math.exp(Lbar[k]) * Abar[k], Z @ A[m], rtol=1e-12)
        assert abs(n * math.exp(Lbar[k]) - Z.sum()) < 1e-12 * Z.sum()
    # equal normalisers: plain mean, lse unchanged
    Abar2, Lbar2 = O.aggregate(A, np.full(N, 3.5), idx, K)
    for k in range(K - 2):
        m = idx == k
        np.testing.assert_allclose(Abar2[k], A[m].mean(0), rtol=1e-12, atol=1e-15)
        assert abs(Lbar2[k] - 3.5) < 1e-13


def test_aggregate_is_merge_of_members_minus_log_n():
    r = rng(6, 1)
    A = r.standard_normal((30, 4))
    LSE = r.uniform(0, 50, 30)
    LSE[5] = -np.inf  # an empty member state contributes nothing
    idx = np.zeros(30, np.int64)
    Abar, Lbar = O.aggregate(A, LSE, idx, 1)
    a, l = A[0], LSE[0]
    for i in range(1, 30):
        a, l = O.merge(a, l, A[i], LSE[i])
    np.testing.assert_allclose(Abar[0], a, rtol=1e-12)
    assert abs(Lbar[0] - (l - math.log(30))) < 1e-12


# ---------------------------------------------------------------- decode

def _memory_exact(r, N, L, d, Hq=1, Hkv=1):
    """Memory with K = N: every calibration query is its own centroid and
    keeps its own prefix state."""
    Q = r.standard_normal((Hq, N, d))
    Kp = r.standard_normal((Hkv, L, d))
    Vp = r.standard_normal((Hkv, L, d))
    scale = 1 / math.sqrt(d)
    _, _, A, LSE = O.build_states(Q, Kp, Vp, 16, scale)
    C = Q.copy()
    return Q, Kp, Vp, C, A, LSE, scale


def test_decode_exact_when_K_equals_N():
    """With one entry per calibration query, decoding a calibration query
    reproduces attention over [prefix; local] (the Fusión step recovers the
    exact output when the stored state is the query's own)."""
    r = rng(7, 0)
    Hq, Hkv, N, L, d = 4, 2, 24, 40, 16
    Q, Kp, Vp, C, A, LSE, scale = _memory_exact(r, N, L, d, Hq, Hkv)
    pick = np.array([3, 17, 0])
    q = Q[:, pick, :].transpose(1, 0, 2)  # [B=3, Hq, d]
    lens = [5, 0, 9]
    K_loc = [r.standard_normal((Hkv, n, d)) for n in lens]
    V_loc = [r.standard_normal((Hkv, n, d)) for n in lens]
    out, out_lse, idx, _, _ = O.decode(q, C, A, LSE, K_loc, V_loc, scale)
    np.testing.assert_array_equal(idx, np.repeat(pick[:, None], Hq, axis=1))
    for b in range(3):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            Kc = np.concatenate([Kp[g], K_loc[b][g]])
            Vc = np.concatenate([Vp[g], V_loc[b][g]])
            s = scale * (Kc @ q[b, h])
            np.testing.assert_allclose(out[b, h], scipy.special.softmax(s) @ Vc,
                                       rtol=1e-11, atol=1e-12)
            assert abs(out_lse[b, h] - scipy.special.logsumexp(s)) < 1e-11


def test_decode_degenerate_cases():
    r = rng(7, 1)
    Hq, Hkv, K, d = 2, 1, 6, 8
    q = r.standard_normal((2, Hq, d))
    C = r.standard_normal((Hq, K, d))
    Abar = r.standard_normal((Hq, K, d))
    LSEbar = r.uniform(0, 4, (Hq, K))
    idx0 = O.assign(q[:, 0], C[0])[0]
    LSEbar[0, idx0[1]] = -np.inf  # sequence 1 head 0 retrieves an empty entry
    Abar[0, idx0[1]] = 0
    K_loc = [np.zeros((Hkv, 0, d)), r.standard_normal((Hkv, 7, d))]
    V_loc = [np.zeros((Hkv, 0, d)), r.standard_normal((Hkv, 7, d))]
    out, out_lse, idx, _, _ = O.decode(q, C, Abar, LSEbar, K_loc, V_loc, 0.35)
    # no local tokens: the output is the memory state
    for h in range(Hq):
        np.testing.assert_array_equal(out[0, h], Abar[h, idx[0, h]])
        assert out_lse[0, h] == LSEbar[h, idx[0, h]]
    # empty memory entry: the output is local attention
    a, l = O.state(q[1, 0], K_loc[1][0], V_loc[1][0], 0.35)
    np.testing.assert_allclose(out[1, 0], a, rtol=1e-15)
    assert out_lse[1, 0] == l
    # both empty: the empty state
    Lb = LSEbar.copy()
    Lb[:] = -np.inf
    out, out_lse = O.decode_with_idx(q[:1], idx[:1], np.zeros_like(Abar), Lb,
                                     K_loc[:1], V_loc[:1], 0.35)
    assert np.all(np.isneginf(out_lse)) and np.all(out == 0)


# ---------------------------------------------------------------- hierarchical lookup

def _unit(deg):
    t = math.radians(deg)
    return np.array([math.cos(t), math.sin(t)])


def test_hier_lookup_hand_worked_probe_miss_and_hit():
    """Supers at 0 and 90 degrees; entries at 0 and 50 degrees belong to the
    first, 80 and 90 degrees to the second.  A query at 60 degrees is nearer
    the second super (cos 30 deg > cos 60 deg), so one probe searches
    {80, 90} and returns the 80-degree entry (cos 20 deg), although the
    50-degree entry is the flat nearest (cos 10 deg); two probes find it."""
    C = np.stack([_unit(0), _unit(50), _unit(80), _unit(90)])
    SC = np.stack([_unit(0), _unit(90)])
    e2s = np.array([0, 0, 1, 1])
    counts = np.array([2, 2])
    q = 3.0 * _unit(60)
    idx1, probes1 = O.lookup_hier(q, C, SC, e2s, counts, 1)
    assert list(probes1) == [1] and idx1 == 2
    idx2, probes2 = O.lookup_hier(q, C, SC, e2s, counts, 2)
    assert list(probes2) == [1, 0] and idx2 == 1
    assert O.assign(q[None], C)[0][0] == 1


def test_hier_lookup_probing_all_supers_is_the_flat_search():
    r = rng(8, 0)
    for trial in range(4):
        K, S, d = 200, 13, 16
        C = r.standard_normal((K, d))
        SC, e2s, counts = O.build_index(C, S, 3, "f32")
        nonempty = int(np.sum(counts > 0))
        Q = r.standard_normal((30, d))
        flat = O.assign(Q, C)[0]
        for i in range(Q.shape[0]):
            idx, probes = O.lookup_hier(Q[i], C, SC, e2s, counts, S)
            assert len(probes) == nonempty
            assert idx == flat[i]


def test_hier_lookup_one_entry_per_super_is_the_flat_search():
    """S = K: first-K initialisation puts every entry in its own super (the
    supers are the entries themselves), so one probe already finds the flat
    nearest entry."""
    r = rng(8, 1)
    C = r.standard_normal((40, 8)).astype(np.float32).astype(np.float64)
    SC, e2s, counts = O.build_index(C, 40, 1, "f32")
    np.testing.assert_array_equal(e2s, np.arange(40))
    np.testing.assert_array_equal(SC, C)
    Q = r.standard_normal((25, 8))
    flat = O.assign(Q, C)[0]
    for i in range(25):
        assert O.lookup_hier(Q[i], C, SC, e2s, counts, 1)[0] == flat[i]


def test_hier_probes_ties_and_empty_supers():
    """Equal super scores go to the lower index; empty supers are never
    probed; the member search breaks ties by the lower entry index."""
    SC = np.stack([_unit(10), _unit(10), _unit(40), _unit(10)])
    counts = np.array([3, 0, 1, 2])
    probes, _ = O.probe_supers(_unit(10), SC, counts, 3)
    assert list(probes) == [0, 3, 2]
    C = np.stack([_unit(30), _unit(20), _unit(20), _unit(80)])
    e2s = np.array([2, 0, 3, 0])
    idx, cand, _ = O.lookup_probed(_unit(20), C, e2s, [0, 3])
    assert list(cand) == [1, 2, 3] and idx == 1


def test_index_members_against_brute_force():
    r = rng(8, 2)
    S = 9
    e2s = r.integers(0, S, 300)
    e2s[e2s == 4] = 5  # an empty super
    offsets, members = O.index_members(e2s, S)
    for s in range(S):
        expect = [k for k in range(300) if e2s[k] == s]
        assert list(members[offsets[s]:offsets[s + 1]]) == expect
    assert offsets[-1] == 300


# ---------------------------------------------------------------- whitening

def test_whiten_hand_worked_2d(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "whiten_2d_hand.json")))
    for case in g["cases"]:
        X = np.array(case["X"], float)
        mu, W = O.whiten_fit(X, ridge=0.0)
        np.testing.assert_allclose(mu, case["mu"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(W, case["W"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(O.whiten_apply(X, mu, W), case["whitened"], rtol=0, atol=1e-14)


def test_whiten_recovers_a_known_covariance_with_its_ridge():
    """Rows mu0 + A z over the 16 sign patterns z in {-1, 1}^4 have mean mu0
    and population covariance A A^T exactly.  With A = H diag(s), H the
    orthonormal 4x4 Hadamard matrix, W must be H diag((s^2 + eps)^-1/2) H^T
    with eps = 1e-6 * trace / 4."""
    Z = np.array([[1 - 2 * ((i >> b) & 1) for b in range(4)] for i in range(16)], float)
    Hd = 0.5 * np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], float)
    s = np.array([1.0, 2.0, 3.0, 0.5])
    mu0 = np.array([0.25, -1.0, 4.0, 2.5])
    X = mu0 + Z @ (Hd * s).T
    mu, W = O.whiten_fit(X)
    eps = 1e-6 * np.sum(s ** 2) / 4
    W_ref = (Hd * (1.0 / np.sqrt(s ** 2 + eps))) @ Hd.T
    np.testing.assert_allclose(mu, mu0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(W, W_ref, rtol=0, atol=1e-12)


def test_whitened_corpus_covariance_closed_form():
    """cov(W (x - mu)) over the corpus is I - eps (Sigma + eps I)^-1 (numpy's
    cov and inv), and exactly I without ridge; the mean is 0."""
    r = rng(40, 1)
    X = r.standard_normal((500, 6)) @ r.standard_normal((6, 6)) + r.standard_normal(6)
    for ridge in (0.0, 1e-6, 1e-2):
        mu, W = O.whiten_fit(X, ridge=ridge)
        Y = O.whiten_apply(X, mu, W)
        S0 = np.cov(X.T, bias=True)
        eps = ridge * np.trace(S0) / 6
        ref = np.eye(6) - eps * np.linalg.inv(S0 + eps * np.eye(6))
        np.testing.assert_allclose(np.cov(Y.T, bias=True), ref, rtol=0, atol=1e-10)
        np.testing.assert_allclose(Y.mean(axis=0), 0.0, rtol=0, atol=1e-12)


def test_whitened_distance_is_mahalanobis():
    """|W (u - v)| is scipy's Mahalanobis distance under the ridged
    covariance: W^T W is the inverse covariance."""
    r = rng(40, 2)
    X = r.standard_normal((300, 5)) * np.array([1.0, 3.0, 0.2, 1.0, 2.0])
    mu, W = O.whiten_fit(X)
    S0 = np.cov(X.T, bias=True)
    VI = np.linalg.inv(S0 + 1e-6 * np.trace(S0) / 5 * np.eye(5))
    for _ in range(5):
        u, v = r.standard_normal(5), r.standard_normal(5)
        ref = scipy.spatial.distance.mahalanobis(u, v, VI)
        assert abs(np.linalg.norm(O.whiten_apply(u, mu, W) - O.whiten_apply(v, mu, W)) - ref) < 1e-12


def test_whitened_cosine_is_affine_invariant():
    """Without ridge, refitting on an affinely transformed corpus (x M + b)
    leaves every whitened cosine unchanged."""
    r = rng(40, 3)
    X = r.standard_normal((400, 4)) @ r.standard_normal((4, 4))
    M = r.standard_normal((4, 4)) + 2 * np.eye(4)
    b = r.standard_normal(4)
    q, C = r.standard_normal((3, 4)), r.standard_normal((7, 4))
    mu, W = O.whiten_fit(X, ridge=0.0)
    mu2, W2 = O.whiten_fit(X @ M + b, ridge=0.0)
    c1 = O.cosine(O.whiten_apply(q, mu, W), O.whiten_apply(C, mu, W))
    c2 = O.cosine(O.whiten_apply(q @ M + b, mu2, W2), O.whiten_apply(C @ M + b, mu2, W2))
    np.testing.assert_allclose(c1, c2, rtol=0, atol=1e-10)


def test_lookup_whitened_identity_transform_is_plain_lookup():
    """mu = 0 and W = I leave bf16 rows unchanged, so the whitened lookup is
    the plain cosine lookup."""
    r = rng(40, 4)
    C = O.round_to_dtype(r.standard_normal((50, 8)), "bf16")
    q = O.round_to_dtype(r.standard_normal((20, 8)), "bf16")
    idx, cs = O.lookup_whitened(q, C, np.zeros(8), np.eye(8), "bf16")
    idx0, cs0, _ = O.assign(q, C)
    np.testing.assert_array_equal(idx, idx0)
    np.testing.assert_array_equal(cs, cs0)


def test_lookup_whitened_hand_worked_2d(golden_dir):
    """A whitened lookup with mu != 0 and W != I, worked by hand, where the
    plain lookup, whitening one side only, whitening without centring and
    Sigma^-1 in place of Sigma^-1/2 each pick a different entry."""
    g = json.load(open(os.path.join(golden_dir, "whiten_lookup_2d_hand.json")))
    mu_fit, W_fit = O.whiten_fit(np.array(g["corpus"], float), ridge=0.0)
    np.testing.assert_allclose(mu_fit, g["mu"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(W_fit, g["W"], rtol=0, atol=1e-14)
    q, C = np.array([g["q"]], float), np.array(g["C"], float)
    mu, W = np.array(g["mu"], float), np.array(g["W"], float)
    for dtype in ("bf16", "f32"):
        np.testing.assert_array_equal(O.whiten_rows(q, mu, W, dtype), [g["whitened_q"]])
        np.testing.assert_array_equal(O.whiten_rows(C, mu, W, dtype), g["whitened_C"])
        idx, cs = O.lookup_whitened(q, C, mu, W, dtype)
        assert idx[0] == g["idx"]
        np.testing.assert_allclose(cs[0], g["cos"], rtol=0, atol=1e-15)
    # the case discriminates: each plausible slip picks another entry
    qw, Cw = O.whiten_apply(q, mu, W), O.whiten_apply(C, mu, W)
    assert O.assign(q, C)[0][0] == g["plain_idx"] != g["idx"]
    assert O.assign(qw, C)[0][0] == g["query_only_idx"] != g["idx"]
    assert O.assign(q, Cw)[0][0] == g["table_only_idx"] != g["idx"]
    assert O.assign(q @ W.T, C @ W.T)[0][0] == g["uncentred_idx"] != g["idx"]
    Winv = W @ W
    assert O.assign((q - mu) @ Winv.T, (C - mu) @ Winv.T)[0][0] == g["inverse_covariance_idx"] != g["idx"]


def test_whiten_fit_singular_covariance_with_ridge():
    """Fewer rows than dimensions: the covariance is singular, and only the
    ridge makes it invertible.  W must then be the symmetric inverse square
    root of the ridged covariance, W (Sigma + eps I) W = I, with eps =
    ridge * trace(Sigma) / d; the null directions of Sigma get the factor
    eps^-1/2 exactly.  Without the ridge the oracle has no finite W."""
    r = rng(40, 9)
    N, d = 6, 10
    X = r.standard_normal((N, d))
    S0 = np.cov(X.T, bias=True)
    assert np.linalg.matrix_rank(S0) < d
    mu, W = O.whiten_fit(X, ridge=1e-6)
    eps = 1e-6 * np.trace(S0) / d
    Sr = S0 + eps * np.eye(d)
    np.testing.assert_allclose(W, W.T, rtol=0, atol=1e-9 * np.abs(W).max())
    np.testing.assert_allclose(W @ Sr @ W, np.eye(d), rtol=0, atol=1e-6)
    # a null direction of the centred corpus is scaled by eps^-1/2
    _, _, Vt = np.linalg.svd(X - X.mean(axis=0))
    v = Vt[-1]
    assert abs(np.linalg.norm(W @ v) - eps ** -0.5) <= 1e-6 * eps ** -0.5
    with np.errstate(all="ignore"):
        _, W0 = O.whiten_fit(X, ridge=0.0)
    assert not np.isfinite(W0).all() or np.abs(W0).max() > 1e6
