"""GPU parity of the offline memory build against the fp64 oracle: prefix
states chunk by chunk (asm_build_states), cosine k-means assignment
(asm_kmeans_assign), centroid means and Z-weighted state aggregation
(asm_aggregate), and the tiny end-to-end build, checked step by step."""
import numpy as np
import pytest
import torch

from attention_state_memory_amd import api, synth
from oracle import asm_oracle as O
from tests.helpers import (A_TOL, LSE_TOL, assert_states_close, check_indices, dev, host,
                           widen)

pytestmark = pytest.mark.gpu


def _rng(*seed):
    return np.random.default_rng([200, *seed])


def _normal(r, shape, dtype):
    x = r.standard_normal(shape, dtype=np.float32)
    return synth.to_bf16_bits(x) if dtype == "bf16" else x


# ---------------------------------------------------------------- prefix states

STATES = [
    # (seed, dtype, Hq, Hkv, N, L, chunk, d)
    (1, "f32", 1, 1, 40, 256, 64, 64),
    (2, "bf16", 4, 2, 130, 300, 64, 128),     # ragged chunk tail, ragged query tail
    (3, "bf16", 8, 1, 64, 97, 128, 64),       # one partial chunk, G = 8
    (4, "bf16", 2, 2, 33, 1024, 256, 128),
    (5, "f32", 3, 1, 17, 50, 7, 32),          # odd sizes on the VALU path
]


@pytest.mark.parametrize("case", STATES, ids=[f"s{c[0]}" for c in STATES])
def test_build_states_matches_oracle(case):
    seed, dtype, Hq, Hkv, N, L, chunk, d = case
    r = _rng(1, seed)
    Q = _normal(r, (Hq, N, d), dtype) if dtype == "f32" else synth.to_bf16_bits(
        r.standard_normal((Hq, N, d), dtype=np.float32) * 1.5)
    Kp = _normal(r, (Hkv, L, d), dtype)
    Vp = _normal(r, (Hkv, L, d), dtype)
    scale = synth.softmax_scale(d)
    A, LSE, Ac, Lc = api.build_states(dev(Q), dev(Kp), dev(Vp), chunk, scale, keep_chunks=True)
    torch.cuda.synchronize()
    Ac_ref, Lc_ref, A_ref, L_ref = O.build_states(widen(Q), widen(Kp), widen(Vp), chunk, scale)
    assert_states_close(host(A), host(LSE), A_ref, L_ref)
    assert_states_close(host(Ac), host(Lc), Ac_ref, Lc_ref)


def test_build_states_values_without_fp16_form_take_the_exact_path():
    """bf16 values of magnitude 65520 or more have no fp16 form: the MFMA
    path must notice and compute every state exactly (finite, within the
    oracle's tolerance scaled by the largest value), and the next call with
    ordinary values must take the fast path again."""
    r = _rng(2, 7)
    Hq, Hkv, N, L, chunk, d = 4, 2, 70, 200, 64, 128
    Q = synth.to_bf16_bits(r.standard_normal((Hq, N, d), dtype=np.float32))
    Kp = synth.to_bf16_bits(r.standard_normal((Hkv, L, d), dtype=np.float32))
    Vf = r.standard_normal((Hkv, L, d), dtype=np.float32)
    Vf[0, 37, 5] = 2.0 ** 17
    Vf[1, 150, 90] = -3.0 * 2.0 ** 16
    Vp = synth.to_bf16_bits(Vf)
    scale = synth.softmax_scale(d)
    A, LSE, Ac, Lc = api.build_states(dev(Q), dev(Kp), dev(Vp), chunk, scale, keep_chunks=True)
    torch.cuda.synchronize()
    Ac_ref, Lc_ref, A_ref, L_ref = O.build_states(widen(Q), widen(Kp), widen(Vp), chunk, scale)
    A, Ac = host(A), host(Ac)
    assert np.isfinite(A).all() and np.isfinite(Ac).all()
    # float32 accumulation of values up to 2^17: about 2^-24 of the largest
    tol = 2e-3 + 1e-6 * float(np.abs(widen(Vp)).max())
    assert np.abs(A - A_ref).max() <= tol
    assert np.abs(Ac - Ac_ref).max() <= tol
    assert np.abs(host(LSE) - L_ref).max() <= LSE_TOL
    assert np.abs(host(Lc) - Lc_ref).max() <= LSE_TOL
    # ordinary values right after: the flag is cleared per call
    Vp2 = synth.to_bf16_bits(r.standard_normal((Hkv, L, d), dtype=np.float32))
    A2, LSE2, _, _ = api.build_states(dev(Q), dev(Kp), dev(Vp2), chunk, scale)
    torch.cuda.synchronize()
    _, _, A2_ref, L2_ref = O.build_states(widen(Q), widen(Kp), widen(Vp2), chunk, scale)
    assert_states_close(host(A2), host(LSE2), A2_ref, L2_ref)


def test_build_states_accumulate_and_empty_prefix():
    """Streaming a prefix in two calls (accumulate=1) equals one call over the
    whole prefix; an empty prefix gives empty states."""
    r = _rng(2, 0)
    Hq, Hkv, N, d = 4, 2, 50, 128
    Q = synth.to_bf16_bits(r.standard_normal((Hq, N, d), dtype=np.float32))
    Kp = synth.to_bf16_bits(r.standard_normal((Hkv, 300, d), dtype=np.float32))
    Vp = synth.to_bf16_bits(r.standard_normal((Hkv, 300, d), dtype=np.float32))
    scale = synth.softmax_scale(d)
    A, LSE, _, _ = api.build_states(dev(Q), dev(Kp[:, :128].copy()), dev(Vp[:, :128].copy()), 64, scale)
    A, LSE, _, _ = api.build_states(dev(Q), dev(Kp[:, 128:].copy()), dev(Vp[:, 128:].copy()), 64,
                                    scale, A=A, LSE=LSE, accumulate=True)
    torch.cuda.synchronize()
    _, _, A_ref, L_ref = O.build_states(widen(Q), widen(Kp), widen(Vp), 64, scale)
    assert_states_close(host(A), host(LSE), A_ref, L_ref)
    A0, L0, _, _ = api.build_states(dev(Q), dev(np.zeros((Hkv, 0, d), np.uint16)),
                                    dev(np.zeros((Hkv, 0, d), np.uint16)), 64, scale)
    torch.cuda.synchronize()
    assert np.all(np.isneginf(host(L0))) and np.all(host(A0) == 0)


# ---------------------------------------------------------------- k-means assignment

ASSIGN = [
    # (seed, dtype, H, N, K, d)
    (1, "f32", 1, 512, 64, 64),
    (2, "bf16", 2, 1000, 300, 128),
    (3, "bf16", 3, 257, 1024, 64),
    (4, "bf16", 1, 4096, 8192, 128),
    (5, "f32", 2, 100, 7, 40),
]


@pytest.mark.parametrize("case", ASSIGN, ids=[f"a{c[0]}" for c in ASSIGN])
def test_kmeans_assign_matches_oracle(case):
    seed, dtype, H, N, K, d = case
    X = synth.mixture_queries([201, seed], H, N, d, M=max(4, K // 8), dtype=dtype)
    C = X[:, :K].copy() if K <= N else _normal(_rng(2, seed), (H, K, d), dtype)
    if K > 8:
        C[:, K - 1] = C[:, 2]  # duplicate centroid: never chosen over index 2
        C[:, 5] = 0            # zero centroid: cosine 0
    Cd = dev(C)
    cinv = api.centroid_inv_norms(Cd)
    idx, best = api.kmeans_assign(dev(X), Cd, cinv, want_best=True)
    torch.cuda.synchronize()
    idx, best = host(idx), host(best)
    X64, C64 = widen(X), widen(C)
    for h in range(H):
        check_indices(idx[h], X64[h], C64[h])
        # the winning score is x.c * cinv (cosine times |x|)
        ref_best = O.cosine(X64[h], C64[h])[np.arange(N), idx[h]] * np.linalg.norm(X64[h], axis=1)
        np.testing.assert_allclose(best[h], ref_best, rtol=1e-5, atol=1e-5)
        if K > 8:
            assert not np.any(idx[h] == K - 1)


def test_kmeans_assign_exact_ties_pick_lowest_index():
    d = 128
    r = _rng(3, 0)
    C = synth.to_bf16_bits(r.standard_normal((1, 300, d), dtype=np.float32))
    C[0, 200] = C[0, 17]
    C[0, 299] = C[0, 17]
    X = np.repeat(C[:, 17:18], 70, axis=1).copy()  # queries identical to centroid 17
    X[0, 1::2] = synth.to_bf16_bits(
        2.0 * O.bf16_bits_to_f64(C[0, 17]).astype(np.float32))  # scaled by 2: same cosine
    Cd = dev(C)
    idx, _ = api.kmeans_assign(dev(X), Cd, api.centroid_inv_norms(Cd))
    torch.cuda.synchronize()
    assert np.all(host(idx) == 17)


# ---------------------------------------------------------------- aggregation

AGG = [
    # (seed, dtype, H, N, K, d)
    (1, "f32", 1, 512, 64, 64),
    (2, "bf16", 3, 2000, 300, 128),
    (3, "bf16", 2, 100, 1000, 64),   # mostly empty clusters
    (4, "bf16", 1, 5000, 1, 128),    # one cluster holds everything
]


@pytest.mark.parametrize("case", AGG, ids=[f"g{c[0]}" for c in AGG])
def test_aggregate_matches_oracle(case):
    seed, dtype, H, N, K, d = case
    r = _rng(4, seed)
    X = synth.mixture_queries([202, seed], H, N, d, M=16, dtype=dtype)
    C0 = _normal(r, (H, K, d), dtype)
    idx = r.integers(0, K, (H, N)).astype(np.int32)
    if K > 10:
        idx[idx == 7] = 8  # cluster 7 empty: keeps its centroid, empty state
    A = r.standard_normal((H, N, d), dtype=np.float32)
    LSE = r.uniform(-3, 30, (H, N)).astype(np.float32)
    if N > 3:
        LSE[0, 3] = -np.inf  # an empty member state
    Cd = dev(C0)
    C, cinv, count, Abar, LSEbar = api.aggregate(dev(X), dev(idx), Cd, A=dev(A), LSE=dev(LSE))
    torch.cuda.synchronize()
    C, cinv, count = host(C), host(cinv), host(count)
    Abar, LSEbar = host(Abar), host(LSEbar)
    X64, C064 = widen(X), widen(C0)
    mismatch = 0
    for h in range(H):
        C_ref, n_ref = O.centroid_update(X64[h], idx[h], C064[h], dtype)
        np.testing.assert_array_equal(count[h], n_ref)
        mismatch += int(np.sum(widen(C[h]) != C_ref))
        np.testing.assert_allclose(cinv[h], O.inv_norms(C_ref), rtol=1e-6)
        Ab_ref, Lb_ref = O.aggregate(A[h].astype(np.float64), LSE[h].astype(np.float64), idx[h], K)
        assert_states_close(Abar[h], LSEbar[h], Ab_ref, Lb_ref, a_tol=1e-5, lse_tol=1e-5)
    # float64 sums of bf16/f32 data are exact here, so the rounded means agree bit for bit
    assert mismatch == 0


# ---------------------------------------------------------------- tiny end to end

def test_tiny_build_and_decode_teacher_forced():
    """The tiny workload end to end: prefix states in 4 chunks, 5 Lloyd
    iterations checked step by step against the oracle applied to the GPU's
    previous centroids, the final aggregation, then a decode step of the 4
    new queries against the built memory."""
    t = synth.tiny()
    Xd, Kp, Vp = dev(t["X"]), dev(t["Kp"]), dev(t["Vp"])
    A, LSE, _, _ = api.build_states(Xd, Kp, Vp, t["chunk"], t["scale"])
    X64 = widen(t["X"])[0]
    _, _, A_ref, L_ref = O.build_states(widen(t["X"]), widen(t["Kp"]), widen(t["Vp"]), t["chunk"],
                                        t["scale"])
    torch.cuda.synchronize()
    assert_states_close(host(A), host(LSE), A_ref, L_ref)
    K = t["K"]
    C = Xd[:, :K].clone()
    cinv = api.centroid_inv_norms(C)
    for it in range(t["iters"]):
        C_prev = host(C)[0].astype(np.float64)
        idx, _ = api.kmeans_assign(Xd, C, cinv)
        last = it == t["iters"] - 1
        _, _, count, Abar, LSEbar = api.aggregate(Xd, idx, C, A=A, LSE=LSE, cinv=cinv,
                                                  with_states=last)
        torch.cuda.synchronize()
        idx_h = host(idx)[0]
        check_indices(idx_h, X64, C_prev)
        C_ref, n_ref = O.centroid_update(X64, idx_h, C_prev, "f32")
        np.testing.assert_array_equal(host(count)[0], n_ref)
        np.testing.assert_array_equal(host(C)[0].astype(np.float64), C_ref)
    Ab_ref, Lb_ref = O.aggregate(host(A)[0].astype(np.float64), host(LSE)[0].astype(np.float64),
                                 idx_h, K)
    assert_states_close(host(Abar)[0], host(LSEbar)[0], Ab_ref, Lb_ref, a_tol=1e-5, lse_tol=1e-5)
    # decode the 4 new queries against the built memory with the 32-token local KV
    q = dev(t["q"])
    out, lse, di = api.decode_step(q, C, cinv, Abar, LSEbar, dev(t["Kl"]), dev(t["Vl"]),
                                   dev(t["kv_start"]), dev(t["kv_len"]), 32, t["scale"])
    torch.cuda.synchronize()
    di = host(di)
    q64 = widen(t["q"])
    check_indices(di[:, 0], q64[:, 0], host(C)[0].astype(np.float64))
    ks = [widen(t["Kl"])] * 4
    vs = [widen(t["Vl"])] * 4
    ref, ref_lse = O.decode_with_idx(q64, di, host(Abar).astype(np.float64),
                                     host(LSEbar).astype(np.float64), ks, vs, t["scale"])
    assert_states_close(host(out), host(lse), ref, ref_lse)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_build_memory_equals_the_call_sequence(dtype, d):
    """asm_build_memory gives the same bits as first-K initialisation,
    centroid_inv_norms and `iters` rounds of kmeans_assign + aggregate."""
    r = _rng(9, d)
    H, N, K, iters = 3, 700, 50, 3
    X = synth.mixture_queries([230, d], H, N, d, M=16, dtype=dtype)
    A = r.standard_normal((H, N, d)).astype(np.float32)
    LSE = r.uniform(5, 12, (H, N)).astype(np.float32)
    Xd, Ad, Ld = dev(X), dev(A), dev(LSE)
    got = api.build_memory(Xd, K, iters, Ad, Ld)
    C = Xd[:, :K, :].clone()
    cinv = api.centroid_inv_norms(C)
    idx = torch.empty((H, N), dtype=torch.int32, device="cuda")
    count = torch.empty((H, K), dtype=torch.int32, device="cuda")
    for t in range(iters):
        api.kmeans_assign(Xd, C, cinv, idx=idx)
        _, _, _, Abar, LSEbar = api.aggregate(Xd, idx, C, A=Ad, LSE=Ld, cinv=cinv, count=count,
                                              with_states=t == iters - 1)
    torch.cuda.synchronize()
    for g, w in zip(got, (C, cinv, count, idx, Abar, LSEbar)):
        assert np.array_equal(host(g), host(w), equal_nan=True)
    # without states: no aggregation outputs, same table
    C2, _, _, idx2, Ab2, Lb2 = api.build_memory(Xd, K, iters)
    torch.cuda.synchronize()
    assert Ab2 is None and Lb2 is None
    assert np.array_equal(host(C2), host(C)) and np.array_equal(host(idx2), host(idx))
