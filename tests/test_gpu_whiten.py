"""GPU parity of whitening at retrieval: asm_whiten_fit against the oracle's
whiten_fit, asm_whiten_rows against whiten_rows, and the whitened decode
step against the oracle's whitened lookup and merge.

Tolerances.  The fit is float64 on both sides with different summation
orders and a different route to Sigma^-1/2 (eigendecomposition in the
oracle, Newton-Schulz on the GPU): mu to 1e-12 relative, W to 2e-12 of its
largest entry (the fits below agree to 1e-13 .. 7e-13).  A whitened row
element x = sum_k W[o,k] (y_k - mu_k) is rounded once from float64; with W
known to 2e-12 * max|W| the GPU's float64 value lies within
delta = 2e-12 * max|W| * sum_k |y_k - mu_k| of the oracle's, so its rounding
must lie between the roundings of x - delta and x + delta (the same value
unless a rounding boundary lies within delta of x); at most 2 elements per
head may take the other side of such a boundary.  The lookup and the
outputs follow the flat search's rules (near-ties within 1e-5; a to 2e-3,
lse to 1e-3)."""
import numpy as np
import pytest
import torch

from attention_state_memory_amd import api, synth
from oracle import asm_oracle as O
from tests.helpers import GAP_TOL, assert_states_close, dev, host, local_lists, widen

pytestmark = pytest.mark.gpu

W_REL = 2e-12
W_REL_RIDGED = 5e-9  # ridged rank-deficient corpus: cond(Sigma) about 1e6, fits agree to 5e-10


def _corpus(seed, H, N, d, dtype, skew=True):
    """Clusterable calibration queries; with skew, dims scaled by 0.25..4 so
    that whitening changes the geometry."""
    X = synth.mixture_queries([220, seed], H, N, d, M=32, dtype="f32")
    if skew:
        X = X * np.geomspace(0.25, 4.0, d, dtype=np.float32)
    return synth.to_bf16_bits(X) if dtype == "bf16" else X.astype(np.float32)


def _check_rows(got_bits_or_vals, Y64, mu, W, dtype):
    """Element-wise against the oracle's whitening of the rows Y64 [M, d]:
    the GPU's rounding must be that of some value within delta (see the
    module docstring) of the oracle's float64 value.  Returns how many
    elements took the other neighbour of a nearby rounding boundary."""
    got = widen(got_bits_or_vals)
    x = O.whiten_apply(Y64, mu, W)
    delta = W_REL * np.max(np.abs(W)) * np.sum(np.abs(Y64 - mu), axis=-1, keepdims=True)
    delta = np.broadcast_to(delta, x.shape)
    exact = O.round_to_dtype(x, dtype)
    bad = got != exact
    if not np.any(bad):
        return 0
    xb, db, g = x[bad], delta[bad], got[bad]
    lo = O.round_to_dtype(xb - db, dtype)
    hi = O.round_to_dtype(xb + db, dtype)
    assert np.all((lo <= g) & (g <= hi)), (np.sum(bad), xb[:5], g[:5], db[:5])
    return int(np.sum(bad))


FIT = [
    # (seed, dtype, H, N, d)
    (1, "bf16", 3, 5000, 128),
    (2, "bf16", 2, 777, 64),
    (3, "f32", 2, 300, 64),
    (4, "bf16", 1, 200, 128),   # N > d but few rows: a wide spread of eigenvalues
]


@pytest.mark.parametrize("case", FIT, ids=[f"f{c[0]}" for c in FIT])
def test_whiten_fit_and_rows_match_oracle(case):
    seed, dtype, H, N, d = case
    X = _corpus(seed, H, N, d, dtype)
    print(f"whiten fit case {case}", flush=True)
    mu, W, resid = api.whiten_fit(dev(X), want_resid=True)
    C = X[:, : min(N, 512)].copy()
    Cw = api.whiten_rows(dev(C), mu, W)
    torch.cuda.synchronize()
    mu, W, resid, Cw = host(mu), host(W), host(resid), host(Cw)
    X64 = widen(X)
    for h in range(H):
        mu_ref, W_ref = O.whiten_fit(X64[h])
        np.testing.assert_allclose(mu[h], mu_ref, rtol=1e-12, atol=1e-14)
        werr = np.max(np.abs(W[h] - W_ref)) / np.max(np.abs(W_ref))
        flips = _check_rows(Cw[h], widen(C[h]), mu_ref, W_ref, dtype)
        print(f"  head {h}: W rel err {werr:.2e}, resid {resid[h]:.2e}, flips {flips} of {Cw[h].size}",
              flush=True)
        assert werr <= W_REL
        assert resid[h] < 1e-10
        assert np.array_equal(W[h], W[h].T)
        assert flips <= 2


def test_whiten_fit_singular_without_ridge_gives_nan():
    """A rank-deficient corpus (fewer rows than dimensions) has no inverse
    square root without the ridge: the fit must say so (W all NaN, residual
    reported at or above 1e-6); with the default ridge it matches the
    oracle.  A constant corpus has zero covariance: NaN whatever the ridge."""
    H, N, d = 2, 40, 64
    X = _corpus(9, H, N, d, "bf16", skew=False)
    mu, W, resid = api.whiten_fit(dev(X), ridge=0.0, want_resid=True)
    torch.cuda.synchronize()
    W, resid = host(W), host(resid)
    assert np.isnan(W).all()
    assert not np.any(resid < 1e-6)  # at or above 1e-6, or NaN once Z overflows
    mu, W, resid = api.whiten_fit(dev(X), want_resid=True)
    torch.cuda.synchronize()
    mu, W, resid = host(mu), host(W), host(resid)
    X64 = widen(X)
    for h in range(H):
        mu_ref, W_ref = O.whiten_fit(X64[h])
        werr = np.max(np.abs(W[h] - W_ref)) / np.max(np.abs(W_ref))
        print(f"  rank-deficient head {h}: W rel err {werr:.2e}, resid {resid[h]:.2e}", flush=True)
        np.testing.assert_allclose(mu[h], mu_ref, rtol=1e-12, atol=1e-14)
        assert np.isfinite(W[h]).all() and resid[h] < 1e-6
        assert werr <= W_REL_RIDGED
    Xc = np.repeat(X[:, :1], N, axis=1)
    _, W, resid = api.whiten_fit(dev(Xc), want_resid=True)
    torch.cuda.synchronize()
    assert np.isnan(host(W)).all()


def _whitened_decode_case(seed, B, Hq, Hkv, K, lens, N=4000, dtype="bf16", d=128):
    inp = synth.decode_inputs([221, seed], B=B, Hq=Hq, Hkv=Hkv, d=d, K=K, kv_lens=lens, dtype=dtype)
    X = _corpus(seed, Hq, N, d, dtype)
    # the table and the queries come from the corpus's distribution
    inp["C"] = X[:, :K].copy()
    r = np.random.default_rng([222, seed])
    pick = r.integers(0, N, (B, Hq))
    q = np.stack([widen(X)[np.arange(Hq), pick[b]] for b in range(B)])
    q = (q + 0.3 * r.standard_normal(q.shape) * np.geomspace(0.25, 4.0, d)).astype(np.float32)
    inp["q"] = synth.to_bf16_bits(q) if dtype == "bf16" else q
    return inp, X


def _run_whitened(inp, X):
    mu, W, _ = api.whiten_fit(dev(X))
    Cw = api.whiten_rows(dev(inp["C"]), mu, W)
    cwinv = api.centroid_inv_norms(Cw)
    out, lse, idx = api.decode_step_whitened(
        dev(inp["q"]), mu, W, Cw, cwinv, dev(inp["Abar"]), dev(inp["LSEbar"]), dev(inp["Kl"]),
        dev(inp["Vl"]), dev(inp["kv_start"]), dev(inp["kv_len"]), int(np.max(inp["kv_len"])),
        inp["scale"])
    torch.cuda.synchronize()
    return host(Cw), host(out), host(lse), host(idx)


def _check_whitened(inp, X, Cw, idx, sample=None, dtype="bf16"):
    """idx against the oracle's whitened cosines: the oracle's whitened
    queries against the GPU's table (checked element by element first).
    Returns how many lookups differ from the unwhitened nearest entry."""
    q64, X64, C64 = widen(inp["q"]), widen(X), widen(inp["C"])
    B, Hq, _ = q64.shape
    changed = 0
    heads = range(Hq) if sample is None else sample
    for h in heads:
        mu, W = O.whiten_fit(X64[h])
        _check_rows(Cw[h], C64[h], mu, W, dtype)
        qw = O.whiten_rows(q64[:, h], mu, W, dtype)
        _, cs, _ = O.assign(qw, widen(Cw[h]))
        assert np.all(O.accept_index(idx[:, h], cs, GAP_TOL)), h
        plain, _, _ = O.assign(q64[:, h], C64[h])
        changed += int(np.sum(plain != idx[:, h]))
    return changed


def test_decode_whitened_matches_oracle():
    inp, X = _whitened_decode_case(1, B=6, Hq=16, Hkv=4, K=512, lens=[300, 0, 17, 1024, 64, 33])
    Cw, out, lse, idx = _run_whitened(inp, X)
    changed = _check_whitened(inp, X, Cw, idx)
    assert changed > 0  # whitening changes some lookups on skewed data
    ks, vs = local_lists(inp)
    ref, ref_lse = O.decode_with_idx(widen(inp["q"]), idx, widen(inp["Abar"]), widen(inp["LSEbar"]),
                                     ks, vs, inp["scale"])
    assert_states_close(out, lse, ref, ref_lse)


def test_decode_whitened_f32_valu_path():
    """float32 rows, d = 64, G = 3: the plain VALU decode path scores the
    whitened queries."""
    inp, X = _whitened_decode_case(3, B=5, Hq=6, Hkv=2, K=300, lens=[40, 0, 129, 7, 64],
                                   dtype="f32", d=64)
    Cw, out, lse, idx = _run_whitened(inp, X)
    _check_whitened(inp, X, Cw, idx, dtype="f32")
    ks, vs = local_lists(inp)
    ref, ref_lse = O.decode_with_idx(widen(inp["q"]), idx, widen(inp["Abar"]), widen(inp["LSEbar"]),
                                     ks, vs, inp["scale"])
    assert_states_close(out, lse, ref, ref_lse)


@pytest.mark.timeout(900)
def test_decode_whitened_full_size_sampled():
    """The batched-decode configuration (32 sequences of 512..4096 local
    tokens, 32 query heads, 8 kv heads, K = 8192): every lookup of 8 sampled
    heads checked, outputs on 64 sampled (sequence, head) pairs."""
    r = np.random.default_rng([223, 0])
    lens = r.integers(512, 4097, 32).tolist()
    inp, X = _whitened_decode_case(2, B=32, Hq=32, Hkv=8, K=8192, lens=lens, N=16384)
    print("whitened full-size inputs ready", flush=True)
    Cw, out, lse, idx = _run_whitened(inp, X)
    heads = sorted(r.choice(32, 8, replace=False).tolist())
    _check_whitened(inp, X, Cw, idx, sample=heads)
    ks, vs = local_lists(inp)
    pairs = [(int(b), int(h)) for b, h in zip(r.integers(0, 32, 64), r.integers(0, 32, 64))]
    q64, A64, L64 = widen(inp["q"]), widen(inp["Abar"]), widen(inp["LSEbar"])
    for b, h in pairs:
        G = 32 // 8
        ref, ref_lse = O.decode_with_idx(q64[b:b + 1, h:h + 1], idx[b:b + 1, h:h + 1],
                                         A64[h:h + 1], L64[h:h + 1], [ks[b][h // G:h // G + 1]],
                                         [vs[b][h // G:h // G + 1]], inp["scale"])
        assert_states_close(out[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], ref, ref_lse)
