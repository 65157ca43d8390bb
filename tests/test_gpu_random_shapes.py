"""GPU parity over seeded random shapes: the entry points of the hot path
(decode, prefix states, assignment and aggregation, the two-level lookup and
whitening) on small problems whose sizes (batch, heads, group, head dim,
table size, lengths, chunk, supers, probes, corpus) are drawn from a fixed
seed list, so that tile tails, empty sequences and both the MFMA and the
VALU paths are crossed in many combinations.  The rules are those of the
fixed-shape tests."""
import numpy as np
import pytest
import torch

from attention_state_memory_amd import api, synth
from oracle import asm_oracle as O
from tests.helpers import (assert_states_close, check_decode, check_indices, dev, host,
                           local_lists, run_decode_gpu, widen)

pytestmark = pytest.mark.gpu

SEEDS = list(range(12))


def _shape(seed):
    r = np.random.default_rng([240, seed])
    dtype = "bf16" if seed % 4 else "f32"
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 3, 4, 8]))
    d = int(r.choice([64, 128])) if dtype == "bf16" else int(r.choice([32, 48, 64, 128]))
    return r, dtype, Hkv, G, d


@pytest.mark.parametrize("seed", SEEDS)
def test_decode_random_shape(seed):
    r, dtype, Hkv, G, d = _shape(seed)
    B = int(r.integers(1, 41))
    K = int(r.integers(1, 700))
    lens = r.integers(0, 600, B)
    lens[r.random(B) < 0.15] = 0
    print(f"decode seed {seed}: {dtype} B={B} Hq={Hkv * G} Hkv={Hkv} d={d} K={K}", flush=True)
    inp = synth.decode_inputs([241, seed], B=B, Hq=Hkv * G, Hkv=Hkv, d=d, K=K,
                              kv_lens=lens.tolist(), dtype=dtype)
    out, lse, idx = run_decode_gpu(inp)
    check_decode(inp, out, lse, idx)


@pytest.mark.parametrize("seed", SEEDS)
def test_build_states_random_shape(seed):
    r, dtype, Hkv, G, d = _shape(seed)
    N = int(r.integers(1, 300))
    L = int(r.integers(0, 700))
    chunk = int(r.choice([16, 64, 100, 256, 1000]))
    print(f"states seed {seed}: {dtype} Hq={Hkv * G} Hkv={Hkv} d={d} N={N} L={L} chunk={chunk}",
          flush=True)
    rr = np.random.default_rng([242, seed])
    mk = (lambda s: synth.to_bf16_bits(rr.standard_normal(s, dtype=np.float32))) if dtype == "bf16" \
        else (lambda s: rr.standard_normal(s, dtype=np.float32))
    Q, Kp, Vp = mk((Hkv * G, N, d)), mk((Hkv, L, d)), mk((Hkv, L, d))
    scale = synth.softmax_scale(d)
    A, LSE, Ac, Lc = api.build_states(dev(Q), dev(Kp), dev(Vp), chunk, scale, keep_chunks=L > 0)
    torch.cuda.synchronize()
    Ac_ref, Lc_ref, A_ref, L_ref = O.build_states(widen(Q), widen(Kp), widen(Vp), chunk, scale)
    assert_states_close(host(A), host(LSE), A_ref, L_ref)
    if L > 0:
        assert_states_close(host(Ac), host(Lc), Ac_ref, Lc_ref)


@pytest.mark.parametrize("seed", SEEDS)
def test_assign_and_aggregate_random_shape(seed):
    r, dtype, _, _, d = _shape(seed)
    H = int(r.integers(1, 4))
    K = int(r.integers(1, 300))
    N = int(r.integers(K, K + 900))
    print(f"assign seed {seed}: {dtype} H={H} N={N} K={K} d={d}", flush=True)
    X = synth.mixture_queries([243, seed], H, N, d, M=16, dtype=dtype)
    rr = np.random.default_rng([244, seed])
    A = rr.standard_normal((H, N, d)).astype(np.float32)
    LSE = rr.uniform(5, 12, (H, N)).astype(np.float32)
    Xd = dev(X)
    C = Xd[:, :K, :].clone()
    cinv = api.centroid_inv_norms(C)
    idx, _ = api.kmeans_assign(Xd, C, cinv)
    C2, cinv2, count, Abar, LSEbar = api.aggregate(Xd, idx, C, A=dev(A), LSE=dev(LSE), cinv=cinv,
                                                   with_states=True)
    torch.cuda.synchronize()
    X64, idx_h = widen(X), host(idx)
    C0 = X64[:, :K]
    for h in range(H):
        check_indices(idx_h[h], X64[h], C0[h])
        C_ref, n_ref = O.centroid_update(X64[h], idx_h[h], C0[h], dtype)
        np.testing.assert_array_equal(host(count)[h], n_ref)
        np.testing.assert_array_equal(widen(host(C2)[h]), C_ref)
        a_ref, l_ref = O.aggregate(widen(A[h]), widen(LSE[h]), idx_h[h], K)
        assert_states_close(host(Abar)[h], host(LSEbar)[h], a_ref, l_ref, a_tol=1e-5, lse_tol=1e-5)


HIER_SEEDS = list(range(8))


@pytest.mark.parametrize("seed", HIER_SEEDS)
def test_decode_hier_random_shape(seed):
    """Two-level lookup (bf16, d = 128) on random batch, group, table size,
    super count and probe count; the rules of the fixed-shape hier tests."""
    from tests.test_gpu_hier import _check_hier, _hier_case, _run_hier
    r = np.random.default_rng([245, seed])
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8]))
    B = int(r.integers(1, 13))
    K = int(r.integers(64, 1500))
    S = int(r.integers(2, min(K, 64) + 1))
    p = int(r.integers(1, min(S, 32) + 1))  # the lookup takes at most 32 probes
    iters = int(r.integers(1, 5))
    lens = r.integers(0, 700, B)
    lens[r.random(B) < 0.2] = 0
    print(f"hier seed {seed}: B={B} Hq={Hkv * G} Hkv={Hkv} K={K} S={S} p={p} iters={iters}", flush=True)
    inp = _hier_case(100 + seed, B=B, Hq=Hkv * G, Hkv=Hkv, K=K, S=S, lens=lens.tolist())
    index, out, lse, idx, probes = _run_hier(inp, S=S, p=p, iters=iters)
    _check_hier(inp, index, idx, probes, p)
    ks, vs = local_lists(inp)
    ref, ref_lse = O.decode_with_idx(widen(inp["q"]), idx, widen(inp["Abar"]), widen(inp["LSEbar"]),
                                     ks, vs, inp["scale"])
    assert_states_close(out, lse, ref, ref_lse)


WHITE_SEEDS = list(range(6))


@pytest.mark.parametrize("seed", WHITE_SEEDS)
def test_decode_whitened_random_shape(seed):
    """Whitening fit, table whitening and the whitened decode step on random
    shapes (bf16 and f32 rows, d in {64, 128}, corpora of 2d to 3000 rows)."""
    from tests.test_gpu_whiten import _check_whitened, _run_whitened, _whitened_decode_case
    r = np.random.default_rng([246, seed])
    dtype = "bf16" if seed % 3 else "f32"
    d = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 3, 4])) if dtype == "f32" else int(r.choice([1, 2, 4]))
    B = int(r.integers(1, 10))
    N = int(r.integers(2 * d, 3000))  # a full-rank corpus: W known to 1e-9
    K = int(r.integers(1, min(N, 600) + 1))
    lens = r.integers(0, 500, B)
    print(f"whitened seed {seed}: {dtype} d={d} B={B} Hq={Hkv * G} Hkv={Hkv} N={N} K={K}", flush=True)
    inp, X = _whitened_decode_case(300 + seed, B=B, Hq=Hkv * G, Hkv=Hkv, K=K, lens=lens.tolist(),
                                   N=N, dtype=dtype, d=d)
    Cw, out, lse, idx = _run_whitened(inp, X)
    _check_whitened(inp, X, Cw, idx, dtype=dtype)
    ks, vs = local_lists(inp)
    ref, ref_lse = O.decode_with_idx(widen(inp["q"]), idx, widen(inp["Abar"]), widen(inp["LSEbar"]),
                                     ks, vs, inp["scale"])
    assert_states_close(out, lse, ref, ref_lse)
