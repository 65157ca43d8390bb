"""GPU parity over seeded random shapes: every entry point of the hot path on
small problems whose sizes (batch, heads, group, head dim, table size,
lengths, chunk) are drawn from a fixed seed list, so that tile tails, empty
sequences and both the MFMA and the VALU paths are crossed in many
combinations.  The rules are those of the fixed-shape tests."""
import numpy as np
import pytest
import torch

from attention_state_memory_amd import api, synth
from oracle import asm_oracle as O
from tests.helpers import (assert_states_close, check_decode, check_indices, dev, host,
                           run_decode_gpu, widen)

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
