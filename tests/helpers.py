"""Shared test plumbing: move seeded inputs to the device, widen them for the
oracle, and compare the HIP results with the oracle under the parity rules:

* nearest-centroid indices must equal the oracle's, except where another
  centroid's cosine is within 1e-5 of the best (then any such index passes);
* a must agree within 2e-3 (max abs) and lse within 1e-3, the reference
  being the oracle evaluated with the GPU's indices, so an accepted near-tie
  pick is not scored as an output error.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import asm_oracle as O

A_TOL = 2e-3
LSE_TOL = 1e-3
GAP_TOL = 1e-5


def dev(x, dtype: str = None, device="cuda"):
    """numpy -> device tensor.  uint16 arrays are bf16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(x).to(device)


def widen(x) -> np.ndarray:
    """Input array -> float64 for the oracle (bf16 bits widened exactly)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return O.bf16_bits_to_f64(x)
    return x.astype(np.float64)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def local_lists(inp):
    """Per-sequence local K/V [Hkv, n_b, d] (float64) from the packed layout."""
    Kl, Vl = widen(inp["Kl"]), widen(inp["Vl"])
    ks, vs = [], []
    for s, n in zip(inp["kv_start"], inp["kv_len"]):
        ks.append(Kl[:, s:s + n, :])
        vs.append(Vl[:, s:s + n, :])
    return ks, vs


def run_decode_gpu(inp, max_kv_len=None, **kw):
    from attention_state_memory_amd import api
    q, C = dev(inp["q"]), dev(inp["C"])
    Abar, LSEbar = dev(inp["Abar"]), dev(inp["LSEbar"])
    cinv = api.centroid_inv_norms(C)
    Kl, Vl = dev(inp["Kl"]), dev(inp["Vl"])
    ks, kn = dev(inp["kv_start"]), dev(inp["kv_len"])
    m = int(np.max(inp["kv_len"])) if max_kv_len is None else max_kv_len
    out, lse, idx = api.decode_step(q, C, cinv, Abar, LSEbar, Kl, Vl, ks, kn, m,
                                    inp["scale"], **kw)
    torch.cuda.synchronize()
    return host(out), host(lse), host(idx)


def check_indices(idx_gpu, X64, C64):
    """idx_gpu [N] vs the oracle's cosine argmax of X64 [N, d] over C64 [K, d].
    Returns the number of accepted near-tie flips; asserts the rest match."""
    ref, cs, gap = O.assign(X64, C64)
    ok = O.accept_index(idx_gpu, cs, GAP_TOL)
    bad = np.nonzero(~ok)[0]
    assert bad.size == 0, (
        f"{bad.size} indices outside tolerance, first rows {bad[:5]}: gpu {idx_gpu[bad[:5]]} "
        f"oracle {ref[bad[:5]]} gap {gap[bad[:5]]}")
    return int(np.sum(idx_gpu != ref))


def check_decode(inp, out, lse, idx):
    q64 = widen(inp["q"])
    C64 = widen(inp["C"])
    B, Hq, _ = q64.shape
    flips = 0
    for h in range(Hq):
        flips += check_indices(idx[:, h], q64[:, h, :], C64[h])
    ks, vs = local_lists(inp)
    ref, ref_lse = O.decode_with_idx(q64, idx, widen(inp["Abar"]), widen(inp["LSEbar"]),
                                     ks, vs, inp["scale"])
    assert_states_close(out, lse, ref, ref_lse)
    return flips


def assert_states_close(a, lse, a_ref, lse_ref, a_tol=A_TOL, lse_tol=LSE_TOL):
    a = np.asarray(a, np.float64)
    lse = np.asarray(lse, np.float64)
    assert np.all(np.isfinite(a)), "non-finite values in a"
    err = np.abs(a - a_ref).max() if a.size else 0.0
    assert err <= a_tol, f"max |a - a_ref| = {err:.3e} > {a_tol}"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), "empty states differ"
    if np.any(~empty):
        lerr = np.abs(lse[~empty] - lse_ref[~empty]).max()
        assert lerr <= lse_tol, f"max |lse - lse_ref| = {lerr:.3e} > {lse_tol}"
    return err
