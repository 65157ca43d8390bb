"""GPU parity of the two-level (hierarchical) lookup: asm_build_index against
the oracle's build_index, and asm_decode_step_hier against the oracle's
probe-then-search lookup evaluated on the GPU's index.

Acceptance follows the flat search's rules: a probe or an entry may differ
from the oracle's only where the oracle's cosines are within 1e-5; outputs
are held to 2e-3 (a) and 1e-3 (lse) against the oracle's merge with the
GPU's index."""
import numpy as np
import pytest
import torch

from attention_state_memory_amd import api, synth
from oracle import asm_oracle as O
from tests.helpers import GAP_TOL, assert_states_close, dev, host, local_lists, widen

pytestmark = pytest.mark.gpu


def _no_near_ties(X64, S, iters):
    """The oracle's k-means on X64 has no assignment within 1e-5 of a tie in
    any of the first `iters` rounds (so the GPU must agree exactly)."""
    C = X64[:S].copy()
    for _ in range(iters):
        idx, _, gap = O.assign(X64, C)
        if np.any(gap < GAP_TOL):
            return False
        C, _ = O.centroid_update(X64, idx, C, "bf16")
    return True


def _gpu_partition(offsets, members, S, K):
    e2s = np.full(K, -1, np.int64)
    for s in range(S):
        e2s[members[offsets[s]:offsets[s + 1]]] = s
    assert np.all(e2s >= 0)
    return e2s


def test_build_index_one_round_teacher_forced():
    """One k-means round: the GPU's partition against the oracle's cosine
    assignment to the first S entries (near-ties accepted), and the super
    means of the GPU's partition bit for bit."""
    H, K, S, d = 3, 1000, 30, 128
    E = synth.mixture_queries([400, 1], H, K, d, M=24, dtype="bf16")
    E64 = widen(E)
    SC, scinv, counts, offsets, members = [host(x) for x in api.build_index(dev(E), S, 1)]
    for h in range(H):
        e2s = _gpu_partition(offsets[h], members[h], S, K)
        _, cs, _ = O.assign(E64[h], E64[h, :S])
        assert np.all(O.accept_index(e2s, cs, GAP_TOL))
        SC_ref, n_ref = O.centroid_update(E64[h], e2s, E64[h, :S], "bf16")
        np.testing.assert_array_equal(counts[h], n_ref)
        np.testing.assert_array_equal(widen(SC[h]), SC_ref)
        np.testing.assert_allclose(scinv[h], O.inv_norms(SC_ref), rtol=1e-6)
        np.testing.assert_array_equal(offsets[h], np.concatenate([[0], np.cumsum(n_ref)]))


def test_build_index_four_rounds_matches_oracle():
    """Four rounds on data whose oracle run has no assignment within 1e-5 of
    a tie (checked here): the GPU index equals the oracle's exactly."""
    H, K, S, d, iters = 2, 1000, 30, 128, 4
    E = synth.mixture_queries([400, 7, iters], H, K, d, M=24, dtype="bf16")
    E64 = widen(E)
    for h in range(H):
        assert _no_near_ties(E64[h], S, iters)
    SC, scinv, counts, offsets, members = [host(x) for x in api.build_index(dev(E), S, iters)]
    for h in range(H):
        SC_ref, e2s_ref, n_ref = O.build_index(E64[h], S, iters, "bf16")
        np.testing.assert_array_equal(widen(SC[h]), SC_ref)
        np.testing.assert_array_equal(counts[h], n_ref)
        np.testing.assert_allclose(scinv[h], O.inv_norms(SC_ref), rtol=1e-6)
        np.testing.assert_array_equal(_gpu_partition(offsets[h], members[h], S, K), e2s_ref)


def _hier_case(seed, B, Hq, Hkv, K, S, lens, M=48):
    """Decode inputs whose memory entries are clusterable (mixture queries),
    as a built memory's are."""
    inp = synth.decode_inputs([401, seed], B=B, Hq=Hq, Hkv=Hkv, d=128, K=K, kv_lens=lens)
    inp["C"] = synth.mixture_queries([402, seed], Hq, K, 128, M=M, dtype="bf16")
    # queries near the entries' mixture: entry rows plus noise
    r = np.random.default_rng([403, seed])
    pick = r.integers(0, K, (B, Hq))
    q = np.stack([widen(inp["C"])[np.arange(Hq), pick[b]] for b in range(B)])
    q = q + 0.3 * r.standard_normal(q.shape)
    inp["q"] = synth.to_bf16_bits(q.astype(np.float32))
    return inp


def _run_hier(inp, S, p, iters=4, grouped=False):
    C = dev(inp["C"])
    cinv = api.centroid_inv_norms(C)
    index = api.build_index(C, S, iters)
    g = api.group_index_rows(C, cinv, index) if grouped else None
    out, lse, idx, probes = api.decode_step_hier(
        dev(inp["q"]), C, cinv, index, p, dev(inp["Abar"]), dev(inp["LSEbar"]), dev(inp["Kl"]),
        dev(inp["Vl"]), dev(inp["kv_start"]), dev(inp["kv_len"]), int(np.max(inp["kv_len"])),
        inp["scale"], grouped=g, want_probes=True)
    torch.cuda.synchronize()
    return [host(x) for x in index], host(out), host(lse), host(idx), host(probes)


def _check_hier(inp, index, idx, probes, p):
    """Probes are a valid top-p of the non-empty supers and idx a valid best
    entry among the probed members, both within 1e-5 in cosine units."""
    SC, _, counts, offsets, members = index
    q64 = widen(inp["q"])
    C64 = widen(inp["C"])
    B, Hq, _ = q64.shape
    misses = 0
    for h in range(Hq):
        e2s = np.empty(C64.shape[1], np.int64)
        for s in range(SC.shape[1]):
            e2s[members[h, offsets[h, s]:offsets[h, s + 1]]] = s
        SC64 = widen(SC[h])
        for b in range(B):
            ref_probes, cs = O.probe_supers(q64[b, h], SC64, counts[h], p)
            got = probes[b, h][probes[b, h] >= 0]
            assert len(got) == len(ref_probes)
            assert len(set(got.tolist())) == len(got) and np.all(counts[h][got] > 0)
            kth = cs[ref_probes[-1]]
            assert np.all(cs[got] >= kth - GAP_TOL), (b, h, got, ref_probes)
            _, cand, ce = O.lookup_probed(q64[b, h], C64[h], e2s, got)
            k = int(idx[b, h])
            assert k in set(cand.tolist())
            assert ce[list(cand).index(k)] >= ce.max() - GAP_TOL
            misses += int(k != O.assign(q64[b, h][None], C64[h])[0][0])
    return misses


def test_decode_hier_matches_oracle():
    inp = _hier_case(1, B=6, Hq=16, Hkv=4, K=2048, S=48, lens=[300, 0, 17, 1024, 64, 33])
    p = 4
    index, out, lse, idx, probes = _run_hier(inp, S=48, p=p)
    misses = _check_hier(inp, index, idx, probes, p)
    ks, vs = local_lists(inp)
    ref, ref_lse = O.decode_with_idx(widen(inp["q"]), idx, widen(inp["Abar"]), widen(inp["LSEbar"]),
                                     ks, vs, inp["scale"])
    assert_states_close(out, lse, ref, ref_lse)
    # clusterable entries: the two-level lookup mostly finds the flat nearest
    assert misses <= idx.size // 4, misses


def test_decode_hier_probing_every_super_is_the_flat_search():
    inp = _hier_case(2, B=4, Hq=8, Hkv=2, K=512, S=20, lens=[100, 5, 0, 77])
    index, out, lse, idx, probes = _run_hier(inp, S=20, p=20)
    q64, C64 = widen(inp["q"]), widen(inp["C"])
    for h in range(8):
        _, cs, _ = O.assign(q64[:, h], C64[h])
        assert np.all(O.accept_index(idx[:, h], cs, GAP_TOL))


def test_decode_hier_one_entry_per_super_with_one_probe():
    """S = K with one k-means round: every entry is its own super, so a
    single probe is the flat search."""
    inp = _hier_case(3, B=3, Hq=4, Hkv=1, K=96, S=96, lens=[10, 40, 0])
    index, out, lse, idx, probes = _run_hier(inp, S=96, p=1, iters=1)
    q64, C64 = widen(inp["q"]), widen(inp["C"])
    for h in range(4):
        _, cs, _ = O.assign(q64[:, h], C64[h])
        assert np.all(O.accept_index(idx[:, h], cs, GAP_TOL))
    ks, vs = local_lists(inp)
    ref, ref_lse = O.decode_with_idx(q64, idx, widen(inp["Abar"]), widen(inp["LSEbar"]), ks, vs,
                                     inp["scale"])
    assert_states_close(out, lse, ref, ref_lse)


def test_decode_hier_batch_beyond_resident_grid():
    """40 sequences x 32 heads x 8 probes = 10240 lookup workgroups, more than
    the device holds at once, ahead of the attention workgroups in the same
    grid: every lookup and output must still follow the oracle."""
    r = np.random.default_rng([404, 0])
    lens = r.integers(0, 300, 40).tolist()
    inp = _hier_case(5, B=40, Hq=32, Hkv=8, K=2048, S=64, lens=lens)
    p = 8
    index, out, lse, idx, probes = _run_hier(inp, S=64, p=p, iters=2)
    _check_hier(inp, index, idx, probes, p)
    ks, vs = local_lists(inp)
    ref, ref_lse = O.decode_with_idx(widen(inp["q"]), idx, widen(inp["Abar"]), widen(inp["LSEbar"]),
                                     ks, vs, inp["scale"])
    assert_states_close(out, lse, ref, ref_lse)


def test_decode_hier_more_probes_than_supers():
    """p = 12 probes over S = 8 supers at 5 sequences: the merge reads one
    candidate state per probe beside the keys, and probe ranks past the
    non-empty supers find nothing and leave their candidate unwritten.  Every
    super is probed, so this is the flat search, and the outputs follow the
    oracle."""
    inp = _hier_case(6, B=5, Hq=8, Hkv=2, K=512, S=8, lens=[64, 0, 1, 200, 31])
    index, out, lse, idx, probes = _run_hier(inp, S=8, p=12, iters=2)
    assert np.all(probes[..., 8:] == -1)
    q64, C64 = widen(inp["q"]), widen(inp["C"])
    for h in range(8):
        _, cs, _ = O.assign(q64[:, h], C64[h])
        assert np.all(O.accept_index(idx[:, h], cs, GAP_TOL))
    ks, vs = local_lists(inp)
    ref, ref_lse = O.decode_with_idx(q64, idx, widen(inp["Abar"]), widen(inp["LSEbar"]), ks, vs,
                                     inp["scale"])
    assert_states_close(out, lse, ref, ref_lse)


def test_index_group_rows_matches_indexing():
    """asm_index_group_rows is a row gather: Cg[h, i] = C[h, members[h, i]],
    cginv likewise; a member outside [0, K) gives a zero row and 0."""
    H, K, d = 3, 700, 128
    C = synth.mixture_queries([405, 0], H, K, d, M=8, dtype="bf16")
    r = np.random.default_rng([405, 1])
    members = np.stack([r.permutation(K) for _ in range(H)]).astype(np.int32)
    members[1, 5], members[2, 0] = -1, K
    Ct = dev(C)
    cinv = api.centroid_inv_norms(Ct)
    index = (None, None, None, None, dev(members))
    Cg, cg = api.group_index_rows(Ct, cinv, index)
    torch.cuda.synchronize()
    Cg, cg, ci = host(Cg), host(cg), host(cinv)
    for h in range(H):
        ok = (members[h] >= 0) & (members[h] < K)
        np.testing.assert_array_equal(Cg[h][ok], C[h][members[h][ok]])
        np.testing.assert_array_equal(cg[h][ok], ci[h][members[h][ok]])
        assert np.all(Cg[h][~ok] == 0) and np.all(cg[h][~ok] == 0)


@pytest.mark.parametrize("case", ["small", "beyond_resident"])
def test_decode_hier_grouped_table_is_identical(case):
    """With the table grouped by super the two-level step reads the same
    rows in another order: indices, probes and outputs are bit-identical to
    the step through the member list, and follow the oracle."""
    if case == "small":
        inp = _hier_case(1, B=6, Hq=16, Hkv=4, K=2048, S=48, lens=[300, 0, 17, 1024, 64, 33])
        S, p, iters = 48, 4, 4
    else:
        lens = np.random.default_rng([404, 0]).integers(0, 300, 40).tolist()
        inp = _hier_case(5, B=40, Hq=32, Hkv=8, K=2048, S=64, lens=lens)
        S, p, iters = 64, 8, 2
    # one index (its member order within a super is unspecified), two lookups
    C = dev(inp["C"])
    cinv = api.centroid_inv_norms(C)
    index_t = api.build_index(C, S, iters)
    res = []
    for g in (None, api.group_index_rows(C, cinv, index_t)):
        r = api.decode_step_hier(
            dev(inp["q"]), C, cinv, index_t, p, dev(inp["Abar"]), dev(inp["LSEbar"]), dev(inp["Kl"]),
            dev(inp["Vl"]), dev(inp["kv_start"]), dev(inp["kv_len"]), int(np.max(inp["kv_len"])),
            inp["scale"], grouped=g, want_probes=True)
        torch.cuda.synchronize()
        res.append([host(x) for x in r])
    (out, lse, idx, probes), (out_g, lse_g, idx_g, probes_g) = res
    index_g = [host(x) for x in index_t]
    np.testing.assert_array_equal(idx_g, idx)
    np.testing.assert_array_equal(probes_g, probes)
    if case == "small":  # a wave per unit: bit-identical run to run
        np.testing.assert_array_equal(out_g, out)
        np.testing.assert_array_equal(lse_g, lse)
    else:  # the pools' split of the local tiles is decided at run time: last bits only
        np.testing.assert_allclose(out_g, out, rtol=0, atol=1e-6)
        np.testing.assert_allclose(lse_g, lse, rtol=0, atol=1e-6)
    _check_hier(inp, index_g, idx_g, probes_g, p)


def test_index_group_rows_float32():
    """The row gather on a float32 table (d=64): the same indexing."""
    H, K, d = 2, 333, 64
    r = np.random.default_rng([405, 2])
    C = r.standard_normal((H, K, d)).astype(np.float32)
    members = np.stack([r.permutation(K) for _ in range(H)]).astype(np.int32)
    Ct = dev(C)
    cinv = api.centroid_inv_norms(Ct)
    Cg, cg = api.group_index_rows(Ct, cinv, (None, None, None, None, dev(members)))
    torch.cuda.synchronize()
    Cg, cg, ci = host(Cg), host(cg), host(cinv)
    for h in range(H):
        np.testing.assert_array_equal(Cg[h], C[h][members[h]])
        np.testing.assert_array_equal(cg[h], ci[h][members[h]])
