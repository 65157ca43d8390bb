"""GPU parity of asm_decode_step against the fp64 oracle (retrieval by cosine,
state gather, local attention, online-softmax merge)."""
import numpy as np
import pytest
import torch

from attention_state_memory_amd import api, synth
from oracle import asm_oracle as O
from tests.helpers import (check_decode, dev, host, run_decode_gpu, widen,
                           assert_states_close)

pytestmark = pytest.mark.gpu


def _case(seed, d, Hq, Hkv, K, lens, dtype="bf16"):
    return synth.decode_inputs([100, seed], B=len(lens), Hq=Hq, Hkv=Hkv, d=d, K=K,
                               kv_lens=lens, dtype=dtype)


SMALL = [
    # (seed, d, Hq, Hkv, K, lens)                         path exercised
    (1, 128, 32, 8, 1000, [0, 37, 300]),                   # MFMA, G=4, ragged, empty seq
    (2, 128, 8, 8, 300, list(range(3, 200, 5))),           # MFMA, G=1, B=40 > 32
    (3, 64, 16, 8, 513, [1, 31, 32, 33, 129]),             # MFMA, d=64, G=2
    (4, 128, 16, 2, 257, [700, 64]),                       # MFMA, G=8
    (5, 128, 12, 4, 64, [50, 10]),                         # VALU bf16 (G=3)
    (6, 96, 4, 2, 40, [20, 5]),                            # VALU bf16 (d=96)
    (7, 128, 32, 8, 256, [4096, 1, 2048, 513]),            # long splits
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}" for c in SMALL])
def test_decode_small_shapes(case):
    inp = _case(*case)
    out, lse, idx = run_decode_gpu(inp)
    check_decode(inp, out, lse, idx)


# Steps small enough that every potential work unit has a wave (the direct
# layout: each wave reads its sequence's bounds itself; two tiles per wave
# and per partial state; with at most 16 scoring units per head and 8
# sequences the scoring units also copy their best entries' states).
DIRECT = [
    # (seed, d, Hq, Hkv, K, lens)                        what it exercises
    (20, 128, 32, 8, 1024, [61]),                         # odd tile count: a wave with one tile
    (21, 128, 32, 8, 1000, [5, 0, 500, 33, 64, 65, 1, 499]),  # 8 sequences (gathering), last unit partial
    (22, 128, 32, 8, 960, [100] * 9),                     # 9 sequences: no gathering
    (23, 64, 16, 2, 1024, [31, 32, 33]),                  # d=64, G=8, 16 units per head
    (24, 128, 8, 8, 1088, [300, 7]),                      # 17 units per head: no gathering, G=1
    (25, 128, 32, 8, 512, [0, 1]),                        # one empty sequence, one with a single token
]


@pytest.mark.parametrize("case", DIRECT, ids=[f"d{c[0]}" for c in DIRECT])
def test_decode_direct_layout_shapes(case):
    inp = _case(*case)
    out, lse, idx = run_decode_gpu(inp)
    check_decode(inp, out, lse, idx)


# Steps too large for a wave per unit at once, but dominated by scoring
# (local attention waves at most a quarter of the scoring units): the direct
# layout as well, its grid running in several waves of workgroups; and one
# step just past that bound, which takes the persistent pools.
SCORING_DIRECT = [
    # (seed, d, Hq, Hkv, K, lens)                        what it exercises
    (26, 128, 32, 8, 8192, [2048]),                       # batch 1 at K=8192: 4352 waves
    (27, 128, 32, 8, 8192, [2048, 0, 1, 777]),            # 4 sequences, ragged, at the bound
    (28, 64, 16, 2, 16384, [3000, 45]),                   # d=64, G=8, 256 units per head
    (29, 128, 32, 8, 8192, [2048] * 5),                   # past the bound: pools
    (30, 64, 8, 8, 16384, [20] * 39 + [0]),               # 40 sequences (queries in two column tiles), G=1
]


@pytest.mark.parametrize("case", SCORING_DIRECT, ids=[f"sd{c[0]}" for c in SCORING_DIRECT])
def test_decode_scoring_dominated_shapes(case):
    inp = _case(*case)
    out, lse, idx = run_decode_gpu(inp)
    check_decode(inp, out, lse, idx)


def test_decode_float32_tiny_shape():
    """One head, d=64, float32, four queries sharing one 32-token local KV."""
    inp = _case(8, 64, 1, 1, 64, [32], dtype="f32")
    rng = np.random.default_rng([100, 80])
    inp["q"] = rng.standard_normal((4, 1, 64)).astype(np.float32)
    inp["kv_start"] = np.zeros(4, np.int32)
    inp["kv_len"] = np.full(4, 32, np.int32)
    out, lse, idx = run_decode_gpu(inp)
    check_decode(inp, out, lse, idx)


def test_decode_float32_generic_gqa():
    inp = _case(9, 128, 8, 2, 700, [0, 100, 333], dtype="f32")
    out, lse, idx = run_decode_gpu(inp)
    check_decode(inp, out, lse, idx)


@pytest.mark.parametrize("layer", range(32))
def test_decode_llama_layer_k1024(layer):
    """Batch-1 decode of one LLaMA-3.1-8B-shaped layer (K=1024, 2048 local
    tokens); all 32 layers with independent seeds."""
    inp = synth.layer_decode(layer)
    out, lse, idx = run_decode_gpu(inp)
    check_decode(inp, out, lse, idx)


def test_decode_batched_k8192_full_size():
    """The full batched workload: K=8192, 32 sequences, ragged 512..4096."""
    inp = synth.batched_decode(0)
    out, lse, idx = run_decode_gpu(inp)
    flips = check_decode(inp, out, lse, idx)
    assert flips <= 5


def test_decode_ties_empty_entries_and_bad_lengths():
    inp = _case(10, 128, 8, 2, 300, [40, 0, 17, 9])
    C = inp["C"].copy()
    q = inp["q"].copy()
    # head 0: make centroid 7 a duplicate of centroid 3 and query 0 point at it:
    # exact float32 tie -> the lower index must win.
    C[0, 7] = C[0, 3]
    q[0, 0] = C[0, 3]
    inp["C"], inp["q"] = C, q
    # head 1: sequence 1 (no local tokens) retrieves an empty entry -> (0, -inf)
    Cw = widen(C)
    k_empty = int(O.assign(widen(q)[1:2, 1], Cw[1])[0][0])
    inp["LSEbar"] = inp["LSEbar"].copy()
    inp["Abar"] = inp["Abar"].copy()
    inp["LSEbar"][1, k_empty] = -np.inf
    inp["Abar"][1, k_empty] = 0.0
    out, lse, idx = run_decode_gpu(inp, max_kv_len=64)
    assert idx[0, 0] == 3
    check_decode(inp, out, lse, idx)
    assert np.isneginf(lse[1, 1]) and np.all(out[1, 1] == 0)
    # sequence 0 with a length beyond max_kv_len: refused, outputs NaN
    bad = dict(inp)
    bad["kv_len"] = inp["kv_len"].copy()
    bad["kv_len"][0] = 65
    out2, lse2, _ = run_decode_gpu(bad, max_kv_len=64)
    assert np.all(np.isnan(out2[0])) and np.all(np.isnan(lse2[0]))
    np.testing.assert_array_equal(out2[1:], out[1:])


def test_decode_strided_kv_and_determinism():
    """Local KV inside a padded cache (token stride 136, head stride of a
    larger buffer); two runs must be bit-identical."""
    inp = _case(11, 128, 16, 4, 2048, [200, 1000, 37])
    Hkv, tot, d = 4, int(inp["kv_len"].sum()), 128
    pad_tok, cap = 136, tot + 50
    Kbig = np.zeros((Hkv, cap, pad_tok), np.uint16)
    Vbig = np.zeros((Hkv, cap, pad_tok), np.uint16)
    Kbig[:, :tot, :d] = inp["Kl"]
    Vbig[:, :tot, :d] = inp["Vl"]
    from attention_state_memory_amd import api as A
    Kt = dev(Kbig)[:, :, :d]
    Vt = dev(Vbig)[:, :, :d]
    q, C = dev(inp["q"]), dev(inp["C"])
    cinv = A.centroid_inv_norms(C)
    Ab, Lb = dev(inp["Abar"]), dev(inp["LSEbar"])
    ks, kn = dev(inp["kv_start"]), dev(inp["kv_len"])
    r1 = A.decode_step(q, C, cinv, Ab, Lb, Kt, Vt, ks, kn, 1000, inp["scale"])
    r2 = A.decode_step(q, C, cinv, Ab, Lb, Kt, Vt, ks, kn, 1000, inp["scale"])
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)
    check_decode(inp, host(r1[0]), host(r1[1]), host(r1[2]))


def test_decode_shared_workspace_across_shapes():
    """One workspace serves calls of different shapes in turn; each result is
    bit-identical to the same call on a fresh zeroed workspace."""
    cases = [
        _case(21, 128, 32, 8, 1000, [0, 37, 300]),
        _case(22, 128, 32, 8, 1024, [2048]),          # one sequence over many waves
        _case(23, 64, 16, 8, 513, [1, 31, 32, 33, 129]),
        _case(24, 128, 16, 2, 257, [700, 64]),
    ]
    nbytes = max(api.decode_step_ws(0, c["B"], c["Hq"], c["Hkv"], c["d"], c["K"], 4096)
                 for c in cases)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for c in cases + cases[:1]:
        shared = run_decode_gpu(c, max_kv_len=4096, workspace=ws)
        fresh = run_decode_gpu(c, max_kv_len=4096)
        for x, y in zip(shared, fresh):
            np.testing.assert_array_equal(x, y)
        check_decode(c, *shared)


def test_decode_batch_beyond_one_launch():
    """2100 sequences: more than one launch's batch on the MFMA path, so the
    call runs as consecutive launches over batch slices sharing the
    workspace.  Short ragged contexts (0..64 tokens) keep the oracle cheap."""
    rng = np.random.default_rng([100, 30])
    lens = rng.integers(0, 65, 2100)
    inp = synth.decode_inputs([100, 31], B=2100, Hq=8, Hkv=2, d=128, K=96, kv_lens=lens)
    out, lse, idx = run_decode_gpu(inp, max_kv_len=64)
    check_decode(inp, out, lse, idx)


@pytest.mark.parametrize("lens", [[2048], [1500, 0, 2600]], ids=["b1", "b3"])
def test_decode_scoring_dominated_capped_grid(lens):
    """K = 8192 with one to three short sequences: the scoring units outnumber
    the attention tiles and the grid is capped at the resident waves, so the
    first waves take the tiles and the rest the scoring units, in proportion.
    The lookup and the merge must be the oracle's, as everywhere."""
    inp = _case(40 + len(lens), 128, 32, 8, 8192, lens)
    out, lse, idx = run_decode_gpu(inp)
    check_decode(inp, out, lse, idx)


def test_decode_one_sequence_long_context_many_pieces():
    """Batch 1 with a 40000-token context: the segment is split over many
    waves (dozens of partial states merged by the combine)."""
    inp = _case(32, 128, 32, 8, 512, [40000])
    out, lse, idx = run_decode_gpu(inp)
    check_decode(inp, out, lse, idx)


def test_centroid_inv_norms_match_definition():
    rng = np.random.default_rng([100, 12])
    C = synth.to_bf16_bits(rng.standard_normal((3, 777, 128)).astype(np.float32))
    C[1, 5] = 0
    cinv = host(api.centroid_inv_norms(dev(C)))
    ref = O.inv_norms(widen(C))
    assert cinv[1, 5] == 0.0
    np.testing.assert_allclose(cinv, ref, rtol=1e-6, atol=0)
