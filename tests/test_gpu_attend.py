"""GPU parity of the full-attention comparator (asm_attend_step): the
attention state of each decode query over its sequence's whole context
(the fixed prefix followed by the local tokens, one KV cache), against the
oracle's `state` over that concatenation ([TS] Resultados Experimentales
time the method against full attention over the prefix).  Also the
method's exactness at the system level ([TS] Fusión): with a memory that
holds each decode query's own exact prefix state (K = N), asm_decode_step
over the local tokens must give what asm_attend_step gives over
[prefix; local]."""
import numpy as np
import pytest
import torch

from attention_state_memory_amd import api, synth
from oracle import asm_oracle as O
from tests.helpers import assert_states_close, dev, host, widen

pytestmark = pytest.mark.gpu


def _oracle_attend(inp):
    q, Kc, Vc = widen(inp["q"]), widen(inp["Kc"]), widen(inp["Vc"])
    B, Hq, d = q.shape
    G = Hq // inp["Hkv"]
    out, lse = np.zeros((B, Hq, d)), np.zeros((B, Hq))
    for b in range(B):
        s, n = inp["ctx_start"][b], inp["ctx_len"][b]
        for h in range(Hq):
            out[b, h], lse[b, h] = O.state(q[b, h], Kc[h // G, s:s + n], Vc[h // G, s:s + n],
                                           inp["scale"])
    return out, lse


CASES = [
    # (seed, B, Hq, Hkv, d, L, local lengths)
    (1, 3, 32, 8, 128, 1000, [0, 70, 513]),
    (2, 8, 8, 8, 64, 300, [1, 31, 32, 33, 64, 65, 200, 0]),   # G = 1, ragged tiles
    (3, 2, 8, 1, 128, 4096, [2048, 17]),                        # G = 8
    (4, 32, 32, 8, 128, 512, list(np.random.default_rng(4).integers(512, 4097, 32))),
]


@pytest.mark.parametrize("case", CASES, ids=[f"a{c[0]}" for c in CASES])
def test_attend_step_matches_oracle(case):
    seed, B, Hq, Hkv, d, L, lens = case
    print(f"attend case {case[:6]}", flush=True)
    inp = synth.attend_inputs([230, seed], B, Hq, Hkv, d, L, lens)
    Kc, Vc = dev(inp["Kc"]), dev(inp["Vc"])
    out, lse = api.attend_step(dev(inp["q"]), Kc, Vc, dev(inp["ctx_start"]), dev(inp["ctx_len"]),
                               int(inp["ctx_len"].max()), inp["scale"])
    torch.cuda.synchronize()
    ref, ref_lse = _oracle_attend(inp)
    assert_states_close(host(out), host(lse), ref, ref_lse)


def test_attend_step_strided_cache_and_empty_sequences():
    """A paged-style cache: each token row padded to 192 elements and the
    kv heads 4096 token slots apart; empty sequences give (0, -inf)."""
    inp = synth.attend_inputs([231, 0], 4, 16, 4, 128, 200, [0, 300, 0, 45])
    Hkv, T, d = 4, int(inp["ctx_len"].sum()), 128
    inp["ctx_len"][[0, 2]] = 0  # sequences 0 and 2: no context at all
    big = torch.zeros((Hkv, 4096, 192), dtype=torch.bfloat16, device="cuda")
    bigv = torch.zeros_like(big)
    big[:, :T, :d] = dev(inp["Kc"])
    bigv[:, :T, :d] = dev(inp["Vc"])
    out, lse = api.attend_step(dev(inp["q"]), big[:, :, :d], bigv[:, :, :d], dev(inp["ctx_start"]),
                               dev(inp["ctx_len"]), int(inp["ctx_len"].max()), inp["scale"])
    torch.cuda.synchronize()
    ref, ref_lse = _oracle_attend(inp)
    assert_states_close(host(out), host(lse), ref, ref_lse)
    assert np.all(host(out)[[0, 2]] == 0) and np.all(np.isneginf(host(lse)[[0, 2]]))


def test_decode_with_exact_prefix_states_equals_full_attention():
    """K = N: the memory's entries are the decode queries themselves, each
    holding its own prefix state (asm_build_states), so every lookup finds
    the query's own entry and the merge with the local state must equal
    full attention over [prefix; local]."""
    B, Hq, Hkv, d, L = 16, 32, 8, 128, 2048
    lens = np.random.default_rng(5).integers(0, 1500, B)
    inp = synth.attend_inputs([232, 0], B, Hq, Hkv, d, L, lens)
    q = dev(inp["q"])
    # memory: entry b of head h is query (b, h) with its exact prefix state
    C = q.transpose(0, 1).contiguous()            # [Hq, B, d]
    Abar, LSEbar, _, _ = api.build_states(C, dev(inp["Kp"]), dev(inp["Vp"]), L, inp["scale"])
    cinv = api.centroid_inv_norms(C)
    out, lse, idx = api.decode_step(q, C, cinv, Abar, LSEbar, dev(inp["Kl"]), dev(inp["Vl"]),
                                    dev(inp["kv_start"]), dev(inp["kv_len"]),
                                    int(inp["kv_len"].max()), inp["scale"])
    fo, flse = api.attend_step(q, dev(inp["Kc"]), dev(inp["Vc"]), dev(inp["ctx_start"]),
                               dev(inp["ctx_len"]), int(inp["ctx_len"].max()), inp["scale"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(idx), np.repeat(np.arange(B)[:, None], Hq, axis=1))
    assert_states_close(host(out), host(lse), host(fo), host(flse))
    ref, ref_lse = _oracle_attend(inp)
    assert_states_close(host(fo), host(flse), ref, ref_lse)
