"""GPU parity at the full-attention comparison's largest shapes, in the
launch configuration its benchmark times (one call per step, 32 query heads,
8 kv heads, d=128, bf16, local lengths of the batched workload's replica 0):

* asm_attend_step, batch 32 over a 16384-token prefix plus the local tokens
  (about 600K context tokens per kv head): the attention state of sampled
  (sequence, head) pairs against the oracle's `state` over the sequence's
  whole context ([TS] Resultados Experimentales, the latency baseline);
* asm_decode_step, batch 32 at K=16384: every index and output of two kv-head
  groups (8 query heads) against the oracle's lookup and merge ([TS]
  Recuperación, Fusión).

The tensors are drawn on the device with seeded generators (GB-sized inputs);
the oracle reads copies of exactly the slices it needs."""
import numpy as np
import pytest
import torch

from attention_state_memory_amd import api, synth
from oracle import asm_oracle as O
from tests.helpers import assert_states_close, check_indices, host, widen

pytestmark = pytest.mark.gpu

Hq, Hkv, d = 32, 8, 128
G = Hq // Hkv


def _lens():
    return [int(x) for x in np.random.default_rng([3, 0]).integers(512, 4097, 32)]


def _starts(lens):
    return np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)


def test_attend_step_batch32_prefix16k_sampled():
    dev = torch.device("cuda")
    L = 16384
    lens = _lens()
    ctx = [L + n for n in lens]
    st = _starts(ctx)
    T = int(sum(ctx))
    print(f"attend B=32 L={L}: {T} context tokens per kv head", flush=True)
    q = synth.device_normal((32, Hq, d), 9001, dev)
    Kc = synth.device_normal((Hkv, T, d), 9002, dev)
    Vc = synth.device_normal((Hkv, T, d), 9003, dev)
    ctx_start = torch.tensor(st, dtype=torch.int32).to(dev)
    ctx_len = torch.tensor(ctx, dtype=torch.int32).to(dev)
    scale = synth.softmax_scale(d)
    out, lse = api.attend_step(q, Kc, Vc, ctx_start, ctx_len, max(ctx), scale)
    torch.cuda.synchronize()
    out, lse = host(out), host(lse)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    r = np.random.default_rng(9004)
    pairs = {(int(np.argmax(ctx)), h) for h in range(Hq)} | {(int(np.argmin(ctx)), h) for h in range(Hq)}
    pairs |= {(int(b), int(h)) for b, h in zip(r.integers(0, 32, 32), r.integers(0, Hq, 32))}
    q64 = widen(host(q))
    by_seg = {}
    for b, h in sorted(pairs):
        by_seg.setdefault((b, h // G), []).append(h)
    ref, ref_lse, got, got_lse = [], [], [], []
    for (b, g), heads in by_seg.items():
        s, n = int(st[b]), ctx[b]
        Kb = widen(host(Kc[g, s:s + n]))
        Vb = widen(host(Vc[g, s:s + n]))
        for h in heads:
            a_, l_ = O.state(q64[b, h], Kb, Vb, scale)
            ref.append(a_), ref_lse.append(l_), got.append(out[b, h]), got_lse.append(lse[b, h])
    print(f"  {len(ref)} sampled states checked", flush=True)
    assert_states_close(np.array(got), np.array(got_lse), np.array(ref), np.array(ref_lse))


def test_decode_batch32_k16384_two_groups():
    dev = torch.device("cuda")
    K = 16384
    lens = _lens()
    st = _starts(lens)
    n_loc = int(sum(lens))
    print(f"decode B=32 K={K}: {n_loc} local tokens per kv head", flush=True)
    q = synth.device_normal((32, Hq, d), 9101, dev)
    C = synth.device_normal((Hq, K, d), 9102, dev)
    Abar = synth.device_normal((Hq, K, d), 9103, dev, torch.float32)
    g_lse = torch.Generator(device=dev)
    g_lse.manual_seed(9104)
    LSEbar = torch.rand((Hq, K), generator=g_lse, device=dev) * 7.0 + 5.0
    Kl = synth.device_normal((Hkv, n_loc, d), 9105, dev)
    Vl = synth.device_normal((Hkv, n_loc, d), 9106, dev)
    kv_start = torch.tensor(st, dtype=torch.int32).to(dev)
    kv_len = torch.tensor(lens, dtype=torch.int32).to(dev)
    scale = synth.softmax_scale(d)
    cinv = api.centroid_inv_norms(C)
    out, lse, idx = api.decode_step(q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len,
                                    max(lens), scale)
    torch.cuda.synchronize()
    out, lse, idx = host(out), host(lse), host(idx)
    groups = (0, Hkv - 1)
    heads = [g * G + j for g in groups for j in range(G)]
    q64 = widen(host(q))[:, heads]
    flips = 0
    for i, h in enumerate(heads):
        flips += check_indices(idx[:, h], q64[:, i], widen(host(C[h])))
    ks, vs = [], []
    Ksel = widen(host(Kl[list(groups)]))
    Vsel = widen(host(Vl[list(groups)]))
    for s, n in zip(st, lens):
        ks.append(Ksel[:, s:s + n])
        vs.append(Vsel[:, s:s + n])
    ref, ref_lse = O.decode_with_idx(q64, idx[:, heads], widen(host(Abar[heads])),
                                     widen(host(LSEbar[heads])), ks, vs, scale)
    print(f"  {len(heads)} heads x 32 sequences, {flips} accepted near-tie flips", flush=True)
    assert_states_close(out[:, heads], lse[:, heads], ref, ref_lse)
    assert flips <= 3
