"""GPU checks of the streamed prefix-state build (asm_build_states_streamed):
the prefix sits in host memory and is copied chunk by chunk while the
previous chunk is encoded.  It must equal the device-resident
asm_build_states with the same chunk bit for bit, and the oracle's chunked
states within the usual tolerances."""
import numpy as np
import pytest
import torch

from attention_state_memory_amd import api, synth
from oracle import asm_oracle as O
from tests.helpers import assert_states_close, dev, host, widen

pytestmark = pytest.mark.gpu


def _case(seed, dtype, Hq, Hkv, N, L, d):
    r = np.random.default_rng([210, seed])
    if dtype == "bf16":
        mk = lambda shape: synth.to_bf16_bits(r.standard_normal(shape, dtype=np.float32))
    else:
        mk = lambda shape: r.standard_normal(shape, dtype=np.float32)
    return mk((Hq, N, d)), mk((Hkv, L, d)), mk((Hkv, L, d))


def _host_tensor(x, pinned=True):
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16) \
        if x.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(x))
    return t.pin_memory() if pinned else t.clone()


CASES = [
    # (seed, dtype, Hq, Hkv, N, L, chunk, d)
    (1, "bf16", 8, 2, 300, 1000, 256, 128),   # ragged last chunk (232 tokens)
    (2, "bf16", 4, 4, 70, 513, 128, 64),      # one-token last chunk, G = 1
    (3, "bf16", 8, 1, 40, 100, 300, 128),     # a single partial chunk, G = 8
    (4, "f32", 3, 1, 17, 90, 32, 48),         # VALU path
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_streamed_equals_resident_and_oracle(case):
    seed, dtype, Hq, Hkv, N, L, chunk, d = case
    Q, Kp, Vp = _case(seed, dtype, Hq, Hkv, N, L, d)
    scale = synth.softmax_scale(d)
    print(f"streamed build case {case}", flush=True)
    A_s, L_s = api.build_states_streamed(dev(Q), _host_tensor(Kp), _host_tensor(Vp), chunk, scale)
    A_r, L_r, _, _ = api.build_states(dev(Q), dev(Kp), dev(Vp), chunk, scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(A_s), host(A_r))
    np.testing.assert_array_equal(host(L_s), host(L_r))
    _, _, A_ref, L_ref = O.build_states(widen(Q), widen(Kp), widen(Vp), chunk, scale)
    assert_states_close(host(A_s), host(L_s), A_ref, L_ref)


def test_streamed_accumulates_pageable_and_one_stream():
    """A resident first part then a streamed second part (accumulate=1),
    from pageable memory with copies on the compute stream itself, equals
    one resident call over the whole prefix."""
    Hq, Hkv, N, d, chunk = 8, 2, 96, 128, 128
    Q, Kp, Vp = _case(5, "bf16", Hq, Hkv, N, 128 + 400, d)
    scale = synth.softmax_scale(d)
    A, LSE, _, _ = api.build_states(dev(Q), dev(Kp[:, :128].copy()), dev(Vp[:, :128].copy()), chunk,
                                    scale)
    cur = torch.cuda.current_stream()
    A, LSE = api.build_states_streamed(dev(Q), _host_tensor(Kp[:, 128:], pinned=False),
                                       _host_tensor(Vp[:, 128:], pinned=False), chunk, scale,
                                       A=A, LSE=LSE, accumulate=True, copy_stream=cur)
    A_r, L_r, _, _ = api.build_states(dev(Q), dev(Kp), dev(Vp), chunk, scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(A), host(A_r))
    np.testing.assert_array_equal(host(LSE), host(L_r))


def test_streamed_empty_prefix_and_workspace_reuse():
    Hq, Hkv, N, d = 4, 2, 20, 64
    Q, Kp, Vp = _case(6, "bf16", Hq, Hkv, N, 300, d)
    scale = synth.softmax_scale(d)
    empty = np.zeros((Hkv, 0, d), np.uint16)
    A0, L0 = api.build_states_streamed(dev(Q), _host_tensor(empty), _host_tensor(empty), 64, scale)
    torch.cuda.synchronize()
    assert np.all(np.isneginf(host(L0))) and np.all(host(A0) == 0)
    # one workspace for two calls in a row with different prefixes
    ws = torch.zeros(int(api.lib().asm_build_states_streamed_ws(api.BF16, Hq, Hkv, N, d, 64)),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for L in (300, 130):
        A, LSE = api.build_states_streamed(dev(Q), _host_tensor(Kp[:, :L]), _host_tensor(Vp[:, :L]),
                                           64, scale, workspace=ws)
        A_r, L_r, _, _ = api.build_states(dev(Q), dev(Kp[:, :L].copy()), dev(Vp[:, :L].copy()), 64,
                                          scale)
        outs.append((A, LSE, A_r, L_r))
    torch.cuda.synchronize()
    for A, LSE, A_r, L_r in outs:
        np.testing.assert_array_equal(host(A), host(A_r))
        np.testing.assert_array_equal(host(LSE), host(L_r))
