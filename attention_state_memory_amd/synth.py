"""Seeded synthetic inputs for attention-state memory workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  The same arrays feed the HIP library (after a copy to the
device) and the CPU oracle (after widening to float64), so both see identical
bits.  Values are drawn in float32 with numpy's PCG64 generator seeded by
``[workload id, replica]``, in the order each function lists; bf16 tensors
are the float32 draws rounded by torch's float32 -> bfloat16 conversion and
are returned as uint16 bit patterns.

Workloads (shapes follow LLaMA-3.1-8B attention heads: 32 query heads, 8 kv
heads, head dim 128, the host model the pages evaluate on):

* ``tiny``: 1 head, d=64, float32; 256-token prefix; 512 calibration queries
  from a 16-centre Gaussian mixture (sigma 0.3); 4 decode queries from the
  same mixture against a 32-token local KV.
* ``layer_decode``: one decode step of one layer, batch 1, K=1024 centroids
  per query head, 2048 local tokens; layer l uses seed [2, l].
* ``batched_decode``: K=8192, batch 32, local lengths uniform in
  [512, 4096], KV packed head-major [Hkv, sum(n_b), d].
* ``prefix_states``: a 16384-token prefix (4 chunks of 4096) and 4096
  calibration queries per head from per-head 64-centre mixtures.
* ``memory_build``: 65536 fresh calibration queries per head from the same
  mixtures as ``prefix_states``, K=8192, 10 Lloyd iterations.
"""
from __future__ import annotations

import numpy as np
import torch


def to_bf16_bits(x) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), rounded by torch's
    float32 -> bfloat16 conversion (nearest, ties to even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_float(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def softmax_scale(d: int) -> float:
    """The attention scale both sides use: float32(1/sqrt(d)) as a Python
    float (exactly representable in float32)."""
    return float(np.float32(1.0 / np.sqrt(np.float32(d))))


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _mixture(rng, centres, n):
    """n draws from an equal-weight mixture of N(centre, 0.3^2 I)."""
    comp = rng.integers(0, centres.shape[0], n)
    noise = _normal(rng, (n, centres.shape[1]))
    return (centres[comp] + np.float32(0.3) * noise).astype(np.float32)


def _store(x, dtype):
    return to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


# ---------------------------------------------------------------------------
# tiny end-to-end workload (float32, one head)
# ---------------------------------------------------------------------------

def tiny(replica: int = 0) -> dict:
    """Draw order: prefix K, prefix V, 16 centres, 512 calibration queries
    (components then noise), 4 decode queries (components then noise), local
    K, local V."""
    rng = np.random.default_rng([1, replica])
    d = 64
    Kp = _normal(rng, (1, 256, d))
    Vp = _normal(rng, (1, 256, d))
    centres = _normal(rng, (16, d))
    X = _mixture(rng, centres, 512)[None]
    q = _mixture(rng, centres, 4)[:, None, :]
    Kl = _normal(rng, (1, 32, d))
    Vl = _normal(rng, (1, 32, d))
    return dict(dtype="f32", d=d, Hq=1, Hkv=1, N=512, L=256, chunk=64, K=64, iters=5,
                scale=softmax_scale(d), Kp=Kp, Vp=Vp, X=X, q=q,
                Kl=Kl, Vl=Vl, kv_start=np.zeros(4, np.int32),
                kv_len=np.full(4, 32, np.int32), shared_kv=True)


# ---------------------------------------------------------------------------
# decode-step workloads
# ---------------------------------------------------------------------------

def decode_inputs(seed, B, Hq, Hkv, d, K, kv_lens, dtype="bf16",
                  lse_range=(5.0, 12.0)) -> dict:
    """A generic decode step.  Draw order: q [B,Hq,d], C [Hq,K,d],
    A_bar [Hq,K,d] (float32), LSE_bar [Hq,K] uniform in lse_range, local K
    then V packed head-major [Hkv, sum(kv_lens), d].  kv_lens is given."""
    rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    total = int(kv_lens.sum())
    q = _normal(rng, (B, Hq, d))
    C = _normal(rng, (Hq, K, d))
    Abar = _normal(rng, (Hq, K, d))
    LSEbar = rng.uniform(lse_range[0], lse_range[1], (Hq, K)).astype(np.float32)
    Kl = _normal(rng, (Hkv, total, d))
    Vl = _normal(rng, (Hkv, total, d))
    kv_start = np.concatenate([[0], np.cumsum(kv_lens)[:-1]]).astype(np.int32)
    return dict(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, d=d, K=K, scale=softmax_scale(d),
                q=_store(q, dtype), C=_store(C, dtype), Abar=Abar, LSEbar=LSEbar,
                Kl=_store(Kl, dtype), Vl=_store(Vl, dtype),
                kv_start=kv_start, kv_len=kv_lens.astype(np.int32),
                kv_head_stride=total * d, kv_tok_stride=d)


def layer_decode(layer: int) -> dict:
    """Batch-1 decode of one LLaMA-3.1-8B-shaped layer: K=1024, 2048 local
    tokens, seed [2, layer]."""
    return decode_inputs([2, layer], B=1, Hq=32, Hkv=8, d=128, K=1024, kv_lens=[2048])


def batched_decode(replica: int) -> dict:
    """Batch-32 decode at K=8192 with ragged local lengths.  Draw order: the
    32 lengths (uniform integers in [512, 4096]) from seed [3, replica], then
    the tensors of `decode_inputs` from seed [3, replica, 1]."""
    rng = np.random.default_rng([3, replica])
    kv_lens = rng.integers(512, 4097, 32)
    return decode_inputs([3, replica, 1], B=32, Hq=32, Hkv=8, d=128, K=8192,
                         kv_lens=kv_lens)


def attend_inputs(seed, B, Hq, Hkv, d, L, kv_lens, dtype="bf16") -> dict:
    """A decode step over a fixed L-token prefix plus ragged local contexts,
    laid out two ways: the local tokens alone (packed head-major as in
    `decode_inputs`) and every sequence's full context, its own copy of the
    prefix followed by its local tokens (packed head-major [Hkv, sum(L +
    n_b), d]).  Draw order: q [B,Hq,d], prefix K then V [Hkv,L,d], local K
    then V [Hkv,sum(n_b),d]."""
    rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    total = int(kv_lens.sum())
    q = _normal(rng, (B, Hq, d))
    Kp = _normal(rng, (Hkv, L, d))
    Vp = _normal(rng, (Hkv, L, d))
    Kl = _normal(rng, (Hkv, total, d))
    Vl = _normal(rng, (Hkv, total, d))
    kv_start = np.concatenate([[0], np.cumsum(kv_lens)[:-1]]).astype(np.int64)
    ctx_len = kv_lens + L
    ctx_start = np.concatenate([[0], np.cumsum(ctx_len)[:-1]]).astype(np.int64)
    Kc = np.empty((Hkv, int(ctx_len.sum()), d), np.float32)
    Vc = np.empty_like(Kc)
    for b in range(B):
        c0, l0, n = ctx_start[b], kv_start[b], kv_lens[b]
        Kc[:, c0:c0 + L], Vc[:, c0:c0 + L] = Kp, Vp
        Kc[:, c0 + L:c0 + L + n], Vc[:, c0 + L:c0 + L + n] = Kl[:, l0:l0 + n], Vl[:, l0:l0 + n]
    return dict(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, d=d, L=L, scale=softmax_scale(d),
                q=_store(q, dtype), Kp=_store(Kp, dtype), Vp=_store(Vp, dtype),
                Kl=_store(Kl, dtype), Vl=_store(Vl, dtype),
                kv_start=kv_start.astype(np.int32), kv_len=kv_lens.astype(np.int32),
                Kc=_store(Kc, dtype), Vc=_store(Vc, dtype),
                ctx_start=ctx_start.astype(np.int32), ctx_len=ctx_len.astype(np.int32))


# ---------------------------------------------------------------------------
# build workloads
# ---------------------------------------------------------------------------

def _prefix_and_centres(Hq=32, Hkv=8, d=128, L=16384, M=64):
    """Seed [4, 0]; draw order: prefix K [Hkv,L,d], prefix V, per-head
    mixture centres [Hq, M, d]."""
    rng = np.random.default_rng([4, 0])
    Kp = _normal(rng, (Hkv, L, d))
    Vp = _normal(rng, (Hkv, L, d))
    centres = _normal(rng, (Hq, M, d))
    return rng, Kp, Vp, centres


def prefix_states(N: int = 4096) -> dict:
    """Prefix-state collection: 16384-token prefix in 4 chunks of 4096, N
    calibration queries per head (seed [4, 0], drawn after the prefix and
    centres, head by head)."""
    rng, Kp, Vp, centres = _prefix_and_centres()
    Q = np.stack([_mixture(rng, centres[h], N) for h in range(centres.shape[0])])
    return dict(dtype="bf16", Hq=32, Hkv=8, d=128, N=N, L=16384, chunk=4096,
                scale=softmax_scale(128), Q=to_bf16_bits(Q),
                Kp=to_bf16_bits(Kp), Vp=to_bf16_bits(Vp))


def memory_build(N: int = 65536, K: int = 8192, iters: int = 10) -> dict:
    """Memory build: the prefix and centres of `prefix_states`, and N fresh
    calibration queries per head from seed [5, 0], head by head."""
    _, Kp, Vp, centres = _prefix_and_centres()
    rng = np.random.default_rng([5, 0])
    X = np.stack([_mixture(rng, centres[h], N) for h in range(centres.shape[0])])
    return dict(dtype="bf16", Hq=32, Hkv=8, d=128, N=N, L=16384, chunk=4096, K=K,
                iters=iters, scale=softmax_scale(128), X=to_bf16_bits(X),
                Kp=to_bf16_bits(Kp), Vp=to_bf16_bits(Vp))


def mixture_queries(seed, H, N, d, M, sigma=0.3, dtype="bf16") -> np.ndarray:
    """Small clusterable query sets for tests: per head, M centres ~ N(0, I)
    then N mixture draws (sigma given)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(H):
        centres = _normal(rng, (M, d))
        comp = rng.integers(0, M, N)
        out.append(centres[comp] + np.float32(sigma) * _normal(rng, (N, d)))
    X = np.stack(out).astype(np.float32)
    return _store(X, dtype)


def device_normal(shape, seed: int, device, dtype=torch.bfloat16):
    """N(0, 1) draws made on the device by torch's seeded generator (float32,
    then rounded to `dtype`): for inputs of GB size, where drawing on the host
    and copying would dominate.  The same seed gives the same bits on every
    call, so a test can copy any slice back for the oracle."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32).to(dtype)
