"""GPU check of asm_decode_step_noalloc, the decode entry point for callers
that cannot allocate device memory.  It runs the kernels of asm_decode_step
with the library's fixed per-GPU scratch in place of a workspace, so its
outputs must match asm_decode_step's: on consecutive calls that share the
scratch (the second a smaller step, the third on the float32 path), and
from a captured HIP graph replayed several times with other calls on the
scratch in between.

Indices must be equal.  The two waves of a pair split their tiles at run
time, so on steps with more work units than waves the partial states (and
the reference each softmax is taken against) differ from run to run; the
probabilities enter the value product split into two bf16 parts (about
2^-17 relative), so two runs may differ by up to 2^-17 * max|V| in `out`
(under 4e-5 here, |V| < 5) and by float32 rounding of the sums in
`out_lse`.  The bounds below hold that with margin; everything else is
exact."""
import pytest
import torch

from attention_state_memory_amd import api, synth
from tests.helpers import dev

pytestmark = pytest.mark.gpu


def _operands(inp):
    q, C = dev(inp["q"]), dev(inp["C"])
    return dict(q=q, C=C, cinv=api.centroid_inv_norms(C), Abar=dev(inp["Abar"]),
                LSEbar=dev(inp["LSEbar"]), Kl=dev(inp["Kl"]), Vl=dev(inp["Vl"]),
                kv_start=dev(inp["kv_start"]), kv_len=dev(inp["kv_len"]),
                max_kv_len=max(1, int(inp["kv_len"].max())), scale=inp["scale"])


def _args(t):
    return (t["q"], t["C"], t["cinv"], t["Abar"], t["LSEbar"], t["Kl"], t["Vl"], t["kv_start"],
            t["kv_len"], t["max_kv_len"], t["scale"])


def _outputs(t):
    B, Hq, d = t["q"].shape
    return (torch.full((B, Hq, d), 7.0, device="cuda"), torch.full((B, Hq), 7.0, device="cuda"),
            torch.full((B, Hq), -7, dtype=torch.int32, device="cuda"))


def _with_workspace(t):
    out, lse, idx = api.decode_step(*_args(t))
    return out, lse, idx


def _noalloc(t):
    out, lse, idx = _outputs(t)
    api.decode_step_noalloc(*_args(t), out=out, out_lse=lse, out_idx=idx)
    return out, lse, idx


OUT_TOL = 1e-4
LSE_TOL = 1e-5


def _assert_identical(got, want, what):
    out, lse, idx = got
    w_out, w_lse, w_idx = want
    assert torch.equal(idx, w_idx), f"{what}: out_idx differs"
    d_out = float((out - w_out).abs().max())
    d_lse = float((lse - w_lse).abs().max())
    print(f"{what}: max |d out| {d_out:.3g}, max |d lse| {d_lse:.3g}", flush=True)
    assert d_out <= OUT_TOL, f"{what}: out differs by {d_out}"
    assert d_lse <= LSE_TOL, f"{what}: out_lse differs by {d_lse}"


STEPS = [
    # the batched step (32 sequences, K=8192, lengths uniform in [512, 4096])
    ("batched K8192", lambda: synth.batched_decode(0)),
    # one sequence at K=8192: scoring dominates, so the direct layout runs
    # in several waves of one-wave workgroups
    ("batch-1 K8192", lambda: synth.decode_inputs([240, 3], B=1, Hq=32, Hkv=8, d=128, K=8192,
                                                  kv_lens=[2048])),
    # smaller: an empty and a ragged sequence, K=512
    ("small ragged", lambda: synth.decode_inputs([240, 1], B=3, Hq=32, Hkv=8, d=128, K=512,
                                                 kv_lens=[0, 70, 513])),
    # float32 tensors take the VALU kernels, which use the scratch too
    ("float32", lambda: synth.decode_inputs([240, 2], B=2, Hq=8, Hkv=2, d=64, K=300,
                                            kv_lens=[40, 257], dtype="f32")),
]


def test_noalloc_matches_decode_step_on_consecutive_calls():
    for name, make in STEPS:
        print(f"noalloc step: {name}", flush=True)
        t = _operands(make())
        want = _with_workspace(t)
        got = _noalloc(t)
        torch.cuda.synchronize()
        _assert_identical(got, want, name)
        # the same step again: the scratch keeps the last call's contents,
        # which must not matter
        got2 = _noalloc(t)
        torch.cuda.synchronize()
        _assert_identical(got2, want, name + " (repeat)")


def test_noalloc_in_a_captured_graph():
    small = _operands(synth.decode_inputs([241, 1], B=4, Hq=32, Hkv=8, d=128, K=1024,
                                          kv_lens=[2048, 5, 0, 777]))
    other = _operands(synth.decode_inputs([241, 2], B=2, Hq=32, Hkv=8, d=128, K=2048,
                                          kv_lens=[300, 4000]))
    want = _with_workspace(small)
    want_other = _with_workspace(other)
    # the first call on a device, which looks up the scratch address, runs
    # outside capture
    _assert_identical(_noalloc(small), want, "eager call before capture")
    torch.cuda.synchronize()
    out, lse, idx = _outputs(small)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        api.decode_step_noalloc(*_args(small), out=out, out_lse=lse, out_idx=idx)
    for rep in range(3):
        print(f"noalloc graph replay {rep}", flush=True)
        for x in (out, lse):
            x.fill_(7.0)
        idx.fill_(-7)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        _assert_identical((out, lse, idx), want, f"replay {rep}")
        # an eager call in between overwrites the shared scratch
        _assert_identical(_noalloc(other), want_other, f"eager call after replay {rep}")
        torch.cuda.synchronize()


def test_noalloc_rejects_a_step_larger_than_its_scratch():
    """2048 sequences at K=8192 need 67 MB of argmax keys alone: refused
    before any launch, with the scratch size in the message."""
    t = _operands(synth.decode_inputs([242, 1], B=1, Hq=32, Hkv=8, d=128, K=64, kv_lens=[64]))
    B, K = 2048, 8192
    assert api.decode_step_ws(api.BF16, B, 32, 8, 128, K, 64) > (16 << 20)
    q = torch.empty((B, 32, 128), dtype=torch.bfloat16, device="cuda")
    C = torch.empty((32, K, 128), dtype=torch.bfloat16, device="cuda")
    cinv = torch.empty((32, K), device="cuda")
    Abar = torch.empty((32, K, 128), device="cuda")
    kv_start = torch.zeros(B, dtype=torch.int32, device="cuda")
    kv_len = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, 32, 128), device="cuda")
    with pytest.raises(api.AsmError, match="holds 16777216"):
        api.decode_step_noalloc(q, C, cinv, Abar, cinv, t["Kl"], t["Vl"], kv_start, kv_len, 64,
                                t["scale"], out=out)
