"""GPU check of asm_decode_step_begin / asm_decode_step_finish, the decode
step split into its two launches ([TS] Fase de Inferencia Online:
Recuperación with the local attention, then Fusión).  Together they must give
what asm_decode_step gives on the same inputs: the same indices, and `out`,
`out_lse` within the run-to-run spread of the step itself (the waves of a
pair split their work units at run time; see the no-allocation test for the
bound).  The first launch must leave the outputs untouched."""
import pytest
import torch

from attention_state_memory_amd import api, synth
from tests.helpers import dev

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-4
LSE_TOL = 1e-5


def _operands(inp):
    q, C = dev(inp["q"]), dev(inp["C"])
    return dict(q=q, C=C, cinv=api.centroid_inv_norms(C), Abar=dev(inp["Abar"]),
                LSEbar=dev(inp["LSEbar"]), Kl=dev(inp["Kl"]), Vl=dev(inp["Vl"]),
                kv_start=dev(inp["kv_start"]), kv_len=dev(inp["kv_len"]),
                max_kv_len=max(1, int(inp["kv_len"].max())), scale=inp["scale"])


def _args(t):
    return (t["q"], t["C"], t["cinv"], t["Abar"], t["LSEbar"], t["Kl"], t["Vl"], t["kv_start"],
            t["kv_len"], t["max_kv_len"], t["scale"])


STEPS = [
    # the batched step: 32 sequences, K=8192, lengths uniform in [512, 4096]
    ("batched K8192", lambda: synth.batched_decode(0)),
    # batch 1, K=1024, 2048 local tokens: a wave for every work unit
    ("batch-1 K1024", lambda: synth.decode_inputs([250, 1], B=1, Hq=32, Hkv=8, d=128, K=1024,
                                                  kv_lens=[2048])),
    # batch 1, K=8192: few tiles against many scoring units
    ("batch-1 K8192", lambda: synth.decode_inputs([250, 2], B=1, Hq=32, Hkv=8, d=128, K=8192,
                                                  kv_lens=[2048])),
    # ragged with an empty sequence, GQA group 8, d=64
    ("ragged G8 d64", lambda: synth.decode_inputs([250, 3], B=3, Hq=16, Hkv=2, d=64, K=700,
                                                  kv_lens=[0, 33, 1500])),
    # no grouping (G=1)
    ("G1", lambda: synth.decode_inputs([250, 4], B=5, Hq=4, Hkv=4, d=128, K=256,
                                       kv_lens=[1, 31, 32, 65, 300])),
]


@pytest.mark.parametrize("name,make", STEPS, ids=[s[0] for s in STEPS])
def test_begin_then_finish_equals_the_step(name, make):
    print(f"two-launch step: {name}", flush=True)
    t = _operands(make())
    B, Hq, d = t["q"].shape
    w_out, w_lse, w_idx = api.decode_step(*_args(t))
    ws = torch.zeros(api.decode_step_ws(api.BF16, B, Hq, t["Kl"].shape[0], d, t["C"].shape[1],
                                        t["max_kv_len"]), dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, d), 7.0, device="cuda")
    lse = torch.full((B, Hq), 7.0, device="cuda")
    idx = torch.full((B, Hq), -7, dtype=torch.int32, device="cuda")
    api.decode_step_begin(*_args(t), out=out, out_lse=lse, out_idx=idx, workspace=ws)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all()) and bool((idx == -7).all()), \
        "the first launch wrote an output"
    api.decode_step_finish(*_args(t), out=out, out_lse=lse, out_idx=idx, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(idx, w_idx), f"{name}: out_idx differs"
    both = torch.isnan(w_out) | torch.isnan(out)
    assert torch.equal(torch.isnan(w_out), torch.isnan(out))
    d_out = float((out - w_out).masked_fill(both, 0).abs().max())
    fin = torch.isfinite(w_lse)
    assert torch.equal(fin, torch.isfinite(lse))
    d_lse = float((lse - w_lse)[fin].abs().max()) if bool(fin.any()) else 0.0
    print(f"{name}: max |d out| {d_out:.3g}, max |d lse| {d_lse:.3g}", flush=True)
    assert d_out <= OUT_TOL and d_lse <= LSE_TOL


def test_finish_repeats_and_interleaves():
    """The workspace holds the first launch's results until the next first
    launch: another step on its own workspace in between changes nothing, and
    a second finish gives the same outputs again."""
    a = _operands(synth.decode_inputs([251, 1], B=4, Hq=32, Hkv=8, d=128, K=2048,
                                      kv_lens=[900, 0, 2048, 64]))
    b = _operands(synth.decode_inputs([251, 2], B=2, Hq=32, Hkv=8, d=128, K=512,
                                      kv_lens=[100, 3000]))
    B, Hq, d = a["q"].shape
    ws = torch.zeros(api.decode_step_ws(api.BF16, B, Hq, 8, d, 2048, a["max_kv_len"]),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, d), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    idx = torch.empty((B, Hq), dtype=torch.int32, device="cuda")
    api.decode_step_begin(*_args(a), out=out, out_lse=lse, out_idx=idx, workspace=ws)
    api.decode_step(*_args(b))
    api.decode_step_finish(*_args(a), out=out, out_lse=lse, out_idx=idx, workspace=ws)
    first = (out.clone(), lse.clone(), idx.clone())
    api.decode_step_finish(*_args(a), out=out, out_lse=lse, out_idx=idx, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first[2], idx)
    assert torch.equal(torch.nan_to_num(first[0], nan=123.0), torch.nan_to_num(out, nan=123.0))
    assert torch.equal(torch.nan_to_num(first[1], nan=123.0), torch.nan_to_num(lse, nan=123.0))
    w_out, w_lse, w_idx = api.decode_step(*_args(a))
    assert torch.equal(idx, w_idx)
    assert float((out - w_out).abs().max()) <= OUT_TOL
