"""Benchmark: attention-state-memory decode at K=8192 on one MI355X.

Workload (synthetic, seeded): LLaMA-3.1-8B attention-head shapes (32 query
heads, 8 kv heads, d=128), K=8192 memory entries per query head, batch 32
with ragged local contexts uniform in [512, 4096]; bf16 q/C/K/V, float32
states.  A step is one asm_decode_step call -- centroid scoring, argmax,
state gather, split-K local attention and the online-softmax merge -- over
one batch.  R replicas of the inputs are resident in HBM and rotated so the
256 MB last-level cache does not hold a step's working set.

Prints one JSON line: whole-job head-queries/s, ms/step, the roofline of the
fused decode kernel (algorithmic bytes / kernel time vs 8 TB/s), and the fp64
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COPY_CALIBRATION_ELEMS = 64 << 20  # float32 elements: 256 MiB read and 256 MiB written


def copy_calibration(torch, dev):
    """A plain streaming copy of known size (elementwise negation, float32),
    whose FETCH_SIZE / WRITE_SIZE readings calibrate the byte counters."""
    src = torch.ones(COPY_CALIBRATION_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def measured_traffic(profile_name: str, sources) -> dict:
    """HBM bytes per step from the committed counter summary, if it was taken
    on the kernel sources as they are now (else None: the kernel changed)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    try:
        out = {"bytes_per_step": float(fields["traffic_bytes_per_step"]),
               "profile": f"profiles/{profile_name}"}
        if "traffic_bytes_main" in fields:
            out["bytes_main"] = float(fields["traffic_bytes_main"])
        return out
    except (KeyError, ValueError):
        return None


# the decode kernels' sources: a change to any of them voids the counters
DECODE_SOURCES = ("attention_state_memory_amd/csrc/decode_fast.hip",
                  "attention_state_memory_amd/csrc/common.hpp",
                  "attention_state_memory_amd/csrc/kernels.hpp",
                  "attention_state_memory_amd/csrc/hier_lookup.hpp")


def algorithmic_bytes_split(inp):
    """Bytes a decode step must move, split by the launch that moves them:
    the main grid reads the centroid table and its inverse norms, the local
    KV of every sequence, the queries and the lengths; the merge gathers the
    winning entries' states and writes the outputs (out, lse, idx).  The
    prefix is never read.  Returns (main, merge)."""
    B, Hq, Hkv, d, K = inp["B"], inp["Hq"], inp["Hkv"], inp["d"], inp["K"]
    e = 2 if inp["dtype"] == "bf16" else 4
    table = Hq * K * d * e + Hq * K * 4
    gathered = B * Hq * (d * 4 + 4)
    kv = int(np.sum(inp["kv_len"])) * Hkv * d * e * 2
    q = B * Hq * d * e
    outs = B * Hq * (d * 4 + 4 + 4)
    lens = B * 8
    return table + kv + q + lens, gathered + outs


def algorithmic_bytes(inp) -> int:
    """All the bytes a decode step must move (both launches)."""
    return sum(algorithmic_bytes_split(inp))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--replicas", type=int, default=4)
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="wall-clock budget of the CPU oracle baseline (0 disables it)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one plain device copy (256 MiB read, 256 MiB written) before any "
                        "workload, as the reference kernel for HBM byte counters")
    p.add_argument("--queries", type=int, default=4096,
                   help="prefix_states / prefix_states_streamed: calibration queries per head "
                        "(65536 is the memory-build scale)")
    p.add_argument("--K", type=int, default=8192, help="layer_decode_hier: entries per head")
    p.add_argument("--supers", type=int, default=128, help="layer_decode_hier: super-centroids S")
    p.add_argument("--probes", type=int, default=8, help="layer_decode_hier: probes p")
    p.add_argument("--layers", type=int, default=32, help="layer_decode_hier: layers in the graph")
    p.add_argument("--workload", default="batched_decode",
                   choices=("batched_decode", "batched_decode_whitened", "layer_decode",
                            "layer_decode_hier", "prefix_states", "prefix_states_streamed",
                            "memory_build", "attention_compare"),
                   help="batched_decode (the headline metric) or one of the offline build "
                        "workloads, reported on their MFMA rooflines")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                                   "no multi-GPU mode"}))
        sys.exit(2)
    if args.copy_calibration:
        import torch
        torch.cuda.set_device(torch.device("cuda:0"))
        copy_calibration(torch, torch.device("cuda:0"))
    if args.workload == "layer_decode":
        run_layers(args)
        return
    if args.workload == "layer_decode_hier":
        run_layers_hier(args)
        return
    if args.workload == "attention_compare":
        run_compare(args)
        return
    if args.workload == "batched_decode_whitened":
        run_whitened(args)
        return
    if args.workload != "batched_decode":
        run_build(args)
        return
    import torch
    from attention_state_memory_amd import api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    reps, host_inputs = [], []
    for r in range(args.replicas):
        inp = synth.batched_decode(r)
        host_inputs.append(inp)
        t = {k: to_dev(inp[k]) for k in ("q", "C", "Abar", "LSEbar", "Kl", "Vl", "kv_start", "kv_len")}
        t["cinv"] = api.centroid_inv_norms(t["C"])
        t["max_kv_len"] = int(np.max(inp["kv_len"]))
        reps.append(t)
        print(f"replica {r} resident", file=sys.stderr, flush=True)
    inp0 = host_inputs[0]
    B, Hq, Hkv, d, K = inp0["B"], inp0["Hq"], inp0["Hkv"], inp0["d"], inp0["K"]
    max_kv = 4096
    code = api.BF16
    ws_bytes = api.decode_step_ws(code, B, Hq, Hkv, d, K, max_kv)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    out_lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    out_idx = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    L = api.lib()
    P = ctypes.c_void_p

    def make_call(t, stream, entry="asm_decode_step"):
        cap = t["Kl"].shape[1]
        argv = (code, B, Hq, Hkv, d, K, ctypes.c_float(inp0["scale"]), P(t["q"].data_ptr()),
                P(t["C"].data_ptr()), P(t["cinv"].data_ptr()), P(t["Abar"].data_ptr()),
                P(t["LSEbar"].data_ptr()), P(t["Kl"].data_ptr()), P(t["Vl"].data_ptr()),
                t["Kl"].stride(0), t["Kl"].stride(1), cap, P(t["kv_start"].data_ptr()),
                P(t["kv_len"].data_ptr()), max_kv, P(out.data_ptr()), P(out_lse.data_ptr()),
                P(out_idx.data_ptr()), P(ws.data_ptr()), ws_bytes, P(stream))
        fn = getattr(L, entry)

        def call():
            st = fn(*argv)
            if st != 0:
                raise RuntimeError(L.asm_last_error().decode())
        return call

    stream = torch.cuda.Stream(dev)
    calls = [make_call(t, stream.cuda_stream) for t in reps]
    R = len(calls)
    steps, warmup = max(1, args.steps), max(0, args.warmup)

    def run_steps(n):
        for i in range(n):
            calls[i % R]()

    graph = warm_graph = None
    if args.no_graph:
        with torch.cuda.stream(stream):
            run_steps(warmup)
        stream.synchronize()
    else:
        # The timed steps are one HIP graph holding exactly `steps` decode
        # calls (replicas in rotation), replayed once; the warmup steps are a
        # graph of their own, so the graph machinery is warm before timing.
        # One replay per timed region keeps graph-launch gaps out of the
        # per-step time.
        if warmup > 0:  # the first warmup step runs eagerly (module load)
            with torch.cuda.stream(stream):
                calls[0]()
            stream.synchronize()
        if warmup > 1:
            warm_graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(warm_graph, stream=stream):
                for i in range(1, warmup):
                    calls[i % R]()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            run_steps(steps)
        if warm_graph is not None:
            with torch.cuda.stream(stream):
                warm_graph.replay()
        stream.synchronize()

    def timed_pass():
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            if graph is None:
                run_steps(steps)
            else:
                graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    ms_total = timed_pass()  # exactly `steps` steps
    ms_step = ms_total / steps
    # spread: further passes after the timed one (not part of `value`)
    extra = [timed_pass() / steps for _ in range(4)]
    per_step = np.array([ms_step] + extra)
    queries = B * Hq
    qps = queries / (ms_step * 1e-3)
    rep_split = [algorithmic_bytes_split(h) for h in host_inputs]
    main_bytes = float(np.mean([rep_split[i % R][0] for i in range(steps)]))
    alg_bytes = float(np.mean([sum(rep_split[i % R]) for i in range(steps)]))
    traffic = measured_traffic("decode_batched_K8192_traffic.txt", DECODE_SOURCES)

    # The dominant kernel on its own: the first of the step's two launches
    # (asm_decode_step_begin, decode_fast_main) `steps` times over the same
    # replicas, then the second (asm_decode_step_finish, decode_fast_combine)
    # `steps` times, each as a graph of its own (eagerly with --no-graph)
    # timed by HIP events on the decode stream around its replay.  Either
    # launch may repeat on its own: the first rewrites the workspace, the
    # second only reads it.  No event sits between two kernels, so the mean
    # is the kernel's own duration plus the launch gap inside a graph.
    begins = [make_call(t, stream.cuda_stream, "asm_decode_step_begin") for t in reps]
    finishes = [make_call(t, stream.cuda_stream, "asm_decode_step_finish") for t in reps]

    def phase_ms(fns):
        g = None
        if graph is not None:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    fns[i % R]()
            with torch.cuda.stream(stream):
                g.replay()  # untimed
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            if g is not None:
                g.replay()
            else:
                for i in range(steps):
                    fns[i % R]()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    main_ms = phase_ms(begins)
    merge_ms = phase_ms(finishes)
    achieved = main_bytes / (main_ms * 1e-3) / 1e9
    step_achieved = alg_bytes / (ms_step * 1e-3) / 1e9

    result = {
        "metric": "ASM decode queries/sec (heads x tokens) at K=8192; achieved HBM GB/s vs peak",
        "value": qps,
        "unit": "head-queries/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/C/K/V, fp32 states, lse~U(5,12))",
        "config": {"workload": "batched_decode", "K": K, "batch": B, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": d, "local_len": "U{512..4096}",
                   "replicas": R, "launch": "eager" if graph is None else "hip_graph"},
        "ms_per_step_p10_p50_p90": [float(np.percentile(per_step, q)) for q in (10, 50, 90)],
        "spread_over": "the timed pass and 4 more passes of the same steps",
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic.get("bytes_main") if traffic else None,
                     "kernel": "decode_fast_main (the first of the step's two launches)",
                     "algorithmic_bytes_per_launch": main_bytes,
                     "kernel_us": main_ms * 1e3,
                     "timed": "HIP events on the decode stream around one replay of a graph of "
                              "`steps` asm_decode_step_begin calls (decode_fast_main only)",
                     "merge_kernel_us": merge_ms * 1e3,
                     "step": {"achieved": step_achieved, "frac": step_achieved / HBM_PEAK_GBS,
                              "algorithmic_bytes_per_step": alg_bytes,
                              "traffic": traffic["bytes_per_step"] if traffic else None,
                              "timed": "HIP events around one replay of a graph of exactly "
                                       "`steps` asm_decode_step calls"}},
    }

    # ---- CPU baseline: the fp64 oracle, bounded sample of the same workload
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(inp0, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def run_whitened(args, n_calib=16384):
    """The batched-decode workload with whitening at retrieval: per head a
    transform fit on 16384 calibration queries (64-centre mixture), the
    table whitened once, and every step whitening its queries before the
    lookup.  Timed beside it in the same process: the plain step on the same
    replicas."""
    import torch
    from attention_state_memory_amd import api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    reps, host_inputs = [], []
    fit_ms, rows_ms = [], []
    for r in range(args.replicas):
        inp = synth.batched_decode(r)
        host_inputs.append(inp)
        t = {k: to_dev(inp[k]) for k in ("q", "C", "Abar", "LSEbar", "Kl", "Vl", "kv_start", "kv_len")}
        t["cinv"] = api.centroid_inv_norms(t["C"])
        X = to_dev(synth.mixture_queries([8, r], inp["Hq"], n_calib, inp["d"], M=64))
        ws_fit = torch.zeros(int(api.lib().asm_whiten_fit_ws(api.BF16, inp["Hq"], n_calib, inp["d"])),
                             dtype=torch.uint8, device=dev)
        fit_ms.append(_timed(lambda: api.whiten_fit(X, workspace=ws_fit), 1))
        t["mu"], t["W"], _ = api.whiten_fit(X, workspace=ws_fit)
        t["Cw"] = torch.empty_like(t["C"])
        rows_ms.append(_timed(lambda: api.whiten_rows(t["C"], t["mu"], t["W"], out=t["Cw"]), 1))
        t["cwinv"] = api.centroid_inv_norms(t["Cw"])
        del X, ws_fit
        reps.append(t)
        print(f"replica {r} resident and whitened", file=sys.stderr, flush=True)
    inp0 = host_inputs[0]
    B, Hq, Hkv, d, K = inp0["B"], inp0["Hq"], inp0["Hkv"], inp0["d"], inp0["K"]
    max_kv = 4096
    code = api.BF16
    ws_w = int(api.lib().asm_decode_step_whitened_ws(code, B, Hq, Hkv, d, K, max_kv))
    ws = torch.zeros(ws_w, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    out_lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    out_idx = torch.empty((B, Hq), dtype=torch.int32, device=dev)

    def step_whitened(t):
        api.decode_step_whitened(t["q"], t["mu"], t["W"], t["Cw"], t["cwinv"], t["Abar"],
                                 t["LSEbar"], t["Kl"], t["Vl"], t["kv_start"], t["kv_len"], max_kv,
                                 inp0["scale"], out=out, out_lse=out_lse, out_idx=out_idx,
                                 workspace=ws)

    def step_plain(t):
        api.decode_step(t["q"], t["C"], t["cinv"], t["Abar"], t["LSEbar"], t["Kl"], t["Vl"],
                        t["kv_start"], t["kv_len"], max_kv, inp0["scale"], out=out,
                        out_lse=out_lse, out_idx=out_idx, workspace=ws)

    def graph_ms(step):
        stream = torch.cuda.Stream(dev)
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                step(reps[i % len(reps)])
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for t in reps:
                step(t)
        n = max(1, args.steps // len(reps))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            g.replay()
            e0.record(stream)
            for _ in range(n):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (n * len(reps)), n * len(reps)

    ms_w, steps = graph_ms(step_whitened)
    ms_p, _ = graph_ms(step_plain)
    alg_bytes = float(np.mean([algorithmic_bytes(h) for h in host_inputs]))
    # plus what whitening adds per step: mu and W of every head (float64)
    alg_bytes += Hq * (d + d * d) * 8
    achieved = alg_bytes / (ms_w * 1e-3) / 1e9
    result = {
        "metric": "ASM decode queries/sec (heads x tokens) at K=8192 with whitening at retrieval",
        "value": B * Hq / (ms_w * 1e-3), "unit": "head-queries/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": ms_w, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (batched-decode inputs; whitening fit on 16384 seeded 64-centre "
                "mixture queries per head)",
        "config": {"workload": "batched_decode_whitened", "K": K, "batch": B, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": d, "local_len": "U{512..4096}",
                   "calibration_queries": n_calib, "replicas": len(reps), "launch": "hip_graph"},
        "plain_ms_per_step": ms_p,
        "whitening_overhead_us": (ms_w - ms_p) * 1e3,
        "fit_ms": float(np.mean(fit_ms)),
        "table_whitening_ms": float(np.mean(rows_ms)),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_step": alg_bytes,
                     "timed": "HIP events around graph replays of asm_decode_step_whitened"},
    }
    print(json.dumps(result), flush=True)


def cpu_baseline(inp, budget_s: float) -> dict:
    from threadpoolctl import threadpool_info
    from oracle import asm_oracle as O
    q64 = O.bf16_bits_to_f64(inp["q"])
    C64 = O.bf16_bits_to_f64(inp["C"])
    Ab = inp["Abar"].astype(np.float64)
    Lb = inp["LSEbar"].astype(np.float64)
    Kl = O.bf16_bits_to_f64(inp["Kl"])
    Vl = O.bf16_bits_to_f64(inp["Vl"])
    B = inp["B"]
    ks = [Kl[:, s:s + n] for s, n in zip(inp["kv_start"], inp["kv_len"])]
    vs = [Vl[:, s:s + n] for s, n in zip(inp["kv_start"], inp["kv_len"])]
    # sample: whole decode steps over replica 0 (all 32 sequences x 32 heads),
    # repeated until the wall-clock budget is spent (at least one step)
    t0 = time.perf_counter()
    passes = 0
    while passes == 0 or (time.perf_counter() - t0) < budget_s:
        O.decode(q64, C64, Ab, Lb, ks, vs, inp["scale"])
        passes += 1
    el = time.perf_counter() - t0
    done = passes * B
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    return {"value": done * inp["Hq"] / el, "unit": "head-queries/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{passes} full decode step(s) of replica 0 ({B} sequences x "
                      f"{inp['Hq']} heads, K={inp['K']} scoring + local attention), {el:.1f} s"}


# --------------------------------------------------------------------------
# batch-1 decode through 32 layers (K=1024 per query head, 2048 local tokens)
# --------------------------------------------------------------------------

def run_compare(args):
    """The method against full attention, both as one decode step on the same
    head shapes (32 query heads, 8 kv heads, d=128, bf16):
      full attention  asm_attend_step over each sequence's whole context, its
                      own copy of an L-token prefix followed by its local
                      tokens, L in {4096, 8192, 16384};
      ASM             asm_decode_step with a K-entry memory over the local
                      tokens only: batch 1 at K in {1024, 8192}, batch 32 at
                      K in {1024, 4096, 8192, 16384}.
    Batch 1 (2048 local tokens) and batch 32 (local lengths uniform in
    [512, 4096], the headline's seeded replica 0 lengths).  Every input is
    drawn on the timing stream itself, so no step can start before its
    inputs and workspace exist.  Enough replicas rotate that a step's working
    set is not held by the 256 MB last-level cache.  Each configuration is
    timed as one HIP graph of `steps` calls.  Prints one JSON line with the
    per-step times and the latency ratio full(L) / ASM(K) for every pair."""
    import torch
    from attention_state_memory_amd import api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    Hq, Hkv, d = 32, 8, 128
    scale = synth.softmax_scale(d)
    stream = torch.cuda.Stream(dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    steps = max(4, args.steps)
    asm_K = {1: (1024, 8192), 32: (1024, 4096, 8192, 16384)}
    Ls = (4096, 8192, 16384)

    def normal(shape, seed):
        gen.manual_seed(seed)
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    def timed(calls):
        R = len(calls)
        for i in range(R):
            calls[i]()
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                calls[i % R]()
        g.replay()  # untimed: first replay
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stream.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        stream.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / steps

    results = {"full_attention_us": {}, "asm_us": {}, "ratio_full_over_asm": {}}
    with torch.cuda.stream(stream):
        for B in (1, 32):
            lens = [2048] if B == 1 else [int(x) for x in np.random.default_rng([3, 0]).integers(512, 4097, 32)]
            n_loc = int(sum(lens))
            kv_start = torch.tensor(np.concatenate([[0], np.cumsum(lens)[:-1]]), dtype=torch.int32).to(dev)
            kv_len = torch.tensor(lens, dtype=torch.int32).to(dev)
            q = normal((B, Hq, d), 1)
            for L in Ls:
                print(f"full attention B={B} L={L}: inputs", file=sys.stderr, flush=True)
                ctx = [L + n for n in lens]
                ctx_start = torch.tensor(np.concatenate([[0], np.cumsum(ctx)[:-1]]), dtype=torch.int32).to(dev)
                ctx_len = torch.tensor(ctx, dtype=torch.int32).to(dev)
                step_bytes = sum(ctx) * Hkv * d * 2 * 2
                R = max(2, -(-(1 << 30) // step_bytes))  # at least 1 GiB over the replicas
                reps = [(normal((Hkv, sum(ctx), d), 10 + r), normal((Hkv, sum(ctx), d), 20 + r)) for r in range(R)]
                out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
                lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
                ws = torch.zeros(max(1, api.lib().asm_attend_step_ws(api.BF16, B, Hq, Hkv, d, max(ctx))),
                                 dtype=torch.uint8, device=dev)

                def mk(kc, vc):
                    return lambda: api.attend_step(q, kc, vc, ctx_start, ctx_len, max(ctx), scale, out=out,
                                                   out_lse=lse, workspace=ws)
                us = timed([mk(kc, vc) for kc, vc in reps])
                results["full_attention_us"][f"B{B}_L{L}"] = us
                print(f"full attention B={B} L={L}: {us:.1f} us", file=sys.stderr, flush=True)
                del reps
                stream.synchronize()
            for K in asm_K[B]:
                print(f"ASM B={B} K={K}: inputs", file=sys.stderr, flush=True)
                step_bytes = Hq * K * (d * 2 + 4) + n_loc * Hkv * d * 4
                R = max(2, -(-(1 << 30) // step_bytes))
                reps = []
                for r in range(R):
                    C = normal((Hq, K, d), 100 + r)
                    t = dict(C=C, cinv=api.centroid_inv_norms(C), Abar=normal((Hq, K, d), 200 + r).float(),
                             LSEbar=torch.full((Hq, K), 8.0, device=dev),
                             Kl=normal((Hkv, n_loc, d), 300 + r), Vl=normal((Hkv, n_loc, d), 400 + r))
                    reps.append(t)
                out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
                lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
                idx = torch.empty((B, Hq), dtype=torch.int32, device=dev)
                ws = torch.zeros(api.decode_step_ws(api.BF16, B, Hq, Hkv, d, K, max(lens)),
                                 dtype=torch.uint8, device=dev)

                def mk(t):
                    return lambda: api.decode_step(q, t["C"], t["cinv"], t["Abar"], t["LSEbar"], t["Kl"],
                                                   t["Vl"], kv_start, kv_len, max(lens), scale, out=out,
                                                   out_lse=lse, out_idx=idx, workspace=ws)
                us = timed([mk(t) for t in reps])
                results["asm_us"][f"B{B}_K{K}"] = us
                print(f"ASM B={B} K={K}: {us:.1f} us", file=sys.stderr, flush=True)
                del reps
                stream.synchronize()
            for L in Ls:
                for K in asm_K[B]:
                    results["ratio_full_over_asm"][f"B{B}_L{L}_K{K}"] = (
                        results["full_attention_us"][f"B{B}_L{L}"] / results["asm_us"][f"B{B}_K{K}"])
    print(json.dumps({"workload": "attention_compare", "unit": "us per decode step", "steps": steps,
                      "config": {"q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "dtype": "bf16",
                                 "local_len": {"B1": 2048, "B32": "U{512..4096}"},
                                 "launch": "hip_graph"},
                      **results}), flush=True)


def run_layers(args):
    """One decode step of batch 1 through 32 LLaMA-3.1-8B-shaped layers, each
    with its own memory (K=1024) and local KV (2048 tokens), the 32 calls
    captured in one HIP graph.  Reports per-layer time and the chain's
    algorithmic GB/s (the 32 layers' inputs, 542 MB, exceed the last-level
    cache)."""
    import torch
    from attention_state_memory_amd import api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    layers, host = [], []
    for l in range(32):
        inp = synth.layer_decode(l)
        host.append(inp)
        t = {k: to_dev(inp[k]) for k in ("q", "C", "Abar", "LSEbar", "Kl", "Vl", "kv_start", "kv_len")}
        t["cinv"] = api.centroid_inv_norms(t["C"])
        layers.append(t)
    print("32 layers resident", file=sys.stderr, flush=True)
    i0 = host[0]
    B, Hq, Hkv, d, K = i0["B"], i0["Hq"], i0["Hkv"], i0["d"], i0["K"]
    max_kv = int(np.max(i0["kv_len"]))
    L = api.lib()
    ws_bytes = api.decode_step_ws(api.BF16, B, Hq, Hkv, d, K, max_kv)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((32, B, Hq, d), dtype=torch.float32, device=dev)
    out_lse = torch.empty((32, B, Hq), dtype=torch.float32, device=dev)
    out_idx = torch.empty((32, B, Hq), dtype=torch.int32, device=dev)
    P = ctypes.c_void_p
    stream = torch.cuda.Stream(dev)

    def call(l):
        t = layers[l]
        st = L.asm_decode_step(api.BF16, B, Hq, Hkv, d, K, ctypes.c_float(i0["scale"]),
                               P(t["q"].data_ptr()), P(t["C"].data_ptr()), P(t["cinv"].data_ptr()),
                               P(t["Abar"].data_ptr()), P(t["LSEbar"].data_ptr()),
                               P(t["Kl"].data_ptr()), P(t["Vl"].data_ptr()), t["Kl"].stride(0),
                               t["Kl"].stride(1), t["Kl"].shape[1], P(t["kv_start"].data_ptr()),
                               P(t["kv_len"].data_ptr()), max_kv, P(out[l].data_ptr()),
                               P(out_lse[l].data_ptr()), P(out_idx[l].data_ptr()),
                               P(ws.data_ptr()), ws_bytes, P(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(L.asm_last_error().decode())

    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup // 8)):
            for l in range(32):
                call(l)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for l in range(32):
            call(l)
    with torch.cuda.stream(stream):
        graph.replay()
    stream.synchronize()
    reps = max(1, args.steps // 8)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms_chain = e0.elapsed_time(e1) / reps
    alg = float(sum(algorithmic_bytes(h) for h in host))
    gbs = alg / (ms_chain * 1e-3) / 1e9
    result = {
        "metric": "ASM decode, batch 1 through 32 layers at K=1024: per-layer latency",
        "value": ms_chain * 1e3 / 32, "unit": "us/layer", "n_gpus": 1, "steps": reps,
        "warmup": args.warmup, "ms_per_step": ms_chain, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/C/K/V, fp32 states, lse~U(5,12))",
        "config": {"workload": "layer_decode", "layers": 32, "K": K, "batch": B, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": d, "local_len": max_kv, "launch": "hip_graph"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_step": alg,
                     "timed": "HIP events around replays of one graph holding the 32 layers' "
                              "asm_decode_step calls"},
    }
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------
# batch-1 decode through 32 layers at K=8192: two-level lookup against flat
# --------------------------------------------------------------------------

def run_layers_hier(args):
    """Batch-1 decode through `--layers` layers (32) with `--K` entries per
    query head (8192), once with the flat search and once with the two-level
    lookup (`--supers` S = 128, `--probes` p = 8).  The entries are clusterable (64-centre mixture
    queries per head, as a built memory's are) and every layer's query is an
    entry plus noise.  The two-level lookup reads the entry table grouped by
    super (asm_index_group_rows); it is also timed through the member list.
    Reports per-layer time of the lookups and the two-level lookup's
    recall@1 against the flat search."""
    import torch
    from attention_state_memory_amd import api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    K, S, p, layers, Hq = args.K, args.supers, args.probes, args.layers, 32
    L = []
    for l in range(layers):
        inp = synth.decode_inputs([6, l], B=1, Hq=Hq, Hkv=8, d=128, K=K, kv_lens=[2048])
        C = synth.mixture_queries([6, l, 1], Hq, K, 128, M=64)
        r = np.random.default_rng([6, l, 2])
        pick = r.integers(0, K, Hq)
        q = synth.bf16_bits_to_float(C)[np.arange(Hq), pick][None] + \
            np.float32(0.3) * r.standard_normal((1, Hq, 128), dtype=np.float32)
        t = {k: to_dev(inp[k]) for k in ("Abar", "LSEbar", "Kl", "Vl", "kv_start", "kv_len")}
        t["q"] = to_dev(synth.to_bf16_bits(q))
        t["C"] = to_dev(C)
        t["cinv"] = api.centroid_inv_norms(t["C"])
        t["index"] = api.build_index(t["C"], S, 4)
        t["grouped"] = api.group_index_rows(t["C"], t["cinv"], t["index"])
        L.append(t)
        print(f"layer {l} resident", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    print("layers and indices resident", file=sys.stderr, flush=True)
    scale = synth.softmax_scale(128)
    out = torch.empty((layers, 1, Hq, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((layers, 1, Hq), dtype=torch.float32, device=dev)
    idx_f = torch.empty((layers, 1, Hq), dtype=torch.int32, device=dev)
    idx_h = torch.empty((layers, 1, Hq), dtype=torch.int32, device=dev)
    ws = torch.zeros(max(api.decode_step_ws(api.BF16, 1, Hq, 8, 128, K, 2048),
                         int(api.lib().asm_decode_step_hier_ws(api.BF16, 1, Hq, 8, 128, K, S, p, 2048))),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(dev)

    def flat(l):
        t = L[l]
        api.decode_step(t["q"], t["C"], t["cinv"], t["Abar"], t["LSEbar"], t["Kl"], t["Vl"],
                        t["kv_start"], t["kv_len"], 2048, scale, out=out[l], out_lse=lse[l],
                        out_idx=idx_f[l], workspace=ws)

    def hier(l, grouped=True):
        t = L[l]
        api.decode_step_hier(t["q"], t["C"], t["cinv"], t["index"], p, t["Abar"], t["LSEbar"],
                             t["Kl"], t["Vl"], t["kv_start"], t["kv_len"], 2048, scale,
                             grouped=t["grouped"] if grouped else None,
                             out=out[l], out_lse=lse[l], out_idx=idx_h[l], workspace=ws)

    def timed(fn):
        with torch.cuda.stream(stream):
            for l in range(layers):
                fn(l)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for l in range(layers):
                fn(l)
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        reps = max(1, args.steps // 8)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps, reps

    ms_flat, _ = timed(flat)
    ms_members, _ = timed(lambda l: hier(l, grouped=False))
    ms_hier, reps = timed(hier)
    recall = float((idx_f == idx_h).float().mean().item())
    rows = p * K / S  # member rows scanned per query head on average
    hier_bytes = layers * (Hq * (S * 128 * 2 + S * 4 + (S + 1) * 4 + rows * (128 * 2 + 4 + 4) + 128 * 2
                                 + (128 * 4 + 4) + (128 * 4 + 8)) + 8 * 2048 * 128 * 2 * 2 + 8)
    gbs = hier_bytes / (ms_hier * 1e-3) / 1e9
    result = {
        "metric": f"ASM decode, batch 1 through {layers} layers at K={K}, two-level lookup: "
                  "per-layer latency",
        "value": ms_hier * 1e3 / layers, "unit": "us/layer", "n_gpus": 1, "steps": reps,
        "warmup": args.warmup, "ms_per_step": ms_hier, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (64-centre mixture entries per head, queries = entries + noise, "
                "N(0,1) bf16 local KV, fp32 states)",
        "config": {"workload": "layer_decode_hier", "layers": layers, "K": K, "supers": S,
                   "probes": p, "batch": 1, "q_heads": Hq, "kv_heads": 8, "head_dim": 128,
                   "local_len": 2048, "launch": "hip_graph"},
        "flat_us_per_layer": ms_flat * 1e3 / layers,
        "through_member_list_us_per_layer": ms_members * 1e3 / layers,
        "speedup_vs_flat": ms_flat / ms_hier,
        "recall_at_1_vs_flat": recall,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_step": hier_bytes,
                     "timed": "HIP events around replays of one graph holding the layers' "
                              "asm_decode_step_hier calls"},
    }
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------
# offline build workloads (MFMA-bound prefix states and k-means assignment)
# --------------------------------------------------------------------------

BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 matrix peak of one MI355X


def _timed(fn, reps):
    """Mean milliseconds of fn() over reps calls, HIP events on the current stream."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_build(args):
    import torch
    from attention_state_memory_amd import api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.workload == "prefix_states":
        w = synth.prefix_states(N=args.queries)
        Q, Kp, Vp = to_dev(w["Q"]), to_dev(w["Kp"]), to_dev(w["Vp"])
        Hq, N, L, d, chunk = w["Hq"], w["N"], w["L"], w["d"], w["chunk"]
        nc = -(-L // chunk)
        A = torch.empty((Hq, N, d), dtype=torch.float32, device=dev)
        LSE = torch.empty((Hq, N), dtype=torch.float32, device=dev)
        Ac = torch.empty((nc, Hq, N, d), dtype=torch.float32, device=dev)
        Lc = torch.empty((nc, Hq, N), dtype=torch.float32, device=dev)

        L_ = api.lib()
        ws_bytes = int(L_.asm_build_states_ws(api.BF16, Hq, w["Hkv"], N, L, d, chunk))
        ws = torch.zeros(max(1, ws_bytes), dtype=torch.uint8, device=dev)
        P = ctypes.c_void_p

        def step_chunks():
            # per-chunk states kept: the workload emits (a, lse) per chunk
            st = L_.asm_build_states(api.BF16, Hq, w["Hkv"], N, L, d, chunk,
                                     ctypes.c_float(w["scale"]),
                                     *(P(t.data_ptr()) for t in (Q, Kp, Vp, Ac, Lc, A, LSE)),
                                     0, P(ws.data_ptr()), ws_bytes,
                                     P(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError(L_.asm_last_error().decode())

        for _ in range(args.warmup):
            step_chunks()
        steps = args.steps
        ms = _timed(step_chunks, steps)
        flops = 4.0 * Hq * N * L * d
        tflops = flops / (ms * 1e-3) / 1e12
        result = {
            "metric": "prefix attention states (query-heads x prefix tokens) per second",
            "value": Hq * N / (ms * 1e-3), "unit": "query-head states/s", "n_gpus": 1,
            "steps": steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded 64-centre mixture queries, N(0,1) bf16 prefix)",
            "config": {"workload": "prefix_states", "q_heads": Hq, "kv_heads": w["Hkv"],
                       "head_dim": d, "queries_per_head": N, "prefix": L, "chunk": chunk,
                       "per_chunk_states": True},
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / BF16_MFMA_PEAK_TFLOPS,
                         "traffic": None, "algorithmic_flops_per_launch": flops,
                         "timed": "asm_build_states (one kernel launch)"},
        }
        if args.cpu_seconds > 0:
            result["cpu_baseline"] = cpu_baseline_states(w, args.cpu_seconds)
        print(json.dumps(result), flush=True)
        return

    if args.workload == "prefix_states_streamed":
        run_streamed(args, w=synth.prefix_states(N=args.queries), to_dev=to_dev)
        return

    # memory_build: states over the prefix, 10 Lloyd iterations, aggregation
    w = synth.memory_build()
    print("memory_build inputs generated", file=sys.stderr, flush=True)
    H, N, K, d, T = w["Hq"], w["N"], w["K"], w["d"], w["iters"]
    X, Kp, Vp = to_dev(w["X"]), to_dev(w["Kp"]), to_dev(w["Vp"])
    A = torch.empty((H, N, d), dtype=torch.float32, device=dev)
    LSE = torch.empty((H, N), dtype=torch.float32, device=dev)
    C = torch.empty((H, K, d), dtype=torch.bfloat16, device=dev)
    cinv = torch.empty((H, K), dtype=torch.float32, device=dev)
    idx = torch.empty((H, N), dtype=torch.int32, device=dev)
    count = torch.empty((H, K), dtype=torch.int32, device=dev)
    Abar = torch.empty((H, K, d), dtype=torch.float32, device=dev)
    LSEbar = torch.empty((H, K), dtype=torch.float32, device=dev)
    ev = {k: [] for k in ("states", "assign", "mean", "aggregate")}

    def mark():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def build(record):
        e = [mark()]
        api.build_states(X, Kp, Vp, w["chunk"], w["scale"], A=A, LSE=LSE)
        e.append(mark())
        C.copy_(X[:, :K, :])
        api.centroid_inv_norms(C, cinv=cinv)
        marks = []
        for t in range(T):
            a0 = mark()
            api.kmeans_assign(X, C, cinv, idx=idx)
            a1 = mark()
            last = t == T - 1
            api.aggregate(X, idx, C, A=A, LSE=LSE, cinv=cinv, count=count, Abar=Abar,
                          LSEbar=LSEbar, with_states=last)
            a2 = mark()
            marks.append((a0, a1, a2, last))
        e.append(mark())
        if record:
            torch.cuda.synchronize()
            ev["states"].append(e[0].elapsed_time(e[1]))
            for a0, a1, a2, last in marks:
                ev["assign"].append(a0.elapsed_time(a1))
                ev["aggregate" if last else "mean"].append(a1.elapsed_time(a2))
            return e[0].elapsed_time(e[2])
        return None

    for _ in range(max(1, args.warmup)):
        build(False)
    torch.cuda.synchronize()
    steps = max(1, args.steps)
    totals = [build(True) for _ in range(steps)]
    ms = float(np.mean(totals))
    assign_ms = float(np.mean(ev["assign"]))
    aflops = 2.0 * H * N * K * d
    atf = aflops / (assign_ms * 1e-3) / 1e12
    sflops = 4.0 * H * N * w["L"] * d
    result = {
        "metric": "ASM memory build wall-clock (states + 10 Lloyd iterations + aggregation)",
        "value": ms * 1e-3, "unit": "s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded 64-centre mixture queries, N(0,1) bf16 prefix)",
        "config": {"workload": "memory_build", "q_heads": H, "head_dim": d,
                   "queries_per_head": N, "K": K, "iterations": T, "prefix": w["L"],
                   "chunk": w["chunk"]},
        "kernels_ms": {k: float(np.mean(v)) for k, v in ev.items()},
        "states_tflops": sflops / (float(np.mean(ev["states"])) * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "achieved": atf, "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": atf / BF16_MFMA_PEAK_TFLOPS, "traffic": None,
                     "algorithmic_flops_per_launch": aflops,
                     "timed": "asm_kmeans_assign (one kernel launch), mean of all iterations"},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_assign(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def run_streamed(args, w, to_dev):
    """The prefix-state workload with the prefix in pinned host memory:
    asm_build_states_streamed copies chunk c + 1 while chunk c is encoded.
    Timed beside it, on the same stream: the resident asm_build_states over
    the same chunks (merged states only) and the plain host-to-device copy
    of the prefix."""
    import torch
    from attention_state_memory_amd import api

    dev = torch.device("cuda:0")
    Hq, Hkv, N, L, d, chunk = w["Hq"], w["Hkv"], w["N"], w["L"], w["d"], w["chunk"]

    def pinned(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).pin_memory()

    Q = to_dev(w["Q"])
    Kh, Vh = pinned(w["Kp"]), pinned(w["Vp"])
    Kd, Vd = Kh.to(dev), Vh.to(dev)
    A = torch.empty((Hq, N, d), dtype=torch.float32, device=dev)
    LSE = torch.empty((Hq, N), dtype=torch.float32, device=dev)
    ws_s = torch.zeros(int(api.lib().asm_build_states_streamed_ws(api.BF16, Hq, Hkv, N, d, chunk)),
                       dtype=torch.uint8, device=dev)
    ws_r = torch.zeros(max(1, int(api.lib().asm_build_states_ws(api.BF16, Hq, Hkv, N, L, d, chunk))),
                       dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream(device=dev)
    Kc, Vc = torch.empty_like(Kd), torch.empty_like(Vd)

    def streamed():
        api.build_states_streamed(Q, Kh, Vh, chunk, w["scale"], A=A, LSE=LSE, workspace=ws_s,
                                  copy_stream=copy_stream)

    def resident():
        api.build_states(Q, Kd, Vd, chunk, w["scale"], A=A, LSE=LSE, workspace=ws_r)

    def copy_only():
        Kc.copy_(Kh, non_blocking=True)
        Vc.copy_(Vh, non_blocking=True)

    for fn in (streamed, resident, copy_only):
        for _ in range(args.warmup):
            fn()
    steps = args.steps
    ms = _timed(streamed, steps)
    ms_res = _timed(resident, steps)
    ms_copy = _timed(copy_only, steps)
    prefix_bytes = 2 * Hkv * L * d * 2
    flops = 4.0 * Hq * N * L * d
    tflops = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "prefix attention states (query-heads x prefix tokens) per second, prefix "
                  "streamed from pinned host memory",
        "value": Hq * N / (ms * 1e-3), "unit": "query-head states/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded 64-centre mixture queries, N(0,1) bf16 prefix in pinned host memory)",
        "config": {"workload": "prefix_states_streamed", "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": d, "queries_per_head": N, "prefix": L, "chunk": chunk},
        "resident_ms": ms_res,
        "copy_only_ms": ms_copy,
        "host_to_device_GBps": prefix_bytes / (ms * 1e-3) / 1e9,
        "copy_only_GBps": prefix_bytes / (ms_copy * 1e-3) / 1e9,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "traffic": None,
                     "algorithmic_flops_per_launch": flops,
                     "timed": "asm_build_states_streamed (copies and one states launch per chunk)"},
    }
    print(json.dumps(result), flush=True)


def _blas_threads():
    from threadpoolctl import threadpool_info
    return int(max((p.get("num_threads", 1) for p in threadpool_info()), default=1))


def cpu_baseline_states(w, budget_s: float) -> dict:
    from oracle import asm_oracle as O
    Kp, Vp = O.bf16_bits_to_f64(w["Kp"]), O.bf16_bits_to_f64(w["Vp"])
    rows = 64
    t0 = time.perf_counter()
    done = 0
    while done == 0 or (time.perf_counter() - t0) < budget_s:
        lo = (done * rows) % w["N"]
        Q = O.bf16_bits_to_f64(w["Q"][:, lo:lo + rows])
        O.build_states(Q, Kp, Vp, w["chunk"], w["scale"])
        done += 1
    el = time.perf_counter() - t0
    return {"value": done * rows * w["Hq"] / el, "unit": "query-head states/s",
            "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{done} pass(es) of {rows} queries x {w['Hq']} heads over the full "
                      f"16384-token prefix in 4 chunks, {el:.1f} s"}


def cpu_baseline_assign(w, budget_s: float) -> dict:
    """The oracle's cosine assignment on row blocks of the first head against
    the first-K centroids; reported as seconds per full assignment pass."""
    from oracle import asm_oracle as O
    X = w["X"]
    K = w["K"]
    C = O.bf16_bits_to_f64(X[0, :K])
    rows = 256
    t0 = time.perf_counter()
    done = 0
    while done == 0 or (time.perf_counter() - t0) < budget_s:
        lo = (done * rows) % w["N"]
        O.assign(O.bf16_bits_to_f64(X[0, lo:lo + rows]), C)
        done += 1
    el = time.perf_counter() - t0
    per_row = el / (done * rows)
    total = per_row * w["N"] * w["Hq"]
    return {"value": total, "unit": "s per assignment pass (all heads, extrapolated)",
            "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{done} block(s) of {rows} rows x K={K} of head 0, {el:.1f} s; "
                      f"one full pass = {w['N']} rows x {w['Hq']} heads"}


if __name__ == "__main__":
    main()
