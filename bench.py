#!/usr/bin/env python3
"""Benchmark of the POP channel-pruned gated-MLP path on one MI355X.

One step is one whole request of the workload with every input already in
HBM: the prefill of every layer (one pop_prefill_ffn_partition call: column
norms, the dense prompt FFN on the matrix cores with the importance taken in
its gate/up pass, the three-region select) followed by every decode step over
every layer (gate/up over R u C with fused scores, candidate top-k, gathered
down-projection).  The layers do not chain: each has its own seeded prompt
and decode inputs (with that layer's outlier channels).  Steps are replayed as
HIP graphs.

Printed: ONE JSON line on stdout.  value = decode tokens per second per layer
over the whole step of the LLaMA-2-7B-shaped batch-1 workload (B * T * layers
/ step time; the prefill is in the denominator).  The same line carries, for
that workload, the decode time per layer-step (median, p10, p90 over steps;
graph replay and eager), its HBM rate on algorithmic bytes against the peak and
against a measured stream-read probe, the dense comparator, the ablation
variants, the prefill partition and the prompt FFN; the roofline of the
dominant kernel (per-kernel HIP events); the CPU oracle baseline with a spot
check of the timed inputs; and a summary of each other workload (batch 16,
the Qwen2-7B shape with drifting outliers and mask churn, the mixture of
experts).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-extra]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "pruned FFN decode tokens/s per layer + HBM GB/s vs peak; prefill partition µs"
HBM_PEAK_GBPS = 8000.0
MAIN_WORKLOAD = "llama2_7b_ffn_b1"
EXTRA_WORKLOADS = ("llama2_7b_ffn_b16", "qwen2_7b_ffn_b4", "mixtral_moe_ffn_t32")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=MAIN_WORKLOAD)
    ap.add_argument("--layers", type=int, default=None, help="default: the workload's layer count")
    ap.add_argument("--decode-steps", type=int, default=None, help="default: the workload's decode steps")
    ap.add_argument("--kernel-steps", type=int, default=4, help="decode steps in the per-kernel timing pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads' summaries")
    ap.add_argument("--extra-steps", type=int, default=2, help="timed whole steps of each other workload")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of each oracle timing sample")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run 3 device-to-device copies of this many MiB (a known-size kernel that "
                         "calibrates the profiler's HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Ev:
    """HIP events on torch's current stream."""

    def __init__(self, torch):
        self.e = torch.cuda.Event(enable_timing=True)

    def record(self):
        self.e.record()
        return self

    def ms(self, other):
        return self.e.elapsed_time(other.e)


def timed(torch, fn, reps):
    torch.cuda.synchronize()
    a = Ev(torch).record()
    for _ in range(reps):
        fn()
    b = Ev(torch).record()
    torch.cuda.synchronize()
    return a.ms(b) / reps


def per_step_ms(torch, step, T):
    """Runs step(t) for t < T back to back with an event between steps;
    returns the T step times (ms)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(T + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for t in range(T):
        step(t)
        ev[t + 1].record()
    torch.cuda.synchronize()
    return [ev[t].elapsed_time(ev[t + 1]) for t in range(T)]


def spread(np, v, scale=1.0, nd=3):
    """median, p10, p90 of v * scale."""
    a = np.asarray(v, dtype=np.float64) * scale
    return {"median": round(float(np.median(a)), nd), "p10": round(float(np.percentile(a, 10)), nd),
            "p90": round(float(np.percentile(a, 90)), nd)}


def copy_probe(torch, dev, mib):
    """Three device-to-device copies of known size (the profiler's byte
    counters are scaled by what they read for these)."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy probe: 3 copies of {mib} MiB ({n} bytes read and written each)")


def hbm_probe(np, torch, pop, dev):
    """Measured HBM stream-read rate: pop_hbm_read_probe over 1 GiB, 1024
    workgroups, alternating between two buffers so that no read is served by
    the 256 MB memory-side cache."""
    nbytes = 1 << 30
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(2)]
    sink = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
    for i in range(4):
        pop.pop_hbm_read_probe(bufs[i % 2], sink, 1024)
    ts = []
    for i in range(10):
        ts.append(timed(torch, lambda: pop.pop_hbm_read_probe(bufs[i % 2], sink, 1024), 1))
    del bufs
    gbps = nbytes / (float(np.median(ts)) * 1e-3) / 1e9
    log(f"[bench] HBM stream-read probe: {gbps:.0f} GB/s ({gbps / HBM_PEAK_GBPS:.3f} of {HBM_PEAK_GBPS:.0f})")
    return {"gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes": nbytes,
            "kernel": "pop_hbm_read_probe: 1024 workgroups x 256 threads, non-temporal 16-byte loads, 8 in flight "
                      "per thread, one contiguous chunk per workgroup; median of 10 event-timed launches"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the path is not sharded across GPUs", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from online_structured_ffn_amd import configs, metrics, pop, synth

    mods = (np, torch, metrics, pop, synth)
    w = configs.BY_NAME[args.workload]
    if "attention" in w.extra:
        bench_layer(args, w, np, torch, metrics, pop, synth)
        return
    dev = torch.device("cuda")
    if args.copy_probe_mib > 0:
        copy_probe(torch, dev, args.copy_probe_mib)
    probe = hbm_probe(np, torch, pop, dev)
    if w.experts:
        res = bench_moe(args, w, mods, args.layers or w.layers, args.decode_steps or w.decode_steps, args.steps,
                        args.warmup, detail=True)
        out = compose(args, w, res, probe, np)
    else:
        res = bench_ffn(args, w, mods, args.layers or w.layers, args.decode_steps or w.decode_steps, args.steps,
                        args.warmup, detail=True)
        spot = res.pop("_spot", None)
        out = compose(args, w, res, probe, np)
        if spot is not None:
            out["oracle_spot_check"] = spot_check(w, spot)
            log(f"[bench] oracle spot check of the timed inputs: {out['oracle_spot_check']}")
        del spot
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(w, res["config"]["decode_steps"], args.cpu_seconds)
            log(f"[bench] cpu baseline: {out['cpu_baseline']}")
    torch.cuda.empty_cache()
    if w.name == MAIN_WORKLOAD and not args.no_extra:
        out["other_workloads"] = {}
        for name in EXTRA_WORKLOADS:
            wx = configs.BY_NAME[name]
            t0 = time.time()
            if wx.experts:
                r = bench_moe(args, wx, mods, wx.layers, wx.decode_steps, args.extra_steps, 1, detail=False)
            else:
                r = bench_ffn(args, wx, mods, wx.layers, wx.decode_steps, args.extra_steps, 1, detail=False)
                r.pop("_spot", None)
            r["wall_s"] = round(time.time() - t0, 1)
            out["other_workloads"][name] = r
            torch.cuda.empty_cache()
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def compose(args, w, res, probe, np):
    """The driver's JSON line around one workload's results."""
    dec = res["decode"]
    out = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": res["data"],
        "config": res["config"],
        "roofline": res.get("roofline"),
        "hbm_read_probe": probe,
    }
    dec["hbm_frac_of_probe"] = round(dec["hbm_gbps"] / probe["gbps"], 4)
    rl = out["roofline"]
    if rl and rl.get("achieved") is not None:
        rl["achieved_vs_read_probe"] = round(rl["achieved"] / probe["gbps"], 4)
    for k_, v in res.items():
        if k_ not in out and k_ not in ("value", "ms_per_step", "data", "config", "roofline"):
            out[k_] = v
    out["cpu_baseline"] = None
    return out


def ffn_inputs(w, mods, L, T, dev):
    """Device-drawn weights, prompts and the decode stream of an FFN stack.
    Each layer's prompt and decode inputs carry that layer's outlier channels;
    with drifting outliers the decode input of step t carries the set O_{t+1}
    (one member swapped per step from the prompt's O_0)."""
    np, torch, _, _, synth = mods
    B, d = w.decode_batch, w.d
    n_tok = w.prompt_batch * w.prompt_len
    Wg, Wu, WdT, X, dec = [], [], [], [], []
    for l in range(L):
        ws_ = synth.torch_layer_weights(w, l, dev)
        Wg.append(ws_["W_gate"])
        Wu.append(ws_["W_up"])
        WdT.append(ws_["W_downT"])
        X.append(synth.torch_activations(w, (n_tok, d), l, 0, dev, synth.outlier_channels(w, l)))
        dec.append(synth.torch_decode_inputs(w, l, T, dev))
    Xdec = torch.stack(dec, dim=1).contiguous()  # [T, L, B, d]
    del dec
    return Wg, Wu, WdT, X, Xdec


def bench_ffn(args, w, mods, L, T, steps, warmup, detail):
    """One FFN-stack workload: whole steps (prefill of every layer + every
    decode step over every layer) replayed as HIP graphs; the decode alone per
    step (median/p10/p90); the dense comparator; the standalone prefill
    partition; mask churn.  With detail: the ablation variants, periodic
    refresh, eager decode, the prompt FFN, the per-kernel pass and roofline,
    and host copies of layer 0 for the oracle's spot check."""
    np, torch, metrics, pop, synth = mods
    from online_structured_ffn_amd import profiling
    B = w.decode_batch
    d, d_ff = w.d, w.d_ff
    e = 2 if w.dtype == "bf16" else 4
    n_tok = w.prompt_batch * w.prompt_len
    dev = torch.device("cuda")
    cnt = pop.pop_partition_counts(d_ff, w.r, w.gamma)
    n_R, n_C, n_P, k = cnt["n_R"], cnt["n_C"], cnt["n_P"], cnt["k"]
    n_A, n_live = n_R + n_C, n_R + k
    log(f"[bench] {w.name}: {L} layers, d={d}, d_ff={d_ff}, prompt {n_tok} tokens, T={T}, B={B}; "
        f"|R|={n_R} |C|={n_C} |P|={n_P} k={k}")
    t0 = time.time()
    Wg, Wu, WdT, X, Xdec = ffn_inputs(w, mods, L, T, dev)
    R = [torch.empty(n_R, dtype=torch.int32, device=dev) for _ in range(L)]
    C = [torch.empty(n_C, dtype=torch.int32, device=dev) for _ in range(L)]
    P = [torch.empty(n_P, dtype=torch.int32, device=dev) for _ in range(L)]
    x_buf = torch.empty((L, B, d), dtype=Xdec.dtype, device=dev)
    y = torch.empty((L, B, d), dtype=torch.float32, device=dev)
    ws_pre = pop.workspace(pop.pop_prefill_workspace_bytes(n_tok, d, d_ff), dev)
    ws_fused = pop.workspace(pop.pop_prefill_ffn_partition_workspace_bytes(n_tok, d, d_ff, w.dtype), dev)
    Yp = torch.empty((n_tok, d), dtype=torch.float32, device=dev)   # prompt FFN output (layers do not chain)
    ws_dec = pop.workspace(pop.pop_decode_workspace_bytes(B, d, d_ff), dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs generated on the device in {time.time() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")

    def partition(l):
        pop.pop_prefill_partition(X[l], Wu[l], w.r, w.gamma, out=(R[l], C[l], P[l], None), ws=ws_pre)

    def prefill():
        # each layer's whole prefill in one call: the importance comes out of
        # the prompt FFN's gate/up pass (one W_up sweep instead of two)
        for l in range(L):
            pop.pop_prefill_ffn_partition(X[l], Wg[l], Wu[l], WdT[l], w.r, w.gamma, Y=Yp,
                                          out=(R[l], C[l], P[l], None), ws=ws_fused)

    def partition_layers():
        for l in range(L):
            partition(l)

    def decode_layers():
        for l in range(L):
            pop.pop_decode_ffn(x_buf[l], Wg[l], Wu[l], WdT[l], R[l], C[l], w.r, y=y[l], ws=ws_dec)

    def dense_layers():
        for l in range(L):
            pop.pop_dense_ffn_decode(x_buf[l], Wg[l], Wu[l], WdT[l], y=y[l], ws=ws_dec)

    fns = [("prefill", prefill), ("partition", partition_layers), ("decode", decode_layers),
           ("dense", dense_layers)]
    if detail:
        ws_ffn = pop.workspace(max(pop.pop_dense_ffn_prefill_workspace_bytes(n_tok, d, d_ff, w.dtype), 256), dev)

        def prompt_ffn_layers():
            for l in range(L):
                pop.pop_dense_ffn_prefill(X[l], Wg[l], Wu[l], WdT[l], Y=Yp, ws=ws_ffn)

        def prefill_unfused():
            for l in range(L):
                pop.pop_dense_ffn_prefill(X[l], Wg[l], Wu[l], WdT[l], Y=Yp, ws=ws_ffn)
                partition(l)

        fns += [("prompt_ffn", prompt_ffn_layers), ("prefill_unfused", prefill_unfused)]

    # ------------------------------------------------------------ graphs
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        x_buf.copy_(Xdec[0])
        for _, fn in fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = {}
    for name, fn in fns:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs[name] = g
    torch.cuda.synchronize()

    def step_of(name):
        def run(t):
            x_buf.copy_(Xdec[t])
            graphs[name].replay()
        return run

    def job():
        graphs["prefill"].replay()
        run = step_of("decode")
        for t in range(T):
            run(t)

    # ------------------------------------------------------------ timed region: whole steps
    for _ in range(warmup):
        job()
    torch.cuda.synchronize()
    ms_step = timed(torch, job, steps)
    value = B * T * L / (ms_step / 1e3)   # B*T tokens through each of the L layers
    log(f"[bench] step {ms_step:.2f} ms -> {value:,.0f} tokens/s/layer")

    # ------------------------------------------------------------ components (graphs)
    dec_ms = per_step_ms(torch, step_of("decode"), T)
    dense_ms = per_step_ms(torch, step_of("dense"), T)
    ms_part = timed(torch, lambda: graphs["partition"].replay(), 5)
    ms_pre = timed(torch, lambda: graphs["prefill"].replay(), 3)
    t_ls = float(np.median(dec_ms)) / L             # ms per layer-step
    t_ls_dense = float(np.median(dense_ms)) / L
    bytes_ls = metrics.decode_bytes(d, n_R, n_C, k, B, e)
    bytes_dense = metrics.dense_decode_bytes(d, d_ff, B, e)
    part_bytes = metrics.partition_bytes(n_tok, d, d_ff, e)
    log(f"[bench] decode {t_ls * 1e3:.1f} us/layer-step ({bytes_ls / (t_ls * 1e-3) / 1e9:.0f} GB/s), dense "
        f"{t_ls_dense * 1e3:.1f} us ({bytes_dense / (t_ls_dense * 1e-3) / 1e9:.0f} GB/s), prefill partition "
        f"{ms_part / L * 1e3:.1f} us/layer, prefill (fused) {ms_pre / L * 1e3:.1f} us/layer")

    # ------------------------------------------------------------ mask churn |S_t xor S_t-1| / k
    churn = None
    if k > 0 and n_C > 0:
        layers_c = sorted({0, L // 2, L - 1})
        n_s = min(T, 32)
        ch = []
        for l in layers_c:
            prev = None
            for t in range(n_s):
                x_buf.copy_(Xdec[t])
                _, S = pop.pop_decode_ffn(x_buf[l], Wg[l], Wu[l], WdT[l], R[l], C[l], w.r, y=y[l], selected=True,
                                          ws=ws_dec)
                cur = S.cpu().numpy()
                if prev is not None:
                    ch.append(len(np.setxor1d(cur, prev)) / k)
                prev = cur
        churn = {"mean": round(float(np.mean(ch)), 4), "max": round(float(np.max(ch)), 4),
                 "layers": layers_c, "steps": n_s,
                 "definition": "|S_t symmetric-difference S_{t-1}| / k over consecutive decode steps (2x the fraction "
                               "of the selected candidates replaced; the decode inputs are drawn independently per "
                               "step)"}
        log(f"[bench] mask churn: mean {churn['mean']:.3f}, max {churn['max']:.3f} (layers {layers_c}, {n_s} steps)")

    res = {
        "value": round(value, 1),
        "ms_per_step": round(ms_step, 4),
        "data": "synthetic (seeded device-drawn weights N(0,0.02^2) and activations with per-layer outlier "
                "channels; no dataset, no trained weights)",
        "config": {
            "workload": w.name, "layers": L, "d": d, "d_ff": d_ff, "r_ffn": w.r, "gamma": w.gamma,
            "prompt_tokens": n_tok, "decode_steps": T, "decode_batch": B, "hip_graphs": True, "streams": 1,
            "outliers": f"{w.outlier_kind}, {w.outlier_channels} channels"
                        + (", drifting by one member per decode step" if w.outlier_kind == "drift_scale" else ""),
            "step": "prefill (fused dense prompt FFN + partition) of every layer + every decode step over every layer",
        },
        "decode": {
            "us_per_layer_step": round(t_ls * 1e3, 3),
            "us_per_layer_step_spread": spread(np, dec_ms, 1e3 / L),
            "tokens_per_s_per_layer": round(B / (t_ls * 1e-3), 1),
            "algorithmic_bytes_per_layer_step": bytes_ls,
            "hbm_gbps": round(bytes_ls / (t_ls * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes_ls / (t_ls * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "timing": "per decode step: HIP events between graph replays (each step copies its inputs into place "
                      "and replays one graph of every layer's pop_decode_ffn); median, p10, p90 over the steps",
        },
        "dense_decode": {
            "us_per_layer_step": round(t_ls_dense * 1e3, 3),
            "us_per_layer_step_spread": spread(np, dense_ms, 1e3 / L),
            "algorithmic_bytes_per_layer_step": bytes_dense,
            "hbm_gbps": round(bytes_dense / (t_ls_dense * 1e-3) / 1e9, 1),
        },
        "speedup_vs_dense": round(t_ls_dense / t_ls, 4),
        "ideal_speedup_bytes": round(bytes_dense / bytes_ls, 4),
        "prefill_partition_us_per_layer": round(ms_part / L * 1e3, 2),
        "prefill_partition_hbm_frac": round(part_bytes / (ms_part / L * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "prefill_fused_us_per_layer": round(ms_pre / L * 1e3, 2),
        "mask_churn": churn,
    }
    if not detail:
        return res

    # ------------------------------------------------------------ ablation variants (POP notes, ablation table)
    # (1) static prefill mask: the n_live channels of highest prefill importance, no candidates;
    # (2) full re-evaluation: every channel a candidate at every step.
    I_l = [torch.empty(d_ff, dtype=torch.float32, device=dev) for _ in range(L)]
    Rs = []
    for l in range(L):
        pop.pop_prefill_partition(X[l], Wu[l], w.r, w.gamma, out=(R[l], C[l], P[l], I_l[l]), ws=ws_pre)
        Rs.append(pop.pop_partition_select(I_l[l], w.r, 0.0)[0])
    R_none = torch.empty(0, dtype=torch.int32, device=dev)
    C_all = torch.arange(d_ff, dtype=torch.int32, device=dev)

    def static_layers():
        for l in range(L):
            pop.pop_decode_ffn(x_buf[l], Wg[l], Wu[l], WdT[l], Rs[l], R_none, w.r, y=y[l], ws=ws_dec)

    def full_layers():
        for l in range(L):
            pop.pop_decode_ffn(x_buf[l], Wg[l], Wu[l], WdT[l], R_none, C_all, w.r, y=y[l], ws=ws_dec)

    for name, fn in (("static", static_layers), ("full", full_layers)):
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs[name] = g
    torch.cuda.synchronize()
    ms_static = float(np.median(per_step_ms(torch, step_of("static"), T)))
    ms_full = float(np.median(per_step_ms(torch, step_of("full"), T)))

    # periodic refresh mode (batch-wise pruning page, figures 1 and 2(b), read into POP's candidate set)
    periodic = {}
    ws_per = pop.workspace(pop.pop_decode_periodic_workspace_bytes(B, d, d_ff), dev)
    for period in (8, 32):
        states = [pop.PeriodicState(d_ff, w.r, n_R, n_C, dev) for _ in range(L)]

        def per_layers(t, states=states, period=period):
            for l in range(L):
                pop.pop_decode_ffn_periodic(x_buf[l], Wg[l], Wu[l], WdT[l], R[l], C[l], w.r, t, period, states[l],
                                            y=y[l], ws=ws_per)

        with torch.cuda.stream(side):
            per_layers(0)
            per_layers(1)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gp = []
        for t in (0, 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                per_layers(t)
            gp.append(g)

        def run(gp=gp, period=period):
            for t in range(T):
                x_buf.copy_(Xdec[t])
                gp[0 if t % period == 0 else 1].replay()

        periodic[period] = timed(torch, run, 1) / (T * L)
        del gp

    # eager decode (no graph): the host enqueues every call
    n_eager = min(T, 16)

    def eager_step(t):
        x_buf.copy_(Xdec[t])
        decode_layers()

    eager_step(0)
    eager_ms = per_step_ms(torch, eager_step, n_eager)
    ms_pffn = timed(torch, lambda: graphs["prompt_ffn"].replay(), 3)
    ms_unfused = timed(torch, lambda: graphs["prefill_unfused"].replay(), 3)
    pffn_flops = metrics.prefill_ffn_flops(n_tok, d, d_ff)
    pffn_tflops = pffn_flops / (ms_pffn / L * 1e-3) / 1e12
    log(f"[bench] static mask {ms_static / L * 1e3:.1f} us, full re-evaluation {ms_full / L * 1e3:.1f} us, "
        + ", ".join(f"periodic every {p}: {v * 1e3:.1f} us" for p, v in periodic.items())
        + f", eager decode {np.median(eager_ms) / L * 1e3:.1f} us/layer-step, prompt FFN {ms_pffn / L * 1e3:.1f} "
        f"us/layer ({pffn_tflops:.0f} TFLOP/s), prefill unfused {ms_unfused / L * 1e3:.1f} us/layer")

    # ------------------------------------------------------------ per-kernel pass (eager, queued ahead)
    # The same calls as the timed region, with libpop's trace hook recording a
    # HIP event before and after every kernel; a spin kernel queued first keeps
    # the GPU busy while the host enqueues, so the traced kernels run back to back.
    S = min(args.kernel_steps, T)
    vec = 8 if e == 2 else 4
    fused = B == 1 and d <= 4 * metrics.LINKED_THREADS * vec
    linked = fused and 0 < n_C <= 4096 and k > 0
    labels_pre = (["k_colsq_slices"] if n_tok <= 8192 else ["k_colsq_partial", "k_sum_chunks(s2)"]) + [
        "k_importance_items", "k_partition"]
    n_pass = -(-n_tok // 4096)
    labels_ffn = (["k_prompt_gateup", "k_prompt_down"] if e == 2 else
                  ["k_prompt_gateup_f32", "k_prompt_down_f32"]) * n_pass
    if linked:
        labels_dec = ["k_pop_linked", "k_pop_finish"]
    elif fused:
        labels_dec = ["k_pop_step.1", "k_pop_step.2", "k_pop_finish"]
    else:
        labels_dec = None
    labels_dense = ["k_pop_step.0(dense)", "k_pop_finish(dense)"] if fused else None

    def kernel_pass(marks):
        for l in range(L):
            if n_tok > 0:
                a = pop.lib.pop_trace_recorded()
                pop.pop_dense_ffn_prefill(X[l], Wg[l], Wu[l], WdT[l], Y=Yp, ws=ws_ffn)
                marks.append((labels_ffn, a, pop.lib.pop_trace_recorded()))
            a = pop.lib.pop_trace_recorded()
            partition(l)
            marks.append((labels_pre, a, pop.lib.pop_trace_recorded()))
        for t in range(S):
            x_buf.copy_(Xdec[t])
            for l in range(L):
                a = pop.lib.pop_trace_recorded()
                pop.pop_decode_ffn(x_buf[l], Wg[l], Wu[l], WdT[l], R[l], C[l], w.r, y=y[l], ws=ws_dec)
                marks.append((labels_dec or ["decode"], a, pop.lib.pop_trace_recorded()))
            for l in range(L):
                a = pop.lib.pop_trace_recorded()
                pop.pop_dense_ffn_decode(x_buf[l], Wg[l], Wu[l], WdT[l], y=y[l], ws=ws_dec)
                marks.append((labels_dense or ["dense"], a, pop.lib.pop_trace_recorded()))

    n_ev = L * (len(labels_pre) + len(labels_ffn) + 3) + S * L * 12 + 8

    def traced(flags):
        tracer = pop.Tracer(n_ev, flags)
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        with tracer:
            kernel_pass([])
        host_s = time.perf_counter() - h0
        torch.cuda.synchronize()
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        a = Ev(torch).record()
        torch.cuda._sleep(20_000_000)
        b = Ev(torch).record()
        torch.cuda.synchronize()
        cyc_per_ms = 20_000_000 / max(a.ms(b), 1e-3)
        lead_ms = max(50.0, 3.0 * host_s * 1e3)
        torch.cuda._sleep(int(cyc_per_ms * lead_ms))
        marks = []
        with tracer:
            kernel_pass(marks)
        torch.cuda.synchronize()
        per = {}
        span = tracer.elapsed_ms(marks[0][1], marks[-1][2] - 1)
        busy = 0.0
        for labels, i0, i1 in marks:
            if i1 - i0 != len(labels) + 1:  # a launch shape other than the one assumed: number them
                labels = [f"{labels[0]}#{j}" for j in range(i1 - i0 - 1)]
            for j, name in enumerate(labels):
                dt = tracer.elapsed_ms(i0 + j, i0 + j + 1)
                per.setdefault(name, []).append(dt)
                busy += dt
        tracer.close()
        kus = {name: float(np.mean(v)) * 1e3 for name, v in per.items()}
        log(f"[bench] kernel pass (event flags {flags:#x}): host enqueue {host_s * 1e3:.1f} ms, "
            f"lead {lead_ms:.0f} ms, traced kernels cover {busy / span:.3f} of the span")
        log("[bench] kernels (us): " + ", ".join(f"{n} {v:.2f}" for n, v in kus.items()))
        return kus, busy / span

    # Events without the system-scope fence disturb the kernels between them
    # least; the default events are reported beside them.
    kus_fenced, _ = traced(0)
    kus, coverage = traced(pop.Tracer.DISABLE_SYSTEM_FENCE)

    roofline = None
    if linked:
        dom, dom_bytes = "k_pop_linked", metrics.linked_bytes(d, n_R, n_C, k, e)
        dom_symbol = metrics.linked_symbol(d, e)
        tb = profiling.traffic_bytes(dom_symbol) if w.name == MAIN_WORKLOAD else None
        dom_us = kus[dom]
        dom_gbps = dom_bytes / (dom_us * 1e-6) / 1e9
        roofline = {
            "kernel": "k_pop_linked (batch-1 decode step: candidate gate/up rows with the in-kernel top-k, every "
                      "retained channel's gate, up and W_downT rows, and the selected candidates' W_downT rows, in "
                      "one launch; k_pop_finish then adds the per-workgroup partial sums)",
            "bound": "hbm",
            "achieved": round(dom_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None if tb is None else tb[0] + tb[1],
            "traffic_source": (None if tb is None else
                               "rocprofv3 L2-to-memory read and write requests per dispatch (every L2 instance), "
                               "checked against a stream-read probe and a fill of known size in the same passes "
                               "(profiles/ffn_kernels_llama2_7b_b1_hbm_traffic.md)"),
            "bytes_per_launch": dom_bytes,
            "avg_launch_us": round(dom_us, 3),
            "achieved_vs_read_probe": None,
        }
    res["roofline"] = roofline
    res["decode"]["eager_us_per_layer_step"] = round(float(np.median(eager_ms)) / L * 1e3, 3)
    res["ablation"] = {
        "static_prefill_mask": {"us_per_layer_step": round(ms_static / L * 1e3, 3),
                                "algorithmic_bytes": metrics.decode_bytes(d, n_live, 0, 0, B, e)},
        "full_reevaluation": {"us_per_layer_step": round(ms_full / L * 1e3, 3),
                              "algorithmic_bytes": metrics.decode_bytes(d, 0, d_ff, n_live, B, e)},
        "pop": {"us_per_layer_step": round(t_ls * 1e3, 3), "algorithmic_bytes": bytes_ls},
        "pop_time_over_static": round(t_ls * L / ms_static - 1.0, 4),
        "full_time_over_static": round(ms_full / ms_static - 1.0, 4),
        "periodic_refresh": {str(p): {"us_per_layer_step": round(v * 1e3, 3), "refresh_every": p,
                                      "kernels": "stage entry points (gate/up, select, down) + memory kernels"}
                             for p, v in periodic.items()},
    }
    res["prefill_layer_us"] = {
        "fused": round(ms_pre / L * 1e3, 2),
        "unfused": round(ms_unfused / L * 1e3, 2),
        "fused_call": "pop_prefill_ffn_partition (column norms, prompt FFN with the importance in its gate/up pass, "
                      "partition); unfused: pop_dense_ffn_prefill + pop_prefill_partition",
    }
    res["prompt_ffn"] = {
        "us_per_layer": round(ms_pffn / L * 1e3, 2),
        "flops_per_layer": pffn_flops,
        "tflops": round(pffn_tflops, 1),
        "mfma_frac_bf16_dense_peak": round(pffn_tflops / 2500.0, 4) if e == 2 else None,
        "kernels": "k_prompt_gateup + k_prompt_down (v_mfma_f32_16x16x32_bf16)" if e == 2 else "fp32 FMA",
    }
    res["kernel_pass_coverage"] = round(coverage, 4)
    res["kernels_us"] = {n: round(v, 3) for n, v in kus.items()}
    res["kernels_us_default_events"] = {n: round(v, 3) for n, v in kus_fenced.items()}
    imp_bytes = metrics.importance_bytes(n_tok, d, d_ff, e)
    res["importance_gbps"] = (round(imp_bytes / (kus["k_importance_items"] * 1e-6) / 1e9, 1)
                              if "k_importance_items" in kus else None)
    # host copies of layer 0 (as timed: the same device-drawn tensors) for the oracle's spot check
    x_buf.copy_(Xdec[0])
    _, S0 = pop.pop_decode_ffn(x_buf[0], Wg[0], Wu[0], WdT[0], R[0], C[0], w.r, y=y[0], selected=True, ws=ws_dec)
    torch.cuda.synchronize()
    f32 = lambda t: t.float().cpu().numpy()
    res["_spot"] = {"W_gate": f32(Wg[0]), "W_up": f32(Wu[0]), "W_downT": f32(WdT[0]), "X": f32(X[0]),
                    "x": f32(Xdec[0, 0]), "R": R[0].cpu().numpy(), "C": C[0].cpu().numpy(),
                    "P": P[0].cpu().numpy(), "I": I_l[0].cpu().numpy(), "S": S0.cpu().numpy(), "y": y[0].cpu().numpy()}
    return res


def bench_moe(args, w, mods, L, T, steps, warmup, detail):
    """The mixture-of-experts workload: per layer, the per-expert partition of
    the prompt (routed tokens only), then every decode step through
    pop_moe_decode_ffn (routing, per-expert POP step, weighted combine).  The
    step is the partition of every layer + every decode step over every layer
    (there is no MoE prompt FFN in this library).  The dense comparator runs
    the same kernels with every channel retained and no candidates."""
    np, torch, metrics, pop, synth = mods
    B, E, d, d_ff = w.decode_batch, w.experts, w.d, w.d_ff
    e = 2 if w.dtype == "bf16" else 4
    n_tok = w.prompt_batch * w.prompt_len
    dev = torch.device("cuda")
    cnt = pop.pop_partition_counts(d_ff, w.r, w.gamma)
    n_R, n_C, n_P, k = cnt["n_R"], cnt["n_C"], cnt["n_P"], cnt["k"]
    log(f"[bench] {w.name}: {L} layers x {E} experts, d={d}, d_ff={d_ff}, prompt {n_tok} tokens, T={T}, "
        f"{B} tokens per step, top-2; per expert |R|={n_R} |C|={n_C} |P|={n_P} k={k}")
    t0 = time.time()
    Wg, Wu, WdT, X = [], [], [], []
    for l in range(L):
        parts = [synth.torch_layer_weights(w, l * E + x, dev) for x in range(E)]
        for dst, name in ((Wg, "W_gate"), (Wu, "W_up"), (WdT, "W_downT")):
            dst.append(torch.stack([q[name] for q in parts]).contiguous())
        del parts
        X.append(synth.torch_activations(w, (n_tok, d), l, 0, dev))
    logits_pre, logits_dec, Xdec = synth.torch_moe_inputs(w, L, T, dev)
    R = [torch.empty((E, n_R), dtype=torch.int32, device=dev) for _ in range(L)]
    C = [torch.empty((E, n_C), dtype=torch.int32, device=dev) for _ in range(L)]
    P = [torch.empty((E, n_P), dtype=torch.int32, device=dev) for _ in range(L)]
    R_all = torch.arange(d_ff, dtype=torch.int32, device=dev).repeat(E, 1).contiguous()
    C_none = torch.empty((E, 0), dtype=torch.int32, device=dev)
    x_buf = torch.empty((L, B, d), dtype=Xdec.dtype, device=dev)
    lg_buf = torch.empty((L, B, E), dtype=torch.float32, device=dev)
    y = torch.empty((L, B, d), dtype=torch.float32, device=dev)
    ws_pre = pop.workspace(int(pop.lib.pop_moe_prefill_workspace_bytes(n_tok, d, d_ff, E)), dev)
    ws_dec = pop.workspace(pop.pop_moe_decode_workspace_bytes(B, d, d_ff, E), dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs generated on the device in {time.time() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")

    def prefill():
        for l in range(L):
            pop.pop_moe_prefill_partition(X[l], logits_pre[l], Wu[l], w.r, w.gamma, out=(R[l], C[l], P[l], None),
                                          ws=ws_pre)

    def decode_layers():
        for l in range(L):
            pop.pop_moe_decode_ffn(x_buf[l], lg_buf[l], Wg[l], Wu[l], WdT[l], R[l], C[l], w.r, y=y[l], ws=ws_dec)

    def dense_layers():
        for l in range(L):
            pop.pop_moe_decode_ffn(x_buf[l], lg_buf[l], Wg[l], Wu[l], WdT[l], R_all, C_none, 0.0, y=y[l], ws=ws_dec)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        x_buf.copy_(Xdec[0])
        lg_buf.copy_(logits_dec[0])
        prefill()
        decode_layers()
        dense_layers()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = {}
    for name, fn in (("prefill", prefill), ("decode", decode_layers), ("dense", dense_layers)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs[name] = g
    torch.cuda.synchronize()

    def step_of(name):
        def run(t):
            x_buf.copy_(Xdec[t])
            lg_buf.copy_(logits_dec[t])
            graphs[name].replay()
        return run

    def job():
        graphs["prefill"].replay()
        run = step_of("decode")
        for t in range(T):
            run(t)

    for _ in range(warmup):
        job()
    torch.cuda.synchronize()
    ms_step = timed(torch, job, steps)
    value = B * T * L / (ms_step / 1e3)
    log(f"[bench] step {ms_step:.2f} ms -> {value:,.0f} tokens/s/layer")
    ms_pre = timed(torch, lambda: graphs["prefill"].replay(), 3)
    dec_ms = per_step_ms(torch, step_of("decode"), T)
    dense_ms = per_step_ms(torch, step_of("dense"), T)
    t_ls, t_ls_dense = float(np.median(dec_ms)) / L, float(np.median(dense_ms)) / L

    # experts reached per step (top-2 of the step's logits), for the byte counts
    top2 = torch.topk(logits_dec, 2, dim=-1).indices.view(T, L, B * 2).cpu().numpy()
    active = float(np.mean([[len(np.unique(top2[t, l])) for l in range(L)] for t in range(T)]))
    bytes_ls = metrics.moe_decode_bytes(d, n_R, n_C, k, active, B, e)
    bytes_dense = metrics.moe_decode_bytes(d, d_ff, 0, 0, active, B, e)
    gateup_bytes = active * (2 * (n_R + n_C) * d * e)
    log(f"[bench] MoE decode {t_ls * 1e3:.1f} us/layer-step ({bytes_ls / (t_ls * 1e-3) / 1e9:.0f} GB/s, "
        f"{active:.2f} experts reached per step), dense {t_ls_dense * 1e3:.1f} us "
        f"({bytes_dense / (t_ls_dense * 1e-3) / 1e9:.0f} GB/s), partition {ms_pre / L * 1e3:.1f} us/layer")
    res = {
        "value": round(value, 1),
        "ms_per_step": round(ms_step, 4),
        "data": "synthetic (seeded device-drawn expert weights N(0,0.02^2), activations and N(0,1) router logits)",
        "config": {
            "workload": w.name, "layers": L, "experts": E, "route_top_k": 2, "d": d, "d_ff": d_ff, "r_ffn": w.r,
            "gamma": w.gamma, "prompt_tokens": n_tok, "decode_steps": T, "tokens_per_step": B, "hip_graphs": True,
            "step": "per-expert prefill partition of every layer + every decode step over every layer",
        },
        "decode": {
            "us_per_layer_step": round(t_ls * 1e3, 3),
            "us_per_layer_step_spread": spread(np, dec_ms, 1e3 / L),
            "experts_reached_per_step": round(active, 3),
            "algorithmic_bytes_per_layer_step": round(bytes_ls),
            "hbm_gbps": round(bytes_ls / (t_ls * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes_ls / (t_ls * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        },
        "dense_decode": {
            "us_per_layer_step": round(t_ls_dense * 1e3, 3),
            "us_per_layer_step_spread": spread(np, dense_ms, 1e3 / L),
            "algorithmic_bytes_per_layer_step": round(bytes_dense),
            "hbm_gbps": round(bytes_dense / (t_ls_dense * 1e-3) / 1e9, 1),
        },
        "speedup_vs_dense": round(t_ls_dense / t_ls, 4),
        "ideal_speedup_bytes": round(bytes_dense / bytes_ls, 4),
        "prefill_partition_us_per_layer": round(ms_pre / L * 1e3, 2),
    }
    if not detail:
        return res

    # per-kernel pass: the decode calls with libpop's trace hook
    S = min(args.kernel_steps, T)
    mfma = e == 2 and B <= 64   # the library's dispatch: bf16 steps of up to 64 tokens on the matrix cores
    topk = n_C > 0 and k > 0
    if mfma:
        gu = "k_gateup_lds"
        labels_dec = (["k_moe_top2", "k_moe_bucket", gu] + (["k_moe_topk"] if topk and n_C > 4096 else [])
                      + ["k_down_stream.R+topk" if topk and n_C <= 4096 else "k_down_stream.R"]
                      + (["k_down_stream.S"] if k > 0 else []) + ["k_moe_combine"])
        labels_dense = ["k_moe_top2", "k_moe_bucket", gu + "(dense)", "k_down_stream.R(dense)", "k_moe_combine"]
    else:
        gu = "k_moe_gateup"
        labels_dec = ["k_moe_top2", "k_moe_bucket", gu] + (["k_moe_topk"] if topk else []) + [
            "k_moe_down", "k_moe_combine"]
        labels_dense = ["k_moe_top2", "k_moe_bucket", gu + "(dense)", "k_moe_down(dense)", "k_moe_combine"]
    tracer = pop.Tracer(S * L * (len(labels_dec) + len(labels_dense) + 2) + 8, pop.Tracer.DISABLE_SYSTEM_FENCE)
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    marks = []
    with tracer:
        for t in range(S):
            x_buf.copy_(Xdec[t])
            lg_buf.copy_(logits_dec[t])
            for l in range(L):
                a = pop.lib.pop_trace_recorded()
                pop.pop_moe_decode_ffn(x_buf[l], lg_buf[l], Wg[l], Wu[l], WdT[l], R[l], C[l], w.r, y=y[l], ws=ws_dec)
                marks.append((labels_dec, a, pop.lib.pop_trace_recorded()))
            for l in range(L):
                a = pop.lib.pop_trace_recorded()
                pop.pop_moe_decode_ffn(x_buf[l], lg_buf[l], Wg[l], Wu[l], WdT[l], R_all, C_none, 0.0, y=y[l],
                                       ws=ws_dec)
                marks.append((labels_dense, a, pop.lib.pop_trace_recorded()))
    torch.cuda.synchronize()
    per = {}
    for labels, i0, i1 in marks:
        if i1 - i0 != len(labels) + 1:
            labels = [f"{labels[0]}#{j}" for j in range(i1 - i0 - 1)]
        for j, name in enumerate(labels):
            per.setdefault(name, []).append(tracer.elapsed_ms(i0 + j, i0 + j + 1))
    tracer.close()
    kus = {n: float(np.mean(v)) * 1e3 for n, v in per.items()}
    log("[bench] kernels (us): " + ", ".join(f"{n} {v:.2f}" for n, v in kus.items()))
    dom_us = kus.get(gu)
    dom_gbps = gateup_bytes / (dom_us * 1e-6) / 1e9 if dom_us else None
    res["roofline"] = {
        "kernel": f"{gu} (MoE decode gate/up over each reached expert's R u C for its routed tokens)",
        "bound": "hbm",
        "achieved": None if dom_gbps is None else round(dom_gbps, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": None if dom_gbps is None else round(dom_gbps / HBM_PEAK_GBPS, 4),
        "traffic": None,
        "bytes_per_launch": round(gateup_bytes),
        "avg_launch_us": None if dom_us is None else round(dom_us, 3),
    }
    res["kernels_us"] = {n: round(v, 3) for n, v in kus.items()}
    return res


def bench_layer(args, w, np, torch, metrics, pop, synth):
    """Chained decoder layers (dense attention, POP's FFN): the prompt's pass
    through every layer (pop_layer_prefill: attention over the prompt, the
    dense prompt FFN and the partition, the key/value caches filled), then every
    decode step through every layer (pop_layer_decode), the position advanced on
    the device inside each step's graph.  The dense comparator runs the same
    layers with the dense FFN."""
    from online_structured_ffn_amd import profiling
    a = w.extra["attention"]
    H, Hkv, hd = a["n_heads"], a["n_kv_heads"], a["head_dim"]
    L = args.layers or w.layers
    T = args.decode_steps or w.decode_steps
    B, N, d, d_ff = w.decode_batch, w.prompt_len, w.d, w.d_ff
    if w.prompt_batch != B:
        raise ValueError("the decoder-layer workload decodes the sequences it prompted (prompt_batch == decode_batch)")
    e = 2 if w.dtype == "bf16" else 4
    Lc = N + T
    dev = torch.device("cuda")
    cnt = pop.pop_partition_counts(d_ff, w.r, w.gamma)
    n_R, n_C, n_P, k = cnt["n_R"], cnt["n_C"], cnt["n_P"], cnt["k"]
    log(f"[bench] {w.name}: {L} chained layers, d={d}, {H} heads ({Hkv} kv) of {hd}, d_ff={d_ff}, "
        f"prompt {B}x{N}, T={T}; FFN |R|={n_R} |C|={n_C} |P|={n_P} k={k}")
    t0 = time.time()
    layers = []
    for l in range(L):
        wts = dict(synth.torch_layer_weights(w, l, dev))
        wts.update(synth.torch_attention_weights(w, l, dev))
        layers.append(pop.Layer(d, H, Hkv, hd, d_ff, Lc, wts, eps=a["eps"], rope_theta=a["rope_theta"]))
    caches = [lay.cache(B) for lay in layers]
    X0 = synth.torch_activations(w, (B * N, d), 0, 0, dev).float().view(B, N, d).contiguous()
    Xdec = synth.torch_activations(w, (T * B, d), 0, 1, dev).float().view(T, B, d).contiguous()
    x_pre = torch.empty_like(X0)
    x_buf = torch.empty((B, d), dtype=torch.float32, device=dev)
    pos = torch.zeros(1, dtype=torch.int32, device=dev)
    R = [torch.empty(n_R, dtype=torch.int32, device=dev) for _ in range(L)]
    C = [torch.empty(n_C, dtype=torch.int32, device=dev) for _ in range(L)]
    P = [torch.empty(n_P, dtype=torch.int32, device=dev) for _ in range(L)]
    ws_pre = pop.workspace(pop.pop_layer_prefill_workspace_bytes(B, N, layers[0]), dev)
    ws_dec = pop.workspace(pop.pop_layer_decode_workspace_bytes(B, layers[0]), dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs generated on the device in {time.time() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")
    if args.copy_probe_mib > 0:  # a copy of known size, to scale the profiler's byte counters
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 3 copies of {args.copy_probe_mib} MiB ({n} bytes read and written each)")
        del src, dst

    def prefill():
        x_pre.copy_(X0)
        for l in range(L):
            pop.pop_layer_prefill(x_pre, layers[l], *caches[l], w.r, w.gamma, out=(R[l], C[l], P[l], None),
                                  ws=ws_pre)
        pos.fill_(N)

    def step(dense):
        def run():
            for l in range(L):
                pop.pop_layer_decode(x_buf, layers[l], *caches[l], pos, R[l], C[l], w.r, dense_ffn=dense, ws=ws_dec)
            pos.add_(1)
        return run

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prefill()
        x_buf.copy_(Xdec[0])
        step(False)()
        step(True)()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = {}
    for name, fn in (("prefill", prefill), ("decode", step(False)), ("dense", step(True))):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs[name] = g
    torch.cuda.synchronize()

    def steps(name):
        def run():
            for t in range(T):
                x_buf.copy_(Xdec[t])
                graphs[name].replay()
        return run

    def job():
        graphs["prefill"].replay()
        steps("decode")()

    def timed(fn, reps, before=None):
        if before is not None:
            before()
        torch.cuda.synchronize()
        a_ = Ev(torch).record()
        for _ in range(reps):
            fn()
        b_ = Ev(torch).record()
        torch.cuda.synchronize()
        return a_.ms(b_) / reps

    for _ in range(args.warmup):
        job()
    torch.cuda.synchronize()
    ms_step = timed(job, args.steps)
    value = B * T * L / (ms_step / 1e3)
    log(f"[bench] step {ms_step:.2f} ms -> {value:,.0f} tokens/s/layer ({B * T / (ms_step / 1e3):,.1f} tokens/s "
        f"through all {L} layers)")
    ms_pre = timed(lambda: graphs["prefill"].replay(), 3)
    reset = lambda: pos.fill_(N)
    ms_dec = timed(steps("decode"), 1, reset)
    ms_dense = timed(steps("dense"), 1, reset)
    t_ls, t_ls_dense = ms_dec / (T * L), ms_dense / (T * L)
    n_keys_avg = N + (T + 1) / 2
    att = metrics.attention_decode_bytes(d, H, Hkv, hd, n_keys_avg, B, e)
    att_bytes = sum(att.values())
    bytes_ls = att_bytes + metrics.decode_bytes(d, n_R, n_C, k, B, e) + 2 * B * d * 4
    bytes_dense = att_bytes + metrics.dense_decode_bytes(d, d_ff, B, e) + 2 * B * d * 4
    log(f"[bench] layer decode {t_ls * 1e3:.1f} us/layer-step ({bytes_ls / (t_ls * 1e-3) / 1e9:.0f} GB/s), "
        f"dense FFN {t_ls_dense * 1e3:.1f} us ({bytes_dense / (t_ls_dense * 1e-3) / 1e9:.0f} GB/s); "
        f"prefill {ms_pre / L * 1e3:.1f} us/layer")

    # per-kernel pass: the decode calls with libpop's trace hook
    S = min(args.kernel_steps, T)
    # the library's batch <= 2 form runs the attention RMSNorm inside the q|k|v projection
    head = ((["k_gemv_kmajor(norm+qkv)"] if B <= 2 else ["k_rmsnorm", "k_gemv_kmajor(qkv)"])
            + ["k_qkv_rope", "k_attn_decode"]
            + (["k_gemv_kmajor(merge+o)"] if B <= 2 else ["k_attn_merge", "k_gemv_kmajor(o)"])
            + ["k_sum_residual", "k_rmsnorm(ffn)", "-"])
    if B >= 12 and e == 2:   # the library bf16 form from 12 tokens: both projections on the matrix cores
        head = [{"k_gemv_kmajor(qkv)": "k_gemm_decode(qkv)", "k_gemv_kmajor(o)": "k_gemm_decode(o)"
                 }.get(n, n) for n in head]
    if B > 1:   # the library's batch-2..64 FFN kernels (bf16, matrix cores), then the residual add
        # the selected rows ride in the retained rows' launch (their chunks' shares of C)
        mfma_tail = (["k_gateup_lds"] + (["k_topk"] if n_C > 4096 else [])
                     + ["k_down_stream.R+S+topk" if n_C <= 4096 else "k_down_stream.R+S", "k_sum_few(y)"])
        dense_tail = ["k_gateup_lds(dense)", "k_down_stream(dense)", "k_sum_few(y)"]
    linked = B == 1 and 0 < n_C <= 4096 and k > 0
    # at batch 1 the FFN's last kernel adds its output into the residual stream (no k_add)
    if B == 1:
        labels_pop = head + (["k_pop_linked", "k_pop_finish(+h)"] if linked else ["ffn#0"])
        labels_dense = head + ["k_pop_step.0(dense)", "k_pop_finish(dense,+h)"]
    else:
        labels_pop = head + mfma_tail + ["k_add"]
        labels_dense = head + dense_tail + ["k_add"]
    tracer = pop.Tracer(S * L * (len(labels_pop) + len(labels_dense) + 2) + 8, pop.Tracer.DISABLE_SYSTEM_FENCE)
    marks = []
    for dense, labels in ((False, labels_pop), (True, labels_dense)):
        pos.fill_(N)
        torch.cuda.synchronize()
        torch.cuda._sleep(50_000_000)
        with tracer:
            for t in range(S):
                x_buf.copy_(Xdec[t])
                for l in range(L):
                    i0 = pop.lib.pop_trace_recorded()
                    pop.pop_layer_decode(x_buf, layers[l], *caches[l], pos, R[l], C[l], w.r, dense_ffn=dense,
                                         ws=ws_dec)
                    marks.append((labels, i0, pop.lib.pop_trace_recorded()))
                pos.add_(1)
        torch.cuda.synchronize()
        # the tracer's events are re-armed for the second pass: read this pass now
        per_pass = {}
        for labels_, a0, a1 in marks:
            if a1 - a0 != len(labels_) + 1:
                labels_ = [f"{labels_[0]}#{j}" for j in range(a1 - a0 - 1)]
            for j, name in enumerate(labels_):
                per_pass.setdefault(name, []).append(tracer.elapsed_ms(a0 + j, a0 + j + 1))
        marks = []
        if not dense:
            per_pop = per_pass
        else:
            per_dense = per_pass
    tracer.close()
    kus = {n: float(np.mean(v)) * 1e3 for n, v in per_pop.items() if n != "-"}
    kus_dense = {n: float(np.mean(v)) * 1e3 for n, v in per_dense.items() if n != "-"}
    log("[bench] kernels (us): " + ", ".join(f"{n} {v:.2f}" for n, v in kus.items()))
    log("[bench] dense-FFN layer kernels (us): " + ", ".join(f"{n} {v:.2f}" for n, v in kus_dense.items()))
    att_k = metrics.attention_decode_bytes(d, H, Hkv, hd, N + (S + 1) / 2, B, e)
    kbytes = {head[0] if B <= 2 else head[1]: att_k["qkv"],
              "k_gemv_kmajor(merge+o)" if B <= 2 else head[5]: att_k["o"], "k_attn_decode": att_k["attn"]}
    if linked:
        kbytes.update({"k_pop_linked": metrics.linked_bytes(d, n_R, n_C, k, e),
                       "k_pop_finish(+h)": metrics.linked_finish_bytes(d, n_R, n_C) + 4 * d})
    dom = max((n for n in kbytes if n in kus), key=lambda n: kus[n], default=None)
    dom_gbps = kbytes[dom] / (kus[dom] * 1e-6) / 1e9 if dom else None
    # the same kernel at the same shape as the FFN workload's profiled one: its counters apply
    same_ffn = dom == "k_pop_linked" and (d, d_ff, w.r, w.gamma, B, w.dtype) == (4096, 11008, 0.299, 0.1, 1, "bf16")
    tb = profiling.traffic_bytes(metrics.linked_symbol(d, e)) if same_ffn else None
    cpu = None if args.no_cpu_baseline else cpu_baseline_layer(w, T, args.cpu_seconds)
    out = {
        "metric": "decoder-layer decode tokens/s per layer (dense attention + POP FFN); HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded device-drawn weights N(0,0.02^2), RMSNorm gains 1, token inputs N(0,1); "
                "no dataset, no trained weights)",
        "config": {
            "workload": w.name, "layers": L, "d": d, "n_heads": H, "n_kv_heads": Hkv, "head_dim": hd,
            "d_ff": d_ff, "r_ffn": w.r, "gamma": w.gamma, "prompt_tokens": B * N, "decode_steps": T,
            "decode_batch": B, "cache_len": Lc, "hip_graphs": True, "streams": 1,
            "step": "the prompt's pass through every chained layer + every decode step through every layer",
        },
        "roofline": {
            "kernel": f"{dom} (the decoder layer's longest decode kernel)",
            "bound": "hbm",
            "achieved": None if dom_gbps is None else round(dom_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": None if dom_gbps is None else round(dom_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None if tb is None else tb[0] + tb[1],
            "traffic_source": (None if tb is None else
                               "rocprofv3 L2-to-memory read and write requests per dispatch of the same kernel at "
                               "the same shape in the FFN workload "
                               "(profiles/ffn_kernels_llama2_7b_b1_hbm_traffic.md)"),
            "bytes_per_launch": None if dom is None else round(kbytes[dom]),
            "avg_launch_us": None if dom is None else round(kus[dom], 3),
        },
        "decode": {
            "us_per_layer_step": round(t_ls * 1e3, 3),
            "tokens_per_s_through_the_stack": round(B / (t_ls * L * 1e-3), 1),
            "algorithmic_bytes_per_layer_step": round(bytes_ls),
            "hbm_gbps": round(bytes_ls / (t_ls * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes_ls / (t_ls * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        },
        "dense_ffn_decode": {
            "us_per_layer_step": round(t_ls_dense * 1e3, 3),
            "algorithmic_bytes_per_layer_step": round(bytes_dense),
            "hbm_gbps": round(bytes_dense / (t_ls_dense * 1e-3) / 1e9, 1),
        },
        "speedup_vs_dense_ffn": round(t_ls_dense / t_ls, 4),
        "ideal_speedup_bytes": round(bytes_dense / bytes_ls, 4),
        "prefill_layer_us": round(ms_pre / L * 1e3, 2),
        "kernels_us": {n: round(v, 3) for n, v in kus.items()},
        "kernels_us_dense_ffn": {n: round(v, 3) for n, v in kus_dense.items()},
        "kernel_bytes": {n: round(v) for n, v in kbytes.items()},
        "cpu_baseline": cpu,
    }
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def cpu_baseline_layer(w, T, budget_s):
    """The layer oracle, as it stands, on layer 0 of the decoder-layer
    workload: the prompt's pass, then as many decode steps as fit in the
    budget, scaled to tokens/s/layer as the GPU value is."""
    import numpy as np

    import oracle
    from online_structured_ffn_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    a = w.extra["attention"]
    cfg = {"H": a["n_heads"], "H_kv": a["n_kv_heads"], "hd": a["head_dim"], "eps": a["eps"],
           "theta": a["rope_theta"]}
    lw = dict(synth.attention_weights(w, 0))
    lw.update(synth.layer_weights(w, 0))
    B, N = w.decode_batch, w.prompt_len
    X = synth.prompt(w, 0).reshape(B, N, w.d)
    t0 = time.perf_counter()
    pre = oracle.layer.layer_prefill(X, lw, cfg, w.r, w.gamma, w.dtype, N + T)
    t_pre = time.perf_counter() - t0
    K, V = pre["K"], pre["V"]
    times = []
    t_start = time.perf_counter()
    step = 0
    while step < T and (time.perf_counter() - t_start) < budget_s:
        x = synth.decode_input(w, 0, step)
        t0 = time.perf_counter()
        oracle.layer.layer_decode(x, lw, cfg, K, V, N + step, pre["R"], pre["C"], w.r, w.dtype)
        times.append(time.perf_counter() - t0)
        step += 1
    t_dec = float(np.median(times))
    value = B * T / (t_pre + T * t_dec)
    return {
        "value": round(value, 3),
        "unit": "tokens/s/layer",
        "cores": blas_threads if blas_threads is not None else len(os.sched_getaffinity(0)),
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"layer 0 of {w.name}: the {N}-token prompt pass ({t_pre:.2f} s) + {len(times)} decode steps "
                  f"(median {t_dec * 1e3:.1f} ms), numpy fp64; value = B*T / (t_prefill + T * t_step)",
    }




def _host_info():
    """CPU model, usable CPUs and the BLAS library numpy calls."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = {"library": libs[0].get("internal_api"), "version": libs[0].get("version"),
                    "threads": libs[0].get("num_threads")}
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "host_cpus": len(os.sched_getaffinity(0)), "blas": blas}


def spot_check(w, spot):
    """The oracle on layer 0 of the timed inputs (the same device-drawn
    tensors, copied to the host): the importance, the partition (exactly, on
    the device's importance; against fp64 with near-tie exclusions) and the
    first decode step's output on the device's selection."""
    import numpy as np

    import oracle
    Wg, Wu, WdT, X, x = (spot[n] for n in ("W_gate", "W_up", "W_downT", "X", "x"))
    R, C, P, I_dev, S, y_dev = (spot[n] for n in ("R", "C", "P", "I", "S", "y"))
    I_ref = oracle.importance(Wu, oracle.column_norm(X))
    I_err = float(np.abs(I_dev - I_ref).max() / max(I_ref.max(), 1e-30))
    eR, eC, eP = oracle.partition(I_dev.astype(np.float64), w.r, w.gamma)
    exact = bool(np.array_equal(R, eR) and np.array_equal(C, eC) and np.array_equal(P, eP))
    oR, oC, _ = oracle.partition(I_ref, w.r, w.gamma)
    lab = lambda a, b: np.isin(np.arange(w.d_ff), a) * 2 + np.isin(np.arange(w.d_ff), b)
    part_diff = int((lab(R, C) != lab(oR, oC)).sum())
    ref = oracle.decode_step(x, Wg, Wu, WdT.T, R, C, w.r)
    sel_diff = int(len(np.setxor1d(S, ref["S"])))
    y_ref = oracle.masked_ffn(x, Wg, Wu, WdT.T, np.concatenate([R, S]))
    y_err = float(np.abs(y_dev - y_ref).max() / max(np.abs(y_ref).max(), 1e-30))
    ok = exact and I_err <= 1e-4 and y_err <= 2e-2
    return {"layer": 0, "decode_step": 0, "importance_max_rel_err": I_err, "partition_exact_on_device_I": exact,
            "partition_channels_differing_from_fp64": part_diff, "selected_differing_from_fp64": sel_diff,
            "y_max_rel_err_on_device_selection": y_err, "pass": bool(ok),
            "bar": "partition exact on the device's importance; importance within 1e-4 and y within 2e-2 of "
                   "max|y| (bf16 weights, fp32 accumulation)"}


def cpu_baseline(w, T, budget_s):
    """The CPU oracle, as it stands, on layer 0 of the same workload: one
    prefill (dense prompt FFN and partition) and as many decode layer-steps as
    fit in the budget, once with every core numpy's BLAS uses and once on one
    thread.  Scaled to tokens/s/layer the way the GPU value is: the prefill's
    time is spread over the T decode steps of the request."""
    import numpy as np

    import oracle
    from online_structured_ffn_amd import synth
    info = _host_info()
    wts = synth.layer_weights(w, 0)
    X = synth.prompt(w, 0)
    B = w.decode_batch

    def sample(budget):
        t0 = time.perf_counter()
        oracle.dense_ffn(X, wts["W_gate"], wts["W_up"], wts["W_down"])
        R, C, _ = oracle.partition(oracle.importance(wts["W_up"], oracle.column_norm(X)), w.r, w.gamma)
        t_part = time.perf_counter() - t0
        times = []
        t_start = time.perf_counter()
        step = 0
        while step < T and (time.perf_counter() - t_start) < budget:
            x = synth.decode_input(w, 0, step)
            t0 = time.perf_counter()
            oracle.decode_step(x, wts["W_gate"], wts["W_up"], wts["W_down"], R, C, w.r)
            times.append(time.perf_counter() - t0)
            step += 1
        t_dec = float(np.median(times))
        return B * T / (t_part + T * t_dec), t_part, t_dec, len(times)

    v_all, tp_all, td_all, n_all = sample(budget_s)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            v1, tp1, td1, n1 = sample(budget_s / 2)
        one = {"value": round(v1, 3), "cores": 1,
               "sample": f"1 prefill ({tp1:.2f} s) + {n1} decode layer-steps (median {td1 * 1e3:.1f} ms)"}
    except Exception as exc:  # noqa: BLE001
        one = {"error": repr(exc)}
    blas_threads = (info["blas"] or {}).get("threads")
    out = {
        "value": round(v_all, 3),
        "unit": "tokens/s/layer",
        "cores": blas_threads if blas_threads is not None else info["host_cpus"],
        "kind": "oracle",
        "sample": f"layer 0 of {w.name}: 1 prefill (dense prompt FFN + partition, {tp_all:.2f} s) + {n_all} "
                  f"decode layer-steps (median {td_all * 1e3:.1f} ms), numpy fp64; "
                  "value = B*T / (t_prefill + T * t_step)",
        "one_thread": one,
        "host": info,
    }
    return out


if __name__ == "__main__":
    main()
