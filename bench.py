#!/usr/bin/env python3
"""Benchmark of the POP channel-pruned gated-MLP path on one MI355X.

One step is one whole request of the workload with every input already in
HBM: the prefill partition of every layer (column norm, importance, three-region
select) followed by every decode step over every layer (gate/up over R u C with
fused scores, candidate top-k, gathered down-projection).  The layers do not
chain: each has its own seeded prompt and decode inputs.  Steps are replayed as
HIP graphs.

Printed: ONE JSON line on stdout.  value = decode tokens per second per layer
over the whole step (B * T * layers / step time), i.e. the prefill partition is
included in the denominator.

Per-kernel durations for the roofline come from a second, eager pass in which
HIP events bracket each stage call; a spin kernel queued first keeps the GPU
busy while the host enqueues, so the events time the kernels back to back.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "pruned FFN decode tokens/s per layer + HBM GB/s vs peak; prefill partition µs"
HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama2_7b_ffn_b1")
    ap.add_argument("--layers", type=int, default=None, help="default: the workload's layer count")
    ap.add_argument("--decode-steps", type=int, default=None, help="default: the workload's decode steps")
    ap.add_argument("--kernel-steps", type=int, default=4, help="decode steps in the per-kernel timing pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle timing sample")
    ap.add_argument("--json-out", default=None)
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

    w = configs.BY_NAME[args.workload]
    if w.experts:
        print("the MoE workload has no bench line yet", file=sys.stderr)
        sys.exit(2)
    L = args.layers or w.layers
    T = args.decode_steps or w.decode_steps
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

    # ------------------------------------------------------------ inputs in HBM
    t0 = time.time()
    Wg, Wu, WdT, X = [], [], [], []
    for l in range(L):
        ws_ = synth.torch_layer_weights(w, l, dev)
        Wg.append(ws_["W_gate"])
        Wu.append(ws_["W_up"])
        WdT.append(ws_["W_downT"])
        chans = synth.outlier_channels(w, l)
        X.append(synth.torch_activations(w, (n_tok, d), l, 0, dev, chans))
    chans0 = synth.outlier_channels(w, 0) if w.outliers_in_decode else None
    Xdec = synth.torch_activations(w, (T * L * B, d), 0, 1, dev, chans0).view(T, L, B, d)
    R = [torch.empty(n_R, dtype=torch.int32, device=dev) for _ in range(L)]
    C = [torch.empty(n_C, dtype=torch.int32, device=dev) for _ in range(L)]
    P = [torch.empty(n_P, dtype=torch.int32, device=dev) for _ in range(L)]
    x_buf = torch.empty((L, B, d), dtype=Xdec.dtype, device=dev)
    y = torch.empty((L, B, d), dtype=torch.float32, device=dev)
    ws_pre = pop.workspace(pop.pop_prefill_workspace_bytes(n_tok, d, d_ff), dev)
    ws_dec = pop.workspace(pop.pop_decode_workspace_bytes(B, d, d_ff), dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs generated on the device in {time.time() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")

    def prefill():
        for l in range(L):
            pop.pop_prefill_partition(X[l], Wu[l], w.r, w.gamma, out=(R[l], C[l], P[l], None), ws=ws_pre)

    def decode_layers():
        for l in range(L):
            pop.pop_decode_ffn(x_buf[l], Wg[l], Wu[l], WdT[l], R[l], C[l], w.r, y=y[l], ws=ws_dec)

    def dense_layers():
        for l in range(L):
            pop.pop_dense_ffn_decode(x_buf[l], Wg[l], Wu[l], WdT[l], y=y[l], ws=ws_dec)

    # ------------------------------------------------------------ graphs
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        x_buf.copy_(Xdec[0])
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

    def job():
        graphs["prefill"].replay()
        for t in range(T):
            x_buf.copy_(Xdec[t])
            graphs["decode"].replay()

    def timed(fn, reps):
        torch.cuda.synchronize()
        a = Ev(torch).record()
        for _ in range(reps):
            fn()
        b = Ev(torch).record()
        torch.cuda.synchronize()
        return a.ms(b) / reps

    # ------------------------------------------------------------ timed region: whole steps
    for _ in range(args.warmup):
        job()
    torch.cuda.synchronize()
    ms_step = timed(job, args.steps)
    # B*T tokens pass through each of the L layers: B*T*L layer-tokens per second of the step
    value = B * T * L / (ms_step / 1e3)
    log(f"[bench] step {ms_step:.2f} ms -> {value:,.0f} tokens/s/layer")

    # ------------------------------------------------------------ component timings (graphs)
    ms_prefill = timed(lambda: graphs["prefill"].replay(), 5)

    def decode_only():
        for t in range(T):
            x_buf.copy_(Xdec[t])
            graphs["decode"].replay()

    def dense_only():
        for t in range(T):
            x_buf.copy_(Xdec[t])
            graphs["dense"].replay()

    ms_dec = timed(decode_only, 1)
    ms_dense = timed(dense_only, 1)
    t_ls = ms_dec / (T * L)          # ms per pruned layer-step
    t_ls_dense = ms_dense / (T * L)
    bytes_ls = metrics.decode_bytes(d, n_R, n_C, k, B, e)
    bytes_dense = metrics.dense_decode_bytes(d, d_ff, B, e)
    log(f"[bench] decode {t_ls * 1e3:.1f} us/layer-step ({bytes_ls / (t_ls * 1e-3) / 1e9:.0f} GB/s), "
        f"dense {t_ls_dense * 1e3:.1f} us ({bytes_dense / (t_ls_dense * 1e-3) / 1e9:.0f} GB/s), "
        f"prefill partition {ms_prefill / L * 1e3:.1f} us/layer")

    # ------------------------------------------------------------ per-kernel pass (eager, queued ahead)
    S = min(args.kernel_steps, T)
    zbuf = torch.empty((B, n_A), dtype=torch.float32, device=dev)
    score = torch.empty(n_C, dtype=torch.float32, device=dev)
    Q = torch.empty(k, dtype=torch.int32, device=dev)
    Ssel = torch.empty(k, dtype=torch.int32, device=dev)
    ws_down = pop.workspace(pop.lib.pop_decode_down_workspace_bytes(B, d, n_live), dev)
    I = torch.empty(d_ff, dtype=torch.float32, device=dev)
    ws_imp = pop.workspace(pop.lib.pop_prefill_importance_workspace_bytes(n_tok, d), dev)

    def kernel_pass(record):
        """Eager stage calls of every layer (prefill) and S decode steps; with
        record=True, events bracket every stage call."""
        out = []
        mk = (lambda: Ev(torch).record()) if record else (lambda: None)
        for l in range(L):
            e0 = mk()
            pop.pop_prefill_importance(X[l], Wu[l], out=I, ws=ws_imp)
            e1 = mk()
            pop.pop_partition_select(I, w.r, w.gamma, out=(R[l], C[l], P[l]))
            e2 = mk()
            out.append(("prefill", e0, e1, e2))
        for t in range(S):
            x_buf.copy_(Xdec[t])
            for l in range(L):
                e0 = mk()
                pop.pop_decode_gateup(x_buf[l], Wg[l], Wu[l], R[l], C[l], z=zbuf, score=score)
                e1 = mk()
                pop.pop_decode_select(score, C[l], k, positions=Q, selected=Ssel)
                e2 = mk()
                pop.pop_decode_down(zbuf, WdT[l], R[l], Ssel, Q, y=y[l], ws=ws_down)
                e3 = mk()
                out.append(("decode", e0, e1, e2, e3))
        return out

    # host enqueue time of the pass, and a warmed-up spin kernel calibrated on a long sleep
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    kernel_pass(True)
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
    start_ev = Ev(torch).record()
    evs = kernel_pass(True)
    end_ev = Ev(torch).record()
    torch.cuda.synchronize()
    span_ms = start_ev.ms(end_ev)
    windows_ms = sum(x[1].ms(x[-1]) for x in evs)
    log(f"[bench] kernel pass: host enqueue {host_s * 1e3:.1f} ms, lead {lead_ms:.0f} ms, "
        f"event windows cover {windows_ms / span_ms:.3f} of the span")
    imp_us = np.mean([x[1].ms(x[2]) for x in evs if x[0] == "prefill"]) * 1e3
    psel_us = np.mean([x[2].ms(x[3]) for x in evs if x[0] == "prefill"]) * 1e3
    gu_us = np.mean([x[1].ms(x[2]) for x in evs if x[0] == "decode"]) * 1e3
    sel_us = np.mean([x[2].ms(x[3]) for x in evs if x[0] == "decode"]) * 1e3
    dn_us = np.mean([x[3].ms(x[4]) for x in evs if x[0] == "decode"]) * 1e3
    gu_bytes = metrics.gateup_bytes(d, n_A, n_C, B, e)
    dn_bytes = metrics.down_bytes(d, n_live, B, e, k)
    imp_bytes = metrics.importance_bytes(n_tok, d, d_ff, e)
    gu_gbps = gu_bytes / (gu_us * 1e-6) / 1e9
    log(f"[bench] kernels (us): importance {imp_us:.1f}, partition-select {psel_us:.1f}, gate/up {gu_us:.1f} "
        f"({gu_gbps:.0f} GB/s), top-k {sel_us:.1f}, down {dn_us:.1f} ({dn_bytes / (dn_us * 1e-6) / 1e9:.0f} GB/s)")

    out = {
        "metric": METRIC,
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
        "data": "synthetic (seeded device-drawn weights N(0,0.02^2) and activations; no dataset, no trained weights)",
        "config": {
            "workload": w.name, "layers": L, "d": d, "d_ff": d_ff, "r_ffn": w.r, "gamma": w.gamma,
            "prompt_tokens": n_tok, "decode_steps": T, "decode_batch": B, "hip_graphs": True,
            "step": "prefill partition of every layer + every decode step over every layer",
        },
        "roofline": {
            "kernel": "k_gateup (decode gate/up over R u C, fused SiLU*up and candidate score)",
            "bound": "hbm",
            "achieved": round(gu_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "bytes_per_launch": gu_bytes,
            "avg_launch_us": round(gu_us, 3),
        },
        "decode": {
            "us_per_layer_step": round(t_ls * 1e3, 3),
            "tokens_per_s_per_layer": round(B / (t_ls * 1e-3), 1),
            "algorithmic_bytes_per_layer_step": bytes_ls,
            "hbm_gbps": round(bytes_ls / (t_ls * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes_ls / (t_ls * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        },
        "dense_decode": {
            "us_per_layer_step": round(t_ls_dense * 1e3, 3),
            "tokens_per_s_per_layer": round(B / (t_ls_dense * 1e-3), 1),
            "algorithmic_bytes_per_layer_step": bytes_dense,
            "hbm_gbps": round(bytes_dense / (t_ls_dense * 1e-3) / 1e9, 1),
        },
        "speedup_vs_dense": round(t_ls_dense / t_ls, 4),
        "ideal_speedup_bytes": round(bytes_dense / bytes_ls, 4),
        "prefill_partition_us_per_layer": round(ms_prefill / L * 1e3, 2),
        "prefill_partition_hbm_frac": round(metrics.partition_bytes(n_tok, d, d_ff, e) / (ms_prefill / L * 1e-3)
                                            / 1e9 / HBM_PEAK_GBPS, 4),
        "kernel_pass_coverage": round(windows_ms / span_ms, 4),
        "kernels_us": {
            "importance (colsq + sum + k_importance)": round(imp_us, 2),
            "partition select (k_partition)": round(psel_us, 2),
            "decode gate/up (k_gateup)": round(gu_us, 2),
            "decode top-k (k_topk)": round(sel_us, 2),
            "decode down (k_down_partial + k_sum_chunks)": round(dn_us, 2),
        },
        "kernel_gbps": {
            "importance": round(imp_bytes / (imp_us * 1e-6) / 1e9, 1),
            "gate/up": round(gu_gbps, 1),
            "down": round(dn_bytes / (dn_us * 1e-6) / 1e9, 1),
        },
        "cpu_baseline": None,
    }

    # ------------------------------------------------------------ CPU baseline: the oracle on a sample
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, T, args.cpu_seconds)
        log(f"[bench] cpu baseline: {out['cpu_baseline']}")

    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def cpu_baseline(w, T, budget_s):
    """The CPU oracle, as it stands, on layer 0 of the same workload: one
    prefill partition and as many decode layer-steps as fit in the budget.
    Scaled to tokens/s/layer the way the GPU value is: the partition's time is
    spread over the T decode steps of the request."""
    import numpy as np

    import oracle
    from online_structured_ffn_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    wts = synth.layer_weights(w, 0)
    X = synth.prompt(w, 0)
    t0 = time.perf_counter()
    R, C, _ = oracle.partition(oracle.importance(wts["W_up"], oracle.column_norm(X)), w.r, w.gamma)
    t_part = time.perf_counter() - t0
    times = []
    t_start = time.perf_counter()
    step = 0
    while step < T and (time.perf_counter() - t_start) < budget_s:
        x = synth.decode_input(w, 0, step)
        t0 = time.perf_counter()
        oracle.decode_step(x, wts["W_gate"], wts["W_up"], wts["W_down"], R, C, w.r)
        times.append(time.perf_counter() - t0)
        step += 1
    t_dec = float(np.median(times))
    B = w.decode_batch
    value = B * T / (t_part + T * t_dec)
    return {
        "value": round(value, 3),
        "unit": "tokens/s/layer",
        "cores": blas_threads if blas_threads is not None else len(os.sched_getaffinity(0)),
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"layer 0 of {w.name}: 1 prefill partition ({t_part:.2f} s) + {len(times)} decode layer-steps "
                  f"(median {t_dec * 1e3:.1f} ms), numpy fp64; value = B*T / (t_partition + T * t_step)",
    }


if __name__ == "__main__":
    main()
