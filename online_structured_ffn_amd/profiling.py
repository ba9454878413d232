"""Profiler evidence for the kernels: a short eager workload to run under
rocprofv3, and summaries of what the counters and the kernel trace recorded.

    # the workload (every kernel launched eagerly, so that each dispatch is
    # counted on its own), run under one rocprofv3 pass per counter set, with
    # the repository root on PYTHONPATH:
    rocprofv3 --pmc <counters> --output-format csv -d DIR -o pmc -- \\
        python3 -m online_structured_ffn_amd.profiling run [--workload layer]
    # the summaries:
    python3 -m online_structured_ffn_amd.profiling traffic --reads DIR1 --writes DIR2 --fetch DIR3 --out FILE
    python3 -m online_structured_ffn_amd.profiling mfma --dir DIR4 --out FILE
    python3 -m online_structured_ffn_amd.profiling stats --dir DIR5 --out FILE

HBM bytes come from the L2-to-memory request counters of every L2 instance:
reads = 32 * TCC_EA0_RDREQ_32B + 64 * TCC_EA0_RDREQ_64B + 128 *
TCC_EA0_RDREQ_128B, writes = 64 * TCC_EA0_WRREQ_64B + 32 * (TCC_EA0_WRREQ -
TCC_EA0_WRREQ_64B).  Every pass also runs kernels of known size, and each
summary reports their readings: pop_hbm_read_probe reads PROBE_BYTES, the fill
of its buffer writes PROBE_BYTES, and the runtime's device-to-device copy
reads and writes COPY_MIB MiB.  The read factor is the probe's, the write
factor the fill's (the copy, whose requests the L2 counters see only in part,
is reported but not used).

A traffic summary is valid only for the kernel sources it was taken on: it
stores a digest of them, and :func:`traffic_bytes` returns None once they
differ.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
KERNEL_SOURCES = ("csrc/decode.hip", "csrc/prefill.hip", "csrc/partition.h", "csrc/pop_device.h",
                  "csrc/pop_internal.h", "csrc/prompt_ffn.hip", "csrc/trace.hip")
LAYER_SOURCES = KERNEL_SOURCES + ("csrc/layer.hip", "csrc/prompt_gemm.h")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "ffn_kernels_llama2_7b_b1_hbm_traffic.md")
LAYER_WORKLOAD = "llama2_7b_layer_b1"
_LINE = re.compile(r"^kernel=(?P<k>.+?) fetch_bytes=(?P<f>\d+) write_bytes=(?P<w>\d+) digest=(?P<d>[0-9a-f]+)$")

COPY_MIB = 256
PROBE_BYTES = 1 << 30
READ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")
WRITE_COUNTERS = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")


def source_digest(files=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(_HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_bytes(kernel: str, path: str = TRAFFIC_SUMMARY):
    """(read, write) HBM bytes per launch of ``kernel`` from the summary, or
    None if there is none or the kernel sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    digest = source_digest()
    with open(path) as fh:
        for line in fh:
            m = _LINE.match(line.strip())
            if m and m["k"] == kernel and m["d"] == digest:
                return int(m["f"]), int(m["w"])
    return None


# --------------------------------------------------------------------- workload
def _known_size_kernels(torch, pop, dev) -> None:
    """Three device copies of COPY_MIB MiB and three stream-read probes of
    PROBE_BYTES (alternating between two buffers, each filled first)."""
    n = COPY_MIB << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    del src, dst
    bufs = [torch.full((PROBE_BYTES,), i + 1, dtype=torch.uint8, device=dev) for i in range(2)]
    sink = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
    for i in range(3):
        pop.pop_hbm_read_probe(bufs[i % 2], sink, 1024)
    torch.cuda.synchronize()
    del bufs


def run(layers: int = 4, steps: int = 4, workload: str = "ffn") -> None:
    """The LLaMA-2-7B-shaped batch-1 FFN workload, eager: per layer the prompt
    FFN, the partition and `steps` pruned and dense decode steps; before it the
    known-size kernels.  workload="layer": the decoder-layer stack instead
    (per layer the prompt's pass, then `steps` decode steps through every
    layer)."""
    import torch

    from . import configs, pop, synth
    dev = torch.device("cuda")
    _known_size_kernels(torch, pop, dev)
    if workload == "layer":
        return _run_layer(torch, configs.BY_NAME[LAYER_WORKLOAD], pop, synth, dev, layers, steps)
    w = configs.BY_NAME["llama2_7b_ffn_b1"]
    n_tok = w.prompt_batch * w.prompt_len
    ws_dec = pop.workspace(pop.pop_decode_workspace_bytes(1, w.d, w.d_ff), dev)
    for l in range(layers):
        wt = synth.torch_layer_weights(w, l, dev)
        X = synth.torch_activations(w, (n_tok, w.d), l, 0, dev, synth.outlier_channels(w, l))
        xs = synth.torch_decode_inputs(w, l, steps, dev)
        pop.pop_dense_ffn_prefill(X, wt["W_gate"], wt["W_up"], wt["W_downT"])
        R, C, P = pop.pop_prefill_partition(X, wt["W_up"], w.r, w.gamma)
        for t in range(steps):
            pop.pop_decode_ffn(xs[t], wt["W_gate"], wt["W_up"], wt["W_downT"], R, C, w.r, ws=ws_dec)
            pop.pop_dense_ffn_decode(xs[t], wt["W_gate"], wt["W_up"], wt["W_downT"], ws=ws_dec)
        torch.cuda.synchronize()
        del wt, X
    print(f"profiling workload done: {layers} layers x {steps} decode steps", flush=True)


def _run_layer(torch, w, pop, synth, dev, layers: int, steps: int) -> None:
    a = w.extra["attention"]
    B, N, d = w.decode_batch, w.prompt_len, w.d
    cnt = pop.pop_partition_counts(w.d_ff, w.r, w.gamma)
    lays = []
    for l in range(layers):
        wts = dict(synth.torch_layer_weights(w, l, dev))
        wts.update(synth.torch_attention_weights(w, l, dev))
        lays.append(pop.Layer(d, a["n_heads"], a["n_kv_heads"], a["head_dim"], w.d_ff, N + steps, wts,
                              eps=a["eps"], rope_theta=a["rope_theta"]))
    caches = [lay.cache(B) for lay in lays]
    x_pre = synth.torch_activations(w, (B * N, d), 0, 0, dev).float().view(B, N, d).contiguous()
    xdec = synth.torch_activations(w, (steps * B, d), 0, 1, dev).float().view(steps, B, d).contiguous()
    R = [torch.empty(cnt["n_R"], dtype=torch.int32, device=dev) for _ in range(layers)]
    C = [torch.empty(cnt["n_C"], dtype=torch.int32, device=dev) for _ in range(layers)]
    P = [torch.empty(cnt["n_P"], dtype=torch.int32, device=dev) for _ in range(layers)]
    ws_pre = pop.workspace(pop.pop_layer_prefill_workspace_bytes(B, N, lays[0]), dev)
    ws_dec = pop.workspace(pop.pop_layer_decode_workspace_bytes(B, lays[0]), dev)
    for l in range(layers):
        pop.pop_layer_prefill(x_pre, lays[l], *caches[l], w.r, w.gamma, out=(R[l], C[l], P[l], None), ws=ws_pre)
    torch.cuda.synchronize()
    pos = torch.full((1,), N, dtype=torch.int32, device=dev)
    x = torch.empty((B, d), dtype=torch.float32, device=dev)
    for t in range(steps):
        x.copy_(xdec[t])
        for l in range(layers):
            pop.pop_layer_decode(x, lays[l], *caches[l], pos, R[l], C[l], w.r, ws=ws_dec)
        pos.add_(1)
    torch.cuda.synchronize()
    print(f"profiling workload done: {w.name}, {layers} layers, a {N}-token prompt, {steps} decode steps", flush=True)


# --------------------------------------------------------------------- summaries
def _rows(d: str):
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    for f in files:
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def _per_dispatch(d: str) -> dict:
    """{(kernel, grid): [ {counter: value} per dispatch ]}"""
    disp = {}
    for r in _rows(d):
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Kernel_Name"], int(float(r["Grid_Size"])))
        disp.setdefault(key, {})[r["Counter_Name"]] = disp.get(key, {}).get(r["Counter_Name"], 0.0) + float(
            r["Counter_Value"])
    out = {}
    for (_, k, g), v in disp.items():
        out.setdefault((k, g), []).append(v)
    return out


def _mean(vals):
    return sum(vals) / len(vals) if vals else 0.0


def _short(k: str) -> str:
    k = re.sub(r"^void ", "", k)
    k = re.sub(r"\(.*\)$", "", k)
    return k.strip()


def _read_bytes(c: dict) -> float:
    return 32 * c.get("TCC_EA0_RDREQ_32B_sum", 0) + 64 * c.get("TCC_EA0_RDREQ_64B_sum", 0) + 128 * c.get(
        "TCC_EA0_RDREQ_128B_sum", 0)


def _write_bytes(c: dict) -> float:
    n64 = c.get("TCC_EA0_WRREQ_64B_sum", 0)
    return 64 * n64 + 32 * (c.get("TCC_EA0_WRREQ_sum", 0) - n64)


def _calibration(per: dict, fn) -> tuple:
    """Mean readings of the known-size kernels: (copy, read probe, fill of
    the probe's buffer)."""
    copies = [fn(c) for (k, _), v in per.items() if "copyBuffer" in k for c in v]
    probes = [fn(c) for (k, _), v in per.items() if "k_read_probe" in k for c in v]
    fills = [fn(c) for (k, g), v in per.items() if "FillFunctor" in k and g * 16 == PROBE_BYTES for c in v]
    return _mean(copies), _mean(probes), _mean(fills)


def _algorithmic_reads(workload: str = "ffn", steps: int = 4):
    """Algorithmic read bytes per launch of the kernels of the workload."""
    from . import configs
    if workload == "layer":
        w = configs.BY_NAME[LAYER_WORKLOAD]
        a = w.extra["attention"]
        H, Hkv, hd, d, e = a["n_heads"], a["n_kv_heads"], a["head_dim"], w.d, 2
        keys = w.prompt_len + (steps + 1) / 2  # the mean key count over the decode steps
        return {
            # the K-major projection weights and the fp32 input row
            "pop::k_gemv_kmajor<pop::bf16s, 1, 1>": d * (H + 2 * Hkv) * hd * e + 4 * d,
            "pop::k_gemv_kmajor<pop::bf16s, 1, 2>": H * hd * d * e,
            # the cached keys and values of every head
            "pop::k_attn_decode<pop::bf16s, 128>": int(2 * Hkv * keys * hd * e),
        }
    w = configs.BY_NAME["llama2_7b_ffn_b1"]
    from .metrics import linked_symbol
    from .pop import pop_partition_counts
    c = pop_partition_counts(w.d_ff, w.r, w.gamma)
    n_tok, d, d_ff, e = w.prompt_batch * w.prompt_len, w.d, w.d_ff, 2
    n_A = c["n_R"] + c["n_C"]
    return {
        # gate and up rows of R u C, W_downT rows of R u S, x, the index lists
        linked_symbol(d, e): (2 * n_A + c["n_R"] + c["k"]) * d * e + d * e + 4 * n_A,
        linked_symbol(d, e).replace("k_pop_linked", "k_pop_step").replace(", false>", ", true, 0>"):
            3 * d_ff * d * e + d * e,
        "pop::k_colsq_slices<pop::bf16s>": n_tok * d * e,
        "pop::k_importance_items<pop::bf16s>": d_ff * d * e + 4 * d,
        "pop::k_read_probe": PROBE_BYTES,
    }


def traffic(reads: str, writes: str, fetch: str | None, out: str, workload: str = "ffn", steps: int = 4) -> None:
    pr, pw = _per_dispatch(reads), _per_dispatch(writes)
    pf = _per_dispatch(fetch) if fetch else {}
    copy_r, probe_r, _ = _calibration(pr, _read_bytes)
    copy_w, _, fill_w = _calibration(pw, _write_bytes)
    known = COPY_MIB << 20
    fr = PROBE_BYTES / probe_r if probe_r else float("nan")
    fw = PROBE_BYTES / fill_w if fill_w else float("nan")
    ff = None
    if pf:
        fsz = lambda c: c.get("FETCH_SIZE", 0) * 1024
        copy_f, probe_f, _ = _calibration(pf, fsz)
        ff = (copy_f, probe_f)
    alg = _algorithmic_reads(workload, steps)
    layer = workload == "layer"
    digest = source_digest(LAYER_SOURCES if layer else KERNEL_SOURCES)
    wl = f" --workload layer --layers 2 --steps {steps}" if layer else ""
    sfx = "_layer" if layer else ""
    lines = [
        "# HBM traffic per dispatch: " + (
            f"the LLaMA-2-7B-shaped decoder-layer stack (2 layers, a 512-token prompt, {steps} decode steps at "
            "batch 1, bf16)" if layer else
            "LLaMA-2-7B-shaped FFN layers, prompt FFN, partition and batch-1 decode (bf16)"),
        "",
        "Counter passes, one rocprofv3 run each (`$R` = repository root on the GPU box):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "export PYTHONPATH=$R",
        "rocprofv3 --pmc " + " ".join(READ_COUNTERS) + f" --output-format csv -d $R/gpurun_out/pmc_rd{sfx} -o pmc -- "
        "python3 -m online_structured_ffn_amd.profiling run" + wl,
        "rocprofv3 --pmc " + " ".join(WRITE_COUNTERS) + f" --output-format csv -d $R/gpurun_out/pmc_wr{sfx} -o pmc -- "
        "python3 -m online_structured_ffn_amd.profiling run" + wl,
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/pmc_fetch{sfx} -o pmc -- "
        "python3 -m online_structured_ffn_amd.profiling run" + wl,
        f"python3 -m online_structured_ffn_amd.profiling traffic --reads $R/gpurun_out/pmc_rd{sfx} "
        f"--writes $R/gpurun_out/pmc_wr{sfx} --fetch $R/gpurun_out/pmc_fetch{sfx}"
        + (f" --workload layer --steps {steps}" if layer else "") + " --out <this file>",
        "```",
        "",
        "Bytes: reads = 32 x RDREQ_32B + 64 x RDREQ_64B + 128 x RDREQ_128B, writes = 64 x WRREQ_64B + 32 x "
        "(WRREQ - WRREQ_64B), summed over the L2 instances, averaged over the dispatches of each kernel and grid.",
        "",
        "Known-size kernels in the same passes:",
        "",
        f"- pop_hbm_read_probe over {PROBE_BYTES} bytes (alternating between two 1 GiB buffers, so that no read "
        f"is served by the memory-side cache): counters read {probe_r:.0f} bytes, {probe_r / PROBE_BYTES:.4f} of "
        f"the bytes it reads (read factor {fr:.4f});",
        f"- the fill of one probe buffer ({PROBE_BYTES} bytes written): counters write {fill_w:.0f} bytes, "
        f"{fill_w / PROBE_BYTES:.4f} of them (write factor {fw:.4f});",
        f"- the runtime's device copy of {COPY_MIB} MiB ({known} bytes read and written): counters read "
        f"{copy_r:.0f} bytes ({copy_r / known:.4f}) and write {copy_w:.0f} bytes ({copy_w / known:.4f}). Its "
        "requests reach the L2 counters only in part, so it cannot calibrate them (it was the calibration of earlier "
        "summaries, whose factors differed between sessions for this reason).",
    ]
    if ff:
        lines.append(f"- the FETCH_SIZE derived counter for comparison: probe {ff[1]:.0f} bytes "
                     f"({ff[1] / PROBE_BYTES:.4f} of the bytes read), copy {ff[0]:.0f} bytes "
                     f"({ff[0] / known:.4f}): its formula counts a 128-byte request as 64 bytes, and the probe's requests are "
                     "all 128 bytes.")
    lines += [
        "",
        "Every figure below is the raw byte count x the factor for its direction (the library's kernels and the "
        "known-size ones; the rest of the workload's kernels are torch's input generation).",
        "",
        "| kernel | grid | dispatches | read MB | write MB | algorithmic read MB | read / algorithmic |",
        "|---|---|---|---|---|---|---|",
    ]
    machine = []
    keep = lambda k, g: (k.startswith("void pop::") or k.startswith("pop::") or "copyBuffer" in k and g > 4096
                         or "FillFunctor" in k and g * 16 == PROBE_BYTES)
    keys = sorted((kg for kg in set(pr) | set(pw) if keep(*kg)), key=lambda kg: (_short(kg[0]), kg[1]))
    for k, g in keys:
        name = _short(k)
        rd = _mean([_read_bytes(c) for c in pr.get((k, g), [])]) * fr
        wr = _mean([_write_bytes(c) for c in pw.get((k, g), [])]) * fw
        a = alg.get(name)
        ratio = f"{rd / a:.3f}" if a else ""
        amb = f"{a / 1e6:.2f}" if a else ""
        lines.append(f"| `{name}` | {g} | {len(pr.get((k, g), []))} | {rd / 1e6:.2f} | {wr / 1e6:.2f} | {amb} | "
                     f"{ratio} |")
        if name.startswith("pop::"):
            machine.append(f"kernel={name} fetch_bytes={int(round(rd))} write_bytes={int(round(wr))} digest={digest}")
    lines += [
        "",
        ("Algorithmic reads: the q|k|v projection (`k_gemv_kmajor<..., 1, 1>`) reads Wqkv_T and the input row; "
         "the output projection (`<..., 1, 2>`) Wo_T (the attention slices it merges are not counted); decode "
         f"attention the cached keys and values of every head at the mean key count of the {steps} steps.  The "
         "FFN's kernels are those of the FFN summary." if layer else
         "Algorithmic reads: k_pop_linked reads the gate and up rows of R u C, the W_downT rows of R u S and x; "
         "k_pop_step<..., true, 0> (the dense step) every row of the three matrices; k_colsq_slices the prompt; "
         "k_importance_items W_up and s2."),
        "",
        "Machine-readable (read by bench.py; valid while the kernel sources hash to the digest):",
        "",
        "```",
        *machine,
        "```",
        "",
    ]
    _write(out, lines)


def mfma(d: str, out: str) -> None:
    per = _per_dispatch(d)
    lines = [
        "# Matrix-core counters: prompt FFN GEMMs of the LLaMA-2-7B-shaped layers (512 tokens, bf16)",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp PYTHONPATH=$R",
        "rocprofv3 --pmc " + " ".join(MFMA_COUNTERS) + " --output-format csv -d $R/gpurun_out/pmc_mfma -o pmc -- "
        "python3 -m online_structured_ffn_amd.profiling run",
        "python3 -m online_structured_ffn_amd.profiling mfma --dir $R/gpurun_out/pmc_mfma --out <this file>",
        "```",
        "",
        "MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CU_CYCLES x 4 SIMDs); flops = 512 x "
        "SQ_INSTS_VALU_MFMA_MOPS_BF16 (the counter's unit); GRBM_GUI_ACTIVE = GPU busy cycles of the dispatch.",
        "",
        "| kernel | grid | dispatches | bf16 MFMA flops | MFMA busy / CU-SIMD busy | GUI active cycles |",
        "|---|---|---|---|---|---|",
    ]
    for (k, g), v in sorted(per.items(), key=lambda kv: _short(kv[0][0])):
        name = _short(k)
        if "k_prompt" not in name and "k_gateup" not in name:
            continue
        fl = _mean([c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) for c in v]) * 512
        busy = _mean([c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) for c in v])
        cu = _mean([c.get("SQ_BUSY_CU_CYCLES", 0) for c in v])
        gui = _mean([c.get("GRBM_GUI_ACTIVE", 0) for c in v])
        util = busy / (4 * cu) if cu else float("nan")
        lines.append(f"| `{name}` | {g} | {len(v)} | {fl:.4g} | {util:.3f} | {gui:.0f} |")
    lines.append("")
    _write(out, lines)


def stats(d: str, out: str, command: str) -> None:
    files = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [
        "# Kernel durations under rocprofv3 --kernel-trace --stats",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        command,
        "```",
        "",
        "| kernel | calls | avg us | min us | max us | % of GPU time |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows:
        name = _short(r["Name"])
        if not name.startswith("pop::"):
            continue
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    lines.append("")
    _write(out, lines)


def _write(out: str, lines) -> None:
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {out}")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(prog="python -m online_structured_ffn_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--layers", type=int, default=4)
    r.add_argument("--steps", type=int, default=4)
    r.add_argument("--workload", choices=("ffn", "layer"), default="ffn")
    t = sub.add_parser("traffic")
    t.add_argument("--workload", choices=("ffn", "layer"), default="ffn")
    t.add_argument("--steps", type=int, default=4)
    t.add_argument("--reads", required=True)
    t.add_argument("--writes", required=True)
    t.add_argument("--fetch", default=None)
    t.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--dir", required=True)
    m.add_argument("--out", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--dir", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "run":
        run(a.layers, a.steps, a.workload)
    elif a.cmd == "traffic":
        traffic(a.reads, a.writes, a.fetch, a.out, a.workload, a.steps)
    elif a.cmd == "mfma":
        mfma(a.dir, a.out)
    else:
        stats(a.dir, a.out, a.command)


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    main()
