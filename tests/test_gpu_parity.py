"""HIP path against the CPU oracle (through the C ABI), on seeded inputs.

Small cases span several tiles with ragged tails and the degenerate cases of
the method; full-size cases use the workloads' real shapes.  The comparison
protocol is in tests/parity.py."""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from online_structured_ffn_amd import configs, pop, synth
from tests.parity import check_decode, check_partition, dev, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    yield
    torch.cuda.synchronize()


def _partition_case(X, W_up, dtype, r, gamma):
    Xd, Wd = dev(X, dtype), dev(W_up, dtype)
    R, C, P, I = pop.pop_prefill_partition(Xd, Wd, r, gamma, importance=True)
    torch.cuda.synchronize()
    I_ref = oracle.importance(W_up, oracle.column_norm(X))
    n_ex = check_partition(R, C, P, I, I_ref, r, gamma)
    return (host(R), host(C), host(P)), n_ex


PART_CASES = [
    # name, n_tokens, d, d_ff, dtype, r, gamma
    ("f32_several_tiles", 300, 1028, 2053, "f32", 0.45, 0.15),
    ("bf16_ragged", 37, 264, 1000, "bf16", 0.3, 0.1),
    ("bf16_r0_dense", 20, 128, 333, "bf16", 0.0, 0.1),
    ("bf16_gamma0_no_candidates", 20, 128, 333, "bf16", 0.4, 0.0),
    ("f32_window_clamped", 20, 64, 97, "f32", 0.5, 0.6),
    ("bf16_d_ff_1", 5, 8, 1, "bf16", 0.3, 0.1),
    ("f32_d_ff_3", 5, 8, 3, "f32", 0.5, 0.2),
    ("bf16_empty_prompt", 0, 128, 500, "bf16", 0.3, 0.1),
    ("bf16_max_d_ff", 4, 64, 32768, "bf16", 0.3, 0.1),
    ("bf16_max_d", 3, 16384, 40, "bf16", 0.3, 0.1),
    ("f32_long_prompt", 5000, 256, 700, "f32", 0.25, 0.1),
    # prompts at and past the one-pass column-norm limit (8192 tokens)
    ("f32_prompt_at_one_pass_limit", 8192, 72, 150, "f32", 0.3, 0.1),
    ("bf16_prompt_past_one_pass", 9000, 136, 300, "bf16", 0.3, 0.1),
]


@pytest.mark.parametrize("name,n,d,d_ff,dtype,r,gamma", PART_CASES, ids=[c[0] for c in PART_CASES])
def test_partition_small(name, n, d, d_ff, dtype, r, gamma):
    say(f"[partition] {name} n={n} d={d} d_ff={d_ff} {dtype} r={r} gamma={gamma}")
    c = synth.random_case(zlib.crc32(name.encode()) % 1000, n, d, d_ff, 1, dtype)
    _, n_ex = _partition_case(c["X"], c["W_up"], dtype, r, gamma)
    say(f"  near-tie exclusions: {n_ex}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_partition_exact_ties(dtype):
    """Small-integer inputs: every I^2 is an exact small integer on both sides,
    so the device partition must equal the fp64 oracle exactly, ties included."""
    g = np.random.default_rng(7)
    X = g.integers(-1, 2, (9, 64)).astype(np.float32)
    W = g.integers(-2, 3, (777, 64)).astype(np.float32)
    say(f"[partition ties] {dtype}")
    (R, C, P), n_ex = _partition_case(X, W, dtype, 0.3, 0.1)
    assert n_ex == 0
    I = oracle.importance(W, oracle.column_norm(X))
    assert len(np.unique(I)) < len(I) // 2   # the case really has many ties
    eR, eC, eP = oracle.partition(I, 0.3, 0.1)
    assert np.array_equal(R, eR) and np.array_equal(C, eC) and np.array_equal(P, eP)


def test_partition_zero_prompt_is_index_order():
    say("[partition] all-zero prompt")
    X = np.zeros((8, 32), np.float32)
    W = np.ones((101, 32), np.float32)
    (R, C, P), _ = _partition_case(X, W, "f32", 0.3, 0.1)
    cnt = oracle.partition_counts(101, 0.3, 0.1)
    assert list(R) == list(range(cnt["n_R"]))
    assert list(P) == list(range(101 - cnt["n_P"], 101))


def test_partition_deterministic():
    c = synth.random_case(11, 700, 1024, 3001, 1, "bf16")
    Xd, Wd = dev(c["X"], "bf16"), dev(c["W_up"], "bf16")
    outs = [pop.pop_prefill_partition(Xd, Wd, 0.3, 0.1, importance=True) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


def test_partition_graph_replay_shared_workspace():
    """Replays of a captured partition (with calls of other shapes on the same
    workspace between them) give the eager outputs bit for bit."""
    say("[partition] graph replays on a shared workspace")
    shapes = [(700, 1024, 3001, 0.3, 0.1), (37, 264, 1000, 0.5, 0.2), (4096, 4096, 11008, 0.299, 0.1)]
    cases = []
    for i, (n, d, d_ff, r, g) in enumerate(shapes):
        c = synth.random_case(60 + i, n, d, d_ff, 1, "bf16")
        cases.append((dev(c["X"], "bf16"), dev(c["W_up"], "bf16"), r, g))
    ws = pop.workspace(max(pop.pop_prefill_workspace_bytes(n, d, d_ff) for n, d, d_ff, _, _ in shapes))
    eager = [pop.pop_prefill_partition(X, W, r, g, importance=True, ws=ws) for X, W, r, g in cases]
    torch.cuda.synchronize()
    outs = tuple(torch.empty_like(t) for t in eager[0])
    X0, W0, r0, g0_ = cases[0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pop.pop_prefill_partition(X0, W0, r0, g0_, out=outs, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pop.pop_prefill_partition(X0, W0, r0, g0_, out=outs, ws=ws)
    for rep in range(4):
        for o in outs:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager[0]):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
        X, W, r, g = cases[1 + rep % 2]
        o = pop.pop_prefill_partition(X, W, r, g, importance=True, ws=ws)
        torch.cuda.synchronize()
        for a, b in zip(o, eager[1 + rep % 2]):
            assert torch.equal(a, b)


# ------------------------------------------------------------------ decode
def _decode_case(X, x_steps, w, dtype, r, gamma, label):
    Xd = dev(X, dtype)
    Wg, Wu, WdT = dev(w["W_gate"], dtype), dev(w["W_up"], dtype), dev(w["W_downT"], dtype)
    R, C, P, I = pop.pop_prefill_partition(Xd, Wu, r, gamma, importance=True)
    torch.cuda.synchronize()
    I_ref = oracle.importance(w["W_up"], oracle.column_norm(X))
    check_partition(R, C, P, I, I_ref, r, gamma)
    Rh, Ch = host(R), host(C)
    errs = []
    for t, x in enumerate(x_steps):
        xd = dev(x, dtype)
        ws = pop.workspace(pop.pop_decode_workspace_bytes(x.shape[0], x.shape[1], w["W_gate"].shape[0]))
        y, S = pop.pop_decode_ffn(xd, Wg, Wu, WdT, R, C, r, selected=True, ws=ws)
        torch.cuda.synchronize()
        err, n_ex = check_decode(y, S, ws, x, w, Rh, Ch, r, dtype)
        errs.append(err)
        say(f"  {label} step {t}: rel err {err:.2e}, near-tie exclusions {n_ex}")
    return errs


DEC_CASES = [
    # name, n_tokens, d, d_ff, batch, dtype, r, gamma
    ("f32_b1", 16, 256, 688, 1, "f32", 0.3, 0.1),
    ("bf16_ragged_b1", 37, 264, 1000, 1, "bf16", 0.3, 0.1),
    ("bf16_b3", 50, 520, 1501, 3, "bf16", 0.3, 0.1),
    ("f32_b5_tiles", 40, 1028, 999, 5, "f32", 0.5, 0.1),
    ("bf16_b9", 30, 1032, 2000, 9, "bf16", 0.299, 0.1),
    ("bf16_b0", 12, 256, 500, 0, "bf16", 0.3, 0.1),
    ("bf16_r0", 12, 256, 500, 2, "bf16", 0.0, 0.1),
    ("bf16_gamma0", 12, 256, 500, 2, "bf16", 0.4, 0.0),
    ("f32_high_r", 12, 128, 300, 1, "f32", 0.95, 0.1),
    # batch 1 past 4096 candidates: the top-k is its own launch, the selected-row helpers do not wait
    ("bf16_b1_wide_C", 20, 264, 6000, 1, "bf16", 0.2, 0.8),
    # matrix-core batches: one, two and four 16-token tiles, ragged d; 65 falls back to the FMA kernels
    ("bf16_b8_mfma", 30, 520, 1501, 8, "bf16", 0.3, 0.1),
    ("bf16_b16_mfma_tail_chunk", 30, 264, 1000, 16, "bf16", 0.3, 0.1),
    ("bf16_b17_mfma", 30, 264, 1000, 17, "bf16", 0.3, 0.1),
    ("bf16_b40_mfma", 30, 1032, 1501, 40, "bf16", 0.299, 0.1),
    ("bf16_b64_mfma", 30, 520, 700, 64, "bf16", 0.5, 0.1),
    # no retained rows: 4000 candidates (top-k alone in the retained launch), 6000 (top-k as its own launch)
    ("bf16_b16_mfma_only_C", 20, 264, 4000, 16, "bf16", 0.2, 0.8),
    ("bf16_b16_mfma_wide_C", 20, 264, 6000, 16, "bf16", 0.2, 0.8),
    ("bf16_b65_fma", 30, 256, 600, 65, "bf16", 0.3, 0.1),
]


@pytest.mark.parametrize("name,n,d,d_ff,b,dtype,r,gamma", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_decode_small(name, n, d, d_ff, b, dtype, r, gamma):
    say(f"[decode] {name} d={d} d_ff={d_ff} B={b} {dtype} r={r} gamma={gamma}")
    c = synth.random_case(zlib.crc32(name.encode()) % 1000, n, d, d_ff, b, dtype)
    xs = [c["x"], synth.random_case(zlib.crc32(name.encode()) % 1000 + 1, 1, d, 1, b, dtype)["x"]]
    _decode_case(c["X"], xs, c, dtype, r, gamma, name)


def test_decode_zero_input_selects_lowest_candidates():
    say("[decode] x = 0")
    c = synth.random_case(5, 20, 256, 640, 2, "bf16")
    x = np.zeros((2, 256), np.float32)
    Xd = dev(c["X"], "bf16")
    Wg, Wu, WdT = dev(c["W_gate"], "bf16"), dev(c["W_up"], "bf16"), dev(c["W_downT"], "bf16")
    R, C, P = pop.pop_prefill_partition(Xd, Wu, 0.3, 0.1)
    y, S = pop.pop_decode_ffn(dev(x, "bf16"), Wg, Wu, WdT, R, C, 0.3, selected=True)
    torch.cuda.synchronize()
    k = len(host(S))
    assert np.array_equal(host(S), host(C)[:k])
    assert float(y.abs().max()) == 0.0


def test_dense_decode_matches_oracle():
    for dtype, b in (("f32", 1), ("bf16", 4), ("bf16", 6)):
        say(f"[dense decode] {dtype} B={b}")
        c = synth.random_case(21 + b, 1, 520, 1300, b, dtype)
        y = pop.pop_dense_ffn_decode(dev(c["x"], dtype), dev(c["W_gate"], dtype), dev(c["W_up"], dtype),
                                     dev(c["W_downT"], dtype))
        torch.cuda.synchronize()
        ref = oracle.dense_ffn(c["x"], c["W_gate"], c["W_up"], c["W_down"])
        err = np.abs(host(y) - ref).max() / np.abs(ref).max()
        say(f"  rel err {err:.2e}")
        assert err <= (1e-5 if dtype == "f32" else 2e-2)


def test_r0_pruned_equals_dense():
    say("[decode] r = 0 equals the dense FFN")
    c = synth.random_case(31, 40, 512, 1111, 3, "bf16")
    Xd, xd = dev(c["X"], "bf16"), dev(c["x"], "bf16")
    Wg, Wu, WdT = dev(c["W_gate"], "bf16"), dev(c["W_up"], "bf16"), dev(c["W_downT"], "bf16")
    R, C, P = pop.pop_prefill_partition(Xd, Wu, 0.0, 0.1)
    assert P.numel() == 0
    y = pop.pop_decode_ffn(xd, Wg, Wu, WdT, R, C, 0.0)
    yd = pop.pop_dense_ffn_decode(xd, Wg, Wu, WdT)
    torch.cuda.synchronize()
    assert float((y - yd).abs().max()) <= 1e-5 * float(yd.abs().max())


def test_decode_deterministic_and_graph_replay():
    say("[decode] determinism and HIP-graph replay")
    c = synth.random_case(41, 64, 1024, 2816, 2, "bf16")
    Xd, xd = dev(c["X"], "bf16"), dev(c["x"], "bf16")
    Wg, Wu, WdT = dev(c["W_gate"], "bf16"), dev(c["W_up"], "bf16"), dev(c["W_downT"], "bf16")
    R, C, P = pop.pop_prefill_partition(Xd, Wu, 0.3, 0.1)
    ws = pop.workspace(pop.pop_decode_workspace_bytes(2, 1024, 2816))
    y0, S0 = pop.pop_decode_ffn(xd, Wg, Wu, WdT, R, C, 0.3, selected=True, ws=ws)
    y1, S1 = pop.pop_decode_ffn(xd, Wg, Wu, WdT, R, C, 0.3, selected=True, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(S0, S1)
    yg = torch.empty_like(y0)
    Sg = torch.empty_like(S0)
    x_in = xd.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pop.pop_decode_ffn(x_in, Wg, Wu, WdT, R, C, 0.3, y=yg, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pop.pop_decode_ffn(x_in, Wg, Wu, WdT, R, C, 0.3, y=yg, ws=ws)
    x2 = dev(synth.random_case(42, 1, 1024, 1, 2, "bf16")["x"], "bf16")
    y2 = pop.pop_decode_ffn(x2, Wg, Wu, WdT, R, C, 0.3)
    torch.cuda.synchronize()
    for rep in range(4):
        x_in.copy_(xd if rep % 2 == 0 else x2)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y0 if rep % 2 == 0 else y2), f"replay {rep} differs from eager"


# ------------------------------------------------------------------ full-size workloads
def test_tiny_workload_end_to_end():
    w = configs.TINY
    say(f"[workload] {w.name}")
    wts = synth.layer_weights(w, 0)
    X = synth.prompt(w, 0)
    xs = [synth.decode_input(w, 0, t) for t in range(w.decode_steps)]
    _decode_case(X, xs, wts, w.dtype, w.r, w.gamma, w.name)


@pytest.mark.parametrize("wname,layer,steps", [
    ("llama2_7b_ffn_b1", 0, 2), ("llama2_7b_ffn_b1", 31, 1), ("qwen2_7b_ffn_b4", 5, 2), ("llama2_7b_ffn_b16", 0, 1),
])
def test_full_size_layer(wname, layer, steps):
    w = configs.BY_NAME[wname]
    say(f"[workload] {w.name} layer {layer}: generating inputs")
    wts = synth.layer_weights(w, layer)
    X = synth.prompt(w, layer)
    sets = synth.drifting_outliers(w, layer, steps) if w.outlier_kind == "drift_scale" else None
    xs = [synth.decode_input(w, layer, t, drift_sets=sets) for t in range(steps)]
    say(f"  X {X.shape}, weights {wts['W_up'].shape}")
    _decode_case(X, xs, wts, w.dtype, w.r, w.gamma, w.name)


@pytest.mark.parametrize("batch,dtype", [(3, "f32"), (3, "bf16"), (16, "bf16")])
def test_stages_compose_bitwise(batch, dtype):
    """The stage entry points run the same kernels as the composite calls (the
    FMA kernels in fp32, the matrix-core ones in bf16)."""
    say(f"[stages] batch {batch} {dtype}: importance + select == partition; gate/up + select + down == decode")
    c = synth.random_case(51, 100, 1032, 2900, batch, dtype)
    Xd, xd = dev(c["X"], dtype), dev(c["x"], dtype)
    Wg, Wu, WdT = dev(c["W_gate"], dtype), dev(c["W_up"], dtype), dev(c["W_downT"], dtype)
    R, C, P, I = pop.pop_prefill_partition(Xd, Wu, 0.3, 0.1, importance=True)
    I2 = pop.pop_prefill_importance(Xd, Wu)
    R2, C2, P2 = pop.pop_partition_select(I2, 0.3, 0.1)
    y, S = pop.pop_decode_ffn(xd, Wg, Wu, WdT, R, C, 0.3, selected=True)
    z, score = pop.pop_decode_gateup(xd, Wg, Wu, R, C)
    k = S.numel()
    Q, S2 = pop.pop_decode_select(score, C, k)
    y2 = pop.pop_decode_down(z, WdT, R, S2, Q)
    torch.cuda.synchronize()
    for a, b in ((I, I2), (R, R2), (C, C2), (P, P2), (S, S2), (y, y2)):
        assert torch.equal(a, b)
    # the dense first half through the identity row map
    zd, _ = pop.pop_decode_gateup(xd, Wg, Wu, None, None, n_R=2900, want_score=False)
    yd = pop.pop_decode_down(zd, WdT, None, None, None, n_R=2900)
    yref = pop.pop_dense_ffn_decode(xd, Wg, Wu, WdT)
    torch.cuda.synchronize()
    assert torch.equal(yd, yref)


@pytest.mark.parametrize("dtype,d,d_ff", [("bf16", 4096, 11008), ("bf16", 1032, 2900), ("f32", 256, 688)])
def test_decode_b1_fused_graph_replay(dtype, d, d_ff):
    """Batch 1 runs the row-streaming kernels: every replay of a captured step
    must match eager, bit for bit."""
    say(f"[decode b1] fused path, graph replay, {dtype} d={d} d_ff={d_ff}")
    c = synth.random_case(61 + d, 64, d, d_ff, 1, dtype)
    Xd = dev(c["X"], dtype)
    Wg, Wu, WdT = dev(c["W_gate"], dtype), dev(c["W_up"], dtype), dev(c["W_downT"], dtype)
    R, C, P = pop.pop_prefill_partition(Xd, Wu, 0.299, 0.1)
    ws = pop.workspace(pop.pop_decode_workspace_bytes(1, d, d_ff))
    xs = [synth.random_case(70 + t, 1, d, 1, 1, dtype)["x"] for t in range(3)]
    eager = []
    for xt in xs:
        y, S = pop.pop_decode_ffn(dev(xt, dtype), Wg, Wu, WdT, R, C, 0.299, selected=True, ws=ws)
        torch.cuda.synchronize()
        check_decode(y, S, ws, xt, c, host(R), host(C), 0.299, dtype)
        eager.append(y)
    x_in = dev(xs[0], dtype)
    yg = torch.empty_like(eager[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pop.pop_decode_ffn(x_in, Wg, Wu, WdT, R, C, 0.299, y=yg, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pop.pop_decode_ffn(x_in, Wg, Wu, WdT, R, C, 0.299, y=yg, ws=ws)
    for rep in range(6):
        t = rep % 3
        x_in.copy_(dev(xs[t], dtype))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, eager[t]), f"replay {rep} differs from eager"


@pytest.mark.parametrize("n,kind", [(1, "rand"), (7, "ties"), (64, "rand"), (65, "ties"), (2201, "rand"),
                                    (2201, "ties"), (3788, "zeros"), (4096, "rand"), (4097, "rand"),
                                    (4097, "ties"), (9000, "rand"), (32768, "ties")])
def test_select_stage_exact(n, kind):
    """pop_decode_select against the oracle's selection rule on the same fp32
    scores, at sizes on both sides of the one-wave limit (4096), with heavy
    ties and every k from 0 to n on small sizes."""
    say(f"[select] n={n} {kind}")
    g = np.random.default_rng(n + len(kind))
    if kind == "rand":
        sc = g.uniform(0, 2, n).astype(np.float32)
    elif kind == "ties":
        sc = g.integers(0, 5, n).astype(np.float32)
    else:
        sc = np.zeros(n, np.float32)
    C = np.sort(g.choice(max(n * 3, 8), n, replace=False)).astype(np.int32)
    ks = range(0, n + 1) if n <= 65 else sorted({0, 1, n // 3, n // 2, n - 1, n})
    scd = torch.from_numpy(sc).cuda()
    Cd = torch.from_numpy(C).cuda()
    for k in ks:
        Q, S = pop.pop_decode_select(scd, Cd, k)
        torch.cuda.synchronize()
        exp_S = oracle.select_candidates(C, sc.astype(np.float64), k)
        assert np.array_equal(host(S), exp_S), (n, kind, k)
        assert np.array_equal(C[host(Q)], exp_S)


@pytest.mark.parametrize("n,kind", [(1, "rand"), (10, "ties"), (688, "ties"), (11008, "rand"), (18944, "ties"),
                                    (32768, "rand")])
def test_partition_select_stage_exact(n, kind):
    """pop_partition_select against the oracle's partition of the same fp32 importance."""
    say(f"[partition select] n={n} {kind}")
    g = np.random.default_rng(7 * n + len(kind))
    I = (g.uniform(0, 3, n) if kind == "rand" else g.integers(0, 4, n)).astype(np.float32)
    Id = torch.from_numpy(I).cuda()
    for r, gam in ((0.3, 0.1), (0.0, 0.1), (0.5, 0.5), (0.9, 0.05)):
        R, C, P = pop.pop_partition_select(Id, r, gam)
        torch.cuda.synchronize()
        eR, eC, eP = oracle.partition(I.astype(np.float64), r, gam)
        assert np.array_equal(host(R), eR) and np.array_equal(host(C), eC) and np.array_equal(host(P), eP), (n, r, gam)


@pytest.mark.parametrize("d,d_ff,r", [(4096, 11008, 0.299), (3584, 18944, 0.5), (1032, 2900, 0.3)])
def test_decode_b1_single_launch_bitwise(d, d_ff, r):
    """The single-launch batch-1 step: the same bits on every call, eager and
    as a captured graph replayed several times with other eager work (on
    another workspace) between replays; one workspace serving batch-1 steps
    and a batch-16 step in turn; the control words zero after every call."""
    say(f"[decode b1 single launch] d={d} d_ff={d_ff} r={r}")
    c = synth.random_case(91 + d, 32, d, d_ff, 1, "bf16")
    Xd = dev(c["X"], "bf16")
    Wg, Wu, WdT = dev(c["W_gate"], "bf16"), dev(c["W_up"], "bf16"), dev(c["W_downT"], "bf16")
    R, C, P = pop.pop_prefill_partition(Xd, Wu, r, 0.1)
    ws1 = pop.workspace(pop.pop_decode_workspace_bytes(16, d, d_ff))
    ws2 = pop.workspace(pop.pop_decode_workspace_bytes(1, d, d_ff))
    Z = pop.DECODE_WS_Z_OFFSET
    ctl_zero = lambda ws: not host(ws[:Z]).any()
    xs = [dev(synth.random_case(95 + t, 1, d, 1, 1, "bf16")["x"], "bf16") for t in range(3)]
    x16 = dev(synth.random_case(99, 1, d, 1, 16, "bf16")["x"], "bf16")
    ref, refS = [], []
    for xt in xs:
        y1, S1 = pop.pop_decode_ffn(xt, Wg, Wu, WdT, R, C, r, selected=True, ws=ws1)
        y16 = pop.pop_decode_ffn(x16, Wg, Wu, WdT, R, C, r, ws=ws1)    # same workspace, batch 16
        y2, S2 = pop.pop_decode_ffn(xt, Wg, Wu, WdT, R, C, r, selected=True, ws=ws2)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(S1, S2)
        assert ctl_zero(ws1) and ctl_zero(ws2)
        ref.append(y1)
        refS.append(S1)
    x_in = xs[0].clone()
    yg = torch.empty_like(ref[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pop.pop_decode_ffn(x_in, Wg, Wu, WdT, R, C, r, y=yg, ws=ws2)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pop.pop_decode_ffn(x_in, Wg, Wu, WdT, R, C, r, y=yg, ws=ws2)
    for rep in range(6):
        t = rep % 3
        x_in.copy_(xs[t])
        g.replay()
        pop.pop_decode_ffn(xs[(t + 1) % 3], Wg, Wu, WdT, R, C, r, ws=ws1)  # other eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(yg, ref[t]), f"replay {rep} differs"
        assert ctl_zero(ws1) and ctl_zero(ws2)


@pytest.mark.parametrize("d,d_ff,r,gamma", [(512, 1376, 0.3, 0.1), (1032, 2900, 0.3, 0.01), (4096, 11008, 0.7, 0.02)])
def test_decode_b1_uneven_shares_tight(d, d_ff, r, gamma):
    """Batch-1 single-launch steps where some workers own no candidate or no
    selected row (k or |C| below the worker count): with bf16 inputs the step
    accumulates in fp32, so y matches the oracle on the device's selection to
    fp32 rounding (1e-5 of max|y|, far below the batched paths' bf16 bar), on
    every one of several calls."""
    say(f"[decode b1 uneven shares] d={d} d_ff={d_ff} r={r} gamma={gamma}")
    c = synth.random_case(77 + d, 32, d, d_ff, 1, "bf16")
    Wg, Wu, WdT = dev(c["W_gate"], "bf16"), dev(c["W_up"], "bf16"), dev(c["W_downT"], "bf16")
    R, C, _ = pop.pop_prefill_partition(dev(c["X"], "bf16"), Wu, r, gamma)
    xd = dev(c["x"], "bf16")
    ys = [pop.pop_decode_ffn(xd, Wg, Wu, WdT, R, C, r, selected=True) for _ in range(4)]
    torch.cuda.synchronize()
    live = np.concatenate([host(R), host(ys[0][1])]).astype(np.int64)
    y_ref = oracle.masked_ffn(c["x"], c["W_gate"], c["W_up"], c["W_down"], live)
    for y, S in ys:
        assert torch.equal(S, ys[0][1])
        err = np.abs(host(y) - y_ref).max() / np.abs(y_ref).max()
        assert err <= 1e-5, f"max|dy|/max|y| = {err:.3e}"
