"""Dense prompt FFN (pop_dense_ffn_prefill) against the CPU oracle's dense
gated MLP, through the C ABI, on seeded inputs.

Tolerances: max|dY| <= 1e-5 max|Y_ref| for fp32 inputs and <= 2e-2 max|Y_ref|
for bf16 inputs (fp32 accumulation; the bf16 path also rounds Z to bf16)."""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from online_structured_ffn_amd import configs, pop, synth
from tests.parity import TOL, dev, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    yield
    torch.cuda.synchronize()


def _run(c, dtype):
    return pop.pop_dense_ffn_prefill(dev(c["X"], dtype), dev(c["W_gate"], dtype), dev(c["W_up"], dtype),
                                     dev(c["W_downT"], dtype))


CASES = [
    # name, n_tokens, d, d_ff, dtype
    ("bf16_one_token_d_ff_1", 1, 8, 1, "bf16"),
    ("bf16_ragged", 37, 264, 1000, "bf16"),
    ("bf16_several_tiles", 300, 1032, 2053, "bf16"),
    ("bf16_exact_tiles", 256, 128, 128, "bf16"),
    ("bf16_tile_plus_one", 129, 72, 65, "bf16"),
    ("f32_ragged", 37, 260, 1000, "f32"),
    ("f32_several_tiles", 100, 516, 700, "f32"),
    ("bf16_two_passes", 4096 + 300, 256, 700, "bf16"),
]


@pytest.mark.parametrize("name,n,d,d_ff,dtype", CASES, ids=[c[0] for c in CASES])
def test_prompt_ffn_small(name, n, d, d_ff, dtype):
    say(f"[prompt ffn] {name}: n={n} d={d} d_ff={d_ff} {dtype}")
    c = synth.random_case(zlib.crc32(name.encode()) % 1000, n, d, d_ff, 1, dtype)
    Y = _run(c, dtype)
    torch.cuda.synchronize()
    ref = oracle.dense_ffn(c["X"], c["W_gate"], c["W_up"], c["W_down"])
    err = np.abs(host(Y) - ref).max() / max(np.abs(ref).max(), 1e-30)
    say(f"  max|dY|/max|Y| = {err:.2e}")
    assert err <= TOL[dtype]


def test_prompt_ffn_empty_prompt():
    say("[prompt ffn] n_tokens = 0")
    c = synth.random_case(5, 1, 64, 100, 1, "bf16")
    W = [dev(c[k], "bf16") for k in ("W_gate", "W_up", "W_downT")]
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    Y = pop.pop_dense_ffn_prefill(X, *W)
    torch.cuda.synchronize()
    assert Y.shape == (0, 64)


def test_prompt_ffn_zero_input():
    say("[prompt ffn] X = 0 gives Y = 0")
    c = synth.random_case(6, 50, 128, 300, 1, "bf16")
    c["X"] = np.zeros_like(c["X"])
    Y = _run(c, "bf16")
    torch.cuda.synchronize()
    assert float(Y.abs().max()) == 0.0


def test_prompt_ffn_deterministic_and_graph_replay():
    say("[prompt ffn] determinism and HIP-graph replay")
    c = synth.random_case(7, 200, 512, 1500, 1, "bf16")
    X, Wg, Wu, WdT = (dev(c[k], "bf16") for k in ("X", "W_gate", "W_up", "W_downT"))
    ws = pop.workspace(pop.pop_dense_ffn_prefill_workspace_bytes(200, 512, 1500, "bf16"))
    Y0 = pop.pop_dense_ffn_prefill(X, Wg, Wu, WdT, ws=ws)
    Y1 = pop.pop_dense_ffn_prefill(X, Wg, Wu, WdT, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1)
    Yg = torch.empty_like(Y0)
    X_in = X.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pop.pop_dense_ffn_prefill(X_in, Wg, Wu, WdT, Y=Yg, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pop.pop_dense_ffn_prefill(X_in, Wg, Wu, WdT, Y=Yg, ws=ws)
    X2 = dev(synth.random_case(8, 200, 512, 1, 1, "bf16")["X"], "bf16")
    Y2 = pop.pop_dense_ffn_prefill(X2, Wg, Wu, WdT)
    torch.cuda.synchronize()
    for rep in range(4):
        X_in.copy_(X if rep % 2 == 0 else X2)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Yg, Y0 if rep % 2 == 0 else Y2), f"replay {rep} differs from eager"


@pytest.mark.parametrize("wname,n_tokens,rows", [
    ("llama2_7b_ffn_b1", None, None),                                   # the whole 512-token prompt
    ("qwen2_7b_ffn_b4", None, [0, 1, 1023, 2048, 4095]),                # 4 x 1024 tokens, sampled rows
    ("llama2_7b_ffn_b16", 4096 + 4096 + 77, [0, 4095, 4096, 8191, 8192, 8268]),  # three passes
])
def test_prompt_ffn_full_size(wname, n_tokens, rows):
    w = configs.BY_NAME[wname]
    say(f"[prompt ffn] {w.name}: generating inputs")
    wts = synth.layer_weights(w, 0)
    X = synth.prompt(w, 0, n_tokens=n_tokens)
    say(f"  X {X.shape}, weights {wts['W_up'].shape}")
    Y = pop.pop_dense_ffn_prefill(dev(X, w.dtype), dev(wts["W_gate"], w.dtype), dev(wts["W_up"], w.dtype),
                                  dev(wts["W_downT"], w.dtype))
    torch.cuda.synchronize()
    Yh = host(Y)
    sel = slice(None) if rows is None else rows
    ref = oracle.dense_ffn(X[sel], wts["W_gate"], wts["W_up"], wts["W_down"])
    err = np.abs(Yh[sel] - ref).max() / np.abs(ref).max()
    say(f"  max|dY|/max|Y| = {err:.2e} over {ref.shape[0]} rows")
    assert err <= TOL[w.dtype]
    assert np.isfinite(Yh).all()


# ---------------------------------------------------------------- fused prefill
# pop_prefill_ffn_partition: the prompt FFN with the importance taken inside
# its gate/up pass, then the partition.  Y against the oracle's dense FFN, I
# and the partition against the oracle's importance and partition rule (near
# ties excluded, see tests/parity.py).
from tests.parity import check_partition  # noqa: E402

FUSED_CASES = [
    # name, n_tokens, d, d_ff, dtype, r, gamma
    ("bf16_ragged", 37, 264, 1000, "bf16", 0.3, 0.1),
    ("bf16_several_tiles", 300, 1032, 2053, "bf16", 0.45, 0.15),
    ("bf16_tile_plus_one", 129, 72, 65, "bf16", 0.3, 0.1),
    ("bf16_d_ff_1", 3, 8, 1, "bf16", 0.3, 0.1),
    ("f32_ragged", 37, 260, 1000, "f32", 0.3, 0.1),
    ("f32_several_tiles", 100, 516, 700, "f32", 0.25, 0.1),
    ("bf16_two_passes", 4096 + 300, 256, 700, "bf16", 0.3, 0.1),   # I from the first pass, s over both
    ("bf16_past_one_pass_norms", 9000, 136, 300, "bf16", 0.3, 0.1),
]


def _fused_check(X, W, dtype, r, gamma, rows=None):
    Y, R, C, P, I = pop.pop_prefill_ffn_partition(dev(X, dtype), dev(W["W_gate"], dtype), dev(W["W_up"], dtype),
                                                  dev(W["W_downT"], dtype), r, gamma, importance=True)
    torch.cuda.synchronize()
    I_ref = oracle.importance(W["W_up"], oracle.column_norm(X))
    n_ex = check_partition(R, C, P, I, I_ref, r, gamma)
    sel = slice(None) if rows is None else rows
    if X.shape[0]:
        ref = oracle.dense_ffn(X[sel], W["W_gate"], W["W_up"], W["W_down"])
        err = np.abs(host(Y)[sel] - ref).max() / max(np.abs(ref).max(), 1e-30)
        say(f"  max|dY|/max|Y| = {err:.2e}, near-tie exclusions {n_ex}")
        assert err <= TOL[dtype]
    return Y, R, C, P, I


@pytest.mark.parametrize("name,n,d,d_ff,dtype,r,gamma", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_prefill_small(name, n, d, d_ff, dtype, r, gamma):
    say(f"[fused prefill] {name}: n={n} d={d} d_ff={d_ff} {dtype}")
    c = synth.random_case(zlib.crc32(name.encode()) % 1000, n, d, d_ff, 1, dtype)
    _fused_check(c["X"], c, dtype, r, gamma)


def test_fused_prefill_empty_prompt_is_index_order():
    say("[fused prefill] n_tokens = 0")
    c = synth.random_case(9, 1, 64, 100, 1, "bf16")
    W = [dev(c[k], "bf16") for k in ("W_gate", "W_up", "W_downT")]
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    Y, R, C, P, I = pop.pop_prefill_ffn_partition(X, *W, 0.3, 0.1, importance=True)
    torch.cuda.synchronize()
    assert float(I.abs().max()) == 0.0
    eR, eC, eP = oracle.partition(np.zeros(100), 0.3, 0.1)
    assert np.array_equal(host(R), eR) and np.array_equal(host(C), eC) and np.array_equal(host(P), eP)


def test_fused_prefill_matches_separate_calls():
    """Same Y as pop_dense_ffn_prefill (bitwise: the same GEMMs), and I within
    fp32 rounding of pop_prefill_importance's (another summation order)."""
    say("[fused prefill] against the separate calls")
    c = synth.random_case(10, 300, 1032, 2053, 1, "bf16")
    X, Wg, Wu, WdT = (dev(c[k], "bf16") for k in ("X", "W_gate", "W_up", "W_downT"))
    Y, R, C, P, I = pop.pop_prefill_ffn_partition(X, Wg, Wu, WdT, 0.3, 0.1, importance=True)
    Y2 = pop.pop_dense_ffn_prefill(X, Wg, Wu, WdT)
    I2 = pop.pop_prefill_importance(X, Wu)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    assert float(((I - I2).abs() / I2.abs().clamp_min(1e-30)).max()) < 1e-5


@pytest.mark.parametrize("wname", ["llama2_7b_ffn_b1"])
def test_fused_prefill_full_size(wname):
    w = configs.BY_NAME[wname]
    say(f"[fused prefill] {w.name}: generating inputs")
    wts = synth.layer_weights(w, 0)
    X = synth.prompt(w, 0)
    _fused_check(X, wts, w.dtype, w.r, w.gamma, rows=[0, 1, 255, 511])
