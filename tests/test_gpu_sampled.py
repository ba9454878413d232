"""Sampled parity at the workloads' full sizes, on the inputs the benchmark
times.

The benchmark draws its weights, prompts and decode streams on the device with
seeded torch generators (synth.torch_*); these tests draw the same tensors,
run the calls the benchmark times (the fused prefill, then pop_decode_ffn in
the same launch configuration), and copy the inputs to the host for the
oracle.  For each FFN stack: layers 0, L/2 and L-1, the partition (exact on the
device's importance, near ties only against fp64), the prompt FFN on sampled
rows, and the first 8 decode steps element by element.  For the mixture of
experts: the same layers, every expert's partition and 8 decode steps of 32
tokens.  The comparison protocol is in tests/parity.py."""
import sys

import numpy as np
import pytest
import torch

import oracle
from online_structured_ffn_amd import configs, pop, synth
from tests.parity import TIE_REL, TOL, VALUE_RTOL, check_decode, check_partition, host, moe_decode_views

pytestmark = pytest.mark.gpu
STEPS = 8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    yield
    torch.cuda.synchronize()


def _h32(t):
    """Host float32 copy (exact for bf16 values)."""
    return t.float().cpu().numpy()


def _layers(w):
    return sorted({0, w.layers // 2, w.layers - 1})


FFN_CASES = [(name, l) for name in ("llama2_7b_ffn_b1", "llama2_7b_ffn_b16", "qwen2_7b_ffn_b4")
             for l in _layers(configs.BY_NAME[name])]


@pytest.mark.parametrize("wname,layer", FFN_CASES, ids=[f"{n}-L{l}" for n, l in FFN_CASES])
def test_sampled_ffn_layer(wname, layer):
    w = configs.BY_NAME[wname]
    dev = torch.device("cuda")
    n_tok, d, d_ff, B = w.prompt_batch * w.prompt_len, w.d, w.d_ff, w.decode_batch
    say(f"[sampled] {w.name} layer {layer}: drawing the benchmark's inputs")
    wt = synth.torch_layer_weights(w, layer, dev)
    Wg, Wu, WdT = wt["W_gate"], wt["W_up"], wt["W_downT"]
    X = synth.torch_activations(w, (n_tok, d), layer, 0, dev, synth.outlier_channels(w, layer))
    xs = synth.torch_decode_inputs(w, layer, w.decode_steps, dev)[:STEPS].contiguous()
    # the timed prefill: prompt FFN + partition in one call
    Y, R, C, P, I = pop.pop_prefill_ffn_partition(X, Wg, Wu, WdT, w.r, w.gamma, importance=True)
    torch.cuda.synchronize()
    Xh = _h32(X)
    hw = {"W_gate": _h32(Wg).astype(np.float64), "W_up": _h32(Wu).astype(np.float64)}
    hw["W_down"] = _h32(WdT).astype(np.float64).T          # [d, d_ff] view of W_downT
    I_ref = oracle.importance(hw["W_up"], oracle.column_norm(Xh))
    n_ex = check_partition(R, C, P, I, I_ref, w.r, w.gamma)
    rows = sorted({0, 1, n_tok // 2, n_tok - 1})
    ref = oracle.dense_ffn(Xh[rows], hw["W_gate"], hw["W_up"], hw["W_down"])
    err = np.abs(host(Y)[rows] - ref).max() / max(np.abs(ref).max(), 1e-30)
    say(f"  partition near-tie exclusions {n_ex}; prompt FFN rows {rows}: max|dY|/max|Y| = {err:.2e}")
    assert err <= TOL[w.dtype]
    del Y, X, Xh
    Rh, Ch = host(R), host(C)
    ws = pop.workspace(pop.pop_decode_workspace_bytes(B, d, d_ff), dev)
    for t in range(STEPS):
        y, S = pop.pop_decode_ffn(xs[t], Wg, Wu, WdT, R, C, w.r, selected=True, ws=ws)
        torch.cuda.synchronize()
        err, n_ex = check_decode(y, S, ws, _h32(xs[t]), hw, Rh, Ch, w.r, w.dtype)
        say(f"  step {t}: max|dy|/max|y| = {err:.2e}, near-tie exclusions {n_ex}")


@pytest.mark.parametrize("layer", _layers(configs.MIXTRAL_MOE))
def test_sampled_moe_layer(layer):
    w = configs.MIXTRAL_MOE
    dev = torch.device("cuda")
    E, d, d_ff, r, gamma = w.experts, w.d, w.d_ff, w.r, w.gamma
    n_tok, B = w.prompt_batch * w.prompt_len, w.decode_batch
    say(f"[sampled] {w.name} layer {layer}: drawing the benchmark's inputs")
    lg_pre, lg_dec, Xdec = synth.torch_moe_inputs(w, w.layers, w.decode_steps, dev)
    parts = [synth.torch_layer_weights(w, layer * E + e, dev) for e in range(E)]
    Wg, Wu, WdT = (torch.stack([q[n] for q in parts]).contiguous() for n in ("W_gate", "W_up", "W_downT"))
    del parts
    X = synth.torch_activations(w, (n_tok, d), layer, 0, dev)
    R, C, P, I = pop.pop_moe_prefill_partition(X, lg_pre[layer], Wu, r, gamma, importance=True)
    torch.cuda.synchronize()
    Xh, Lp = _h32(X), _h32(lg_pre[layer])
    ex, _ = oracle.moe_route_top2(Lp)
    Rh, Ch = host(R).astype(np.int64), host(C).astype(np.int64)
    n_R, n_C = Rh.shape[1], Ch.shape[1]
    # per expert: the partition, then the expert's rows R u C on the host (f64)
    rex = []
    for e in range(E):
        toks = np.flatnonzero((ex == e).any(axis=1))
        Wu_e = _h32(Wu[e])
        I_ref = oracle.importance(Wu_e, oracle.column_norm(Xh[toks]))
        n_ex = check_partition(R[e], C[e], P[e], I[e], I_ref, r, gamma)
        say(f"  expert {e}: {len(toks)} prompt tokens, near-tie exclusions {n_ex}")
        A = np.concatenate([Rh[e], Ch[e]])
        rex.append({"W_gate": _h32(Wg[e])[A].astype(np.float64), "W_up": Wu_e[A].astype(np.float64),
                    "W_down": _h32(WdT[e])[A].astype(np.float64).T})
        del Wu_e
    # Restricted to R u C, expert e's channels are renumbered 0..n_A-1 (R
    # first, C after, both ascending): the order of C is kept, so the
    # selection rule (score, then lower index) is unchanged, and every channel
    # outside R u C is zero in the oracle's output anyway.
    k = oracle.partition_counts(d_ff, r, 0.0)["n_live"] - n_R
    k = max(0, min(k, n_C))
    Rr, Cr = np.arange(n_R), n_R + np.arange(n_C)
    ws = pop.workspace(pop.pop_moe_decode_workspace_bytes(B, d, d_ff, E), dev)
    for t in range(STEPS):
        x, Ld = Xdec[t, layer].contiguous(), lg_dec[t, layer].contiguous()
        y, S = pop.pop_moe_decode_ffn(x, Ld, Wg, Wu, WdT, R, C, r, selected=True, ws=ws)
        torch.cuda.synchronize()
        xh, Lh = _h32(x), _h32(Ld)
        S = host(S).astype(np.int64)
        assert S.shape == (E, k)
        ext, _ = oracle.moe_route_top2(Lh)
        z_dev, sc_dev = moe_decode_views(ws, B, d_ff, E, n_R + n_C, n_C)
        off, sel = 0, [None] * E
        for e in range(E):
            rows = np.sort(np.nonzero(ext == e)[0], kind="stable")
            if len(rows) == 0:
                continue
            zr = oracle.restricted_forward(xh[rows], rex[e]["W_gate"], rex[e]["W_up"], Rr, Cr)
            scale = max(np.abs(zr).max(), 1e-30)
            zd = z_dev[off: off + len(rows)].astype(np.float64)
            assert np.abs(zd - zr).max() <= VALUE_RTOL * scale, f"step {t} expert {e}: z differs"
            sr = oracle.candidate_scores(zr, n_R)
            sd = sc_dev[e].astype(np.float64)
            np.testing.assert_allclose(sd, sr, rtol=VALUE_RTOL, atol=1e-6 * scale)
            assert np.array_equal(S[e], oracle.select_candidates(Ch[e], sd, k)), f"step {t} expert {e}: selection"
            S_ref = oracle.select_candidates(Ch[e], sr, k)
            srt = np.sort(sr)[::-1]
            cuts = [srt[j] for j in (k - 1, k) if 0 <= j < n_C]
            for ch in np.setxor1d(S[e], S_ref):
                v = sr[np.searchsorted(Ch[e], ch)]
                assert any(abs(v - c) <= TIE_REL * max(c, 1e-30) for c in cuts), f"step {t} expert {e}: {ch}"
            sel[e] = n_R + np.searchsorted(Ch[e], S[e])      # the device's selection, renumbered
            off += len(rows)
        parts_r = [(Rr, Cr, None)] * E
        y_ref, _ = oracle.moe_decode_step(xh, Lh, rex, parts_r, r, selections=sel)
        err = np.abs(host(y) - y_ref).max() / max(np.abs(y_ref).max(), 1e-30)
        say(f"  step {t}: max|dy|/max|y| = {err:.2e}")
        assert err <= TOL[w.dtype]
