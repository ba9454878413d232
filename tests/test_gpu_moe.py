"""Mixture-of-experts form of the path (routing, per-expert partition,
per-expert decode step and weighted combine) against the oracle's MoE
functions, through the C ABI, on seeded inputs.

Selections follow the protocol of tests/parity.py: exact against the oracle's
rule on the device's own values, and against fp64 up to near-ties."""
import sys

import numpy as np
import pytest
import torch

import oracle
from online_structured_ffn_amd import configs, pop, synth
from tests.parity import TIE_REL, TOL, VALUE_RTOL, check_partition, dev, host, moe_decode_views

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    yield
    torch.cuda.synchronize()


def _logits(seed, T, E, kind="rand", idle=()):
    g = np.random.default_rng(seed)
    L = g.integers(-2, 3, size=(T, E)).astype(np.float32) if kind == "ties" else g.standard_normal((T, E)).astype(
        np.float32)
    for e in idle:
        L[:, e] = -50.0
    return L


def _experts(seed, E, d, d_ff, dtype):
    return [synth.random_case(seed * 100 + e, 1, d, d_ff, 1, dtype) for e in range(E)]


def _stack(exps, key, dtype):
    return torch.stack([dev(c[key], dtype) for c in exps]).contiguous()


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("T,E,kind", [(1, 2, "rand"), (5, 3, "ties"), (32, 8, "rand"), (1000, 8, "ties"),
                                      (8195, 8, "rand"), (300, 64, "rand"), (0, 8, "rand")])
def test_moe_route(T, E, kind):
    say(f"[moe route] T={T} E={E} {kind}")
    L = _logits(T + E, T, E, kind)
    ex, wt, off, tok, slot = pop.pop_moe_route_top2(dev(L, "f32"))
    torch.cuda.synchronize()
    ex, wt, off, tok, slot = (host(a) for a in (ex, wt, off, tok, slot))
    if T == 0:
        assert (off == 0).all()
        return
    ex_ref, wt_ref = oracle.moe_route_top2(L)
    assert np.array_equal(ex, ex_ref)
    np.testing.assert_allclose(wt, wt_ref, rtol=0, atol=2e-6)
    counts = np.array([(ex_ref == e).any(axis=1).sum() for e in range(E)])
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(counts)]))
    for e in range(E):
        assert np.array_equal(tok[off[e]:off[e + 1]], np.flatnonzero((ex_ref == e).any(axis=1)))
    for t in range(T):
        for j in range(2):
            p = slot[t, j]
            assert tok[p] == t and off[ex[t, j]] <= p < off[ex[t, j] + 1]


# ------------------------------------------------------------------ prefill
PREFILL = [
    # name, n_tokens, d, d_ff, E, dtype, idle experts
    ("f32_E4", 50, 64, 200, 4, "f32", ()),
    ("bf16_E8", 300, 520, 700, 8, "bf16", ()),
    ("bf16_E8_idle_expert", 100, 128, 300, 8, "bf16", (5,)),
    ("f32_E2", 40, 32, 100, 2, "f32", ()),
    ("bf16_E32", 200, 64, 150, 32, "bf16", ()),
    ("bf16_empty_prompt", 0, 64, 150, 4, "bf16", ()),
]


@pytest.mark.parametrize("name,n,d,d_ff,E,dtype,idle", PREFILL, ids=[c[0] for c in PREFILL])
def test_moe_prefill(name, n, d, d_ff, E, dtype, idle):
    say(f"[moe prefill] {name}")
    r, gamma = 0.3, 0.1
    X = synth.random_case(n + d, n, d, 1, 1, dtype)["X"]
    L = _logits(n + 7, n, E, idle=idle)
    exps = _experts(n + 3, E, d, d_ff, dtype)
    R, C, P, I = pop.pop_moe_prefill_partition(dev(X, dtype), dev(L, "f32"), _stack(exps, "W_up", dtype), r, gamma,
                                               importance=True)
    torch.cuda.synchronize()
    ex, _ = oracle.moe_route_top2(L) if n else (np.zeros((0, 2), np.int64), None)
    for e in range(E):
        toks = np.flatnonzero((ex == e).any(axis=1))
        s = oracle.column_norm(X[toks]) if len(toks) else np.zeros(d)
        I_ref = oracle.importance(exps[e]["W_up"], s)
        n_ex = check_partition(R[e], C[e], P[e], I[e], I_ref, r, gamma)
        if n_ex:
            say(f"  expert {e}: near-tie exclusions {n_ex}")


# ------------------------------------------------------------------ decode
def _check_moe_step(x, L, exps, parts, r, dtype, y, S, ws):
    """Checks one MoE decode step; returns the relative error of y."""
    T = x.shape[0]
    E = len(exps)
    d_ff = exps[0]["W_gate"].shape[0]
    ex, _ = oracle.moe_route_top2(L)
    n_R, n_C = len(parts[0][0]), len(parts[0][1])
    z_dev, sc_dev = moe_decode_views(ws, T, d_ff, E, n_R + n_C, n_C)
    S = host(S).astype(np.int64)
    off = 0
    k = S.shape[1]
    sel_dev = [None] * E
    for e in range(E):
        rows, slot = np.nonzero(ex == e)
        order = np.argsort(rows, kind="stable")
        rows, slot = rows[order], slot[order]
        if len(rows) == 0:
            continue
        R_e, C_e, _ = parts[e]
        zr = oracle.restricted_forward(x[rows], exps[e]["W_gate"], exps[e]["W_up"], R_e, C_e)
        scale = max(np.abs(zr).max(), 1e-30)
        zd = z_dev[off: off + len(rows)].astype(np.float64)
        assert np.abs(zd - zr).max() <= VALUE_RTOL * scale, f"expert {e}: z differs"
        sr = oracle.candidate_scores(zr, len(R_e))
        sd = sc_dev[e].astype(np.float64)
        np.testing.assert_allclose(sd, sr, rtol=VALUE_RTOL, atol=1e-6 * scale)
        # exact selection on the device's scores
        assert np.array_equal(S[e], oracle.select_candidates(C_e, sd, k)), f"expert {e}: selection"
        # against fp64: near-ties only
        S_ref = oracle.select_candidates(C_e, sr, k)
        for ch in np.setxor1d(S[e], S_ref):
            srt = np.sort(sr)[::-1]
            cuts = [srt[j] for j in (k - 1, k) if 0 <= j < len(C_e)]
            v = sr[np.searchsorted(C_e, ch)]
            assert any(abs(v - t) <= TIE_REL * max(t, 1e-30) for t in cuts), f"expert {e}: candidate {ch}"
        sel_dev[e] = S[e]
        off += len(rows)
    # the output: the oracle's MoE step (routing, per-expert steps, weighted
    # combine) evaluated on the device's selections
    y_ref, _ = oracle.moe_decode_step(x, L, exps, parts, r, selections=sel_dev)
    err = np.abs(host(y) - y_ref).max() / max(np.abs(y_ref).max(), 1e-30)
    assert err <= TOL[dtype], f"max|dy|/max|y| = {err:.3e}"
    return err


DECODE = [
    # name, T, d, d_ff, E, dtype, r, idle
    ("f32_T5_E4", 5, 64, 200, 4, "f32", 0.3, ()),
    ("bf16_T32_E8", 32, 256, 600, 8, "bf16", 0.3, ()),
    ("bf16_T9_E8_idle", 9, 128, 333, 8, "bf16", 0.299, (2, 6)),
    ("bf16_T1_E8", 1, 520, 700, 8, "bf16", 0.3, ()),
    ("f32_T20_E3_r0", 20, 64, 150, 3, "f32", 0.0, ()),
    ("bf16_T64_E16", 64, 128, 300, 16, "bf16", 0.5, ()),
    # past 4096 candidates per expert: the per-expert top-k as its own launch
    ("bf16_T8_E4_wide_C", 8, 64, 21000, 4, "bf16", 0.3, ()),
    # past 64 tokens: the FMA kernels
    ("bf16_T80_E8_fma", 80, 128, 300, 8, "bf16", 0.3, ()),
]


@pytest.mark.parametrize("name,T,d,d_ff,E,dtype,r,idle", DECODE, ids=[c[0] for c in DECODE])
def test_moe_decode(name, T, d, d_ff, E, dtype, r, idle):
    say(f"[moe decode] {name}")
    gamma = 0.1
    exps = _experts(T + 11, E, d, d_ff, dtype)
    Xp = synth.random_case(T + 12, 64, d, 1, 1, dtype)["X"]
    parts = oracle.moe_partitions(Xp, _logits(T + 13, 64, E), [c["W_up"] for c in exps], r, gamma)
    x = synth.random_case(T + 14, 1, d, 1, T, dtype)["x"]
    L = _logits(T + 15, T, E, idle=idle)
    R = torch.from_numpy(np.stack([p[0] for p in parts]).astype(np.int32)).cuda()
    C = torch.from_numpy(np.stack([p[1] for p in parts]).astype(np.int32)).cuda()
    ws = pop.workspace(pop.pop_moe_decode_workspace_bytes(T, d, d_ff, E))
    y, S = pop.pop_moe_decode_ffn(dev(x, dtype), dev(L, "f32"), _stack(exps, "W_gate", dtype),
                                  _stack(exps, "W_up", dtype), _stack(exps, "W_downT", dtype), R, C, r,
                                  selected=True, ws=ws)
    torch.cuda.synchronize()
    err = _check_moe_step(x, L, exps, parts, r, dtype, y, S, ws)
    say(f"  rel err {err:.2e}")


def test_moe_decode_deterministic_and_graph_replay():
    say("[moe decode] determinism and HIP-graph replay")
    T, d, d_ff, E, dtype, r = 16, 256, 500, 8, "bf16", 0.3
    exps = _experts(91, E, d, d_ff, dtype)
    parts = oracle.moe_partitions(synth.random_case(92, 40, d, 1, 1, dtype)["X"], _logits(93, 40, E),
                                  [c["W_up"] for c in exps], r, 0.1)
    R = torch.from_numpy(np.stack([p[0] for p in parts]).astype(np.int32)).cuda()
    C = torch.from_numpy(np.stack([p[1] for p in parts]).astype(np.int32)).cuda()
    Wg, Wu, WdT = (_stack(exps, k, dtype) for k in ("W_gate", "W_up", "W_downT"))
    x1 = dev(synth.random_case(94, 1, d, 1, T, dtype)["x"], dtype)
    x2 = dev(synth.random_case(95, 1, d, 1, T, dtype)["x"], dtype)
    L1, L2 = dev(_logits(96, T, E), "f32"), dev(_logits(97, T, E), "f32")
    ws = pop.workspace(pop.pop_moe_decode_workspace_bytes(T, d, d_ff, E))
    y1 = pop.pop_moe_decode_ffn(x1, L1, Wg, Wu, WdT, R, C, r, ws=ws)
    y1b = pop.pop_moe_decode_ffn(x1, L1, Wg, Wu, WdT, R, C, r, ws=ws)
    y2 = pop.pop_moe_decode_ffn(x2, L2, Wg, Wu, WdT, R, C, r)
    torch.cuda.synchronize()
    assert torch.equal(y1, y1b)
    x_in, L_in, yg = x1.clone(), L1.clone(), torch.empty_like(y1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pop.pop_moe_decode_ffn(x_in, L_in, Wg, Wu, WdT, R, C, r, y=yg, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pop.pop_moe_decode_ffn(x_in, L_in, Wg, Wu, WdT, R, C, r, y=yg, ws=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        x_in.copy_(x1 if rep % 2 == 0 else x2)
        L_in.copy_(L1 if rep % 2 == 0 else L2)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y1 if rep % 2 == 0 else y2), f"replay {rep} differs from eager"


def test_moe_full_size():
    """The Mixtral-like layer: 8 experts of 4096 x 14336, 8192 prompt tokens,
    one decode step of 32 tokens."""
    w = configs.MIXTRAL_MOE
    E, d, d_ff, r, gamma = w.experts, w.d, w.d_ff, w.r, w.gamma
    n = w.prompt_batch * w.prompt_len
    say(f"[moe full size] {w.name}: generating {E} experts")
    exps = [synth.layer_weights(w, e) for e in range(E)]
    X = synth.prompt(w, 0)
    Lp = synth.router_logits(w, n, 0)
    x = synth.decode_input(w, 0, 0)
    Ld = synth.router_logits(w, x.shape[0], 1)
    Wu = _stack(exps, "W_up", w.dtype)
    say("  prefill partition")
    R, C, P, I = pop.pop_moe_prefill_partition(dev(X, w.dtype), dev(Lp, "f32"), Wu, r, gamma, importance=True)
    torch.cuda.synchronize()
    ex, _ = oracle.moe_route_top2(Lp)
    parts = []
    for e in range(E):
        toks = np.flatnonzero((ex == e).any(axis=1))
        I_ref = oracle.importance(exps[e]["W_up"], oracle.column_norm(X[toks]))
        n_ex = check_partition(R[e], C[e], P[e], I[e], I_ref, r, gamma)
        say(f"  expert {e}: {len(toks)} prompt tokens, near-tie exclusions {n_ex}")
        parts.append((host(R[e]).astype(np.int64), host(C[e]).astype(np.int64), host(P[e]).astype(np.int64)))
    say("  decode step")
    ws = pop.workspace(pop.pop_moe_decode_workspace_bytes(x.shape[0], d, d_ff, E))
    y, S = pop.pop_moe_decode_ffn(dev(x, w.dtype), dev(Ld, "f32"), _stack(exps, "W_gate", w.dtype), Wu,
                                  _stack(exps, "W_downT", w.dtype), R, C, r, selected=True, ws=ws)
    torch.cuda.synchronize()
    err = _check_moe_step(x, Ld, exps, parts, r, w.dtype, y, S, ws)
    say(f"  decode rel err {err:.2e}")
