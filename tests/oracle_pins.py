"""Pins of the CPU oracle to facts outside itself.

Each ``pin_*`` takes an oracle module ``o`` and raises AssertionError when the
oracle disagrees with a hand-worked example, a closed form, an independent
library routine (torch CPU / scipy), brute force on tiny inputs or an
invariant of the method.  ``test_oracle_pins`` runs them on the real oracle;
``test_oracle_mutants`` runs them on copies of the oracle with planted mistakes
and requires that at least one pin fails for each.
"""
from __future__ import annotations

import json
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _brute_rank(I):
    """rank_i = number of channels less important than i (larger value more
    important; equal value: lower index more important), by direct counting."""
    n = len(I)
    rank = np.zeros(n, dtype=np.int64)
    for i in range(n):
        for j in range(n):
            if I[j] < I[i] or (I[j] == I[i] and j > i):
                rank[i] += 1
    return rank


def _torch_ffn(x, Wg, Wu, Wd):
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    x = t(x)
    return (F.silu(F.linear(x, t(Wg))) * F.linear(x, t(Wu))).matmul(t(Wd).T).numpy()


# ------------------------------------------------------------------ counts
def pin_counts_table(o):
    for row in _load("partition_counts.json")["rows"]:
        c = o.partition_counts(row["d_ff"], row["r"], row["gamma"])
        for key in ("n_P", "n_C", "n_R", "n_live", "k"):
            assert c[key] == row[key], (row, key, c)


def pin_counts_invariants(o):
    g = _rng(1)
    for _ in range(400):
        n = int(g.integers(1, 3000))
        r = float(g.uniform(0, 0.95))
        gam = float(g.uniform(0, 0.5))
        c = o.partition_counts(n, r, gam)
        assert c["n_P"] + c["n_C"] + c["n_R"] == n
        assert min(c["n_P"], c["n_C"], c["n_R"]) >= 0
        assert 0 <= c["k"] <= c["n_C"]
        live = int(np.floor((1 - r) * n + 0.5))
        if c["n_R"] <= live <= c["n_R"] + c["n_C"]:
            assert c["n_R"] + c["k"] == live
        if gam <= r <= 1 - gam:   # unclamped window: candidate share is 2*delta
            assert abs(c["n_C"] / n - 2 * gam) <= 1.0 / n + 1e-12


# ------------------------------------------------------------------ prefill
def pin_hand_partition(o):
    h = _load("partition_hand_example.json")
    X = np.array(h["X"], dtype=float)
    W = np.array(h["W_up"], dtype=float)
    s = o.column_norm(X)
    np.testing.assert_allclose(s ** 2, h["s_squared"], rtol=1e-15, atol=1e-15)
    I = o.importance(W, s)
    np.testing.assert_allclose(I ** 2, h["I_squared"], rtol=1e-14, atol=1e-14)
    c = o.partition_counts(len(W), h["r"], h["gamma"])
    for k, v in h["counts"].items():
        assert c[k] == v, (k, c)
    for form in (o.partition, o.partition_by_sort):
        R, C, P = form(I, h["r"], h["gamma"])
        assert list(R) == h["R"] and list(C) == h["C"] and list(P) == h["P"], (form.__name__, R, C, P)


def pin_column_norm_library(o):
    g = _rng(2)
    X = g.standard_normal((3, 7, 11))
    np.testing.assert_allclose(o.column_norm(X), np.linalg.norm(X.reshape(-1, 11), axis=0), rtol=1e-14)
    e = np.zeros((5, 6))
    e[3, 4] = 1.0
    np.testing.assert_array_equal(o.column_norm(e), np.eye(6)[4])


def pin_importance_closed_forms(o):
    g = _rng(3)
    W = g.standard_normal((9, 13))
    np.testing.assert_allclose(o.importance(W, np.ones(13)), np.linalg.norm(W, axis=1), rtol=1e-14)
    # one nonzero per row: I_i = |w_i| * s_{k_i}
    s = g.uniform(0.5, 3.0, 13)
    cols = g.integers(0, 13, 9)
    w = g.standard_normal(9)
    W1 = np.zeros((9, 13))
    W1[np.arange(9), cols] = w
    np.testing.assert_allclose(o.importance(W1, s), np.abs(w) * s[cols], rtol=1e-14)
    # a non-square, non-symmetric case against torch's vector norm
    Wr = g.standard_normal((5, 8))
    sr = g.uniform(0.1, 4.0, 8)
    ref = torch.linalg.vector_norm(torch.as_tensor(Wr) * torch.as_tensor(sr)[None, :], dim=1).numpy()
    np.testing.assert_allclose(o.importance(Wr, sr), ref, rtol=1e-14)


def _check_partition(o, I, r, gam):
    c = o.partition_counts(len(I), r, gam)
    rank = _brute_rank(I)
    exp_P = np.flatnonzero(rank < c["c_low"])
    exp_C = np.flatnonzero((rank >= c["c_low"]) & (rank < c["c_high"]))
    exp_R = np.flatnonzero(rank >= c["c_high"])
    for form in (o.partition, o.partition_by_sort):
        R, C, P = form(I, r, gam)
        assert np.array_equal(R, exp_R) and np.array_equal(C, exp_C) and np.array_equal(P, exp_P), \
            (form.__name__, I, r, gam)


def pin_partition_brute_force(o):
    g = _rng(4)
    for trial in range(300):
        n = int(g.integers(1, 40))
        r = float(g.uniform(0, 0.95))
        gam = float(g.uniform(0, 0.5))
        if trial % 2:
            I = g.integers(0, 4, n).astype(float)    # many exact ties
        else:
            I = g.uniform(0, 1, n)
        _check_partition(o, I, r, gam)


def pin_partition_invariances(o):
    g = _rng(5)
    X = g.standard_normal((12, 16))
    W = g.standard_normal((60, 16))
    base = o.partition(o.importance(W, o.column_norm(X)), 0.3, 0.1)
    # scaling X or W_up by a positive constant
    for X2, W2 in ((3.0 * X, W), (X, 0.25 * W)):
        got = o.partition(o.importance(W2, o.column_norm(X2)), 0.3, 0.1)
        assert all(np.array_equal(a, b) for a, b in zip(base, got))
    # rescaling input channel k by c and W_up[:, k] by 1/c (powers of two: exact)
    X3, W3 = X.copy(), W.copy()
    X3[:, 5] *= 8.0
    W3[:, 5] /= 8.0
    got = o.partition(o.importance(W3, o.column_norm(X3)), 0.3, 0.1)
    assert all(np.array_equal(a, b) for a, b in zip(base, got))
    # permuting W_up rows permutes the partition
    perm = g.permutation(60)
    Rp, Cp, Pp = o.partition(o.importance(W[perm], o.column_norm(X)), 0.3, 0.1)
    inv = np.argsort(perm)
    for a, b in zip(base, (Rp, Cp, Pp)):
        assert np.array_equal(np.sort(inv[a]), b)
    # order: every P below every C below every R
    I = o.importance(W, o.column_norm(X))
    R, C, P = base
    assert I[P].max() <= I[C].min() and I[C].max() <= I[R].min()


def pin_partition_all_equal(o):
    # X = 0 makes every importance 0: R is the lowest-index channels, P the highest
    W = _rng(6).standard_normal((50, 8))
    R, C, P = o.partition(o.importance(W, o.column_norm(np.zeros((4, 8)))), 0.3, 0.1)
    c = o.partition_counts(50, 0.3, 0.1)
    assert list(R) == list(range(c["n_R"]))
    assert list(P) == list(range(50 - c["n_P"], 50))


# ------------------------------------------------------------------ decode
def pin_silu_library(o):
    a = np.concatenate([np.linspace(-50, 50, 1001), [-800.0, 800.0, 0.0]])
    np.testing.assert_allclose(o.silu(a), a * scipy.special.expit(a), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(o.silu(a), F.silu(torch.as_tensor(a)).numpy(), rtol=1e-14, atol=1e-300)
    assert o.silu(np.array([0.0]))[0] == 0.0


def pin_restricted_forward_library(o):
    g = _rng(7)
    d, dff, b = 10, 23, 3
    Wg, Wu, x = g.standard_normal((dff, d)), g.standard_normal((dff, d)), g.standard_normal((b, d))
    R, C = np.array([1, 4, 9, 20]), np.array([0, 7, 22])
    A = np.concatenate([R, C])
    t = lambda a: torch.as_tensor(a)
    ref = (F.silu(F.linear(t(x), t(Wg[A]))) * F.linear(t(x), t(Wu[A]))).numpy()
    np.testing.assert_allclose(o.restricted_forward(x, Wg, Wu, R, C), ref, rtol=1e-13, atol=1e-14)


def pin_scores_and_selection(o):
    # score is the max over the batch of |z| on candidate columns only
    z = np.array([[1.0, -5.0, 2.0, -0.5], [-3.0, 1.0, -4.0, 0.25]])
    np.testing.assert_array_equal(o.candidate_scores(z, 1), [5.0, 4.0, 0.5])
    g = _rng(8)
    for trial in range(300):
        n = int(g.integers(0, 30))
        C = np.sort(g.choice(1000, n, replace=False))
        sc = g.integers(0, 4, n).astype(float) if trial % 2 else g.uniform(0, 1, n)
        k = int(g.integers(0, n + 1))
        S = o.select_candidates(C, sc, k)
        # brute force: candidate j is selected iff fewer than k candidates beat it
        beats = np.array([sum((sc[m] > sc[j]) or (sc[m] == sc[j] and C[m] < C[j]) for m in range(n))
                          for j in range(n)], dtype=np.int64)
        assert np.array_equal(S, C[beats < k]), (C, sc, k, S)


def pin_dense_library(o):
    g = _rng(9)
    d, dff, b = 12, 31, 4
    Wg, Wu, Wd, x = (g.standard_normal((dff, d)), g.standard_normal((dff, d)),
                     g.standard_normal((d, dff)), g.standard_normal((b, d)))
    np.testing.assert_allclose(o.dense_ffn(x, Wg, Wu, Wd), _torch_ffn(x, Wg, Wu, Wd), rtol=1e-12, atol=1e-12)


def pin_r0_is_dense(o):
    g = _rng(10)
    d, dff, b = 16, 40, 2
    Wg, Wu, Wd = g.standard_normal((dff, d)), g.standard_normal((dff, d)), g.standard_normal((d, dff))
    X, x = g.standard_normal((9, d)), g.standard_normal((b, d))
    R, C, P = o.partition(o.importance(Wu, o.column_norm(X)), 0.0, 0.1)
    assert len(P) == 0
    out = o.decode_step(x, Wg, Wu, Wd, R, C, 0.0)
    assert out["k"] == len(C)
    np.testing.assert_allclose(out["y"], _torch_ffn(x, Wg, Wu, Wd), rtol=1e-11, atol=1e-11)


def pin_gather_equals_mask(o):
    g = _rng(11)
    for trial in range(20):
        d, dff, b = int(g.integers(2, 20)), int(g.integers(5, 80)), int(g.integers(1, 5))
        r = float(g.uniform(0.05, 0.8))
        Wg, Wu, Wd = g.standard_normal((dff, d)), g.standard_normal((dff, d)), g.standard_normal((d, dff))
        X, x = g.standard_normal((7, d)), g.standard_normal((b, d))
        R, C, P = o.partition(o.importance(Wu, o.column_norm(X)), r, 0.1)
        out = o.decode_step(x, Wg, Wu, Wd, R, C, r)
        c = o.partition_counts(dff, r, 0.1)
        assert len(R) + len(out["S"]) == c["n_live"] == len(R) + c["k"]
        live = np.concatenate([R, out["S"]])
        # the gather form equals the dense FFN (torch) with every other channel's W_down column zeroed
        Wd_m = np.zeros_like(Wd)
        Wd_m[:, live] = Wd[:, live]
        np.testing.assert_allclose(out["y"], _torch_ffn(x, Wg, Wu, Wd_m), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(out["y"], o.masked_ffn(x, Wg, Wu, Wd, live), rtol=1e-11, atol=1e-12)
        # selection is the top-k of max_b |z| over C (recomputed with torch)
        t = lambda a: torch.as_tensor(a)
        zc = (F.silu(F.linear(t(x), t(Wg[C]))) * F.linear(t(x), t(Wu[C]))).abs().amax(0).numpy()
        if len(out["S"]) and len(out["S"]) < len(C):
            inS = np.isin(C, out["S"])
            assert zc[inS].min() >= zc[~inS].max() - 1e-12


def pin_hand_decode(o):
    h = _load("partition_hand_example.json")
    d, dff = 3, 10
    Wg = np.zeros((dff, d))
    Wu = np.zeros((dff, d))
    for ch, row in h["W_gate_rows"].items():
        Wg[int(ch)] = row
    for ch, row in h["W_up_rows_for_decode"].items():
        Wu[int(ch)] = row
    Wd = np.ones((d, dff))
    out = o.decode_step(np.array(h["decode_x"], dtype=float), Wg, Wu, Wd, h["R"], h["C"], h["r"])
    assert list(out["S"]) == h["S"], out["S"]


def pin_zero_input_decode(o):
    g = _rng(12)
    d, dff = 8, 30
    Wg, Wu, Wd = g.standard_normal((dff, d)), g.standard_normal((dff, d)), g.standard_normal((d, dff))
    R, C, P = o.partition(g.uniform(0, 1, dff), 0.4, 0.1)
    out = o.decode_step(np.zeros((2, d)), Wg, Wu, Wd, R, C, 0.4)
    assert list(out["S"]) == list(C[:out["k"]])
    assert np.all(out["y"] == 0)


def pin_batch_properties(o):
    g = _rng(13)
    d, dff = 9, 37
    Wg, Wu, Wd = g.standard_normal((dff, d)), g.standard_normal((dff, d)), g.standard_normal((d, dff))
    R, C, P = o.partition(g.uniform(0, 1, dff), 0.3, 0.1)
    x1 = g.standard_normal((1, d))
    a = o.decode_step(x1, Wg, Wu, Wd, R, C, 0.3)
    b = o.decode_step(np.repeat(x1, 4, axis=0), Wg, Wu, Wd, R, C, 0.3)
    assert np.array_equal(a["S"], b["S"])
    np.testing.assert_allclose(b["y"], np.repeat(a["y"], 4, axis=0), rtol=1e-13, atol=1e-14)
    xb = g.standard_normal((5, d))
    perm = g.permutation(5)
    c1 = o.decode_step(xb, Wg, Wu, Wd, R, C, 0.3)
    c2 = o.decode_step(xb[perm], Wg, Wu, Wd, R, C, 0.3)
    assert np.array_equal(c1["S"], c2["S"])
    np.testing.assert_allclose(c2["y"], c1["y"][perm], rtol=1e-13, atol=1e-14)
    # the shared mask ranks candidates by the batch max, not by any single row
    zc = np.abs(o.restricted_forward(xb, Wg, Wu, R, C)[:, len(R):]).max(0)
    inS = np.isin(C, c1["S"])
    assert zc[inS].min() >= zc[~inS].max()


# ------------------------------------------------------------------ MoE
def pin_moe_routing(o):
    L = np.array([[0.0, 2.0, 1.0, 2.0], [5.0, 5.0, 5.0, -1.0], [1.0, -2.0, 3.0, 0.5]])
    ex, wt = o.moe_route_top2(L)
    assert ex.tolist() == [[1, 3], [0, 1], [2, 0]]
    np.testing.assert_allclose(wt.sum(1), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(wt[0], [0.5, 0.5])
    e = np.exp(np.array([3.0, 1.0]))
    np.testing.assert_allclose(wt[2], e / e.sum(), rtol=1e-15)


def pin_moe_identical_experts(o):
    # two identical experts share every routed token: the output equals the
    # single-expert POP decode of the tokens they share (weights sum to 1)
    g = _rng(14)
    d, dff, E = 8, 25, 2
    w = {"W_gate": g.standard_normal((dff, d)), "W_up": g.standard_normal((dff, d)),
         "W_down": g.standard_normal((d, dff))}
    X = g.standard_normal((6, d))
    x = g.standard_normal((3, d))
    logits_p = g.standard_normal((6, E))
    logits_d = g.standard_normal((3, E))
    parts = o.moe_partitions(X, logits_p, [w["W_up"]] * E, 0.3, 0.1)
    single = o.partition(o.importance(w["W_up"], o.column_norm(X)), 0.3, 0.1)
    for p in parts:
        assert all(np.array_equal(a, b) for a, b in zip(p, single))
    y, _ = o.moe_decode_step(x, logits_d, [w] * E, parts, 0.3)
    ref = o.decode_step(x, w["W_gate"], w["W_up"], w["W_down"], *single[:2], 0.3)["y"]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def _dense_by_hand(x, w):
    """W_down (SiLU(W_gate x) * (W_up x)) per row, SiLU from scipy's expit."""
    g = x @ w["W_gate"].T
    u = x @ w["W_up"].T
    return (g * scipy.special.expit(g) * u) @ w["W_down"].T


def pin_moe_weighted_combine_by_hand(o):
    # 2 tokens, 3 distinct experts, r = 0 (each expert's step is its dense FFN,
    # pinned by pin_r0_is_dense): logits chosen so the top-2 softmax weights
    # are exact and unequal.  Token 0: experts 1 (ln 3) and 0 (0) -> 3/4, 1/4.
    # Token 1: experts 2 (ln 4) and 1 (0) -> 4/5, 1/5.
    g = _rng(17)
    d, dff, E = 5, 9, 3
    exps = [{"W_gate": g.standard_normal((dff, d)), "W_up": g.standard_normal((dff, d)),
             "W_down": g.standard_normal((d, dff))} for _ in range(E)]
    X = g.standard_normal((4, d))
    parts = o.moe_partitions(X, g.standard_normal((4, E)), [e["W_up"] for e in exps], 0.0, 0.1)
    x = g.standard_normal((2, d))
    L = np.array([[0.0, np.log(3.0), -5.0], [-3.0, 0.0, np.log(4.0)]])
    y, _ = o.moe_decode_step(x, L, exps, parts, 0.0)
    ref = np.stack([0.75 * _dense_by_hand(x[:1], exps[1])[0] + 0.25 * _dense_by_hand(x[:1], exps[0])[0],
                    0.8 * _dense_by_hand(x[1:], exps[2])[0] + 0.2 * _dense_by_hand(x[1:], exps[1])[0]])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def pin_moe_zeroed_expert(o):
    # distinct experts, one with W_down = 0: a token routed to it and to expert
    # e gets exactly w_e * y_e(token), its POP step on expert e alone
    g = _rng(18)
    d, dff, E = 6, 30, 4
    exps = [{"W_gate": g.standard_normal((dff, d)), "W_up": g.standard_normal((dff, d)),
             "W_down": g.standard_normal((d, dff))} for _ in range(E)]
    exps[2]["W_down"] = np.zeros((d, dff))
    X = g.standard_normal((12, d))
    parts = o.moe_partitions(X, g.standard_normal((12, E)), [e["W_up"] for e in exps], 0.3, 0.1)
    T = 7
    x = g.standard_normal((T, d))
    L = g.standard_normal((T, E))
    L[:, 2] = 10.0  # expert 2 is every token's first choice
    ex, wt = o.moe_route_top2(L)
    y, _ = o.moe_decode_step(x, L, exps, parts, 0.3)
    for e in (0, 1, 3):
        rows = np.flatnonzero(ex[:, 1] == e)
        if len(rows) == 0:
            continue
        R, C, _ = parts[e]
        ye = o.decode_step(x[rows], exps[e]["W_gate"], exps[e]["W_up"], exps[e]["W_down"], R, C, 0.3)["y"]
        np.testing.assert_allclose(y[rows], wt[rows, 1][:, None] * ye, rtol=1e-12, atol=1e-13)
        assert np.all(wt[rows, 1] < 0.5)  # the second weight is the smaller one here


def pin_moe_expert_subsets(o):
    # each expert's partition uses exactly the prompt tokens routed to it
    g = _rng(15)
    d, dff, E = 6, 20, 4
    X = g.standard_normal((10, d))
    Wus = [g.standard_normal((dff, d)) for _ in range(E)]
    logits = g.standard_normal((10, E))
    ex, _ = o.moe_route_top2(logits)
    parts = o.moe_partitions(X, logits, Wus, 0.3, 0.1)
    for e in range(E):
        toks = [t for t in range(10) if e in ex[t]]
        s = np.sqrt((X[toks] ** 2).sum(0)) if toks else np.zeros(d)
        I = np.sqrt(((Wus[e] * s) ** 2).sum(1))
        rank = _brute_rank(I)
        c = o.partition_counts(dff, 0.3, 0.1)
        assert np.array_equal(parts[e][2], np.flatnonzero(rank < c["c_low"]))
        assert np.array_equal(parts[e][0], np.flatnonzero(rank >= c["c_high"]))


def pin_ablation_variants(o):
    g = _rng(16)
    d, dff = 7, 30
    Wg, Wu, Wd = g.standard_normal((dff, d)), g.standard_normal((dff, d)), g.standard_normal((d, dff))
    x = g.standard_normal((2, d))
    full = o.full_reeval_ffn(x, Wg, Wu, Wd, 0.3)
    c = o.partition_counts(dff, 0.3, 0.1)
    assert len(full["S"]) == c["n_live"]
    Wd_m = np.zeros_like(Wd)
    Wd_m[:, full["S"]] = Wd[:, full["S"]]
    np.testing.assert_allclose(full["y"], _torch_ffn(x, Wg, Wu, Wd_m), rtol=1e-12, atol=1e-12)
    R, C, P = o.partition(g.uniform(0, 1, dff), 0.3, 0.1)
    S0 = C[: c["k"]]
    Wd_s = np.zeros_like(Wd)
    live = np.concatenate([R, S0])
    Wd_s[:, live] = Wd[:, live]
    np.testing.assert_allclose(o.static_mask_ffn(x, Wg, Wu, Wd, R, C, S0), _torch_ffn(x, Wg, Wu, Wd_s),
                               rtol=1e-12, atol=1e-12)


def pin_periodic_special_cases(o):
    """Refreshing every step is POP's per-step selection; never refreshing
    after step 0 is the dense FFN with the step-0 mask (torch)."""
    g = _rng(17)
    d, dff, T = 6, 40, 5
    Wg, Wu, Wd = g.standard_normal((dff, d)), g.standard_normal((dff, d)), g.standard_normal((d, dff))
    R, C, P = o.partition(g.uniform(0, 1, dff), 0.3, 0.1)
    xs = [g.standard_normal((2, d)) for _ in range(T)]
    every = o.periodic_decode(xs, Wg, Wu, Wd, R, C, 0.3, 1)
    for t in range(T):
        ref = o.decode_step(xs[t], Wg, Wu, Wd, R, C, 0.3)
        assert np.array_equal(every[t]["S"], ref["S"]) and every[t]["refresh"]
        np.testing.assert_allclose(every[t]["y"], ref["y"], rtol=1e-12, atol=1e-13)
    once = o.periodic_decode(xs, Wg, Wu, Wd, R, C, 0.3, T + 3)
    S0 = o.decode_step(xs[0], Wg, Wu, Wd, R, C, 0.3)["S"]
    live = np.concatenate([R, S0])
    Wd_m = np.zeros_like(Wd)
    Wd_m[:, live] = Wd[:, live]
    for t in range(1, T):
        assert np.array_equal(once[t]["S"], S0) and not once[t]["refresh"]
        np.testing.assert_allclose(once[t]["y"], _torch_ffn(xs[t], Wg, Wu, Wd_m), rtol=1e-12, atol=1e-12)


def pin_periodic_brute_force(o):
    """The refresh schedule and the activation memory, simulated on the dense
    activations of every channel (torch) with an explicit lexicographic
    ranking; at least one refresh must pick differently from the step's own
    scores, so the memory is exercised."""
    g = _rng(18)
    t_ = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    memory_mattered = False
    for trial in range(12):
        d, dff, T = int(g.integers(3, 9)), int(g.integers(20, 60)), 7
        period = int(g.integers(2, 4))
        Wg, Wu, Wd = g.standard_normal((dff, d)), g.standard_normal((dff, d)), g.standard_normal((d, dff))
        R, C, P = o.partition(g.uniform(0, 1, dff), 0.3, 0.1)
        k = o.partition_counts(dff, 0.3, 0.1)["k"]
        xs = [g.standard_normal((int(g.integers(1, 4)), d)) for _ in range(T)]
        got = o.periodic_decode(xs, Wg, Wu, Wd, R, C, 0.3, period)
        mem = np.zeros(len(C))
        keep = np.zeros(0, dtype=np.int64)          # positions into C
        for t in range(T):
            zf = (F.silu(F.linear(t_(xs[t]), t_(Wg))) * F.linear(t_(xs[t]), t_(Wu))).numpy()
            sc = np.abs(zf[:, C]).max(axis=0)
            if t % period == 0:
                mem = mem + sc
                order = np.lexsort((C, -mem))          # memory descending, then channel ascending
                keep = np.sort(order[:k])
                alone = np.sort(np.lexsort((C, -sc))[:k])
                memory_mattered |= not np.array_equal(alone, keep)
                mem = np.zeros(len(C))
            else:
                mem[keep] += sc[keep]
            live = np.concatenate([R, C[keep]])
            Wd_m = np.zeros_like(Wd)
            Wd_m[:, live] = Wd[:, live]
            assert np.array_equal(got[t]["S"], C[keep]), (trial, t)
            np.testing.assert_allclose(got[t]["memory"], mem, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(got[t]["y"], zf @ Wd_m.T, rtol=1e-10, atol=1e-11)
    assert memory_mattered


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
