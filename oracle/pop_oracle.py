"""Plain, slow, float64 CPU oracle of POP (Partition-guided Online Pruning).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the device path.

Sources (cited by title and section; the pages are web notes and abstracts):
  [POP]  "POP: Online Structural Pruning Enables Efficient Inference of Large
         Foundation Models" (paper notes), sections "Overall framework",
         "Key design 1" (prefill three-region partition, importance equation),
         "Key design 2" (decode candidate-local masking, H_t equation),
         "Key design 3" (FFN only), "Loss / training strategy" (gamma = 0.1,
         Wanda metric, online masking from the second step).
  [ABS]  "POP: Online Structural Pruning ..." abstract page (retained,
         candidate and pruned regions).
  [BWP]  "Batch-wise adaptive pruning ... for language reasoning models",
         section 3.1 equation (1) (gated MLP), section 1 and figure 2(a) (a
         batch shares one mask; per-sample scores aggregated by element-wise
         max), figure 1 and figure 2(b) (the mask refreshed by a top-k only
         periodically, an activation memory carrying importance to the next
         refresh).

Everything is float64.  Inputs given in bf16 enter as the exact float64 value
of their bits.  Each stage follows the pages' steps in their order; where the
pages leave a step open the reading taken is named in the docstring:

  R1  importance uses row i of W_up: I_i = || W_up[i,:] * s ||_2 (the printed
      W_{:,i} is ill-typed against s in R^{C_in}; an output channel of W_up is
      a row).
  R2  delta = gamma (gamma = 0.1 gives a candidate share of about 20%).
  R3  q_p is the order statistic at cut rank round(p * D_FF); p is clamped to
      [0, 1]; round is half away from zero.
  R4  one total order everywhere: larger value = more important; on equal
      values the lower channel index is more important.
  R5  the decode score of candidate i is max over the batch of |z_i| with
      z = SiLU(W_gate x) * (W_up x).
  R6  live count = round((1 - r) * D_FF); k = live - |R|, kept in [0, |C|].
  R7  no biases; SiLU(a) = a * sigmoid(a).
  R8  MoE: top-2 routing (ties to the lower expert), weights = softmax of the
      two chosen logits; one partition per expert over its routed prompt
      tokens; per step, the batch max runs over the tokens routed to it.
  R17 periodic refresh ([BWP] figures 1 and 2(b); its own definition is cut
      off in the pages): inside POP's candidate set, step t refreshes the
      selection when t % period == 0.  The activation memory holds, per
      candidate, the sum of its step scores (R5) over the steps since the last
      refresh on which it was computed (every candidate on a refresh step, the
      selected ones in between); a refresh ranks the candidates by the memory
      including its own step's scores, keeps the k best (R4, R6) and clears it;
      the other steps compute R plus the kept selection only.

Parity unpinned by the pages (no worked example is printed): the decode score
formula (R5), the quantile convention (R3) and the tie rule (R4) are fixed
readings; the tests pin the oracle against closed forms, brute force and
invariants instead.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "round_half_away", "partition_counts", "column_norm", "importance",
    "total_order", "partition", "partition_by_sort", "silu", "restricted_forward",
    "candidate_scores", "select_candidates", "pruned_ffn", "masked_ffn",
    "dense_ffn", "decode_step", "moe_route_top2", "moe_partitions", "moe_decode_step",
    "static_mask_ffn", "full_reeval_ffn", "periodic_decode",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------------------ counts
def round_half_away(v: float) -> int:
    """Round half away from zero (reading R3/R6)."""
    f = math.floor(v)
    frac = v - f
    if v >= 0:
        return int(f + 1) if frac >= 0.5 else int(f)
    return -round_half_away(-v)


def partition_counts(d_ff: int, r: float, gamma: float) -> dict:
    """Sizes of P, C, R and the per-step top-k count.

    [POP] Key design 1: thresholds q_{r-delta} and q_{r+delta}; Key design 2:
    |R| plus the selected candidates equals exactly the live count that r
    requires.  Readings R2 (delta = gamma), R3, R6.
    """
    n = int(d_ff)
    delta = float(gamma)
    p_lo = min(max(float(r) - delta, 0.0), 1.0)
    p_hi = min(max(float(r) + delta, 0.0), 1.0)
    c_low = round_half_away(p_lo * n)
    c_high = round_half_away(p_hi * n)
    n_live = round_half_away((1.0 - float(r)) * n)
    c_mid = min(max(n - n_live, c_low), c_high)
    return {
        "d_ff": n, "c_low": c_low, "c_high": c_high,
        "n_P": c_low, "n_C": c_high - c_low, "n_R": n - c_high,
        "n_live": n_live, "k": c_high - c_mid,
    }


# ------------------------------------------------------------------ prefill
def column_norm(X) -> np.ndarray:
    """s_k = || X[:, :, k] ||_2 over every prompt token of every sequence.

    [POP] Key design 1, importance equation (s).  X may be [B, L, C_in] or
    already flattened to [B*L, C_in]."""
    X = _f64(X)
    X = X.reshape(-1, X.shape[-1])
    acc = np.zeros(X.shape[1])
    for row in X:                       # plain sum of squares, token by token
        acc += row * row
    return np.sqrt(acc)


def importance(W_up, s) -> np.ndarray:
    """I_i = || W_up[i, :] (elementwise*) s ||_2 for every intermediate channel i.

    [POP] Key design 1 (importance equation) under reading R1; the Wanda-style
    |W| * ||X||_2 metric of "Loss / training strategy" (the absolute value is
    immaterial under the square)."""
    W = _f64(W_up)
    s = _f64(s)
    return np.sqrt(((W * s[None, :]) ** 2).sum(axis=1))


def total_order(values) -> np.ndarray:
    """Channel indices from least to most important (reading R4)."""
    v = _f64(values)
    idx = np.arange(len(v))
    return np.lexsort((-idx, v))        # primary: value ascending; ties: higher index first


def _least_important(values: np.ndarray, c: int) -> np.ndarray:
    """Boolean mask of the c least important channels, found with a value
    order statistic (the quantile) and the index tie rule R4."""
    n = len(values)
    m = np.zeros(n, dtype=bool)
    if c <= 0:
        return m
    if c >= n:
        m[:] = True
        return m
    tau = np.sort(values)[c - 1]        # the quantile value q at this cut rank
    below = values < tau
    m |= below
    ties = np.flatnonzero(values == tau)           # ascending channel indices
    need = c - int(below.sum())
    if need > 0:
        m[ties[len(ties) - need:]] = True          # higher index is less important
    return m


def partition(I, r: float, gamma: float):
    """Three-region partition of the channels by the quantile thresholds.

    [POP] Key design 1: tau_low = q_{r-delta}, tau_high = q_{r+delta};
    P = {I <= tau_low}, R = {I >= tau_high}, C = strictly between; the three
    sets are disjoint.  Channels equal to a threshold are split by rule R4 so
    that the sizes are exactly those of :func:`partition_counts`.
    Returns (R, C, P) as ascending int64 index arrays."""
    I = _f64(I)
    cnt = partition_counts(len(I), r, gamma)
    in_P = _least_important(I, cnt["c_low"])
    below_high = _least_important(I, cnt["c_high"])
    in_R = ~below_high
    in_C = below_high & ~in_P
    return np.flatnonzero(in_R), np.flatnonzero(in_C), np.flatnonzero(in_P)


def partition_by_sort(I, r: float, gamma: float):
    """Second formulation: rank slices of one brute-force full sort."""
    cnt = partition_counts(len(I), r, gamma)
    pi = total_order(I)
    P = np.sort(pi[:cnt["c_low"]])
    C = np.sort(pi[cnt["c_low"]:cnt["c_high"]])
    R = np.sort(pi[cnt["c_high"]:])
    return R, C, P


# ------------------------------------------------------------------ decode
def silu(a) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a), with the sigmoid evaluated without overflow."""
    a = _f64(a)
    out = np.empty_like(a)
    pos = a >= 0
    out[pos] = a[pos] / (1.0 + np.exp(-a[pos]))
    e = np.exp(a[~pos])
    out[~pos] = a[~pos] * e / (1.0 + e)
    return out


def restricted_forward(x, W_gate, W_up, R, C) -> np.ndarray:
    """H_t = f(X_t; R u C): the gated-MLP intermediate activation restricted
    to the rows R then C of W_gate and W_up.

    [POP] Key design 2 (H_t equation); [BWP] section 3.1 eq. (1):
    z = SiLU(W_g x) * (W_1 x).  Returns z as [B, |R| + |C|], R columns first."""
    x = _f64(x).reshape(-1, np.shape(x)[-1])
    A = np.concatenate([np.asarray(R, dtype=np.int64), np.asarray(C, dtype=np.int64)])
    g = x @ _f64(W_gate)[A].T
    u = x @ _f64(W_up)[A].T
    return silu(g) * u


def candidate_scores(z, n_R: int) -> np.ndarray:
    """Step-local importance of each candidate: max over the batch of |z_i|
    (reading R5; [BWP] figure 2(a) for the batch max)."""
    z = _f64(z)
    return np.abs(z[:, n_R:]).max(axis=0) if z.shape[0] else np.zeros(z.shape[1] - n_R)


def select_candidates(C, scores, k: int) -> np.ndarray:
    """[POP] Key design 2: sort the candidates by their step score, highest
    first (ties: lower index first, rule R4), and keep the first k.
    Returns the selected channel indices in ascending order."""
    C = np.asarray(C, dtype=np.int64)
    scores = _f64(scores)
    ranked = sorted(range(len(C)), key=lambda j: (-scores[j], C[j]))
    return np.sort(C[ranked[:k]])


def _k_for(d_ff: int, r: float, n_R: int, n_C: int) -> int:
    n_live = round_half_away((1.0 - float(r)) * int(d_ff))
    return min(max(n_live - n_R, 0), n_C)


def decode_step(x, W_gate, W_up, W_down, R, C, r: float):
    """One decode step of POP on one layer, gather form.

    [POP] Overall framework and Key design 2: H_t over R u C, candidate
    scores, top-k over C so that |R| + k is the live count, then the FFN on R
    plus the selected candidates.  W_down is [D, D_FF] (eq. (1) layout).
    Returns dict(y [B, D], S, z, scores, k)."""
    R = np.asarray(R, dtype=np.int64)
    C = np.asarray(C, dtype=np.int64)
    d_ff = _f64(W_gate).shape[0]
    z = restricted_forward(x, W_gate, W_up, R, C)
    scores = candidate_scores(z, len(R))
    k = _k_for(d_ff, r, len(R), len(C))
    S = select_candidates(C, scores, k)
    pos = {int(c): j for j, c in enumerate(C)}
    live = np.concatenate([R, S])
    zpos = np.concatenate([np.arange(len(R)), len(R) + np.array([pos[int(c)] for c in S], dtype=np.int64)])
    Wd = _f64(W_down)
    y = z[:, zpos] @ Wd[:, live].T
    return {"y": y, "S": S, "z": z, "scores": scores, "k": k}


def pruned_ffn(x, W_gate, W_up, W_down, R, C, r: float) -> np.ndarray:
    return decode_step(x, W_gate, W_up, W_down, R, C, r)["y"]


def masked_ffn(x, W_gate, W_up, W_down, live) -> np.ndarray:
    """Second formulation: the dense gated MLP over all D_FF channels with
    every channel outside ``live`` zeroed before W_down."""
    x = _f64(x).reshape(-1, np.shape(x)[-1])
    d_ff = _f64(W_gate).shape[0]
    m = np.zeros(d_ff)
    m[np.asarray(live, dtype=np.int64)] = 1.0
    z = silu(x @ _f64(W_gate).T) * (x @ _f64(W_up).T)
    return (z * m[None, :]) @ _f64(W_down).T


def dense_ffn(x, W_gate, W_up, W_down) -> np.ndarray:
    """[BWP] eq. (1): y = W_2 (SiLU(W_g x) * (W_1 x)), no channel removed.
    Also the prefill forward, which POP runs dense ([POP] "online masking from
    the second step")."""
    x = _f64(x).reshape(-1, np.shape(x)[-1])
    return (silu(x @ _f64(W_gate).T) * (x @ _f64(W_up).T)) @ _f64(W_down).T


# ------------------------------------------------------------------ ablation variants
def static_mask_ffn(x, W_gate, W_up, W_down, R, C, S_prefill) -> np.ndarray:
    """[POP] ablation table, variant (1): the mask fixed at prefill (R plus a
    prefill-chosen subset of C) reused at every decode step."""
    live = np.concatenate([np.asarray(R, dtype=np.int64), np.asarray(S_prefill, dtype=np.int64)])
    return masked_ffn(x, W_gate, W_up, W_down, live)


def full_reeval_ffn(x, W_gate, W_up, W_down, r: float):
    """[POP] ablation table, variant (2): every channel re-scored at every
    step (same score as R5), keep the round((1-r) D_FF) best."""
    d_ff = _f64(W_gate).shape[0]
    allc = np.arange(d_ff)
    z = restricted_forward(x, W_gate, W_up, np.zeros(0, dtype=np.int64), allc)
    sc = candidate_scores(z, 0)
    n_live = round_half_away((1.0 - float(r)) * d_ff)
    S = select_candidates(allc, sc, n_live)
    return {"y": z[:, S] @ _f64(W_down)[:, S].T, "S": S}


# ------------------------------------------------------------------ periodic refresh
def periodic_decode(xs, W_gate, W_up, W_down, R, C, r: float, period: int):
    """[BWP] figure 1 and figure 2(b) read into POP's candidate set (reading
    R17): the candidate selection is refreshed by a top-k only every
    ``period`` steps, ranking by an activation memory of accumulated step
    scores.  xs: the inputs of consecutive steps, each [B, D].  Returns one
    dict per step: y [B, D], S (selected channels, ascending), refresh (bool)
    and memory (after the step, per position of C)."""
    R = np.asarray(R, dtype=np.int64)
    C = np.asarray(C, dtype=np.int64)
    n_R = len(R)
    d_ff = _f64(W_gate).shape[0]
    k = _k_for(d_ff, r, n_R, len(C))
    Wd = _f64(W_down)
    pos_of = {int(c): j for j, c in enumerate(C)}
    memory = np.zeros(len(C))
    S = np.zeros(0, dtype=np.int64)
    out = []
    for t, x in enumerate(xs):
        refresh = t % int(period) == 0
        if refresh:
            # every candidate computed: its score joins the memory, which ranks them
            z = restricted_forward(x, W_gate, W_up, R, C)
            memory = memory + candidate_scores(z, n_R)
            S = select_candidates(C, memory, k)
            spos = np.array([pos_of[int(c)] for c in S], dtype=np.int64)
            z_live = np.concatenate([z[:, :n_R], z[:, n_R + spos]], axis=1)
            memory = np.zeros(len(C))
        else:
            # R plus the kept selection: only the selected candidates are observed
            z_live = restricted_forward(x, W_gate, W_up, R, S)
            spos = np.array([pos_of[int(c)] for c in S], dtype=np.int64)
            memory[spos] += candidate_scores(z_live, n_R)
        live = np.concatenate([R, S])
        y = z_live @ Wd[:, live].T
        out.append({"y": y, "S": S.copy(), "refresh": refresh, "memory": memory.copy()})
    return out


# ------------------------------------------------------------------ MoE
def moe_route_top2(logits):
    """Top-2 routing: each token's two largest logits (ties to the lower
    expert id) and softmax weights over the two (reading R8)."""
    L = _f64(logits)
    T, E = L.shape
    experts = np.zeros((T, 2), dtype=np.int64)
    weights = np.zeros((T, 2))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-L[t, e], e))
        e1, e2 = order[0], order[1]
        m = max(L[t, e1], L[t, e2])
        w1, w2 = math.exp(L[t, e1] - m), math.exp(L[t, e2] - m)
        experts[t] = (e1, e2)
        weights[t] = (w1 / (w1 + w2), w2 / (w1 + w2))
    return experts, weights


def moe_partitions(X, logits, experts_W_up, r: float, gamma: float):
    """One (R, C, P) per expert over the prompt tokens routed to it
    ([POP] "Loss / training strategy": partitions built in the first prefill
    pass under dynamic routing)."""
    X = _f64(X).reshape(-1, np.shape(X)[-1])
    ex, _ = moe_route_top2(logits)
    parts = []
    for e, Wu in enumerate(experts_W_up):
        toks = np.flatnonzero((ex == e).any(axis=1))
        s = column_norm(X[toks]) if len(toks) else np.zeros(X.shape[1])
        parts.append(partition(importance(Wu, s), r, gamma))
    return parts


def moe_decode_step(x, logits, experts, parts, r: float, selections=None):
    """One MoE decode step: each expert runs POP decode on the tokens routed
    to it (batch max over them), outputs combined with the routing weights:
    y_tok = sum over the token's two experts of w_e * y_e(tok) (reading R8).
    ``experts`` is a list of dicts with W_gate, W_up, W_down.
    ``selections`` (optional, per expert: its selected candidates, or None)
    replaces each expert's own selection step, so that the output can be
    evaluated on another implementation's selection (the parity protocol's
    step for admissible near-tie flips); the rest of the step is unchanged."""
    x = _f64(x).reshape(-1, np.shape(x)[-1])
    ex, wt = moe_route_top2(logits)
    y = np.zeros((x.shape[0], _f64(experts[0]["W_down"]).shape[0]))
    sel = []
    for e, ew in enumerate(experts):
        rows, slot = np.nonzero(ex == e)
        if len(rows) == 0:
            sel.append(None)
            continue
        R, C, _ = parts[e]
        if selections is not None and selections[e] is not None:
            S = np.asarray(selections[e], dtype=np.int64)
            ye = masked_ffn(x[rows], ew["W_gate"], ew["W_up"], ew["W_down"], np.concatenate([R, S]))
        else:
            out = decode_step(x[rows], ew["W_gate"], ew["W_up"], ew["W_down"], R, C, r)
            S, ye = out["S"], out["y"]
        y[rows] += wt[rows, slot][:, None] * ye
        sel.append(S)
    return y, sel
