"""Comparison of the HIP path with the CPU oracle.

Selections (partition regions, selected candidates) are integer results decided
by floating point.  They are checked twice:
  1. exactly, against the oracle's selection rule applied to the device's own
     fp32 values (importance I, candidate scores): the same decision in the
     same precision, so any difference is a selection bug;
  2. against the fp64 oracle end to end, where a channel may differ only if its
     fp64 value lies within ``TIE_REL`` (relative) of a cut value; such
     channels are counted and reported.
Outputs are compared element by element against the oracle evaluated on the
device's selection (so an admissible near-tie flip cannot fail the output
check), with max|dy| <= tol * max|y_ref|:
  fp32 inputs: tol = 1e-5;  bf16 inputs with fp32 accumulation: tol = 2e-2.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from online_structured_ffn_amd import pop

TIE_REL = 1e-4
Z_OFFSET = pop.DECODE_WS_Z_OFFSET
TOL = {"f32": 1e-5, "bf16": 2e-2}
# Device importance / scores against fp64: fp32 sums of non-negative terms
# (chunked, depth well under 200 additions) stay within 200 * 2^-24 ~ 1.2e-5;
# 1e-4 leaves margin and matches the tie window.
VALUE_RTOL = 1e-4


def dev(a, dtype: str, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)   # exact: the values are bf16-representable
    return t.to(device).contiguous()


def host(t):
    return t.detach().to("cpu").numpy()


def check_partition(R, C, P, I_dev, I_ref, r, gamma):
    """Returns the number of near-tie exclusions against the fp64 oracle."""
    R, C, P = (np.asarray(host(t), dtype=np.int64) for t in (R, C, P))
    I_dev = np.asarray(host(I_dev), dtype=np.float64)
    cnt = oracle.partition_counts(len(I_ref), r, gamma)
    assert (len(P), len(C), len(R)) == (cnt["n_P"], cnt["n_C"], cnt["n_R"])
    # values
    np.testing.assert_allclose(I_dev, I_ref, rtol=VALUE_RTOL, atol=1e-30)
    # 1. same decision on the device's own values: exact
    eR, eC, eP = oracle.partition(I_dev, r, gamma)
    assert np.array_equal(R, eR), "R differs from the oracle rule on the device's importance"
    assert np.array_equal(C, eC), "C differs from the oracle rule on the device's importance"
    assert np.array_equal(P, eP), "P differs from the oracle rule on the device's importance"
    # 2. against fp64, with near-tie exclusions at the four cut values
    oR, oC, oP = oracle.partition(I_ref, r, gamma)
    n = len(I_ref)
    lab_dev = np.zeros(n, dtype=np.int8)
    lab_dev[C], lab_dev[R] = 1, 2
    lab_ref = np.zeros(n, dtype=np.int8)
    lab_ref[oC], lab_ref[oR] = 1, 2
    diff = np.flatnonzero(lab_dev != lab_ref)
    if len(diff):
        pi = oracle.total_order(I_ref)
        cuts = [I_ref[pi[c]] for c in (cnt["c_low"] - 1, cnt["c_low"], cnt["c_high"] - 1, cnt["c_high"])
                if 0 <= c < n]
        for i in diff:
            near = any(abs(I_ref[i] - t) <= TIE_REL * max(t, 1e-30) for t in cuts)
            assert near, f"channel {i} differs and is not a near tie (I={I_ref[i]!r})"
    return len(diff)


def check_decode(y, S, ws, x, w, R, C, r, dtype, z_ref=None):
    """w: dict with W_gate, W_up, W_down (fp32/bf16 values as float arrays).
    ws: the device workspace after the call (z then scores).
    Returns (relative max error of y, near-tie exclusions)."""
    R = np.asarray(R, dtype=np.int64)
    C = np.asarray(C, dtype=np.int64)
    B = x.shape[0]
    n_R, n_C = len(R), len(C)
    d_ff = w["W_gate"].shape[0]
    k = oracle.partition_counts(d_ff, r, 0.0)["n_live"] - n_R
    k = max(0, min(k, n_C))
    S = np.asarray(host(S), dtype=np.int64)
    assert len(S) == k
    ref = oracle.decode_step(x, w["W_gate"], w["W_up"], w["W_down"], R, C, r)
    n_A = n_R + n_C
    raw = host(ws)
    # the first POP_DECODE_WS_Z_OFFSET bytes are control words, zero after every completed call
    ctl = raw[:Z_OFFSET].view(np.uint32)
    assert not ctl.any(), f"decode control words not zero after the call: {np.flatnonzero(ctl)}"
    wsf = raw.view(np.float32)[Z_OFFSET // 4:]    # z starts at byte POP_DECODE_WS_Z_OFFSET
    z_dev = wsf[: B * n_A].reshape(B, n_A).astype(np.float64)
    zb = (B * d_ff * 4 + 16 + 255) // 256 * 256 // 4   # scores: Z_OFFSET + align_up(4*B*d_ff + 16, 256) bytes
    sc_dev = wsf[zb: zb + n_C].astype(np.float64)
    # intermediate and scores
    zr = ref["z"]
    scale = max(np.abs(zr).max(), 1e-30) if zr.size else 1.0
    if B:
        assert np.abs(z_dev - zr).max() <= VALUE_RTOL * scale, "z differs"
    if n_C:
        np.testing.assert_allclose(sc_dev, ref["scores"], rtol=VALUE_RTOL, atol=1e-6 * scale)
    # 1. exact selection on the device's own scores
    eS = oracle.select_candidates(C, sc_dev, k)
    assert np.array_equal(S, eS), "selection differs from the oracle rule on the device's scores"
    # 2. against fp64 with near-tie exclusions
    diff = np.setxor1d(S, ref["S"])
    if len(diff):
        srt = np.sort(ref["scores"])[::-1]
        cuts = [srt[j] for j in (k - 1, k) if 0 <= j < n_C]
        pos = {int(c): j for j, c in enumerate(C)}
        for ch in diff:
            v = ref["scores"][pos[int(ch)]]
            assert any(abs(v - t) <= TIE_REL * max(t, 1e-30) for t in cuts), f"candidate {ch} is not a near tie"
    # output against the oracle on the device's selection
    live = np.concatenate([R, S])
    y_ref = oracle.masked_ffn(x, w["W_gate"], w["W_up"], w["W_down"], live)
    y_dev = host(y).astype(np.float64)
    if B == 0:
        return 0.0, len(diff)
    m = max(np.abs(y_ref).max(), 1e-30)
    err = np.abs(y_dev - y_ref).max() / m
    assert err <= TOL[dtype], f"max|dy|/max|y| = {err:.3e} > {TOL[dtype]}"
    return err, len(diff)


def moe_decode_views(ws, n_tokens, d_ff, n_experts, n_A, n_C):
    """(z [2T, n_A], scores [E, n_C]) of a pop_moe_decode_ffn workspace, after
    the layout the header documents."""
    a = lambda b: (b + 255) // 256 * 256
    P = 2 * max(n_tokens, 1)
    o = a(P * 4) + a(P * 4) + a((n_experts + 1) * 4) + a(P * 4) + a(P * 4)
    raw = host(ws)
    z = raw[o: o + P * n_A * 4].view(np.float32).reshape(P, n_A)
    o += a(P * d_ff * 4)
    sc = raw[o: o + n_experts * n_C * 4].view(np.float32).reshape(n_experts, n_C)
    return z, sc
