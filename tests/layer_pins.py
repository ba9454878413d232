"""Pins of the decoder-layer oracle to facts outside itself.

Each ``pin_*`` takes the layer-oracle module ``lo`` and raises AssertionError
when it disagrees with a closed form, an independent library routine (torch
CPU: bfloat16 conversion, rms_norm, scaled_dot_product_attention, complex
multiplication), brute force in plain Python on tiny inputs, or an invariant
of the layer (causality, cache consistency between the prompt pass and a
decode step).  ``test_layer_oracle`` runs them on the real oracle and on
copies with planted mistakes.
"""
from __future__ import annotations

import cmath
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def _weights(g, D, H, Hkv, hd, dff, std=0.2):
    return {
        "attn_norm": g.uniform(0.5, 1.5, D), "ffn_norm": g.uniform(0.5, 1.5, D),
        "Wqkv_T": g.normal(0, std, (D, (H + 2 * Hkv) * hd)), "Wo_T": g.normal(0, std, (H * hd, D)),
        "W_gate": g.normal(0, std, (dff, D)), "W_up": g.normal(0, std, (dff, D)),
        "W_down": g.normal(0, std, (D, dff)),
    }


def _cfg(H, Hkv, hd, eps=1e-5, theta=10000.0):
    return {"H": H, "H_kv": Hkv, "hd": hd, "eps": eps, "theta": theta}


# ------------------------------------------------------------------ bf16 storage
def pin_round_bf16_library(lo):
    g = _rng(11)
    a = g.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    # exact ties: low 16 bits 0x8000 with both parities of the kept bit
    bits = (g.integers(0x3c000000, 0x44000000, 4000, dtype=np.uint32) & np.uint32(0xffff0000)) | np.uint32(0x8000)
    a = np.concatenate([a, bits.view(np.float32), -bits.view(np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(lo.round_bf16(a.astype(np.float64)), ref)


# ------------------------------------------------------------------ RMSNorm
def pin_rms_norm(lo):
    g = _rng(12)
    D = 24
    w = g.uniform(0.5, 2.0, D)
    for c in (3.0, -0.25):                         # constant vector: c / sqrt(c^2 + eps)
        got = lo.rms_norm(np.full(D, c), w, 1e-5)
        np.testing.assert_allclose(got, w * c / math.sqrt(c * c + 1e-5), rtol=1e-13)
    e = np.zeros(D)
    e[5] = 2.0                                     # one spike: mean square = 4 / D
    got = lo.rms_norm(e, w, 0.0)
    np.testing.assert_allclose(got[5], w[5] * 2.0 / math.sqrt(4.0 / D), rtol=1e-13)
    v = g.standard_normal((3, 7, D))
    ref = F.rms_norm(_t(v), (D,), weight=_t(w), eps=1e-5).numpy()
    np.testing.assert_allclose(lo.rms_norm(v, w, 1e-5), ref, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ rotary embedding
def pin_rope_complex_form(lo):
    """RoFormer's complex form: pair (2i, 2i+1) read as x_{2i} + j x_{2i+1}
    is multiplied by exp(j pos theta^(-2i/hd))."""
    g = _rng(13)
    n_heads, hd, theta = 3, 8, 10000.0
    for pos in (0, 1, 7, 513):
        v = g.standard_normal((n_heads, hd))
        got = lo.rope(v[None], np.array([pos]), theta)[0]
        for h in range(n_heads):
            for i in range(hd // 2):
                zc = complex(v[h, 2 * i], v[h, 2 * i + 1]) * cmath.exp(1j * pos * theta ** (-2.0 * i / hd))
                assert abs(got[h, 2 * i] - zc.real) < 1e-12 and abs(got[h, 2 * i + 1] - zc.imag) < 1e-12


def pin_rope_relative(lo):
    """<R(m) q, R(n) k> depends on m - n only; R(0) is the identity."""
    g = _rng(14)
    hd = 16
    q, k = g.standard_normal((1, hd)), g.standard_normal((1, hd))
    np.testing.assert_allclose(lo.rope(q[None], np.array([0]), 500.0)[0], q, rtol=0, atol=0)
    dots = []
    for s in (0, 3, 40):
        a = lo.rope(q[None], np.array([9 + s]), 500.0)[0, 0]
        b = lo.rope(k[None], np.array([4 + s]), 500.0)[0, 0]
        dots.append(a @ b)
    np.testing.assert_allclose(dots, dots[0], rtol=1e-11)


# ------------------------------------------------------------------ attention
def pin_attend_brute_force(lo):
    g = _rng(15)
    H, Hkv, hd, L = 4, 2, 3, 6
    q = g.standard_normal((H, hd))
    K, V = g.standard_normal((Hkv, L, hd)), g.standard_normal((Hkv, L, hd))
    for n in (1, 4, 6):
        got = lo.attend(q, K, V, n)
        for h in range(H):
            kv = h // (H // Hkv)
            s = [sum(q[h, c] * K[kv, j, c] for c in range(hd)) / math.sqrt(hd) for j in range(n)]
            w = [math.exp(v - max(s)) for v in s]
            for c in range(hd):
                ref = sum(w[j] * V[kv, j, c] for j in range(n)) / sum(w)
                assert abs(got[h, c] - ref) < 1e-12, (n, h, c)
    # one key: its value; equal keys: the mean of the values
    np.testing.assert_allclose(lo.attend(q, K, V, 1), V[[0, 0, 1, 1], 0], rtol=1e-13)
    Ke = np.repeat(K[:, :1], L, axis=1)
    np.testing.assert_allclose(lo.attend(q, Ke, V, L), V.mean(axis=1)[[0, 0, 1, 1]], rtol=1e-12)


def _torch_attention_block(x, lw, cfg, act_round):
    """The prompt pass's attention branch from torch routines: rms_norm,
    complex rotation (torch.polar), scaled_dot_product_attention(is_causal)."""
    B, T, D = x.shape
    H, Hkv, hd = cfg["H"], cfg["H_kv"], cfg["hd"]
    xn = act_round(F.rms_norm(_t(x), (D,), weight=_t(lw["attn_norm"]), eps=cfg["eps"]))
    qkv = xn @ _t(lw["Wqkv_T"])
    q = qkv[..., : H * hd].reshape(B, T, H, hd)
    k = qkv[..., H * hd: (H + Hkv) * hd].reshape(B, T, Hkv, hd)
    v = qkv[..., (H + Hkv) * hd:].reshape(B, T, Hkv, hd)
    i = torch.arange(hd // 2, dtype=torch.float64)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * cfg["theta"] ** (-2.0 * i / hd)
    rot = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]

    def rotate(a):
        c = torch.view_as_complex(a.reshape(*a.shape[:-1], hd // 2, 2).contiguous()) * rot
        return torch.view_as_real(c).reshape(a.shape)

    q, k = rotate(q), act_round(rotate(k))
    v = act_round(v)
    rep = H // Hkv
    kk = k.transpose(1, 2).repeat_interleave(rep, dim=1)
    vv = v.transpose(1, 2).repeat_interleave(rep, dim=1)
    o = F.scaled_dot_product_attention(q.transpose(1, 2), kk, vv, is_causal=True)
    o = act_round(o.transpose(1, 2).reshape(B, T, H * hd))
    return (_t(x) + o @ _t(lw["Wo_T"])).numpy(), k.numpy(), v.numpy()


def pin_attention_block_library(lo):
    g = _rng(16)
    for (B, T, D, H, Hkv, hd, act) in ((2, 9, 16, 4, 4, 4, "f32"), (1, 11, 24, 4, 2, 6, "f32"),
                                       (2, 7, 16, 2, 1, 8, "bf16")):
        cfg = _cfg(H, Hkv, hd, theta=100.0)
        lw = _weights(g, D, H, Hkv, hd, 8)
        x = g.standard_normal((B, T, D))
        K = np.zeros((B, Hkv, T + 3, hd))
        V = np.zeros_like(K)
        got = lo.attention_block(x, lw, cfg, K, V, 0, act)
        rnd = (lambda a: a.to(torch.bfloat16).to(torch.float64)) if act == "bf16" else (lambda a: a)
        ref, k, v = _torch_attention_block(x, lw, cfg, rnd)
        tol = 1e-12 if act == "f32" else 1e-9
        np.testing.assert_allclose(got, ref, rtol=tol, atol=tol)
        np.testing.assert_allclose(K[:, :, :T], k.transpose(0, 2, 1, 3), rtol=tol, atol=tol)
        np.testing.assert_allclose(V[:, :, :T], v.transpose(0, 2, 1, 3), rtol=tol, atol=tol)
        assert not K[:, :, T:].any() and not V[:, :, T:].any()


def pin_attention_causal(lo):
    """Changing later tokens changes nothing at earlier positions."""
    g = _rng(17)
    B, T, D, H, Hkv, hd = 1, 8, 16, 2, 2, 4
    cfg = _cfg(H, Hkv, hd)
    lw = _weights(g, D, H, Hkv, hd, 8)
    x = g.standard_normal((B, T, D))
    y = x.copy()
    y[:, 5:] = g.standard_normal((B, T - 5, D))
    K1, K2 = np.zeros((B, Hkv, T, hd)), np.zeros((B, Hkv, T, hd))
    a = lo.attention_block(x, lw, cfg, K1, K1.copy(), 0, "f32")
    b = lo.attention_block(y, lw, cfg, K2, K2.copy(), 0, "f32")
    np.testing.assert_allclose(a[:, :5], b[:, :5], rtol=1e-13)
    assert np.abs(a[:, 5:] - b[:, 5:]).max() > 1e-3


# ------------------------------------------------------------------ whole layer
def pin_prefill_then_decode(lo):
    """The prompt pass over N + 1 tokens, last row, equals the prompt pass over
    N tokens followed by one decode step with the dense FFN (and with POP at
    r = 0, where every channel stays live)."""
    g = _rng(18)
    for act in ("f32", "bf16"):
        B, N, D, H, Hkv, hd, dff = 2, 6, 16, 4, 2, 4, 12
        cfg = _cfg(H, Hkv, hd, theta=50.0)
        lw = _weights(g, D, H, Hkv, hd, dff)
        X = g.standard_normal((B, N + 1, D))
        full = lo.layer_prefill(X, lw, cfg, 0.3, 0.1, act, N + 1)
        pre = lo.layer_prefill(X[:, :N], lw, cfg, 0.3, 0.1, act, N + 1)
        for dense, r in ((True, 0.3), (False, 0.0)):
            K, V = pre["K"].copy(), pre["V"].copy()
            R, C = (pre["R"], pre["C"]) if dense else oracle.partition(pre["I"], 0.0, 0.1)[:2]
            st = lo.layer_decode(X[:, N], lw, cfg, K, V, N, R, C, r, act, dense_ffn=dense)
            np.testing.assert_allclose(st["x"], full["x"][:, N], rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(K, full["K"], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(V, full["V"], rtol=1e-12, atol=1e-12)


def pin_layer_composition(lo):
    """With Wo = 0 the attention branch vanishes (h = x); with the FFN's down
    projection zero the FFN branch vanishes; the decode step's FFN is the POP
    step of the FFN oracle on RMSNorm_f(h)."""
    g = _rng(19)
    B, D, H, Hkv, hd, dff, pos = 3, 16, 2, 2, 8, 20, 5
    cfg = _cfg(H, Hkv, hd)
    lw = _weights(g, D, H, Hkv, hd, dff)
    x = g.standard_normal((B, D))
    K, V = g.standard_normal((B, Hkv, 8, hd)), g.standard_normal((B, Hkv, 8, hd))
    R, C, _ = oracle.partition(g.uniform(0, 1, dff), 0.3, 0.1)
    z = dict(lw, Wo_T=np.zeros_like(lw["Wo_T"]))
    st = lo.layer_decode(x, z, cfg, K.copy(), V.copy(), pos, R, C, 0.3, "f32")
    xn = lw["ffn_norm"] * x / np.sqrt((x * x).mean(axis=1, keepdims=True) + cfg["eps"])
    ref = oracle.decode_step(xn, lw["W_gate"], lw["W_up"], lw["W_down"], R, C, 0.3)
    np.testing.assert_allclose(st["h"], x, rtol=0, atol=0)
    np.testing.assert_allclose(st["x"], x + ref["y"], rtol=1e-12, atol=1e-12)
    assert np.array_equal(st["S"], ref["S"])
    z = dict(lw, W_down=np.zeros_like(lw["W_down"]))
    st = lo.layer_decode(x, z, cfg, K.copy(), V.copy(), pos, R, C, 0.3, "f32")
    np.testing.assert_allclose(st["x"], st["h"], rtol=0, atol=0)
    assert np.abs(st["h"] - x).max() > 1e-3


def pin_bf16_storage_points(lo):
    """act='bf16' stores bf16 values where R22 says and leaves the residual
    stream unrounded."""
    g = _rng(20)
    B, N, D, H, Hkv, hd, dff = 1, 5, 16, 2, 2, 8, 12
    cfg = _cfg(H, Hkv, hd)
    lw = _weights(g, D, H, Hkv, hd, dff)
    X = g.standard_normal((B, N, D))
    p = lo.layer_prefill(X, lw, cfg, 0.3, 0.1, "bf16", N)
    for a in (p["K"], p["V"], p["xn2"]):
        assert np.array_equal(a, torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy())
    assert not np.array_equal(p["h"], torch.from_numpy(p["h"]).to(torch.bfloat16).to(torch.float64).numpy())
    f = lo.layer_prefill(X, lw, cfg, 0.3, 0.1, "f32", N)
    assert 0 < np.abs(p["x"] - f["x"]).max() < 0.05 * np.abs(f["x"]).max()


def pin_ffn_budget(lo):
    """[POP] Key design 3 prints 29.9% for a 20% global rate on LLaMA-2-7B
    (multi-head attention, 32 heads of 128)."""
    with open(os.path.join(GOLDEN, "ffn_budget.json")) as f:
        gld = json.load(f)
    r = lo.ffn_prune_rate(gld["global_rate"], gld["d"], gld["d_ff"], 32, 32, 128)
    assert round(100 * r, 1) == gld["printed_ffn_rate_percent"]
    # grouped-query attention holds fewer attention weights, so less moves to the FFN
    assert lo.ffn_prune_rate(0.2, 4096, 11008, 32, 8, 128) < r
    assert abs(lo.ffn_prune_rate(0.2, 8, 16, 1, 1, 8) - 0.2 * (4 * 64 + 3 * 128) / (3 * 128)) < 1e-15


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
