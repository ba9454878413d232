"""Float64 CPU oracle of a whole decoder layer whose FFN is pruned by POP.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the device path.

Sources:
  [POP]  "POP: Online Structural Pruning Enables Efficient Inference of Large
         Foundation Models" (paper notes), "Key design 3": the attention
         block keeps all of its parameters and runs dense; the whole pruning
         budget goes to the FFN (a global 20% on LLaMA-2-7B becomes 29.9% of
         the FFN's channels).  "Limitations": no channel of self-attention is
         pruned.  "Loss / training strategy": the prompt's forward pass runs
         dense and yields the partition; masking starts at the second step.
  The pages evaluate on LLaMA-family models but define none of the attention
  block, so its parts are taken from their published definitions:
  [RMS]  Zhang and Sennrich, "Root Mean Square Layer Normalization" (2019),
         equation (4).
  [ROPE] Su et al., "RoFormer: Enhanced Transformer with Rotary Position
         Embedding" (2021), section 3.2, equations (14)-(15).
  [ATT]  Vaswani et al., "Attention Is All You Need" (2017), section 3.2.1
         (scaled dot-product attention), with the decoder's causal mask.
  [LLAMA] Touvron et al., "Llama 2" (2023) and "LLaMA" (2023), section 2.2:
         pre-normalisation with RMSNorm, SwiGLU FFN, rotary embeddings;
         grouped-query attention for the largest model.

Readings (the pages leave these open):
  R18 the layer is pre-norm with two residual branches:
        h = x + Attn(RMSNorm_a(x)),  out = h + FFN(RMSNorm_f(h)),
      and the FFN is POP's pruned gated MLP (the FFN oracle of this package).
  R19 RMSNorm(v) = v / sqrt(mean(v^2) + eps) * g, eps given (1e-5 for
      LLaMA-2), the gain g per feature.
  R20 rotary embedding as RoFormer's block-diagonal rotation of consecutive
      feature pairs (2i, 2i+1) of each head by the angle
      pos * theta^(-2i / hd), theta given (10000), applied to q and k; the
      angle is exact (no rounding of pos * frequency).
  R21 causal scaled dot-product attention with scale 1/sqrt(hd); head h reads
      the key/value head h // (H / H_kv) (H_kv = H is plain multi-head
      attention).  The query at position p sees the keys at positions 0..p.
  R22 storage precision.  With act="bf16" the values a bf16 model stores are
      rounded to bf16 (round to nearest, ties to even) where it stores them:
      the two RMSNorm outputs (the inputs of the projections and of the FFN),
      the key and value cache entries and the attention output (the input of
      the output projection).  q stays unrounded through the attention; the
      residual stream (x, h, out) is never rounded.  With act="f32" nothing
      is rounded.
  R23 projection layout: Wqkv_T [D, (H + 2 H_kv) hd] holds the q, k and v
      projections column blocks in that order (y = x Wqkv_T); Wo_T [H hd, D].
      The FFN weights follow the FFN oracle (W_gate, W_up [D_FF, D], W_down
      [D, D_FF]).
"""
from __future__ import annotations

import math

import numpy as np

from . import pop_oracle as pop

__all__ = [
    "round_bf16", "rms_norm", "rope", "attend", "attention_block", "layer_prefill",
    "layer_decode", "ffn_prune_rate",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def round_bf16(a) -> np.ndarray:
    """Nearest bf16 value (8 significant bits), ties to even (reading R22).

    frexp writes a = m * 2^e with 0.5 <= |m| < 1; m * 256 then carries the 8
    significant bits above the binary point, and rint rounds the rest away,
    half to even.  Normal range only (no bf16 subnormal or overflow)."""
    m, e = np.frexp(_f64(a))
    return np.ldexp(np.rint(m * 256.0), e - 8)


def _store(a, act: str):
    return round_bf16(a) if act == "bf16" else _f64(a)


def rms_norm(v, g, eps: float) -> np.ndarray:
    """[RMS] equation (4) over the last axis (reading R19)."""
    v = _f64(v)
    ms = (v * v).mean(axis=-1, keepdims=True)
    return v / np.sqrt(ms + float(eps)) * _f64(g)


def rope(v, pos, theta: float) -> np.ndarray:
    """[ROPE] equations (14)-(15) (reading R20).

    v [..., n_heads, hd]; pos holds one position per leading index (shape
    v.shape[:-2]).  Pair i = (2i, 2i+1) of every head turns by
    pos * theta^(-2i/hd)."""
    v = _f64(v)
    hd = v.shape[-1]
    i = np.arange(hd // 2, dtype=np.float64)
    freq = float(theta) ** (-2.0 * i / hd)
    ang = _f64(pos)[..., None, None] * freq
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def attend(q, K, V, n_keys: int) -> np.ndarray:
    """[ATT] for one query position (reading R21).

    q [H, hd]; K, V [H_kv, L, hd] (the cache of one sequence); attends to the
    first n_keys positions.  Returns [H, hd]."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    H, hd = q.shape
    group = H // K.shape[0]
    out = np.empty((H, hd))
    for h in range(H):
        kk = K[h // group, :n_keys]
        vv = V[h // group, :n_keys]
        s = kk @ q[h] / math.sqrt(hd)
        p = np.exp(s - s.max())
        out[h] = (p / p.sum()) @ vv
    return out


def attention_block(x, lw, cfg, K, V, pos0: int, act: str) -> np.ndarray:
    """h = x + Attn(RMSNorm_a(x)) for T new tokens per sequence (readings
    R18-R23).

    x [B, T, D] are the tokens at positions pos0 .. pos0 + T - 1; K, V
    [B, H_kv, L, hd] are the caches, updated in place at those positions.
    cfg: dict with H, H_kv, hd, eps, theta."""
    x = _f64(x)
    B, T, D = x.shape
    H, Hkv, hd = cfg["H"], cfg["H_kv"], cfg["hd"]
    xn = _store(rms_norm(x, lw["attn_norm"], cfg["eps"]), act)
    qkv = xn @ _f64(lw["Wqkv_T"])
    q = qkv[..., : H * hd].reshape(B, T, H, hd)
    k = qkv[..., H * hd: (H + Hkv) * hd].reshape(B, T, Hkv, hd)
    v = qkv[..., (H + Hkv) * hd:].reshape(B, T, Hkv, hd)
    pos = np.broadcast_to(pos0 + np.arange(T), (B, T))
    q = rope(q, pos, cfg["theta"])
    k = rope(k, pos, cfg["theta"])
    K[:, :, pos0: pos0 + T] = _store(k, act).transpose(0, 2, 1, 3)
    V[:, :, pos0: pos0 + T] = _store(v, act).transpose(0, 2, 1, 3)
    o = np.empty((B, T, H, hd))
    for b in range(B):
        for t in range(T):
            o[b, t] = attend(q[b, t], K[b], V[b], pos0 + t + 1)
    o = _store(o.reshape(B, T, H * hd), act)
    return x + o @ _f64(lw["Wo_T"])


def layer_prefill(X, lw, cfg, r: float, gamma: float, act: str, L: int):
    """The prompt's pass through one layer: dense attention, then the dense
    FFN, whose input also yields the partition ([POP] "Loss / training
    strategy", Key design 1; readings R18-R23).

    X [B, N, D]; L >= N is the cache length.  Returns dict(x [B, N, D], h,
    xn2 [B*N, D] (the FFN's input), K, V [B, H_kv, L, hd], I, R, C, P)."""
    X = _f64(X)
    B, N, D = X.shape
    K = np.zeros((B, cfg["H_kv"], L, cfg["hd"]))
    V = np.zeros_like(K)
    h = attention_block(X, lw, cfg, K, V, 0, act)
    xn2 = _store(rms_norm(h, lw["ffn_norm"], cfg["eps"]), act).reshape(B * N, D)
    I = pop.importance(lw["W_up"], pop.column_norm(xn2))
    R, C, P = pop.partition(I, r, gamma)
    Y = pop.dense_ffn(xn2, lw["W_gate"], lw["W_up"], lw["W_down"])
    return {"x": h + Y.reshape(B, N, D), "h": h, "xn2": xn2, "K": K, "V": V, "I": I, "R": R, "C": C, "P": P}


def layer_decode(x, lw, cfg, K, V, pos: int, R, C, r: float, act: str, dense_ffn: bool = False):
    """One decode step of one layer: dense attention over the cache, then
    POP's pruned FFN step on R u C ([POP] Key design 2 and 3; readings
    R18-R23).  dense_ffn=True runs the FFN over every channel instead.

    x [B, D] is the token at position pos of every sequence; K, V are updated
    in place at pos.  Returns dict(x, h, xn2, y, S, scores)."""
    x = _f64(x)
    h = attention_block(x[:, None, :], lw, cfg, K, V, pos, act)[:, 0]
    xn2 = _store(rms_norm(h, lw["ffn_norm"], cfg["eps"]), act)
    if dense_ffn:
        y = pop.dense_ffn(xn2, lw["W_gate"], lw["W_up"], lw["W_down"])
        return {"x": h + y, "h": h, "xn2": xn2, "y": y, "S": None, "scores": None}
    st = pop.decode_step(xn2, lw["W_gate"], lw["W_up"], lw["W_down"], R, C, r)
    return {"x": h + st["y"], "h": h, "xn2": xn2, "y": st["y"], "S": st["S"], "scores": st["scores"]}


def ffn_prune_rate(r_global: float, d: int, d_ff: int, n_heads: int, n_kv_heads: int, hd: int) -> float:
    """[POP] Key design 3: the parameters a global rate removes from a layer,
    all taken from the FFN.  Attention holds D (H + 2 H_kv) hd + H hd D
    weights, the FFN 3 D D_FF; the FFN rate is r_global * (attention + FFN) /
    FFN."""
    attn = d * (n_heads + 2 * n_kv_heads) * hd + n_heads * hd * d
    ffn = 3 * d * d_ff
    return float(r_global) * (attn + ffn) / ffn
