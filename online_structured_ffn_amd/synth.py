"""Seeded synthetic inputs for the pruned gated-MLP path.

This is the only module that both the CPU oracle's tests and the HIP path's
tests and benchmark use.  It draws random numbers and rounds them to the
element type of the workload; it holds none of the method's arithmetic (no
norms, no importance, no selection, no FFN).

Seeds: every tensor comes from its own PCG64 stream keyed by
``SeedSequence([0x504F50, workload_id, layer, tensor_id, *extra])`` so that any
single layer, step or expert can be regenerated on its own.

bf16 handling: there is no ``ml_dtypes`` here, so float32 -> bf16 uses
round-to-nearest-even on the bit pattern.  Arrays returned to callers are
float32 arrays whose values are exactly representable in bf16 when the
workload is bf16, plus the raw uint16 bits for upload to the device.
"""
from __future__ import annotations

import numpy as np

from .configs import WORKLOADS, Workload

SEED_ROOT = 0x504F50
T_GATE, T_UP, T_DOWN, T_PROMPT, T_DECODE, T_OUTLIER, T_ROUTER, T_QKV, T_O = range(9)


def workload_id(w: Workload) -> int:
    return [x.name for x in WORKLOADS].index(w.name) + 1 if w in WORKLOADS else 99


def rng(wid: int, layer: int, tensor: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([SEED_ROOT, wid, layer, tensor, *extra])))


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Float32 values as stored in the workload's element type."""
    a = np.asarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a))
    raise ValueError(dtype)


# ---------------------------------------------------------------- weights
def layer_weights(w: Workload, layer: int, wid: int | None = None) -> dict:
    """W_gate, W_up: [D_FF, D]; W_down: [D, D_FF] (nn.Linear layout) and its
    transpose W_downT: [D_FF, D] (the layout the device path reads).
    All entries ~ N(0, weight_std^2), rounded to the workload dtype."""
    wid = workload_id(w) if wid is None else wid
    out = {}
    for name, tid, shape in (("W_gate", T_GATE, (w.d_ff, w.d)),
                             ("W_up", T_UP, (w.d_ff, w.d)),
                             ("W_down", T_DOWN, (w.d, w.d_ff))):
        g = rng(wid, layer, tid)
        a = g.standard_normal(shape, dtype=np.float32) * np.float32(w.weight_std)
        out[name] = to_dtype(a, w.dtype)
    out["W_downT"] = np.ascontiguousarray(out["W_down"].T)
    return out


def attention_weights(w: Workload, layer: int, wid: int | None = None) -> dict:
    """The attention half of a decoder layer: Wqkv_T [D, (H + 2 H_kv) hd] and
    Wo_T [H hd, D] ~ N(0, weight_std^2) rounded to the workload dtype, RMSNorm
    gains of 1 (fp32)."""
    wid = workload_id(w) if wid is None else wid
    a = w.extra["attention"]
    H, Hkv, hd = a["n_heads"], a["n_kv_heads"], a["head_dim"]
    out = {}
    for name, tid, shape in (("Wqkv_T", T_QKV, (w.d, (H + 2 * Hkv) * hd)), ("Wo_T", T_O, (H * hd, w.d))):
        g = rng(wid, layer, tid)
        out[name] = to_dtype(g.standard_normal(shape, dtype=np.float32) * np.float32(w.weight_std), w.dtype)
    out["attn_norm"] = np.ones(w.d, dtype=np.float32)
    out["ffn_norm"] = np.ones(w.d, dtype=np.float32)
    return out


# ---------------------------------------------------------------- activations
def outlier_channels(w: Workload, layer: int, wid: int | None = None) -> np.ndarray:
    wid = workload_id(w) if wid is None else wid
    if w.outlier_channels == 0:
        return np.zeros(0, dtype=np.int64)
    g = rng(wid, layer, T_OUTLIER)
    return np.sort(g.choice(w.d, size=w.outlier_channels, replace=False))


def drifting_outliers(w: Workload, layer: int, steps: int, wid: int | None = None) -> list:
    """Outlier sets O_0 (prompt) .. O_steps: at each decode step one member of
    the previous set is swapped for a uniformly drawn non-member."""
    wid = workload_id(w) if wid is None else wid
    cur = outlier_channels(w, layer, wid)
    sets = [cur.copy()]
    g = rng(wid, layer, T_OUTLIER, 1)
    for _ in range(steps):
        out_pos = int(g.integers(len(cur)))
        non = np.setdiff1d(np.arange(w.d), cur, assume_unique=True)
        new = int(non[g.integers(len(non))])
        cur = np.sort(np.concatenate([np.delete(cur, out_pos), [new]]))
        sets.append(cur.copy())
    return sets


def _apply_outliers(w: Workload, a: np.ndarray, chans: np.ndarray, g: np.random.Generator) -> np.ndarray:
    if len(chans) == 0 or w.outlier_kind == "none":
        return a
    if w.outlier_kind in ("scale", "drift_scale"):
        a[:, chans] *= np.float32(w.outlier_factor)
    elif w.outlier_kind == "student_t":
        a[:, chans] = g.standard_t(w.student_nu, size=(a.shape[0], len(chans))).astype(np.float32)
    else:
        raise ValueError(w.outlier_kind)
    return a


def prompt(w: Workload, layer: int, wid: int | None = None, n_tokens: int | None = None) -> np.ndarray:
    """Prompt FFN-input activations X as [B*L, D] (token-major rows)."""
    wid = workload_id(w) if wid is None else wid
    n = w.prompt_batch * w.prompt_len if n_tokens is None else n_tokens
    g = rng(wid, layer, T_PROMPT)
    a = g.standard_normal((n, w.d), dtype=np.float32)
    a = _apply_outliers(w, a, outlier_channels(w, layer, wid), g)
    return to_dtype(a, w.dtype)


def decode_input(w: Workload, layer: int, step: int, wid: int | None = None,
                 batch: int | None = None, drift_sets: list | None = None) -> np.ndarray:
    """Decode-step FFN input x_t as [B, D]."""
    wid = workload_id(w) if wid is None else wid
    b = w.decode_batch if batch is None else batch
    g = rng(wid, layer, T_DECODE, step)
    a = g.standard_normal((b, w.d), dtype=np.float32)
    if w.outliers_in_decode:
        if w.outlier_kind == "drift_scale":
            sets = drift_sets if drift_sets is not None else drifting_outliers(w, layer, step + 1, wid)
            chans = sets[step + 1]
        else:
            chans = outlier_channels(w, layer, wid)
        a = _apply_outliers(w, a, chans, g)
    return to_dtype(a, w.dtype)


def router_logits(w: Workload, n_tokens: int, stream: int, wid: int | None = None) -> np.ndarray:
    """Router logits [n_tokens, experts] ~ N(0,1); stream 0 = prompt, t+1 = step t."""
    wid = workload_id(w) if wid is None else wid
    g = rng(wid, 0, T_ROUTER, stream)
    return g.standard_normal((n_tokens, w.experts)).astype(np.float32)


def random_case(seed: int, n_tokens: int, d: int, d_ff: int, batch: int, dtype: str = "f32",
                weight_std: float = 0.02) -> dict:
    """A small free-form case (ragged shapes for parity tests)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 1000, seed])))
    f = np.float32
    c = {
        "X": to_dtype(g.standard_normal((n_tokens, d), dtype=f), dtype),
        "W_gate": to_dtype(g.standard_normal((d_ff, d), dtype=f) * f(weight_std), dtype),
        "W_up": to_dtype(g.standard_normal((d_ff, d), dtype=f) * f(weight_std), dtype),
        "W_down": to_dtype(g.standard_normal((d, d_ff), dtype=f) * f(weight_std), dtype),
        "x": to_dtype(g.standard_normal((batch, d), dtype=f), dtype),
    }
    c["W_downT"] = np.ascontiguousarray(c["W_down"].T)
    return c


# ---------------------------------------------------------------- device-side
def torch_layer_weights(w: Workload, layer: int, device, wid: int | None = None):
    """Throughput-only weights drawn on the device (same distribution as
    :func:`layer_weights`, different random stream).  Returns bf16/fp32
    tensors W_gate, W_up, W_downT, each [D_FF, D]."""
    import torch
    wid = workload_id(w) if wid is None else wid
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {}
    for name, tid in (("W_gate", T_GATE), ("W_up", T_UP), ("W_downT", T_DOWN)):
        gen = torch.Generator(device=device)
        gen.manual_seed((SEED_ROOT << 24) ^ (wid << 16) ^ (layer << 4) ^ tid)
        t = torch.randn((w.d_ff, w.d), generator=gen, device=device, dtype=torch.float32)
        out[name] = (t * w.weight_std).to(dt).contiguous()
    return out


def torch_attention_weights(w: Workload, layer: int, device, wid: int | None = None):
    """Device-drawn counterpart of :func:`attention_weights` (same
    distribution, different random stream)."""
    import torch
    wid = workload_id(w) if wid is None else wid
    a = w.extra["attention"]
    H, Hkv, hd = a["n_heads"], a["n_kv_heads"], a["head_dim"]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {}
    for name, tid, shape in (("Wqkv_T", T_QKV, (w.d, (H + 2 * Hkv) * hd)), ("Wo_T", T_O, (H * hd, w.d))):
        gen = torch.Generator(device=device)
        gen.manual_seed((SEED_ROOT << 24) ^ (wid << 16) ^ (layer << 4) ^ tid)
        out[name] = (torch.randn(shape, generator=gen, device=device) * w.weight_std).to(dt).contiguous()
    out["attn_norm"] = torch.ones(w.d, dtype=torch.float32, device=device)
    out["ffn_norm"] = torch.ones(w.d, dtype=torch.float32, device=device)
    return out


def torch_activations(w: Workload, shape, layer: int, tag: int, device, chans=None):
    """Device-drawn N(0,1) activations (bf16/fp32) with the workload's
    outlier treatment on ``chans``."""
    import torch
    wid = workload_id(w)
    gen = torch.Generator(device=device)
    gen.manual_seed((SEED_ROOT << 24) ^ (wid << 16) ^ (layer << 4) ^ (T_PROMPT + 16 * tag))
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if chans is not None and len(chans) and w.outlier_kind != "none":
        idx = torch.as_tensor(np.asarray(chans), device=device, dtype=torch.long)
        if w.outlier_kind in ("scale", "drift_scale"):
            t[:, idx] *= w.outlier_factor
        elif w.outlier_kind == "student_t":
            # Student-t(nu) = N / sqrt(chi2_nu / nu); chi2_nu = sum of nu squared normals
            nu = int(round(w.student_nu))
            z = torch.randn((t.shape[0], len(idx), nu + 1), generator=gen, device=device)
            t[:, idx] = z[..., 0] / torch.sqrt((z[..., 1:] ** 2).sum(-1) / nu)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return t.to(dt).contiguous()


def torch_decode_inputs(w: Workload, layer: int, steps: int, device):
    """Device-drawn decode inputs of one layer for ``steps`` steps as
    [steps, B, D]: N(0,1) with the layer's outlier channels (the prompt's set,
    or with drifting outliers the set O_{t+1} at step t, one member swapped per
    step as :func:`drifting_outliers` draws them)."""
    import torch
    B, d = w.decode_batch, w.d
    if w.outlier_kind == "drift_scale" and w.outliers_in_decode:
        sets = drifting_outliers(w, layer, steps)
        mult = np.ones((steps, d), dtype=np.float32)
        for t in range(steps):
            mult[t, sets[t + 1]] = w.outlier_factor
        base = torch_activations(w, (steps * B, d), layer, 1, device).float().view(steps, B, d)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        return (base * torch.from_numpy(mult).to(device)[:, None, :]).to(dt).contiguous()
    chans = outlier_channels(w, layer) if w.outliers_in_decode else None
    return torch_activations(w, (steps * B, d), layer, 1, device, chans).view(steps, B, d)


def torch_moe_inputs(w: Workload, layers: int, steps: int, device):
    """Device-drawn inputs of a mixture-of-experts stack: N(0,1) router logits
    of every layer's prompt [layers, n_tokens, E] and of every decode step
    [steps, layers, B, E], and the decode inputs [steps, layers, B, D]."""
    import torch
    n_tok, E, B, d = w.prompt_batch * w.prompt_len, w.experts, w.decode_batch, w.d
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED_ROOT ^ 0x5EED)
    logits_pre = torch.randn((layers, n_tok, E), generator=gen, device=device, dtype=torch.float32)
    logits_dec = torch.randn((steps, layers, B, E), generator=gen, device=device, dtype=torch.float32)
    x = torch_activations(w, (steps * layers * B, d), 0, 1, device).view(steps, layers, B, d)
    return logits_pre, logits_dec, x
