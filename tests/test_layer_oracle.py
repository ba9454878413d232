"""The decoder-layer oracle against its pins, and planted mistakes in copies
of it that at least one pin must catch."""
import os
import types

import pytest

import oracle.layer_oracle as real
from tests.layer_pins import ALL_PINS

SRC = open(real.__file__).read()

MUTANTS = [
    ("bf16 rounding truncates", "np.rint(m * 256.0)", "np.trunc(m * 256.0)"),
    ("RMSNorm over the sum of squares", "ms = (v * v).mean(axis=-1, keepdims=True)", "ms = (v * v).sum(axis=-1, keepdims=True)"),
    ("RMSNorm eps outside the root", "v / np.sqrt(ms + float(eps))", "v / (np.sqrt(ms) + float(eps))"),
    ("RMSNorm without its gain", "return v / np.sqrt(ms + float(eps)) * _f64(g)", "return v / np.sqrt(ms + float(eps))"),
    ("rotation sign flipped", "out[..., 0::2] = a * c - b * s", "out[..., 0::2] = a * c + b * s"),
    ("rotary frequency exponent halved", "freq = float(theta) ** (-2.0 * i / hd)", "freq = float(theta) ** (-1.0 * i / hd)"),
    ("rotary pairs split by halves", "a, b = v[..., 0::2], v[..., 1::2]", "a, b = v[..., : hd // 2], v[..., hd // 2:]"),
    ("positions off by one", "pos = np.broadcast_to(pos0 + np.arange(T), (B, T))",
     "pos = np.broadcast_to(pos0 + 1 + np.arange(T), (B, T))"),
    ("attention scale without the root", "s = kk @ q[h] / math.sqrt(hd)", "s = kk @ q[h] / hd"),
    ("causal window one key short", "attend(q[b, t], K[b], V[b], pos0 + t + 1)", "attend(q[b, t], K[b], V[b], max(pos0 + t, 1))"),
    ("grouped heads interleaved", "kk = K[h // group, :n_keys]", "kk = K[h % K.shape[0], :n_keys]"),
    ("k and v blocks swapped", "k = qkv[..., H * hd: (H + Hkv) * hd]", "k = qkv[..., (H + Hkv) * hd:]"),
    ("k cache not rounded", "K[:, :, pos0: pos0 + T] = _store(k, act)", "K[:, :, pos0: pos0 + T] = _f64(k)"),
    ("attention output not rounded", "o = _store(o.reshape(B, T, H * hd), act)", "o = o.reshape(B, T, H * hd)"),
    ("attention residual dropped", "return x + o @ _f64(lw[\"Wo_T\"])", "return o @ _f64(lw[\"Wo_T\"])"),
    ("decode FFN norm on x instead of h", "xn2 = _store(rms_norm(h, lw[\"ffn_norm\"], cfg[\"eps\"]), act)\n    if dense_ffn:",
     "xn2 = _store(rms_norm(x, lw[\"ffn_norm\"], cfg[\"eps\"]), act)\n    if dense_ffn:"),
    ("FFN norm uses the attention gain", "xn2 = _store(rms_norm(h, lw[\"ffn_norm\"], cfg[\"eps\"]), act).reshape",
     "xn2 = _store(rms_norm(h, lw[\"attn_norm\"], cfg[\"eps\"]), act).reshape"),
    ("FFN residual dropped", "return {\"x\": h + st[\"y\"]", "return {\"x\": st[\"y\"]"),
    ("budget counts four square attention matrices",
     "attn = d * (n_heads + 2 * n_kv_heads) * hd + n_heads * hd * d", "attn = 4 * d * d"),
]


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(real)


def _load_mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle.layer_oracle_mutant")
    mod.__file__ = os.path.join(os.path.dirname(real.__file__), "layer_oracle_mutant.py")
    mod.__package__ = "oracle"
    exec(compile(SRC.replace(old, new), mod.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure of a pin counts as caught
            return
    pytest.fail(f"no pin caught the planted mistake: {name}")
