"""The decoder-layer entry points on a machine without a GPU: argument
validation and workspace sizing.  Every device call here fails validation,
which happens before anything is enqueued."""
import ctypes

import pytest

from online_structured_ffn_amd import pop

OK, INVALID, DTYPE, SHAPE, MISALIGNED, WS = 0, 1, 2, 3, 4, 5
A = 1 << 20   # a fake, 16-byte-aligned "device address": never dereferenced


def _shape(**kw):
    f = dict(d=256, n_heads=4, n_kv_heads=2, head_dim=64, d_ff=688, cache_len=96, eps=1e-5, rope_theta=1e4)
    f.update(kw)
    return pop.LayerShape(*[f[n] for n, _ in pop.LayerShape._fields_])


def _weights(**kw):
    f = {n: A for n, _ in pop.LayerWeights._fields_}
    f.update(kw)
    return pop.LayerWeights(*[f[n] for n, _ in pop.LayerWeights._fields_])


def _decode(x=A, b=1, shape=None, w=None, dt=1, K=A, V=A, pos=A, R=A, nR=413, C=A, nC=137, r=0.3, dense=0,
            S=None, ws=A, wsb=1 << 30, null_shape=False, null_w=False):
    sp = None if null_shape else ctypes.byref(shape or _shape())
    wp = None if null_w else ctypes.byref(w or _weights())
    return pop.lib.pop_layer_decode(x, b, sp, wp, dt, K, V, pos, R, nR, C, nC, r, dense, S, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(null_shape=True), INVALID), (dict(dt=7), DTYPE), (dict(shape=_shape(d=96)), SHAPE),
    (dict(shape=_shape(d=0)), SHAPE), (dict(shape=_shape(head_dim=96)), SHAPE),
    (dict(shape=_shape(n_heads=6, n_kv_heads=4)), SHAPE), (dict(shape=_shape(n_kv_heads=0)), SHAPE),
    (dict(shape=_shape(d_ff=0)), SHAPE), (dict(shape=_shape(d_ff=40000)), SHAPE),
    (dict(shape=_shape(cache_len=0)), SHAPE), (dict(shape=_shape(eps=-1.0)), INVALID),
    (dict(shape=_shape(rope_theta=0.0)), INVALID), (dict(null_w=True), INVALID),
    (dict(w=_weights(Wo_T=None)), INVALID), (dict(w=_weights(ffn_norm=A + 4)), MISALIGNED),
    (dict(b=0), SHAPE), (dict(b=65), SHAPE), (dict(x=None), INVALID), (dict(pos=None), INVALID),
    (dict(K=None), INVALID), (dict(x=A + 8), MISALIGNED), (dict(V=A + 2), MISALIGNED), (dict(dense=2), INVALID),
    (dict(wsb=1024), WS), (dict(r=1.0), INVALID), (dict(nR=600), INVALID), (dict(R=None), INVALID),
    (dict(nC=-1), INVALID),
])
def test_layer_decode_validation(kw, status):
    assert _decode(**kw) == status
    assert pop.lib.pop_last_error().decode() != ""


def _prefill(x=A, b=1, n=16, shape=None, w=None, dt=1, K=A, V=A, r=0.3, g=0.1, R=A, C=A, P=A, I=None, ws=A,
             wsb=1 << 30):
    return pop.lib.pop_layer_prefill(x, b, n, ctypes.byref(shape or _shape()), ctypes.byref(w or _weights()), dt,
                                     K, V, r, g, R, C, P, I, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), SHAPE), (dict(n=97), SHAPE), (dict(b=0), SHAPE), (dict(dt=3), DTYPE),
    (dict(shape=_shape(head_dim=32)), SHAPE), (dict(r=1.5), INVALID), (dict(g=-0.1), INVALID),
    (dict(R=None), INVALID), (dict(P=None), INVALID), (dict(x=None), INVALID), (dict(ws=None), INVALID),
    (dict(I=A + 4), MISALIGNED), (dict(K=A + 4), MISALIGNED), (dict(wsb=4096), WS),
    (dict(w=_weights(W_up=None)), INVALID),
])
def test_layer_prefill_validation(kw, status):
    assert _prefill(**kw) == status
    assert pop.lib.pop_last_error().decode() != ""


def test_layer_workspace_sizes():
    s = _shape()
    dec = lambda b, sh=s, dt=1: pop.lib.pop_layer_decode_workspace_bytes(b, ctypes.byref(sh), dt)
    pre = lambda b, n, sh=s, dt=1: pop.lib.pop_layer_prefill_workspace_bytes(b, n, ctypes.byref(sh), dt)
    # the FFN step's own workspace is inside, plus the layer's buffers
    assert dec(1) > pop.pop_decode_workspace_bytes(1, 256, 688)
    assert dec(4) > pop.pop_decode_workspace_bytes(4, 256, 688) and dec(1, _shape(cache_len=1000)) > dec(1)
    assert dec(1, dt=0) > dec(1)                 # fp32 activations take more room
    assert dec(0) == 0 and dec(65) == 0 and dec(1, _shape(head_dim=80)) == 0
    M, d = 3 * 40, 256
    big = pre(3, 40)
    assert big >= M * d * 2 + M * (4 + 2 * 2) * 64 * 4 + pop.pop_prefill_ffn_partition_workspace_bytes(M, d, 688, "bf16")
    assert pre(3, 97) == 0 and pre(0, 4) == 0 and pre(1, 0) == 0
    # the LLaMA-2-7B-shaped layer at batch 1 and a 512-token prompt stays far below HBM
    ll = _shape(d=4096, n_heads=32, n_kv_heads=32, head_dim=128, d_ff=11008, cache_len=1024)
    assert 0 < dec(1, ll) < (64 << 20)
    assert 0 < pre(1, 512, ll) < (1 << 30)
