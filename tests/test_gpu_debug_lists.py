"""The checking build libpop_debug.so: with valid index lists it gives the
same results as libpop.so, bit for bit (the same kernels run); with an
invalid list it returns POP_ERR_INVALID_ARGUMENT before anything is
enqueued, so the output buffer keeps its contents.  The lists planted here
are wrong in order or overlap but hold channel ids inside [0, d_ff), and the
device code clamps ids in any case, so nothing here can address outside a
weight matrix."""
import os

import numpy as np
import pytest
import torch

import oracle
from online_structured_ffn_amd import pop, synth
from tests.parity import dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not os.path.exists(pop.DEBUG_LIB_PATH),
                                                  reason="libpop_debug.so is not built")]

INVALID = 1
D, D_FF, BATCH, R_RATE = 128, 300, 2, 0.3


def _case(dtype):
    c = synth.random_case(11, 24, D, D_FF, BATCH, dtype)
    R, C, _ = oracle.partition(oracle.importance(c["W_up"], oracle.column_norm(c["X"])), R_RATE, 0.1)
    t = {k: dev(c[k], dtype) for k in ("x", "W_gate", "W_up", "W_downT")}
    return t, torch.from_numpy(R.astype(np.int32)).cuda(), torch.from_numpy(C.astype(np.int32)).cuda()


def _bad_lists(R, C):
    """(name, R, C) with one planted mistake each."""
    Rh, Ch = R.cpu().numpy(), C.cpu().numpy()
    out = []
    swapped = Rh.copy()
    swapped[[0, 1]] = swapped[[1, 0]]
    out.append(("R out of order", swapped, Ch))
    out.append(("channel in R and C", Rh, np.sort(np.concatenate([Ch[1:], Rh[:1]]))))
    dup = Ch.copy()
    dup[1] = dup[0]
    out.append(("repeat in C", Rh, dup))
    return [(n, torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda(),
             torch.from_numpy(np.ascontiguousarray(b, dtype=np.int32)).cuda()) for n, a, b in out]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("entry", ["pop_decode_ffn", "pop_decode_ffn_noalloc"])
def test_decode_matches_and_rejects(dtype, entry):
    t, R, C = _case(dtype)
    args = (t["x"], t["W_gate"], t["W_up"], t["W_downT"])
    y0, S0 = getattr(pop, entry)(*args, R, C, R_RATE, selected=True)
    with pop.using_library(pop.DEBUG_LIB_PATH):
        y1, S1 = getattr(pop, entry)(*args, R, C, R_RATE, selected=True)
        for name, Rb, Cb in _bad_lists(R, C):
            y = torch.full((BATCH, D), 7.0, device="cuda")
            with pytest.raises(pop.PopError) as e:
                getattr(pop, entry)(*args, Rb, Cb, R_RATE, y=y)
            assert e.value.status == INVALID, name
            torch.cuda.synchronize()
            assert bool((y == 7.0).all()), f"{entry}: {name}: output written"
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(S0, S1)


def test_gateup_and_periodic_match_and_reject():
    t, R, C = _case("bf16")
    z0, s0 = pop.pop_decode_gateup(t["x"], t["W_gate"], t["W_up"], R, C)
    st0 = pop.PeriodicState(D_FF, R_RATE, R.numel(), C.numel(), "cuda")
    p0 = [pop.pop_decode_ffn_periodic(t["x"], t["W_gate"], t["W_up"], t["W_downT"], R, C, R_RATE, s, 2, st0).clone()
          for s in range(3)]
    with pop.using_library(pop.DEBUG_LIB_PATH):
        z1, s1 = pop.pop_decode_gateup(t["x"], t["W_gate"], t["W_up"], R, C)
        st1 = pop.PeriodicState(D_FF, R_RATE, R.numel(), C.numel(), "cuda")
        p1 = [pop.pop_decode_ffn_periodic(t["x"], t["W_gate"], t["W_up"], t["W_downT"], R, C, R_RATE, s, 2,
                                          st1).clone() for s in range(3)]
        for name, Rb, Cb in _bad_lists(R, C):
            with pytest.raises(pop.PopError) as e:
                pop.pop_decode_gateup(t["x"], t["W_gate"], t["W_up"], Rb, Cb)
            assert e.value.status == INVALID, name
            st = pop.PeriodicState(D_FF, R_RATE, Rb.numel(), Cb.numel(), "cuda")
            for step in (0, 1):  # a refresh step and a kept step
                with pytest.raises(pop.PopError) as e:
                    pop.pop_decode_ffn_periodic(t["x"], t["W_gate"], t["W_up"], t["W_downT"], Rb, Cb, R_RATE, step,
                                                2, st)
                assert e.value.status == INVALID, (name, step)
    torch.cuda.synchronize()
    assert torch.equal(z0, z1) and torch.equal(s0, s1)
    for a, b in zip(p0, p1):
        assert torch.equal(a, b)


def test_layer_decode_matches_and_rejects():
    g = np.random.default_rng(5)
    Dl, H, Hkv, hd, dff, L = 256, 4, 2, 64, 688, 16
    lw = {"attn_norm": g.uniform(0.5, 1.5, Dl), "ffn_norm": g.uniform(0.5, 1.5, Dl),
          "Wqkv_T": g.normal(0, Dl ** -0.5, (Dl, (H + 2 * Hkv) * hd)), "Wo_T": g.normal(0, (H * hd) ** -0.5, (H * hd, Dl)),
          "W_gate": g.normal(0, Dl ** -0.5, (dff, Dl)), "W_up": g.normal(0, Dl ** -0.5, (dff, Dl)),
          "W_downT": g.normal(0, dff ** -0.5, (dff, Dl))}
    layer = pop.Layer(Dl, H, Hkv, hd, dff, L, {k: torch.from_numpy(v.astype(np.float32)).cuda() for k, v in lw.items()})
    R, C, _ = oracle.partition(g.random(dff), R_RATE, 0.1)
    R, C = (torch.from_numpy(a.astype(np.int32)).cuda() for a in (R, C))
    x0 = torch.from_numpy(g.standard_normal((1, Dl)).astype(np.float32)).cuda()
    pos = torch.tensor([3], dtype=torch.int32, device="cuda")
    K, V = layer.cache(1)
    K.normal_()
    V.normal_()
    xa = x0.clone()
    pop.pop_layer_decode(xa, layer, K, V, pos, R, C, R_RATE)
    with pop.using_library(pop.DEBUG_LIB_PATH):
        xb = x0.clone()
        pop.pop_layer_decode(xb, layer, K, V, pos, R, C, R_RATE)
        for name, Rb, Cb in _bad_lists(R, C):
            xc = x0.clone()
            with pytest.raises(pop.PopError) as e:
                pop.pop_layer_decode(xc, layer, K, V, pos, Rb, Cb, R_RATE)
            assert e.value.status == INVALID, name
            torch.cuda.synchronize()
            assert torch.equal(xc, x0), f"layer: {name}: x written"
    torch.cuda.synchronize()
    assert torch.equal(xa, xb)
