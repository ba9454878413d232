"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/pop.h declares, and its host-only logic (counts, argument
validation, workspace sizing) behaves as documented.  No call here reaches the
device: every device entry point is called with arguments that fail
validation, which happens before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle
from online_structured_ffn_amd import pop

OK, INVALID, DTYPE, SHAPE, MISALIGNED, WS = 0, 1, 2, 3, 4, 5


def test_exports_every_declared_symbol():
    names = pop.declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(pop.lib, n), n


def test_debug_library_exports_and_checks():
    """libpop_debug.so (built beside libpop.so) exports the same functions."""
    import os
    if not os.path.exists(pop.DEBUG_LIB_PATH):
        pytest.skip("libpop_debug.so is not built")
    with pop.using_library(pop.DEBUG_LIB_PATH) as dbg:
        for n in pop.declared_functions():
            assert hasattr(dbg, n), n
        with pytest.raises(pop.PopError):
            pop.pop_check_lists([2, 1], [], 4)
    assert pop.lib is not dbg


def test_counts_match_oracle_everywhere():
    g = np.random.default_rng(0)
    for _ in range(3000):
        n = int(g.integers(1, 32769))
        r = float(g.uniform(0, 0.999))
        gam = float(g.uniform(0, 0.999))
        if g.integers(4) == 0:  # exact binary fractions hit the rounding halves
            r = float(g.integers(0, 64)) / 64
            gam = float(g.integers(0, 64)) / 64
            if r >= 1.0:
                continue
        got = pop.pop_partition_counts(n, r, gam)
        exp = oracle.partition_counts(n, r, gam)
        for k in ("c_low", "c_high", "n_P", "n_C", "n_R", "n_live", "k"):
            assert got[k] == exp[k], (n, r, gam, k, got, exp)


@pytest.mark.parametrize("args,status", [
    ((0, 0.3, 0.1), SHAPE), ((32769, 0.3, 0.1), SHAPE), ((10, -0.1, 0.1), INVALID),
    ((10, 1.0, 0.1), INVALID), ((10, 0.3, -0.01), INVALID), ((10, 0.3, 1.0), INVALID),
    ((10, float("nan"), 0.1), INVALID),
])
def test_counts_errors(args, status):
    c = pop.PopCounts()
    assert pop.lib.pop_partition_counts(*args, ctypes.byref(c)) == status
    assert pop.lib.pop_last_error().decode() != ""


def test_decode_topk_count_matches_oracle():
    """k for existing lists: the oracle's live count less |R|, clamped to [0, |C|]
    (the oracle's decode step selects exactly that many)."""
    g = np.random.default_rng(3)
    for _ in range(2000):
        n = int(g.integers(1, 32769))
        r = float(g.uniform(0, 0.999))
        n_R = int(g.integers(0, n + 1))
        n_C = int(g.integers(0, n - n_R + 1))
        live = oracle.partition_counts(n, r, 0.0)["n_live"]
        assert pop.pop_decode_topk_count(n, r, n_R, n_C) == min(max(live - n_R, 0), n_C), (n, r, n_R, n_C)
    # the partition's own sizes give the partition's k
    for n, r, gam in ((688, 0.3, 0.1), (11008, 0.299, 0.1), (18944, 0.5, 0.1), (14336, 0.3, 0.1)):
        c = oracle.partition_counts(n, r, gam)
        assert pop.pop_decode_topk_count(n, r, c["n_R"], c["n_C"]) == c["k"]


@pytest.mark.parametrize("args,status", [
    ((0, 0.3, 0, 0), SHAPE), ((32769, 0.3, 0, 0), SHAPE), ((10, 1.0, 2, 2), INVALID),
    ((10, -0.5, 2, 2), INVALID), ((10, 0.3, -1, 2), INVALID), ((10, 0.3, 6, 5), INVALID),
])
def test_decode_topk_count_errors(args, status):
    k = ctypes.c_int32(-7)
    assert pop.lib.pop_decode_topk_count(*args, ctypes.byref(k)) == status
    assert k.value == -7 and pop.lib.pop_last_error().decode() != ""
    assert pop.lib.pop_decode_topk_count(10, 0.3, 2, 2, None) == INVALID


def test_counts_null_out():
    assert pop.lib.pop_partition_counts(10, 0.3, 0.1, None) == INVALID
    assert pop.status_string(INVALID) == "POP_ERR_INVALID_ARGUMENT"
    assert pop.status_string(99) == "POP_ERR_UNKNOWN"


def test_workspace_sizes():
    assert pop.pop_prefill_workspace_bytes(512, 4096, 11008) >= 4 * (4096 + 11008)
    assert pop.pop_prefill_workspace_bytes(0, 256, 688) > 0
    assert pop.pop_prefill_workspace_bytes(-1, 256, 688) == 0
    a = pop.pop_decode_workspace_bytes(1, 4096, 11008)
    b = pop.pop_decode_workspace_bytes(16, 4096, 11008)
    # control and hand-over words, then z and the candidate scores
    Z = pop.DECODE_WS_Z_OFFSET
    assert Z % 256 == 0 and Z >= 1024 + 2 * 4096 * 8
    assert a >= Z + 4 * 11008 * 2 and b >= Z + 4 * 16 * 11008 + 4 * 11008
    assert pop.pop_decode_workspace_bytes(0, 4096, 11008) > 0


A = 1 << 20   # a fake, 16-byte-aligned "device address": never dereferenced (validation fails first)


def _prefill(X=A, n=16, d=256, W=A, d_ff=688, dt=0, r=0.3, g=0.1, R=A, C=A, P=A, I=None, ws=A, wsb=1 << 30):
    return pop.lib.pop_prefill_partition(X, n, d, W, d_ff, dt, r, g, R, C, P, I, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), DTYPE), (dict(d=0), SHAPE), (dict(d=250), SHAPE), (dict(d=12, dt=1), SHAPE),
    (dict(d_ff=0), SHAPE), (dict(d_ff=40000), SHAPE), (dict(n=-1), SHAPE), (dict(r=1.5), INVALID),
    (dict(X=None), INVALID), (dict(W=None), INVALID), (dict(R=None), INVALID), (dict(ws=None), INVALID),
    (dict(X=A + 4), MISALIGNED), (dict(I=A + 8), MISALIGNED), (dict(wsb=16), WS),
])
def test_prefill_validation(kw, status):
    assert _prefill(**kw) == status
    assert pop.lib.pop_last_error().decode()


def _decode(x=A, b=1, d=256, Wg=A, Wu=A, Wd=A, d_ff=688, dt=0, R=A, nR=413, C=A, nC=137, r=0.3, y=A, S=None,
            ws=A, wsb=1 << 30):
    return pop.lib.pop_decode_ffn(x, b, d, Wg, Wu, Wd, d_ff, dt, R, nR, C, nC, r, y, S, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=3), DTYPE), (dict(d=4, dt=1), SHAPE), (dict(b=-1), SHAPE), (dict(b=100000), SHAPE),
    (dict(nR=600), INVALID), (dict(nR=-1), INVALID), (dict(R=None), INVALID), (dict(x=None), INVALID),
    (dict(Wd=A + 2), MISALIGNED), (dict(y=A + 4), MISALIGNED), (dict(wsb=100), WS), (dict(r=1.0), INVALID),
])
def test_decode_validation(kw, status):
    assert _decode(**kw) == status


def _periodic(x=A, b=1, d=256, Wg=A, Wu=A, Wd=A, d_ff=688, dt=0, R=A, nR=413, C=A, nC=137, r=0.3, step=0, period=4,
              mem=A, pos=A, S=A, rows=A, y=A, ws=A, wsb=1 << 30):
    return pop.lib.pop_decode_ffn_periodic(x, b, d, Wg, Wu, Wd, d_ff, dt, R, nR, C, nC, r, step, period, mem, pos, S,
                                           rows, y, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(period=0), INVALID), (dict(step=-1), INVALID), (dict(r=1.0), INVALID), (dict(nR=600), INVALID),
    (dict(mem=None), INVALID), (dict(S=None), INVALID), (dict(C=None), INVALID), (dict(rows=None), INVALID),
    (dict(ws=A + 4), MISALIGNED),
    (dict(wsb=100), WS),
    (dict(dt=3), DTYPE), (dict(d=4, dt=1), SHAPE), (dict(b=-1), SHAPE), (dict(d_ff=0), SHAPE),
    (dict(x=None), INVALID), (dict(y=None), INVALID), (dict(Wg=None), INVALID),
    (dict(Wd=A + 2), MISALIGNED), (dict(y=A + 4), MISALIGNED),
])
def test_periodic_validation(kw, status):
    assert _periodic(**kw) == status
    assert pop.lib.pop_last_error().decode()


def test_periodic_workspace_sizes():
    f = pop.pop_decode_periodic_workspace_bytes
    for b in (1, 4, 16, 64):
        n = f(b, 4096, 11008)
        assert n >= pop.lib.pop_decode_down_workspace_bytes(b, 4096, 11008) + 4 * b * 11008
        assert n % 256 == 0
    assert f(-1, 4096, 11008) == 0 and f(1, 0, 11008) == 0


def test_dense_decode_validation():
    f = pop.lib.pop_dense_ffn_decode
    assert f(A, 1, 256, A, A, A, 688, 0, A, A, 10, None) == WS
    assert f(A, 1, 256, None, A, A, 688, 0, A, A, 1 << 30, None) == INVALID


def _prompt(X=A, n=512, d=256, Wg=A, Wu=A, Wd=A, d_ff=688, dt=1, Y=A, ws=A, wsb=1 << 30):
    return pop.lib.pop_dense_ffn_prefill(X, n, d, Wg, Wu, Wd, d_ff, dt, Y, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), DTYPE), (dict(d=12), SHAPE), (dict(d=0), SHAPE), (dict(d=32768), SHAPE), (dict(d_ff=0), SHAPE),
    (dict(d_ff=40000), SHAPE), (dict(n=-3), SHAPE), (dict(Wg=None), INVALID), (dict(Wd=None), INVALID),
    (dict(X=None), INVALID), (dict(Y=None), INVALID), (dict(ws=None), INVALID), (dict(Wu=A + 2), MISALIGNED),
    (dict(Y=A + 4), MISALIGNED), (dict(wsb=1000), WS),
])
def test_prompt_ffn_validation(kw, status):
    assert _prompt(**kw) == status
    assert pop.lib.pop_last_error().decode()


def test_prompt_ffn_workspace_sizes():
    f = pop.pop_dense_ffn_prefill_workspace_bytes
    # Z for one pass of up to 4096 tokens, rows padded to 128, pitch d_ff rounded up to 64
    assert f(512, 4096, 11008, "bf16") >= 512 * 11008 * 2
    assert f(512, 4096, 11008, "f32") >= 512 * 11008 * 4
    assert f(32768, 4096, 11008, "bf16") == f(4096, 4096, 11008, "bf16")
    assert f(1, 256, 688, "bf16") >= 128 * 704 * 2
    assert f(0, 256, 688, "bf16") == 0
    assert pop.lib.pop_dense_ffn_prefill_workspace_bytes(-1, 256, 688, 1) == 0


def _fused(X=A, n=512, d=256, Wg=A, Wu=A, Wd=A, d_ff=688, dt=1, r=0.3, g=0.1, Y=A, R=A, C=A, P=A, I=None, ws=A,
           wsb=1 << 30):
    return pop.lib.pop_prefill_ffn_partition(X, n, d, Wg, Wu, Wd, d_ff, dt, r, g, Y, R, C, P, I, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), DTYPE), (dict(d=12), SHAPE), (dict(d=0), SHAPE), (dict(d=32768), SHAPE), (dict(d_ff=0), SHAPE),
    (dict(d_ff=40000), SHAPE), (dict(n=-3), SHAPE), (dict(r=1.5), INVALID), (dict(g=-0.1), INVALID),
    (dict(Wg=None), INVALID), (dict(Wu=None), INVALID), (dict(Wd=None), INVALID), (dict(X=None), INVALID),
    (dict(Y=None), INVALID), (dict(ws=None), INVALID), (dict(R=None), INVALID), (dict(C=None), INVALID),
    (dict(P=None), INVALID), (dict(Wu=A + 2), MISALIGNED), (dict(Y=A + 4), MISALIGNED),
    (dict(I=A + 8), MISALIGNED), (dict(wsb=1000), WS),
])
def test_fused_prefill_validation(kw, status):
    assert _fused(**kw) == status
    assert pop.lib.pop_last_error().decode()


def test_fused_prefill_empty_prompt_needs_no_activations():
    # n_tokens = 0: X and Y may be NULL; validation passes up to the workspace size check
    assert _fused(X=None, Y=None, n=0, wsb=16) == WS


def test_fused_prefill_workspace_sizes():
    f = pop.pop_prefill_ffn_partition_workspace_bytes
    for n, d, d_ff, dt in ((512, 4096, 11008, "bf16"), (1, 256, 688, "f32"), (0, 256, 688, "bf16"),
                           (9000, 136, 300, "bf16")):
        # the prompt FFN's Z buffer, the column-norm workspace and I
        assert f(n, d, d_ff, dt) >= (pop.pop_dense_ffn_prefill_workspace_bytes(n, d, d_ff, dt)
                                     + 4 * d + 4 * d_ff)
    assert pop.lib.pop_prefill_ffn_partition_workspace_bytes(-1, 256, 688, 1) == 0
    assert pop.lib.pop_prefill_ffn_partition_workspace_bytes(5, 256, 688, 9) == 0


def test_moe_validation():
    lib = pop.lib
    # routing: expert count range, NULL outputs
    assert lib.pop_moe_route_top2(A, 4, 1, A, A, A, A, A, None) == SHAPE
    assert lib.pop_moe_route_top2(A, 4, 65, A, A, A, A, A, None) == SHAPE
    assert lib.pop_moe_route_top2(A, -1, 8, A, A, A, A, A, None) == SHAPE
    assert lib.pop_moe_route_top2(A, 4, 8, None, A, A, A, A, None) == INVALID
    assert lib.pop_moe_route_top2(A, 4, 8, A, A, None, A, A, None) == INVALID
    # prefill
    f = lib.pop_moe_prefill_partition
    ok = dict(X=A, n=64, d=256, L=A, E=8, W=A, d_ff=688, dt=1, r=0.3, g=0.1, R=A, C=A, P=A, I=None, ws=A,
              wsb=1 << 30)

    def pre(**kw):
        a = dict(ok, **kw)
        return f(a["X"], a["n"], a["d"], a["L"], a["E"], a["W"], a["d_ff"], a["dt"], a["r"], a["g"], a["R"],
                 a["C"], a["P"], a["I"], a["ws"], a["wsb"], None)
    assert pre(E=1) == SHAPE and pre(E=33) == SHAPE and pre(E=65, dt=0) == SHAPE
    assert pre(L=None) == INVALID and pre(R=None) == INVALID and pre(r=1.2) == INVALID
    assert pre(L=A + 4) == MISALIGNED and pre(wsb=64) == WS and pre(dt=4) == DTYPE
    # decode
    g = lib.pop_moe_decode_ffn
    okd = dict(x=A, T=32, d=256, L=A, E=8, Wg=A, Wu=A, Wd=A, d_ff=688, dt=1, R=A, nR=413, C=A, nC=137, r=0.3,
               y=A, S=None, ws=A, wsb=1 << 30)

    def dec(**kw):
        a = dict(okd, **kw)
        return g(a["x"], a["T"], a["d"], a["L"], a["E"], a["Wg"], a["Wu"], a["Wd"], a["d_ff"], a["dt"], a["R"],
                 a["nR"], a["C"], a["nC"], a["r"], a["y"], a["S"], a["ws"], a["wsb"], None)
    assert dec(E=1) == SHAPE and dec(T=300) == SHAPE and dec(d=12) == SHAPE
    assert dec(nR=600) == INVALID and dec(L=None) == INVALID and dec(C=None) == INVALID and dec(r=1.0) == INVALID
    assert dec(y=A + 8) == MISALIGNED and dec(wsb=1000) == WS


def test_moe_workspace_sizes():
    assert pop.lib.pop_moe_prefill_workspace_bytes(8192, 4096, 14336, 8) >= 8 * (4096 + 14336) * 4
    assert pop.lib.pop_moe_prefill_workspace_bytes(8192, 4096, 14336, 1) == 0
    b = pop.pop_moe_decode_workspace_bytes(32, 4096, 14336, 8)
    assert b >= 64 * 14336 * 4 + 8 * 14336 * 4   # z of every routed pair, scores of every expert
    assert pop.pop_moe_decode_workspace_bytes(32, 4096, 14336, 100) == 0
