"""The decoder layer (pop_layer_prefill, pop_layer_decode) against the
float64 layer oracle, element by element.

Inputs are seeded and synthetic: weights N(0, std^2) with std = 1/sqrt(fan-in)
on the small shapes and 0.02 on the LLaMA-2-7B shape, RMSNorm gains U(0.5,
1.5), activations N(0, 1), caches N(0, 1) where a test fills them directly.
bf16 values are rounded on the device and enter the oracle as the exact
float64 value of their bits.

Selections are integer results decided by floating point.  The FFN's input
(RMSNorm(h), left in the workspace) is first compared with the oracle's; the
FFN's candidate selection is then compared with the oracle's selection rule
applied to that device input (the same decision on the same values; a channel
may differ only as a near tie of the fp32 arithmetic), and the layer output
with the oracle's layer evaluated on the device's selection.  How many
channels the fp64 chain would have chosen differently is reported, not
asserted: in bf16 the FFN input carries rounding flips of the attention half.
Tolerances: max|d| <= tol * max|ref|, tol = 1e-5 (fp32), 2e-2 (bf16).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, check_partition, host

pytestmark = pytest.mark.gpu

lo = oracle.layer
TIE_REL = 1e-4   # fp32 scores against fp64 on the same input


def _pop():
    from online_structured_ffn_amd import pop
    return pop


def _seed(name):
    return zlib.crc32(name.encode())


class Case:
    def __init__(self, name, dtype, D, H, Hkv, hd, dff, L, std=None, eps=1e-5, theta=10000.0):
        self.name, self.dtype, self.D, self.H, self.Hkv, self.hd, self.dff, self.L = name, dtype, D, H, Hkv, hd, dff, L
        self.std, self.eps, self.theta = std, eps, theta
        self.cfg = {"H": H, "H_kv": Hkv, "hd": hd, "eps": eps, "theta": theta}

    def tdtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


def _param(g, shape, std, tdt, mean=0.0, uniform=None):
    if uniform is not None:
        a = torch.from_numpy(g.uniform(*uniform, size=shape).astype(np.float32))
    else:
        a = torch.from_numpy((mean + std * g.standard_normal(shape)).astype(np.float32))
    d = a.to(tdt).cuda().contiguous()
    return d, d.float().cpu().numpy().astype(np.float64)


def _layer(case, g):
    pop = _pop()
    t = case.tdtype()
    D, H, Hkv, hd, dff = case.D, case.H, case.Hkv, case.hd, case.dff
    sd = lambda fan: case.std if case.std is not None else 1.0 / np.sqrt(fan)
    dev, ref = {}, {}
    dev["attn_norm"], ref["attn_norm"] = _param(g, (D,), 0, torch.float32, uniform=(0.5, 1.5))
    dev["ffn_norm"], ref["ffn_norm"] = _param(g, (D,), 0, torch.float32, uniform=(0.5, 1.5))
    dev["Wqkv_T"], ref["Wqkv_T"] = _param(g, (D, (H + 2 * Hkv) * hd), sd(D), t)
    dev["Wo_T"], ref["Wo_T"] = _param(g, (H * hd, D), sd(H * hd), t)
    dev["W_gate"], ref["W_gate"] = _param(g, (dff, D), sd(D), t)
    dev["W_up"], ref["W_up"] = _param(g, (dff, D), sd(D), t)
    dev["W_downT"], wdT = _param(g, (dff, D), sd(dff), t)
    ref["W_down"] = wdT.T.copy()
    layer = pop.Layer(D, H, Hkv, hd, dff, case.L, dev, eps=case.eps, rope_theta=case.theta)
    return layer, ref


def _close(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    m = max(np.abs(ref).max(), 1e-30)
    err = np.abs(got - ref).max() / m
    assert err <= TOL[dtype], f"{what}: max|d|/max|ref| = {err:.3e} > {TOL[dtype]}"
    return err


def _check_xn2(got, ref, dtype):
    """The FFN input against the oracle's.  bf16: most elements equal; the
    others differ where the fp32 value sat near a rounding boundary (the
    attention half's own rounding flips move h by about 1e-4 relative, so a
    few percent of the elements cross one)."""
    got = np.asarray(got, dtype=np.float64)
    if dtype == "bf16":
        frac = (got != ref).mean()
        assert frac <= 0.10, f"{frac:.3%} of the FFN inputs differ"
    return _close(got, ref, dtype, "FFN input")


def _check_selection(S_dev, xn2_dev, ref, R, C, r, k, fp64_S=None):
    """S_dev against the oracle's rule on the device's FFN input; returns the
    sorted selection and how many channels differ from ``fp64_S``."""
    S_dev = np.sort(np.asarray(host(S_dev), dtype=np.int64))
    assert len(S_dev) == k and len(np.unique(S_dev)) == k and np.isin(S_dev, C).all()
    st = oracle.decode_step(xn2_dev, ref["W_gate"], ref["W_up"], ref["W_down"], R, C, r)
    diff = np.setxor1d(S_dev, st["S"])
    if len(diff):
        srt = np.sort(st["scores"])[::-1]
        cuts = [srt[j] for j in (k - 1, k) if 0 <= j < len(C)]
        where = {int(c): j for j, c in enumerate(C)}
        for ch in diff:
            v = st["scores"][where[int(ch)]]
            assert any(abs(v - t) <= TIE_REL * max(t, 1e-30) for t in cuts), f"candidate {ch} is not a near tie"
    return S_dev, (0 if fp64_S is None else len(np.setxor1d(S_dev, fp64_S)))


# ---------------------------------------------------------------- prefill
PREFILL = [
    # name, dtype, D, H, Hkv, hd, d_ff, L, batch, n_tokens
    ("f32_gqa_b1_n37", "f32", 256, 4, 2, 64, 688, 96, 1, 37),
    ("bf16_gqa_b3_n37", "bf16", 256, 4, 2, 64, 688, 96, 3, 37),
    ("bf16_mha_hd128_b2_n16", "bf16", 512, 4, 4, 128, 1376, 40, 2, 16),
    ("f32_mha_hd128_b2_n50", "f32", 512, 4, 4, 128, 1376, 64, 2, 50),
    ("bf16_one_token", "bf16", 256, 4, 1, 64, 688, 8, 2, 1),
    # several 64-query and 64-key tiles of the matrix-core prompt attention, ragged ends
    ("bf16_hd128_n150", "bf16", 512, 4, 4, 128, 1376, 160, 1, 150),
    ("bf16_gqa_hd64_b2_n100", "bf16", 256, 4, 2, 64, 688, 128, 2, 100),
    # the largest model width the library accepts (q|k|v narrower than D)
    ("bf16_max_d_16384_n33", "bf16", 16384, 2, 2, 128, 688, 40, 1, 33),
]


@pytest.mark.parametrize("spec", PREFILL, ids=[p[0] for p in PREFILL])
def test_layer_prefill_parity(spec):
    pop = _pop()
    name, dtype, D, H, Hkv, hd, dff, L, B, N = spec
    case = Case(name, dtype, D, H, Hkv, hd, dff, L)
    g = np.random.default_rng(_seed(name))
    layer, ref = _layer(case, g)
    X = g.standard_normal((B, N, D))
    x = torch.from_numpy(X.astype(np.float32)).cuda()
    Xr = x.double().cpu().numpy()
    K, V = layer.cache(B)
    ws = pop.workspace(pop.pop_layer_prefill_workspace_bytes(B, N, layer))
    R, C, P, I = pop.pop_layer_prefill(x, layer, K, V, 0.3, 0.1, importance=True, ws=ws)
    torch.cuda.synchronize()
    o = lo.layer_prefill(Xr, ref, case.cfg, 0.3, 0.1, dtype, L)
    Kd, Vd = K.double().cpu().numpy(), V.double().cpu().numpy()
    _close(Kd[:, :, :N], o["K"][:, :, :N], dtype, "K cache")
    _close(Vd[:, :, :N], o["V"][:, :, :N], dtype, "V cache")
    assert not Kd[:, :, N:].any() and not Vd[:, :, N:].any(), "cache positions past the prompt were written"
    esz = 2 if dtype == "bf16" else 4
    xn2 = ws[: B * N * D * esz].view(case.tdtype()).double().cpu().numpy().reshape(B * N, D)
    _check_xn2(xn2, o["xn2"], dtype)
    check_partition(R, C, P, I, o["I"], 0.3, 0.1)
    _close(host(x), o["x"], dtype, "layer output")


# ---------------------------------------------------------------- decode
DECODE = [
    # name, dtype, D, H, Hkv, hd, d_ff, L, batch, pos
    ("f32_gqa_b1_pos40", "f32", 256, 4, 2, 64, 688, 96, 1, 40),
    ("bf16_gqa_b3_pos95_last_slot", "bf16", 256, 4, 2, 64, 688, 96, 3, 95),
    ("bf16_pos0_first_token", "bf16", 256, 4, 4, 64, 688, 96, 2, 0),
    ("f32_hd128_b2_pos700", "f32", 512, 4, 4, 128, 1376, 800, 2, 700),
    ("bf16_hd128_b16_pos333", "bf16", 512, 8, 2, 128, 1376, 400, 16, 333),
    ("bf16_b64_pos63", "bf16", 256, 4, 2, 64, 688, 64, 64, 63),
    # fp32 above batch 2 (separate merge kernel, plain projections); bf16 at the matrix-core projections' threshold
    ("f32_gqa_b5_pos77", "f32", 256, 4, 2, 64, 688, 96, 5, 77),
    ("bf16_hd128_b12_pos130", "bf16", 512, 4, 2, 128, 1376, 160, 12, 130),
    # matrix-core projections past one stage: 96-row reduction slices of the
    # q|k|v projection (3 stages), a 64-column partial tile of the output
    # projection, and a partial second 16-token group (batch 20)
    ("bf16_d4160_b20_pos40", "bf16", 4160, 4, 2, 128, 688, 64, 20, 40),
    # the largest model width, and a 4096-position cache at its last slot (64 slices merged)
    ("bf16_max_d_16384_b2_pos50", "bf16", 16384, 2, 1, 128, 688, 64, 2, 50),
    ("f32_cache_4096_last_slot", "f32", 256, 4, 2, 64, 688, 4096, 1, 4095),
]


def _k(dff, r, R, C):
    """Candidates the step selects for these lists: clamp(live - |R|, 0, |C|)."""
    return min(max(oracle.partition_counts(dff, r, 0.0)["n_live"] - len(R), 0), len(C))


def _decode_inputs(case, g, B, pos, r=0.3):
    t = case.tdtype()
    shp = (B, case.Hkv, case.L, case.hd)
    K = torch.zeros(shp, dtype=t, device="cuda")
    V = torch.zeros(shp, dtype=t, device="cuda")
    if pos > 0:
        K[:, :, :pos] = torch.from_numpy(g.standard_normal((B, case.Hkv, pos, case.hd)).astype(np.float32)).to(t).cuda()
        V[:, :, :pos] = torch.from_numpy(g.standard_normal((B, case.Hkv, pos, case.hd)).astype(np.float32)).to(t).cuda()
    x = torch.from_numpy(g.standard_normal((B, case.D)).astype(np.float32)).cuda()
    R, C, _ = oracle.partition(g.uniform(0, 1, case.dff), r, 0.1)
    return K, V, x, R, C


@pytest.mark.parametrize("spec", DECODE, ids=[p[0] for p in DECODE])
@pytest.mark.parametrize("dense", [False, True], ids=["pop", "dense_ffn"])
def test_layer_decode_parity(spec, dense):
    pop = _pop()
    name, dtype, D, H, Hkv, hd, dff, L, B, pos = spec
    case = Case(name, dtype, D, H, Hkv, hd, dff, L)
    g = np.random.default_rng(_seed(name))
    layer, ref = _layer(case, g)
    K, V, x, R, C = _decode_inputs(case, g, B, pos)
    Kr, Vr, xr = K.double().cpu().numpy(), V.double().cpu().numpy(), x.double().cpu().numpy()
    k = _k(dff, 0.3, R, C)
    S = torch.empty(k, dtype=torch.int32, device="cuda")
    Rd = torch.from_numpy(R.astype(np.int32)).cuda()
    Cd = torch.from_numpy(C.astype(np.int32)).cuda()
    posd = torch.tensor([pos], dtype=torch.int32, device="cuda")
    ws = pop.workspace(pop.pop_layer_decode_workspace_bytes(B, layer))
    pop.pop_layer_decode(x, layer, K, V, posd, Rd, Cd, 0.3, dense_ffn=dense, selected=None if dense else S, ws=ws)
    torch.cuda.synchronize()
    o = lo.layer_decode(xr, ref, case.cfg, Kr, Vr, pos, R, C, 0.3, dtype, dense_ffn=dense)
    Kd, Vd = K.double().cpu().numpy(), V.double().cpu().numpy()
    _close(Kd[:, :, pos], Kr[:, :, pos], dtype, "K cache entry")
    _close(Vd[:, :, pos], Vr[:, :, pos], dtype, "V cache entry")
    mask = np.ones(L, dtype=bool)
    mask[pos] = False
    assert np.array_equal(Kd[:, :, mask], Kr[:, :, mask]) and np.array_equal(Vd[:, :, mask], Vr[:, :, mask]), \
        "cache entries other than pos changed"
    esz = 2 if dtype == "bf16" else 4
    xn2 = ws[: B * D * esz].view(case.tdtype()).double().cpu().numpy().reshape(B, D)
    _check_xn2(xn2, o["xn2"], dtype)
    if dense:
        want = o["x"]
    else:
        S_dev, _ = _check_selection(S, xn2, ref, R, C, 0.3, k, o["S"])
        live = np.concatenate([R, S_dev])
        want = o["h"] + oracle.masked_ffn(o["xn2"], ref["W_gate"], ref["W_up"], ref["W_down"], live)
    _close(host(x), want, dtype, "layer output")


def test_layer_decode_bad_position_touches_nothing():
    """pos outside [0, cache_len): no cache entry is written (x is undefined)."""
    pop = _pop()
    case = Case("bad_pos", "bf16", 256, 4, 2, 64, 688, 32)
    g = np.random.default_rng(5)
    layer, _ = _layer(case, g)
    K, V, x, R, C = _decode_inputs(case, g, 2, 32)
    K0, V0 = K.clone(), V.clone()
    for bad in (32, -1):
        posd = torch.tensor([bad], dtype=torch.int32, device="cuda")
        pop.pop_layer_decode(x, layer, K, V, posd, torch.from_numpy(R.astype(np.int32)).cuda(),
                             torch.from_numpy(C.astype(np.int32)).cuda(), 0.3)
        torch.cuda.synchronize()
        assert torch.equal(K, K0) and torch.equal(V, V0)


# ---------------------------------------------------------------- prompt, then decode steps
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_prefill_then_decode_steps(dtype):
    """The prompt pass, then four decode steps (pos advanced on the device),
    each against the oracle's chain from the same inputs; the partition is the
    device's, checked against the oracle's first."""
    pop = _pop()
    case = Case(f"chain_{dtype}", dtype, 256, 4, 2, 64, 688, 64)
    g = np.random.default_rng(_seed(case.name))
    layer, ref = _layer(case, g)
    B, N, steps = 2, 21, 4
    X = torch.from_numpy(g.standard_normal((B, N, case.D)).astype(np.float32)).cuda()
    Xr = X.double().cpu().numpy()
    K, V = layer.cache(B)
    R, C, P, I = pop.pop_layer_prefill(X, layer, K, V, 0.3, 0.1, importance=True)
    torch.cuda.synchronize()
    o = lo.layer_prefill(Xr, ref, case.cfg, 0.3, 0.1, dtype, case.L)
    check_partition(R, C, P, I, o["I"], 0.3, 0.1)
    Rn, Cn = host(R).astype(np.int64), host(C).astype(np.int64)
    Kr, Vr = o["K"], o["V"]
    posd = torch.tensor([N], dtype=torch.int32, device="cuda")
    k = _k(case.dff, 0.3, Rn, Cn)
    S = torch.empty(k, dtype=torch.int32, device="cuda")
    ws = pop.workspace(pop.pop_layer_decode_workspace_bytes(B, layer))
    xs = g.standard_normal((steps, B, case.D))
    for t in range(steps):
        x = torch.from_numpy(xs[t].astype(np.float32)).cuda()
        xr = x.double().cpu().numpy()
        pop.pop_layer_decode(x, layer, K, V, posd, R, C, 0.3, selected=S, ws=ws)
        posd += 1
        torch.cuda.synchronize()
        st = lo.layer_decode(xr, ref, case.cfg, Kr, Vr, N + t, Rn, Cn, 0.3, dtype)
        esz = 2 if dtype == "bf16" else 4
        xn2 = ws[: B * case.D * esz].view(case.tdtype()).double().cpu().numpy().reshape(B, case.D)
        _check_xn2(xn2, st["xn2"], dtype)
        S_dev, _ = _check_selection(S, xn2, ref, Rn, Cn, 0.3, k, st["S"])
        want = st["h"] + oracle.masked_ffn(st["xn2"], ref["W_gate"], ref["W_up"], ref["W_down"],
                                          np.concatenate([Rn, S_dev]))
        _close(host(x), want, dtype, f"step {t} output")
        _close(K.double().cpu().numpy()[:, :, : N + t + 1], Kr[:, :, : N + t + 1], dtype, f"step {t} K cache")
    assert int(posd.item()) == N + steps


def test_layer_decode_graph_replay_matches_eager():
    """A captured decode step (the position advanced inside the graph) replays
    bit for bit like the eager calls, step after step."""
    pop = _pop()
    case = Case("graph", "bf16", 256, 4, 2, 64, 688, 64)
    g = np.random.default_rng(_seed(case.name))
    layer, _ = _layer(case, g)
    B, pos0 = 3, 10
    K, V, x, R, C = _decode_inputs(case, g, B, pos0)
    Rd, Cd = torch.from_numpy(R.astype(np.int32)).cuda(), torch.from_numpy(C.astype(np.int32)).cuda()
    xs = torch.from_numpy(g.standard_normal((5, B, case.D)).astype(np.float32)).cuda()
    # eager reference on copies
    Ke, Ve = K.clone(), V.clone()
    pe = torch.tensor([pos0], dtype=torch.int32, device="cuda")
    eager = []
    wse = pop.workspace(pop.pop_layer_decode_workspace_bytes(B, layer))
    for t in range(5):
        xe = xs[t].clone()
        pop.pop_layer_decode(xe, layer, Ke, Ve, pe, Rd, Cd, 0.3, ws=wse)
        pe += 1
        eager.append(xe)
    torch.cuda.synchronize()
    # graph
    xg = torch.empty_like(xs[0])
    pg = torch.tensor([pos0], dtype=torch.int32, device="cuda")
    wsg = pop.workspace(pop.pop_layer_decode_workspace_bytes(B, layer))
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        pop.pop_layer_decode(xg, layer, K, V, pg, Rd, Cd, 0.3, ws=wsg, stream=s)
        pg.add_(1)
    torch.cuda.synchronize()
    for t in range(5):
        xg.copy_(xs[t])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(xg, eager[t]), f"replay {t} differs from the eager step"
    assert torch.equal(K, Ke) and torch.equal(V, Ve)
    assert int(pg.item()) == pos0 + 5


# ---------------------------------------------------------------- LLaMA-2-7B shape
def test_layer_llama2_7b_shape_decode_and_prefill():
    """The LLaMA-2-7B layer shape (D 4096, 32 heads of 128, D_FF 11008, bf16,
    weights N(0, 0.02^2)) at batch 1: a 32-token prompt pass, then a decode step
    at position 700 of a cache filled with N(0, 1) entries."""
    pop = _pop()
    case = Case("llama2_7b_layer", "bf16", 4096, 32, 32, 128, 11008, 1024, std=0.02)
    g = np.random.default_rng(_seed(case.name))
    layer, ref = _layer(case, g)
    # prompt pass
    N = 32
    X = torch.from_numpy(g.standard_normal((1, N, case.D)).astype(np.float32)).cuda()
    Xr = X.double().cpu().numpy()
    K, V = layer.cache(1)
    R, C, P, I = pop.pop_layer_prefill(X, layer, K, V, 0.299, 0.1, importance=True)
    torch.cuda.synchronize()
    o = lo.layer_prefill(Xr, ref, case.cfg, 0.299, 0.1, "bf16", N)
    check_partition(R, C, P, I, o["I"], 0.299, 0.1)
    _close(host(X), o["x"], "bf16", "prompt output")
    _close(K.double().cpu().numpy()[:, :, :N], o["K"], "bf16", "prompt K cache")
    del o
    # decode step at position 700
    pos = 700
    K2, V2, x, Rr, Cr = _decode_inputs(case, g, 1, pos, r=0.299)
    Kr, Vr, xr = K2.double().cpu().numpy(), V2.double().cpu().numpy(), x.double().cpu().numpy()
    k = _k(case.dff, 0.299, Rr, Cr)
    S = torch.empty(k, dtype=torch.int32, device="cuda")
    ws = pop.workspace(pop.pop_layer_decode_workspace_bytes(1, layer))
    pop.pop_layer_decode(x, layer, K2, V2, torch.tensor([pos], dtype=torch.int32, device="cuda"),
                         torch.from_numpy(Rr.astype(np.int32)).cuda(), torch.from_numpy(Cr.astype(np.int32)).cuda(),
                         0.299, selected=S, ws=ws)
    torch.cuda.synchronize()
    st = lo.layer_decode(xr, ref, case.cfg, Kr, Vr, pos, Rr, Cr, 0.299, "bf16")
    xn2 = ws[: case.D * 2].view(torch.bfloat16).double().cpu().numpy().reshape(1, case.D)
    _check_xn2(xn2, st["xn2"], "bf16")
    S_dev, n_flip = _check_selection(S, xn2, ref, Rr, Cr, 0.299, k, st["S"])
    print(f"selection: {n_flip} of {k} channels differ from the fp64 chain's")
    want = st["h"] + oracle.masked_ffn(st["xn2"], ref["W_gate"], ref["W_up"], ref["W_down"],
                                      np.concatenate([Rr, S_dev]))
    _close(host(x), want, "bf16", "decode output")
    _close(K2.double().cpu().numpy()[:, :, pos], Kr[:, :, pos], "bf16", "decode K entry")
