"""The periodic-refresh decode mode (pop_decode_ffn_periodic) against the
oracle's periodic_decode, step by step: the selection exactly (the cases are
checked to hold no near-tie at a refresh, where either choice would be
admissible and the sequences would part), the activation memory to
VALUE_RTOL and y to TOL of max|y|."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from online_structured_ffn_amd import pop, synth
from tests.parity import TIE_REL, TOL, VALUE_RTOL, dev, host

pytestmark = pytest.mark.gpu

CASES = [
    # name, d, d_ff, batch, dtype, r, period, steps
    ("f32_b1_p3", 64, 300, 1, "f32", 0.3, 3, 7),
    ("bf16_b1_p1", 128, 500, 1, "bf16", 0.3, 1, 4),
    ("bf16_b4_p2", 256, 700, 4, "bf16", 0.3, 2, 6),
    ("bf16_b16_p4", 264, 1000, 16, "bf16", 0.299, 4, 9),
    ("f32_b3_p5_high_r", 64, 200, 3, "f32", 0.8, 5, 6),
]


def _setup(seed, d, d_ff, batch, dtype, r, steps):
    c = synth.random_case(seed, 40, d, d_ff, batch, dtype)
    g = np.random.default_rng(seed + 7)
    xs = [synth.to_dtype(g.standard_normal((batch, d)).astype(np.float32), dtype) for _ in range(steps)]
    R, C, _ = oracle.partition(oracle.importance(c["W_up"], oracle.column_norm(c["X"])), r, 0.1)
    return c, xs, R, C


def _min_refresh_gap(ref, xs, c, R, C, r, period):
    """Smallest relative gap between the k-th and (k+1)-th ranking value over
    the refreshes (inf when every candidate or none is kept)."""
    k = len(ref[0]["S"])
    gap = np.inf
    mem = np.zeros(len(C))
    for t, x in enumerate(xs):
        if t % period == 0:
            h = mem + oracle.candidate_scores(oracle.restricted_forward(x, c["W_gate"], c["W_up"], R, C), len(R))
            if 0 < k < len(C):
                v = np.sort(h)[::-1]
                gap = min(gap, (v[k - 1] - v[k]) / max(v[k - 1], 1e-30))
        mem = ref[t]["memory"]
    return gap


@pytest.mark.parametrize("name,d,d_ff,batch,dtype,r,period,steps", CASES, ids=[c[0] for c in CASES])
def test_periodic_matches_oracle(name, d, d_ff, batch, dtype, r, period, steps):
    print(f"[periodic] {name}", flush=True)
    c, xs, R, C = _setup(zlib.crc32(name.encode()) % 1000, d, d_ff, batch, dtype, r, steps)
    ref = oracle.periodic_decode(xs, c["W_gate"], c["W_up"], c["W_down"], R, C, r, period)
    gap = _min_refresh_gap(ref, xs, c, R, C, r, period)
    assert gap > TIE_REL, f"case {name} holds a near-tie at a refresh (gap {gap:.2e}); pick another seed"
    Wg, Wu, WdT = dev(c["W_gate"], dtype), dev(c["W_up"], dtype), dev(c["W_downT"], dtype)
    Rd = torch.from_numpy(R.astype(np.int32)).cuda()
    Cd = torch.from_numpy(C.astype(np.int32)).cuda()
    state = pop.PeriodicState(d_ff, r, len(R), len(C), "cuda")
    ws = pop.workspace(pop.pop_decode_periodic_workspace_bytes(batch, d, d_ff))
    for t in range(steps):
        y = pop.pop_decode_ffn_periodic(dev(xs[t], dtype), Wg, Wu, WdT, Rd, Cd, r, t, period, state, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(host(state.selected)), ref[t]["S"]), f"step {t}: selection differs"
        assert np.array_equal(np.sort(C[host(state.positions)]), ref[t]["S"]), f"step {t}: positions differ"
        np.testing.assert_allclose(host(state.memory), ref[t]["memory"], rtol=VALUE_RTOL,
                                   atol=VALUE_RTOL * max(np.abs(ref[t]["memory"]).max(), 1e-30))
        y_ref = ref[t]["y"]
        err = np.abs(host(y) - y_ref).max() / max(np.abs(y_ref).max(), 1e-30)
        assert err <= TOL[dtype], f"step {t}: max|dy|/max|y| = {err:.3e}"
        print(f"  step {t} ({'refresh' if ref[t]['refresh'] else 'kept'}): rel err {err:.2e}", flush=True)


def test_periodic_deterministic_and_graph_replay():
    """Two runs of the same sequence give the same bits; the refresh and the
    in-between step captured in HIP graphs replay like eager calls."""
    print("[periodic] determinism and graph replay", flush=True)
    d, d_ff, batch, dtype, r, period, steps = 256, 700, 2, "bf16", 0.3, 2, 6
    c, xs, R, C = _setup(5, d, d_ff, batch, dtype, r, steps)
    Wg, Wu, WdT = dev(c["W_gate"], dtype), dev(c["W_up"], dtype), dev(c["W_downT"], dtype)
    Rd = torch.from_numpy(R.astype(np.int32)).cuda()
    Cd = torch.from_numpy(C.astype(np.int32)).cuda()
    ws = pop.workspace(pop.pop_decode_periodic_workspace_bytes(batch, d, d_ff))
    xd = [dev(x, dtype) for x in xs]

    def run():
        st = pop.PeriodicState(d_ff, r, len(R), len(C), "cuda")
        return [pop.pop_decode_ffn_periodic(xd[t], Wg, Wu, WdT, Rd, Cd, r, t, period, st, ws=ws).clone()
                for t in range(steps)]

    a, b = run(), run()
    torch.cuda.synchronize()
    for t in range(steps):
        assert torch.equal(a[t], b[t]), f"step {t} differs between runs"
    st = pop.PeriodicState(d_ff, r, len(R), len(C), "cuda")
    x_in, y_out = xd[0].clone(), torch.empty((batch, d), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in (0, 1):
            pop.pop_decode_ffn_periodic(x_in, Wg, Wu, WdT, Rd, Cd, r, t, period, st, y=y_out, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = []
    for t in (0, 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            pop.pop_decode_ffn_periodic(x_in, Wg, Wu, WdT, Rd, Cd, r, t, period, st, y=y_out, ws=ws)
        graphs.append(g)
    st.memory.zero_()
    torch.cuda.synchronize()
    for t in range(steps):
        x_in.copy_(xd[t])
        graphs[t % period].replay()
        torch.cuda.synchronize()
        assert torch.equal(y_out, a[t]), f"graph replay of step {t} differs from eager"
