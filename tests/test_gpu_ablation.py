"""The two ablation variants of the POP notes ("Key experimental data",
ablation table) on the GPU, against the oracle, plus the empty-R stage calls
they rely on.

Both variants run through the existing entry points:
  variant (1), static prefill mask: the live set is fixed at prefill to the
    round((1 - r) d_ff) channels of highest prefill importance, which is R
    plus the k most important candidates (reading taken: the pages say only
    that the prefill mask is reused).  pop_partition_select(I, r, gamma=0)
    yields it as its R list; every step is pop_decode_ffn over that list with
    no candidates.
  variant (2), full re-evaluation: pop_decode_ffn with R empty and every
    channel a candidate, so the step scores all d_ff channels and keeps the
    round((1 - r) d_ff) best.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from online_structured_ffn_amd import configs, pop, synth
from tests.parity import TOL, check_decode, dev, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    yield
    torch.cuda.synchronize()


def _case(kind, seed, n, d, d_ff, b, dtype):
    if kind == "llama":
        w = configs.BY_NAME["llama2_7b_ffn_b1"]
        c = dict(synth.layer_weights(w, 3))
        c["X"] = synth.prompt(w, 3)
        c["x"] = synth.decode_input(w, 3, 0)
        return c
    return synth.random_case(seed, n, d, d_ff, b, dtype)


CASES = [
    # kind, seed, n_tokens, d, d_ff, batch, dtype, r
    ("rand", 61, 40, 256, 688, 1, "f32", 0.3),
    ("rand", 62, 33, 1032, 2900, 1, "bf16", 0.3),
    ("rand", 63, 20, 520, 1501, 4, "bf16", 0.299),
    ("llama", 0, 0, 4096, 11008, 1, "bf16", 0.299),
]
IDS = [f"{c[0]}_{c[4]}_b{c[5]}_{c[6]}" for c in CASES]


@pytest.mark.parametrize("kind,seed,n,d,d_ff,b,dtype,r", CASES, ids=IDS)
def test_static_prefill_mask(kind, seed, n, d, d_ff, b, dtype, r):
    say(f"[ablation static] d={d} d_ff={d_ff} B={b} {dtype}")
    c = _case(kind, seed, n, d, d_ff, b, dtype)
    Xd, xd = dev(c["X"], dtype), dev(c["x"], dtype)
    Wg, Wu, WdT = dev(c["W_gate"], dtype), dev(c["W_up"], dtype), dev(c["W_downT"], dtype)
    R, C, P, I = pop.pop_prefill_partition(Xd, Wu, r, 0.1, importance=True)
    Rs, Cs, Ps = pop.pop_partition_select(I, r, 0.0)
    y = pop.pop_decode_ffn(xd, Wg, Wu, WdT, Rs, Cs, r)
    torch.cuda.synchronize()
    cnt = oracle.partition_counts(d_ff, r, 0.1)
    assert Cs.numel() == 0 and Rs.numel() == cnt["n_live"]
    I_dev = host(I).astype(np.float64)
    Rh, Ch = host(R).astype(np.int64), host(C).astype(np.int64)
    # the static live set is R plus the k most important candidates (same decision, device values)
    S0 = oracle.select_candidates(Ch, I_dev[Ch], cnt["k"])
    assert np.array_equal(host(Rs), np.sort(np.concatenate([Rh, S0])))
    assert np.array_equal(host(Rs), oracle.partition(I_dev, r, 0.0)[0])
    ref = oracle.static_mask_ffn(c["x"], c["W_gate"], c["W_up"], c["W_down"], Rh, Ch, S0)
    err = np.abs(host(y) - ref).max() / np.abs(ref).max()
    say(f"  rel err {err:.2e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("kind,seed,n,d,d_ff,b,dtype,r", CASES, ids=IDS)
def test_full_reevaluation(kind, seed, n, d, d_ff, b, dtype, r):
    say(f"[ablation full] d={d} d_ff={d_ff} B={b} {dtype}")
    c = _case(kind, seed, n, d, d_ff, b, dtype)
    xd = dev(c["x"], dtype)
    Wg, Wu, WdT = dev(c["W_gate"], dtype), dev(c["W_up"], dtype), dev(c["W_downT"], dtype)
    R = torch.empty(0, dtype=torch.int32, device="cuda")
    C = torch.arange(d_ff, dtype=torch.int32, device="cuda")
    ws = pop.workspace(pop.pop_decode_workspace_bytes(c["x"].shape[0], d, d_ff))
    y, S = pop.pop_decode_ffn(xd, Wg, Wu, WdT, R, C, r, selected=True, ws=ws)
    torch.cuda.synchronize()
    n_live = oracle.partition_counts(d_ff, r, 0.0)["n_live"]
    assert S.numel() == n_live
    err, n_ex = check_decode(y, S, ws, c["x"], c, np.zeros(0, np.int64), np.arange(d_ff), r, dtype)
    say(f"  rel err {err:.2e}, near-tie exclusions {n_ex}")
    full = oracle.full_reeval_ffn(c["x"], c["W_gate"], c["W_up"], c["W_down"], r)
    if np.array_equal(host(S), full["S"]):
        e2 = np.abs(host(y) - full["y"]).max() / np.abs(full["y"]).max()
        assert e2 <= TOL[dtype]


def test_stage_calls_with_null_empty_R():
    """R == NULL with n_R == 0 and candidates present: the candidate rows must
    come from C (not be taken as identity rows)."""
    say("[stages] NULL empty R")
    c = synth.random_case(71, 1, 256, 600, 3, "bf16")
    xd = dev(c["x"], "bf16")
    Wg, Wu, WdT = dev(c["W_gate"], "bf16"), dev(c["W_up"], "bf16"), dev(c["W_downT"], "bf16")
    Ch = np.sort(np.random.default_rng(5).choice(600, 150, replace=False)).astype(np.int32)
    C = torch.from_numpy(Ch).cuda()
    z, score = pop.pop_decode_gateup(xd, Wg, Wu, None, C, n_R=0)
    k = 40
    pos, sel = pop.pop_decode_select(score, C, k)
    y = pop.pop_decode_down(z, WdT, None, sel, pos, n_R=0)
    torch.cuda.synchronize()
    zr = oracle.restricted_forward(c["x"], c["W_gate"], c["W_up"], np.zeros(0, np.int64), Ch.astype(np.int64))
    assert np.abs(host(z) - zr).max() <= 1e-4 * np.abs(zr).max()
    S = host(sel).astype(np.int64)
    assert np.array_equal(S, oracle.select_candidates(Ch.astype(np.int64), host(score).astype(np.float64), k))
    ref = oracle.masked_ffn(c["x"], c["W_gate"], c["W_up"], c["W_down"], S)
    assert np.abs(host(y) - ref).max() <= TOL["bf16"] * np.abs(ref).max()
