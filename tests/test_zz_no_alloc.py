"""The allocation-free decode entry point (pop_decode_ffn_noalloc) against
pop_decode_ffn with a caller workspace, through the C ABI: the same kernels on
the same inputs, so the outputs must agree bit for bit (stronger than the
parity bar), on calls in a row whose second input is smaller, including the
single-launch batch-1 step that carries control words between calls."""
import sys

import numpy as np
import pytest
import torch

from online_structured_ffn_amd import pop, synth
from tests.parity import dev, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(seed, d, d_ff, batch, r):
    c = synth.random_case(seed, 24, d, d_ff, batch, "bf16")
    Wg, Wu, WdT = dev(c["W_gate"], "bf16"), dev(c["W_up"], "bf16"), dev(c["W_downT"], "bf16")
    R, C, _ = pop.pop_prefill_partition(dev(c["X"], "bf16"), Wu, r, 0.1)
    return dev(c["x"], "bf16"), Wg, Wu, WdT, R, C


# each list: calls in a row on one GPU, the second with a smaller input
SEQUENCES = [
    [(1024, 2816, 4, 0.3), (512, 1376, 1, 0.3)],
    [(4096, 11008, 1, 0.299), (1024, 2816, 1, 0.3), (512, 1376, 2, 0.5)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["b4_then_b1", "llama_b1_then_smaller"])
def test_noalloc_matches_workspace_call(seq):
    for i, (d, d_ff, batch, r) in enumerate(seq):
        say(f"[noalloc] call {i}: d={d} d_ff={d_ff} batch={batch} r={r}")
        x, Wg, Wu, WdT, R, C = _case(40 + i, d, d_ff, batch, r)
        y_ref, S_ref = pop.pop_decode_ffn(x, Wg, Wu, WdT, R, C, r, selected=True)
        y, S = pop.pop_decode_ffn_noalloc(x, Wg, Wu, WdT, R, C, r, selected=True)
        torch.cuda.synchronize()
        assert torch.equal(S, S_ref), f"call {i}: selection differs"
        assert torch.equal(y, y_ref), f"call {i}: max |dy| = {(y - y_ref).abs().max().item():.3e}"
        # again, as the same call after other work: the scratch keeps nothing that changes the result
        y2 = pop.pop_decode_ffn_noalloc(x, Wg, Wu, WdT, R, C, r)
        torch.cuda.synchronize()
        assert torch.equal(y2, y_ref), f"call {i}: repeated call differs"


def test_noalloc_rejects_beyond_scratch():
    x = torch.zeros((64, 16384), dtype=torch.bfloat16, device="cuda")
    # sizes are checked before any pointer is used: NULL weights with a too-large shape
    st = pop.lib.pop_decode_ffn_noalloc(pop._ptr(x), 64, 16384, None, None, None, 32768, pop.POP_BF16,
                                        None, 0, None, 0, 0.3, None, None, pop._stream(None))
    assert st == 5, pop.status_string(st)
    assert "scratch" in pop.lib.pop_last_error().decode()
