"""Plant plausible mistakes in a copy of the oracle (on the CPU) and require
that at least one pin catches each: a dropped term, a wrong sign or index, a
transposed or swapped operand, an off-by-one count, a flipped tie rule."""
import os
import types

import pytest

import oracle.pop_oracle as real
from tests.oracle_pins import ALL_PINS

SRC = open(real.__file__).read()

MUTANTS = [
    ("importance drops the square root",
     "return np.sqrt(((W * s[None, :]) ** 2).sum(axis=1))", "return ((W * s[None, :]) ** 2).sum(axis=1)"),
    ("importance ignores s",
     "return np.sqrt(((W * s[None, :]) ** 2).sum(axis=1))", "return np.sqrt((W ** 2).sum(axis=1))"),
    ("column norm uses |x| instead of x^2", "acc += row * row", "acc += np.abs(row)"),
    ("column norm over the first token only", "for row in X:", "for row in X[:1]:"),
    ("tie rule flipped in the sort form", "np.lexsort((-idx, v))", "np.lexsort((idx, v))"),
    ("tie rule flipped in the threshold form", "m[ties[len(ties) - need:]] = True", "m[ties[:need]] = True"),
    ("upper cut truncated", "c_high = round_half_away(p_hi * n)", "c_high = int(p_hi * n)"),
    ("round half down", "return int(f + 1) if frac >= 0.5 else int(f)", "return int(f + 1) if frac > 0.5 else int(f)"),
    ("delta = gamma / 2", "delta = float(gamma)", "delta = float(gamma) / 2"),
    ("k off by one", '"k": c_high - c_mid,', '"k": c_high - c_mid - 1,'),
    ("live count ignores rounding", "n_live = round_half_away((1.0 - float(r)) * n)", "n_live = int((1.0 - float(r)) * n)"),
    ("regions swapped", "return np.flatnonzero(in_R), np.flatnonzero(in_C), np.flatnonzero(in_P)",
     "return np.flatnonzero(in_P), np.flatnonzero(in_C), np.flatnonzero(in_R)"),
    ("sigmoid sign flipped", "out[pos] = a[pos] / (1.0 + np.exp(-a[pos]))", "out[pos] = a[pos] / (1.0 + np.exp(a[pos]))"),
    ("gate and up swapped", "    return silu(g) * u\n", "    return silu(u) * g\n"),
    ("score is the batch mean", "return np.abs(z[:, n_R:]).max(axis=0)", "return np.abs(z[:, n_R:]).mean(axis=0)"),
    ("score is signed", "return np.abs(z[:, n_R:]).max(axis=0)", "return z[:, n_R:].max(axis=0)"),
    ("score over R instead of C", "return np.abs(z[:, n_R:]).max(axis=0)", "return np.abs(z[:, :z.shape[1] - n_R]).max(axis=0)"),
    ("selection keeps the lowest scores", "key=lambda j: (-scores[j], C[j])", "key=lambda j: (scores[j], C[j])"),
    ("selection tie toward the higher index", "key=lambda j: (-scores[j], C[j])", "key=lambda j: (-scores[j], -C[j])"),
    ("z position off by one",
     "zpos = np.concatenate([np.arange(len(R)), len(R) + np.array(",
     "zpos = np.concatenate([np.arange(len(R)), len(R) - 1 + np.array("),
    ("down projection reads the wrong channels", "y = z[:, zpos] @ Wd[:, live].T", "y = z[:, zpos] @ Wd[:, np.sort(live)].T"),
    ("dense FFN uses W_gate twice", "return (silu(x @ _f64(W_gate).T) * (x @ _f64(W_up).T)) @ _f64(W_down).T",
     "return (silu(x @ _f64(W_gate).T) * (x @ _f64(W_gate).T)) @ _f64(W_down).T"),
    ("routing tie toward the higher expert", "key=lambda e: (-L[t, e], e)", "key=lambda e: (-L[t, e], -e)"),
    ("routing weights not normalised", "weights[t] = (w1 / (w1 + w2), w2 / (w1 + w2))", "weights[t] = (w1, w2)"),
    ("expert partition over all prompt tokens", "toks = np.flatnonzero((ex == e).any(axis=1))", "toks = np.arange(len(X))"),
    ("a token's two routing weights swapped", "y[rows] += wt[rows, slot][:, None] * ye",
     "y[rows] += wt[rows, 1 - slot][:, None] * ye"),
    ("constant routing weights of one half", "y[rows] += wt[rows, slot][:, None] * ye", "y[rows] += 0.5 * ye"),
    ("an expert's output added without its weight", "y[rows] += wt[rows, slot][:, None] * ye", "y[rows] += ye"),
    ("full re-evaluation keeps one channel too few", "S = select_candidates(allc, sc, n_live)", "S = select_candidates(allc, sc, n_live - 1)"),
    ("periodic memory kept across a refresh", "            memory = np.zeros(len(C))\n        else:", "        else:"),
    ("periodic memory ignores the steps between refreshes", "memory[spos] += candidate_scores(z_live, n_R)",
     "memory[spos] += 0.0"),
    ("periodic refresh ranks by its own step only", "S = select_candidates(C, memory, k)",
     "S = select_candidates(C, candidate_scores(z, n_R), k)"),
    ("periodic refresh every other period", "refresh = t % int(period) == 0", "refresh = t % (2 * int(period)) == 0"),
]


def _load_mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("pop_oracle_mutant")
    mod.__file__ = os.path.join(os.path.dirname(real.__file__), "pop_oracle_mutant.py")
    exec(compile(SRC.replace(old, new), mod.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"no pin caught the planted mistake: {name}"
