"""Property tests (Hypothesis) of the oracle's partition and selection and of
the library's host logic: counts, top-k sizes and the index-list check.

Each property is one that the method fixes at every size, so that Hypothesis
may search freely and shrink a failure to a small case:
  * the three regions of a partition are disjoint, cover every channel, have
    exactly the counts of the quantile thresholds ([POP] Key design 1) and
    are ordered by importance (every P channel at most every C channel at
    most every R channel, ties split by the index rule);
  * the selection keeps k candidates whose scores no unselected candidate
    beats ([POP] Key design 2), and |R| + k equals the live count whenever
    C is large enough;
  * the library's pop_partition_counts and pop_decode_topk_count agree with
    the oracle's, and pop_check_lists accepts exactly the lists a plain
    Python check accepts.
No call here reaches a GPU."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from online_structured_ffn_amd import pop

OK, INVALID, SHAPE = 0, 1, 3
SETTINGS = settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])

rates = st.floats(min_value=0.0, max_value=0.999, allow_nan=False)
gammas = st.floats(min_value=0.0, max_value=0.999, allow_nan=False)


@st.composite
def importances(draw, max_n=300):
    """Importance vectors with many ties (drawn from a small value set) or
    none (continuous values)."""
    n = draw(st.integers(1, max_n))
    seed = draw(st.integers(0, 2**32 - 1))
    g = np.random.default_rng(seed)
    if draw(st.booleans()):
        return g.integers(0, draw(st.integers(1, 6)), n).astype(np.float64)
    return g.random(n)


@SETTINGS
@given(st.integers(1, 32768), rates, gammas)
def test_counts_library_matches_oracle(n, r, gamma):
    got = pop.pop_partition_counts(n, r, gamma)
    exp = oracle.partition_counts(n, r, gamma)
    assert {k: got[k] for k in exp} == exp
    assert got["n_P"] + got["n_C"] + got["n_R"] == n
    assert 0 <= got["k"] <= got["n_C"]
    # the live count is met exactly unless C is too small for it
    if got["n_R"] <= got["n_live"] <= got["n_R"] + got["n_C"]:
        assert got["n_R"] + got["k"] == got["n_live"]


@SETTINGS
@given(st.integers(1, 32768), rates, st.data())
def test_topk_count_library_matches_oracle(n, r, data):
    n_R = data.draw(st.integers(0, n))
    n_C = data.draw(st.integers(0, n - n_R))
    assert pop.pop_decode_topk_count(n, r, n_R, n_C) == oracle.pop_oracle._k_for(n, r, n_R, n_C)


@SETTINGS
@given(importances(), rates, gammas)
def test_partition_invariants(I, r, gamma):
    R, C, P = oracle.partition(I, r, gamma)
    cnt = oracle.partition_counts(len(I), r, gamma)
    assert (len(R), len(C), len(P)) == (cnt["n_R"], cnt["n_C"], cnt["n_P"])
    allc = np.concatenate([R, C, P])
    assert np.array_equal(np.sort(allc), np.arange(len(I)))          # disjoint and covering
    for a in (R, C, P):
        assert np.all(np.diff(a) > 0)                                  # ascending
    # importance order between regions; at equal importance the higher index
    # is the less important channel
    key = lambda i: (I[i], -i)
    if len(P) and len(C):
        assert max(map(key, P)) < min(map(key, C))
    if len(C) and len(R):
        assert max(map(key, C)) < min(map(key, R))
    if len(P) and len(R):
        assert max(map(key, P)) < min(map(key, R))
    # the same sets as the full-sort formulation
    for a, b in zip((R, C, P), oracle.partition_by_sort(I, r, gamma)):
        assert np.array_equal(a, b)
    # and the library's check accepts them
    pop.pop_check_lists(R, C, len(I), P)


@SETTINGS
@given(st.integers(0, 200), st.integers(0, 2**32 - 1), st.data())
def test_selection_invariants(n_C, seed, data):
    g = np.random.default_rng(seed)
    C = np.sort(g.choice(1000, n_C, replace=False)) if n_C else np.zeros(0, np.int64)
    scores = g.integers(0, 5, n_C).astype(np.float64) if data.draw(st.booleans()) else g.random(n_C)
    k = data.draw(st.integers(0, n_C))
    S = oracle.select_candidates(C, scores, k)
    assert len(S) == k and np.all(np.diff(S) > 0) and np.isin(S, C).all()
    sel = np.isin(C, S)
    if 0 < k < n_C:
        # nothing left out beats anything kept; at equal score the lower index wins
        kept = [(scores[j], -C[j]) for j in np.flatnonzero(sel)]
        left = [(scores[j], -C[j]) for j in np.flatnonzero(~sel)]
        assert min(kept) > max(left)


def _python_check(lists, d_ff):
    """A plain restatement of what pop_check_lists accepts."""
    seen = set()
    for a in lists:
        for i, c in enumerate(a):
            if not (0 <= c < d_ff) or (i and c <= a[i - 1]) or c in seen:
                return False
            seen.add(c)
    return sum(map(len, lists)) <= d_ff


@st.composite
def list_triples(draw):
    d_ff = draw(st.integers(1, 64))
    owner = draw(st.lists(st.integers(-1, 2), min_size=d_ff, max_size=d_ff))
    lists = [[c for c in range(d_ff) if owner[c] == l] for l in range(3)]
    mutation = draw(st.sampled_from(["none", "swap", "dup", "cross", "low", "high"]))
    l = draw(st.integers(0, 2))
    a = lists[l]
    if mutation == "swap" and len(a) >= 2:
        i = draw(st.integers(0, len(a) - 2))
        a[i], a[i + 1] = a[i + 1], a[i]
    elif mutation == "dup" and a:
        i = draw(st.integers(0, len(a) - 1))
        a.insert(i, a[i])
    elif mutation == "cross" and a:
        other = lists[(l + 1) % 3]
        c = draw(st.sampled_from(a))
        other.append(c)
        other.sort()
    elif mutation == "low":
        a.insert(0, -draw(st.integers(1, 5)))
    elif mutation == "high":
        a.append(d_ff + draw(st.integers(0, 5)))
    return lists, d_ff


@SETTINGS
@given(list_triples())
def test_check_lists_matches_python(case):
    lists, d_ff = case
    expect = _python_check(lists, d_ff)
    if expect:
        pop.pop_check_lists(lists[0], lists[1], d_ff, lists[2])
    else:
        with pytest.raises(pop.PopError) as e:
            pop.pop_check_lists(lists[0], lists[1], d_ff, lists[2])
        assert e.value.status == INVALID


def test_check_lists_errors():
    with pytest.raises(pop.PopError) as e:
        pop.pop_check_lists([0], [], 0)
    assert e.value.status == SHAPE
    with pytest.raises(pop.PopError) as e:
        pop.pop_check_lists([0, 1], [2], 2)
    assert e.value.status == INVALID and "inconsistent" in str(e.value)
    with pytest.raises(pop.PopError) as e:
        pop.pop_check_lists([3, 1], [], 8)
    assert "R[1] = 1" in str(e.value)
    with pytest.raises(pop.PopError) as e:
        pop.pop_check_lists([1, 3], [3], 8)
    assert "channel 3 is in R and C" in str(e.value)
    # a NULL list with a nonzero count, through the raw entry point
    assert pop.lib.pop_check_lists(None, 2, None, 0, None, 0, 8) == INVALID
    assert pop.lib.pop_check_lists(None, 0, None, 0, None, 0, 8) == OK
