"""Property tests of the oracle on generated tiny cases (hypothesis): top-k
against subset enumeration with injected ties, and the dispatch's
invariants (capacity, packing, rank-major order, greedy drops) for every
overflow policy. These pin the oracle, not the GPU path."""
import itertools

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=200, deadline=None)


def _brute_topc(key, C):
    """Ordered top-C by (key desc, index asc): the chosen set dominates its
    complement under that order, found by enumerating subsets."""
    E = len(key)
    better = lambda a, b: key[a] > key[b] or (key[a] == key[b] and a < b)
    for S in itertools.combinations(range(E), C):
        rest = [e for e in range(E) if e not in S]
        if all(better(a, b) for a in S for b in rest):
            return sorted(S, key=lambda a: (-float(key[a]), a))
    raise AssertionError("no dominant subset")


@st.composite
def routing_case(draw):
    E = draw(st.integers(1, 6))
    k = draw(st.integers(1, min(3, E)))
    C = k + draw(st.integers(0, 1 if k < E else 0))
    N = draw(st.integers(1, 8))
    vals = st.sampled_from([-1.0, 0.0, 0.5, 2.0])  # few values: many ties
    l = np.array(draw(st.lists(st.lists(vals, min_size=E, max_size=E), min_size=N, max_size=N)),
                 np.float32)
    bias = None
    if draw(st.booleans()):
        bias = np.array(draw(st.lists(st.sampled_from([0.0, -0.0, 0.25]), min_size=E,
                                      max_size=E)), np.float32)
    return l, k, C, draw(st.booleans()), bias


@SETTINGS
@given(routing_case())
def test_topk_is_the_dominant_subset(case):
    l, k, C, renorm, bias = case
    r = oracle.route(l, k, C, renorm, bias)
    for t in range(l.shape[0]):
        key = r["s"][t] + bias if bias is not None else r["s"][t]
        assert list(r["cand_ids"][t]) == _brute_topc(key.astype(np.float32), C)
        if renorm:
            assert abs(float(np.sum(r["gates"][t].astype(np.float64))) - 1.0) < 1e-6


@st.composite
def dispatch_case(draw):
    policy = draw(st.sampled_from([oracle.DROPLESS, oracle.DROP, oracle.REROUTE]))
    E = draw(st.integers(2, 6))
    k = 1 if policy == oracle.REROUTE else draw(st.integers(1, min(3, E)))
    C = 2 if policy == oracle.REROUTE else k
    N = draw(st.integers(1, 12))
    cand = np.array([draw(st.permutations(list(range(E))))[:C] for _ in range(N)], np.int32)
    cap = -1 if policy == oracle.DROPLESS else draw(st.integers(1, max(1, N * k // E + 1)))
    return cand, E, k, policy, cap


@SETTINGS
@given(dispatch_case())
def test_dispatch_invariants(case):
    cand, E, k, policy, cap = case
    N, C = cand.shape
    cs = np.linspace(0.9, 0.1, C, dtype=np.float32)[None, :].repeat(N, 0)
    gates = cs[:, :k].copy()
    d = oracle.dispatch(cand, cs, gates, E, k, policy, cap)
    row_of, exp_of, kept = d["row_of"], d["expert_of"], d["counts_kept"]
    offs = d["offsets"]
    assert offs[0] == 0 and np.array_equal(np.diff(offs), kept) and d["R"] == offs[-1]
    assert int((row_of >= 0).sum()) == int(kept.sum())
    if policy == oracle.DROPLESS:
        assert (row_of >= 0).all() and np.array_equal(kept, d["counts_routed"])
    else:
        assert (kept <= cap).all()
    # packing: row r of expert e holds a kept assignment of e; perm inverts row_of
    rank = {}  # row -> (slot j, token t, candidate index used)
    for t in range(N):
        for j in range(k):
            r = row_of[t, j]
            if r < 0:
                continue
            e = exp_of[t, j]
            assert offs[e] <= r < offs[e + 1] and d["perm_token"][r] == t
            used = list(cand[t]).index(e)
            assert used == j or (policy == oracle.REROUTE and used == 1)
            # rank-major: slot j of every token before slot j + 1; a reroute's
            # second phase comes after every first choice
            rank[r] = (used, t) if policy == oracle.REROUTE else (j, t)
            if used == 1 and policy == oracle.REROUTE:
                assert kept[cand[t, 0]] == cap  # rerouted only off a full expert
    # within an expert, rows in rank-major order (all first choices, then second ...)
    for e in range(E):
        keys = [rank[r] for r in range(offs[e], offs[e + 1])]
        assert keys == sorted(keys)
    # greedy: a dropped first choice means its expert filled up with assignments
    # that come earlier in rank-major order
    for t in range(N):
        for j in range(k):
            if policy == oracle.DROP and row_of[t, j] < 0:
                e = cand[t, j]
                assert kept[e] == cap
                assert all(rank[r] < (j, t) for r in range(offs[e], offs[e + 1]))
            if policy == oracle.REROUTE and row_of[t, 0] < 0:
                # dropped after trying both candidates: both experts full
                assert kept[cand[t, 0]] == cap and kept[cand[t, 1]] == cap
