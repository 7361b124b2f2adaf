"""Pins of the golden-label oracle (oracle/labels.py) against what the mathematics fixes:
a worked example by hand, exact rational arithmetic, closed forms, invariances and a
brute-force construction with plain Python sets.  CPU only.
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import labels as OL


def test_worked_example():
    # P = (0.5, 0.3, 0.2): cumulative 0.5, 0.8, 1.0
    s = np.log([0.5, 0.3, 0.2])
    assert OL.nucleus(s, p=0.6).tolist() == [0]
    assert OL.nucleus(s, p=0.85).tolist() == [0, 1]
    assert OL.nucleus(s, p=0.45).tolist() == []          # the largest P alone exceeds p
    assert OL.nucleus(s[::-1], p=0.85).tolist() == [1, 2]  # order follows the score
    # "at most p" is inclusive: equal scores, masses 1/4 each, p = 1/2 exactly (binary exact)
    assert OL.nucleus(np.zeros(4), p=0.5).tolist() == [0, 1]
    assert OL.nucleus(np.zeros(2), p=0.5).tolist() == [0]


def _exact_nucleus(weights, p):
    """Members by exact rationals: P_j = a_j / sum(a), sorted by (a desc, j asc)."""
    tot = sum(weights)
    order = sorted(range(len(weights)), key=lambda j: (-weights[j], j))
    out, c = [], Fraction(0)
    for j in order:
        c += Fraction(weights[j], tot)
        if c <= p:
            out.append(j)
    return sorted(out), order


def test_exact_rationals():
    rng = random.Random(11)
    checked = 0
    for trial in range(300):
        n = rng.randint(1, 40)
        a = [rng.randint(1, 20) for _ in range(n)]
        p = Fraction(rng.randint(1, 99), 100)
        ref, order = _exact_nucleus(a, p)
        # skip draws whose exact cumulative mass lands within 1e-12 of p (fp64 may round across)
        tot, c, near = sum(a), Fraction(0), False
        for j in order:
            c += Fraction(a[j], tot)
            near |= abs(float(c - p)) < 1e-12
        if near:
            continue
        got = OL.nucleus(np.log(np.asarray(a, np.float64)), p=float(p))
        assert got.tolist() == ref, (a, p)
        checked += 1
    assert checked > 250



def test_cumulative_mass_matches_exact_rationals():
    """cumulative_mass (which sets the decision band of the GPU label checks) against exact
    fractions: scores log(a_j) with integer a_j give P_j = a_j / sum(a), so the order is
    (a descending, index ascending) and the k-th inclusive mass is sum of the first k a over
    sum(a).  Entries at or past n_valid and -inf / NaN scores are not candidates."""
    rng = random.Random(5)
    for trial in range(200):
        n = rng.randint(1, 60)
        a = [rng.randint(1, 30) for _ in range(n)]
        x = np.log(np.asarray(a, np.float64))
        n_valid = rng.randint(1, n)
        excl = set(rng.sample(range(n_valid), rng.randint(0, n_valid - 1)))
        for j in excl:
            x[j] = -np.inf if j % 2 else np.nan
        cand = [j for j in range(n_valid) if j not in excl]
        tot = sum(a[j] for j in cand)
        order = sorted(cand, key=lambda j: (-a[j], j))
        got_order, got_c = OL.cumulative_mass(x, n_valid)
        assert got_order.tolist() == order
        c = Fraction(0)
        for j, g in zip(order, got_c):
            c += Fraction(a[j], tot)
            assert abs(g - float(c)) <= 1e-14, (a, j)
        assert got_c[-1] == 1.0
    o, c = OL.cumulative_mass(np.full(4, -np.inf))
    assert o.size == 0 and c.size == 0


def test_uniform_scores_closed_form():
    # equal scores: equal masses 1/n, ties to the lower index, so the nucleus is the first
    # floor(p n) entries (cases with p n an integer are left out: rounding decides those)
    for n in (1, 7, 100, 4096):
        for p in (0.05, 0.33, 0.6, 0.97):
            if abs(p * n - round(p * n)) < 1e-6:
                continue
            got = OL.nucleus(np.full(n, 2.5), p=p)
            assert got.tolist() == list(range(int(math.floor(p * n))))


def test_invariances_and_edges():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(500) * 3
    base = OL.nucleus(x, p=0.6)
    assert np.array_equal(OL.nucleus(x + 17.25, p=0.6), base)        # softmax shift
    prev = np.array([], np.int64)
    for p in (0.1, 0.3, 0.6, 0.9, 0.999):                              # monotone in p
        cur = OL.nucleus(x, p=p)
        assert set(prev.tolist()) <= set(cur.tolist())
        prev = cur
    assert OL.nucleus(x, p=1.0).tolist() == list(range(500))          # p = 1: everything
    y = x.copy()
    y[::3] = -np.inf                                                    # never candidates
    assert not set(OL.nucleus(y, p=0.9).tolist()) & set(range(0, 500, 3))
    assert OL.nucleus(x, n_valid=200, p=0.9).max() < 200               # past n_valid: none
    assert OL.nucleus(np.full(5, -np.inf), p=0.9).size == 0
    # members are the top of the order: every member scores at least every non-member
    m = OL.nucleus(x, p=0.6)
    out = np.setdiff1d(np.arange(500), m)
    assert x[m].min() >= x[out].max()


def _brute_labels(S, n_valid, p, min_votes, tau):
    """Plain-Python construction: per-token sets, vote dictionaries, set unions."""
    T, L, ld = S.shape
    golden = []
    for i in range(T):
        votes = {}
        for l in range(L):
            row = [float(v) for v in S[i, l, :n_valid[i]]]
            cand = [j for j, v in enumerate(row) if v != -math.inf]
            if not cand:
                continue
            m = max(row[j] for j in cand)
            w = {j: math.exp(row[j] - m) for j in cand}
            tot = math.fsum(w.values())
            c = 0.0
            for j in sorted(cand, key=lambda j: (-row[j], j)):
                c += w[j] / tot
                if c > p + 1e-12:
                    break
                votes[j] = votes.get(j, 0) + 1
        golden.append({j for j, v in votes.items() if v >= min_votes})
    out = []
    for t in range(T - tau + 1):
        ys = set().union(*golden[t:t + tau])
        out.append({j: sum(j in golden[i] for i in range(t, t + tau)) / tau for j in ys})
    return out


@pytest.mark.parametrize("tau,min_votes", [(1, 1), (3, 2), (5, 3)])
def test_labels_against_brute_force(tau, min_votes):
    rng = np.random.default_rng(tau * 10 + min_votes)
    T, L, ld = 9, 4, 40
    S = rng.standard_normal((T, L, ld)) * 2
    hot = rng.choice(ld, 6, replace=False)
    S[:, :, hot] += 4.0
    n_valid = rng.integers(ld // 2, ld + 1, T)
    ptr, idx, score = OL.golden_labels(S, n_valid, p=0.6, min_votes=min_votes, tau=tau)
    ref = _brute_labels(S, n_valid, 0.6, min_votes, tau)
    assert ptr.size == T - tau + 2 and ptr[0] == 0
    for t, r in enumerate(ref):
        got = dict(zip(idx[ptr[t]:ptr[t + 1]].tolist(), score[ptr[t]:ptr[t + 1]].tolist()))
        assert got == r
        assert np.all(np.diff(idx[ptr[t]:ptr[t + 1]]) > 0)             # ascending


def test_window_union_grows_with_tau():
    rng = np.random.default_rng(5)
    S = rng.standard_normal((12, 5, 64)) * 3
    prev = None
    for tau in (1, 2, 4, 8):
        ptr, idx, _ = OL.golden_labels(S, p=0.6, min_votes=2, tau=tau)
        y0 = set(idx[ptr[0]:ptr[1]].tolist())
        if prev is not None:
            assert prev <= y0
        prev = y0


def test_single_layer_single_vote_is_the_nucleus():
    rng = np.random.default_rng(8)
    S = rng.standard_normal((4, 1, 100)) * 2.5
    ptr, idx, score = OL.golden_labels(S, p=0.6, min_votes=1, tau=1)
    for t in range(4):
        assert idx[ptr[t]:ptr[t + 1]].tolist() == OL.nucleus(S[t, 0], p=0.6).tolist()
        assert np.all(score[ptr[t]:ptr[t + 1]] == 1.0)
