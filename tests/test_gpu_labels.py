"""GPU parity of the golden-label construction (fm_golden_labels) against the fp64 oracle.

The membership decision compares a cumulative softmax mass with p.  The GPU sums masses in
2^-44 fixed point (exact integer sums of rounded float32 exponentials), so its cumulative mass
ratios agree with the oracle's to within 3e-6 in the worst case; entries whose oracle
cumulative mass lies within BAND = 1e-5 of p are "band" entries and may go either way.  Everything downstream is compared exactly
where no band entry can change it: a golden decision is certain when the certain votes alone
reach min_votes or cannot reach it with every band vote; a label (and its score) is certain
when every token of its window is certain for it.  With equal scores (no rounding in the
order) and in the cases below without band entries, the comparison is exact everywhere.
"""
import numpy as np
import pytest
import torch

from oracle import labels as OL
from tests import gpu_util as G
from top_selection_fm_amd import api
from top_selection_fm_amd import workloads as W

pytestmark = pytest.mark.gpu

BAND = 1e-5


def gpu_labels(S, n_valid, p=0.6, min_votes=3, tau=64, cap=None, with_score=True):
    T, L, ld = S.shape
    dev = "cuda:0"
    St = torch.from_numpy(np.ascontiguousarray(S, np.float32)).to(dev)
    nv = None if n_valid is None else torch.from_numpy(np.asarray(n_valid, np.int32)).to(dev)
    nb = api.fm_golden_workspace_bytes(T, L, ld, tau)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    ptr = torch.empty(T - tau + 2, dtype=torch.int32, device=dev)
    if cap is None:   # count first, then write
        api.fm_golden_labels(St, ld, T, L, nv, p, min_votes, tau, ptr, None, None, 0, ws, nb)
        cap = int(ptr[-1].item())
    idx = torch.full((max(cap, 1),), -7, dtype=torch.int32, device=dev)
    sc = torch.full((max(cap, 1),), -7.0, dtype=torch.float32, device=dev) if with_score else None
    api.fm_golden_labels(St, ld, T, L, nv, p, min_votes, tau, ptr, idx, sc, cap, ws, nb)
    torch.cuda.synchronize()
    return (ptr.cpu().numpy().astype(np.int64), idx.cpu().numpy()[:cap],
            None if sc is None else sc.cpu().numpy()[:cap])


def oracle_with_band(S, n_valid, p):
    """Oracle membership M and band flags B, both [T, L, ld] bool."""
    T, L, ld = S.shape
    M = np.zeros((T, L, ld), bool)
    B = np.zeros((T, L, ld), bool)
    for i in range(T):
        nv = ld if n_valid is None else int(n_valid[i])
        for l in range(L):
            order, c = OL.cumulative_mass(S[i, l], nv)
            M[i, l, OL.nucleus(S[i, l], nv, p)] = True
            B[i, l, order[np.abs(c - p) <= BAND]] = True
    return M, B


def check_labels(tag, S, n_valid, p, min_votes, tau, got):
    ptr, idx, sc = got
    T, L, ld = S.shape
    M, B = oracle_with_band(S, n_valid, p)
    # the oracle proper, for the record and the exact case
    rptr, ridx, rsc = OL.golden_labels(S, n_valid, p, min_votes, tau)
    vc = (M & ~B).sum(1)
    nband = B.sum(1)
    a_true = vc >= min_votes
    a_false = vc + nband < min_votes
    a_unc = ~(a_true | a_false)
    assert ptr.shape[0] == T - tau + 2 and ptr[0] == 0
    uncertain = 0
    for t in range(T - tau + 1):
        ys = idx[ptr[t]:ptr[t + 1]]
        assert np.all(np.diff(ys) > 0), f"{tag} window {t}: not ascending"
        assert ys.size == 0 or (ys.min() >= 0 and ys.max() < ld)
        yset = np.zeros(ld, bool)
        yset[ys] = True
        win_true = a_true[t:t + tau].any(0)
        win_false = a_false[t:t + tau].all(0)
        sure = ~a_unc[t:t + tau].any(0)
        uncertain += int((~sure).sum())
        assert np.all(yset[win_true]), f"{tag} window {t}: a certain label is missing"
        assert not np.any(yset[win_false]), f"{tag} window {t}: a certain non-label is present"
        if sc is not None:
            hits = a_true[t:t + tau].sum(0)
            ok = sure[ys]
            np.testing.assert_array_equal(sc[ptr[t]:ptr[t + 1]][ok], (hits[ys][ok] / tau).astype(np.float32),
                                          err_msg=f"{tag} window {t}: scores")
    if uncertain == 0:
        assert np.array_equal(ptr, rptr) and np.array_equal(idx, ridx)
        if sc is not None:
            assert np.array_equal(sc, rsc.astype(np.float32))
    G.note(tag, windows=T - tau + 1, labels=int(ptr[-1]), band_entries=int(B.sum()),
           uncertain_labels=uncertain)
    return rptr


def test_labels_small_ragged():
    rng = np.random.default_rng(31)
    T, L, ld = 20, 5, 1000
    S = (rng.standard_normal((T, L, ld)) * 1.5).astype(np.float32)
    S[:, :, rng.choice(ld, 30, replace=False)] += 4.0
    n_valid = rng.integers(0, ld + 1, T).astype(np.int32)
    n_valid[3] = 0                                   # a token with no candidate
    S[5, 2, ::2] = -np.inf                          # non-candidates inside a row
    got = gpu_labels(S, n_valid, p=0.6, min_votes=2, tau=4)
    check_labels("labels small ragged", S, n_valid, 0.6, 2, 4, got)


@pytest.mark.parametrize("p", [0.6, 0.3, 1.0])
def test_labels_nucleus_alone(p):
    """One layer, one vote, a window of one token: the labels of window t are the nucleus of
    token t itself, so this checks every membership bit (outside the band)."""
    rng = np.random.default_rng(32)
    T, ld = 9, 5000
    S = (rng.standard_normal((T, 1, ld)) * rng.uniform(0.5, 4, (T, 1, 1))).astype(np.float32)
    got = gpu_labels(S, None, p=p, min_votes=1, tau=1)
    check_labels(f"nucleus alone p={p}", S, None, p, 1, 1, got)


def test_labels_ties_split_by_index():
    """Equal scores: every mass is equal, the nucleus is the lowest floor(p n) entries; the
    boundary score's entries are split by entry index (the boundary-rank path)."""
    T, L, ld = 4, 3, 3000
    S = np.zeros((T, L, ld), np.float32)
    S[1] = 1.5
    S[2, :, 100:] = -np.inf                          # 100 equal candidates
    S[3, :, :] = np.float32(-2.0)
    S[3, :, 7:3000:5] = np.float32(-2.5)
    got = gpu_labels(S, None, p=0.55, min_votes=3, tau=1)
    rptr = check_labels("ties", S, None, 0.55, 3, 1, got)
    ptr, idx, _ = got
    assert idx[ptr[0]:ptr[1]].tolist() == list(range(int(np.floor(0.55 * ld))))
    assert idx[ptr[2]:ptr[3]].tolist() == list(range(55))


@pytest.mark.parametrize("p", [0.3, 0.5, 0.7])
def test_labels_ties_in_small_boundary_bin(p):
    """Ten equal scores carry most of each row's mass and the boundary falls among them, with
    few scores in their bin: the boundary is resolved by one wave comparing the gathered scores
    pairwise, and the tied entries are split by entry index (floor(p Z / w) of them)."""
    rng = np.random.default_rng(34)
    T, ld = 6, 4096
    S = rng.standard_normal((T, 1, ld)).astype(np.float32)
    for t in range(T):
        S[t, 0, rng.choice(ld, 10, replace=False)] = np.float32(8.0)
    got = gpu_labels(S, None, p=p, min_votes=1, tau=1)
    check_labels(f"ties in a small bin p={p}", S, None, p, 1, 1, got)


def test_labels_far_from_zero():
    """Scores near +-10,000 (the boundary-bin gather compares every entry exactly there) and a
    row whose whole mass sits on one entry (an empty nucleus for p below 1)."""
    rng = np.random.default_rng(35)
    T, L, ld = 4, 2, 3000
    S = (rng.standard_normal((T, L, ld)) * 2).astype(np.float32)
    S[0] += np.float32(10000.0)
    S[1] -= np.float32(10000.0)
    S[2, :, 17] = np.float32(60.0)
    got = gpu_labels(S, None, p=0.6, min_votes=1, tau=1)
    check_labels("far from zero", S, None, 0.6, 1, 1, got)


def test_labels_boundary_bin_overflow():
    """More than 4,096 candidates share the boundary's score bin (here: equal scores), so the
    radix search reads the row again from memory instead of the gathered list."""
    T, L, ld = 3, 3, 20000
    S = np.zeros((T, L, ld), np.float32)
    S[1, :, ::2] = -1.0                             # two levels: 10,000 entries at each
    S[2] = (np.arange(ld) % 7).astype(np.float32) * np.float32(0.001)   # 7 close levels
    got = gpu_labels(S, None, p=0.55, min_votes=3, tau=1)
    check_labels("boundary bin overflow", S, None, 0.55, 3, 1, got)
    ptr, idx, _ = got
    assert idx[ptr[0]:ptr[1]].tolist() == list(range(11000))


@pytest.mark.timeout(300)
def test_labels_page_shapes():
    """The benchmarked call: 128 future tokens x 21 layers x 65,536 entries (256K context at
    4:1), p = 0.6, 3 votes, tau = 64 (65 windows), on the same seeded scores, against the
    oracle; a repeat call is bit-identical."""
    g = W.selector_scores()
    got = gpu_labels(g.scores, g.n_valid)
    check_labels("labels 128 x 21 x 65536", g.scores, g.n_valid, 0.6, 3, 64, got)
    again = gpu_labels(g.scores, g.n_valid)
    for a, b in zip(got, again):
        assert np.array_equal(a, b)


def test_labels_cap_and_count_only():
    rng = np.random.default_rng(33)
    T, L, ld = 10, 4, 700
    S = (rng.standard_normal((T, L, ld)) * 2).astype(np.float32)
    full = gpu_labels(S, None, p=0.6, min_votes=2, tau=3)
    total = int(full[0][-1])
    assert total > 10
    cap = total // 2
    ptr, idx, sc = gpu_labels(S, None, p=0.6, min_votes=2, tau=3, cap=cap)
    assert np.array_equal(ptr, full[0])                     # pointers always in full
    assert np.array_equal(idx, full[1][:cap]) and np.array_equal(sc, full[2][:cap])
    ptr2, idx2, sc2 = gpu_labels(S, None, p=0.6, min_votes=2, tau=3, cap=total, with_score=False)
    assert np.array_equal(idx2, full[1]) and sc2 is None


@pytest.mark.parametrize("T,L,ld,tau,min_votes", [(1, 1, 1, 1, 1), (3, 2, 31, 3, 1), (5, 4, 33, 2, 2),
                                                  (6, 3, 257, 6, 3), (4, 64, 100, 2, 40)])
def test_labels_small_shapes(T, L, ld, tau, min_votes):
    """Word and chunk edges (ld 1, 31, 33, 257), one window (tau = T), 64 layers."""
    rng = np.random.default_rng(T * 1000 + ld)
    S = (rng.standard_normal((T, L, ld)) * 2).astype(np.float32)
    got = gpu_labels(S, None, p=0.6, min_votes=min_votes, tau=tau)
    check_labels(f"labels T={T} L={L} ld={ld}", S, None, 0.6, min_votes, tau, got)
