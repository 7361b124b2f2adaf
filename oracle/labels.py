"""fp64 oracle of the retriever's golden-label construction (training-side labels).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP library.

What it computes follows the FlashMemory-DeepSeek-V4 paper summary, section 4 (label
construction from the future native selector's attention), step by step in the page's order:

    P[i,l,s]  = exp(S[i,l,s]) / sum_j exp(S[i,l,j])          softmax over token i's candidates
    M[i,l]    = the prefix of the candidates sorted by P descending whose cumulative mass is at
                most p (p = 0.6 on the page)
    V[i,s]    = sum_l [s in M[i,l]]                            votes across layers
    A[i]      = {s : V[i,s] >= 3}                              golden chunks of token i
    Y[t]      = union of A[i] for i = t .. t + tau - 1         labels of time t (tau = 64)

Readings where the page leaves a step open (each also listed in the design notes):
  * candidates of token i are the entries s < n_valid[i] whose score is not -inf (or NaN);
  * "sorted" breaks ties (equal scores, hence equal P) by the lower entry index first;
  * "at most p" is inclusive and literal: the element whose inclusion would take the cumulative
    mass above p is not a member, so a token whose largest P exceeds p has an empty nucleus;
  * labels are emitted for the windows that lie wholly inside the given tokens,
    t = 0 .. T - tau, in the CSR layout the page's training data uses (pointers, ascending
    indices, scores);
  * the page does not define the label score; the score of s in Y[t] is the fraction of the
    window's tau tokens whose golden set holds s.
"""
from __future__ import annotations

import numpy as np


def _ordered_mass(scores, n_valid):
    x = np.asarray(scores, np.float64)
    n = x.shape[0] if n_valid is None else int(n_valid)
    cand = np.arange(n)[~np.isnan(x[:n]) & ~np.isneginf(x[:n])]
    if cand.size == 0:
        return cand, np.zeros(0)
    xc = x[cand]
    order = np.lexsort((cand, -xc))           # score descending, then lower index
    e = np.exp(xc[order] - xc.max())          # P up to the common factor 1 / sum
    return cand[order], np.cumsum(e)


def cumulative_mass(scores, n_valid: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Token i's candidates in nucleus order (score descending, then lower index) and their
    inclusive cumulative softmax mass, fp64 (the last one exactly 1).  Scores are finite or
    -inf (NaN counts as -inf)."""
    order, C = _ordered_mass(scores, n_valid)
    return order, (C / C[-1] if C.size else C)


def nucleus(scores, n_valid: int | None = None, p: float = 0.6) -> np.ndarray:
    """Member indices (ascending) of the top-p nucleus of one row of scores: the sorted prefix
    whose cumulative mass is at most p.  The mass is compared unnormalised, C_k <= p * C_n, so
    that p = 1 takes every candidate exactly; C only grows along the order, so the members form
    a prefix."""
    order, C = _ordered_mass(scores, n_valid)
    if C.size == 0:
        return order
    return np.sort(order[C <= p * C[-1]])


def golden_sets(S, n_valid=None, p: float = 0.6, min_votes: int = 3):
    """Membership M [T, L, ld] (bool), votes V [T, ld] and golden sets A [T, ld] (bool)."""
    S = np.asarray(S, np.float64)
    T, L, ld = S.shape
    M = np.zeros((T, L, ld), bool)
    for i in range(T):
        nv = ld if n_valid is None else int(n_valid[i])
        for l in range(L):
            M[i, l, nucleus(S[i, l], nv, p)] = True
    V = M.sum(axis=1)
    return M, V, V >= min_votes


def golden_labels(S, n_valid=None, p: float = 0.6, min_votes: int = 3, tau: int = 64):
    """CSR labels of the windows t = 0 .. T - tau: (label_ptr [T - tau + 2], label_idx, label_score)."""
    S = np.asarray(S, np.float64)
    T = S.shape[0]
    _, _, A = golden_sets(S, n_valid, p, min_votes)
    ptr, idx, score = [0], [], []
    for t in range(T - tau + 1):
        hits = A[t:t + tau].sum(axis=0)
        ys = np.nonzero(hits)[0]
        idx.append(ys)
        score.append(hits[ys] / tau)
        ptr.append(ptr[-1] + ys.size)
    cat = (lambda a, dt: np.concatenate(a).astype(dt) if a else np.zeros(0, dt))
    return np.asarray(ptr, np.int64), cat(idx, np.int64), cat(score, np.float64)
