"""Pins for the fp64 oracle: each test checks it against something other than itself.

Sources of truth used here: torch's float8_e4m3fn / bfloat16 decoders and the OCP FP8 spec
table (element decoding); exact-rational brute force (logits); closed forms (rank-1 keys,
sigmoid threshold); numpy.matmul, numpy.lexsort and reshape/any (special cases and
selection); invariants the definitions imply (head permutation, positive rescaling,
threshold monotonicity, union = max of sigmoids, two-level = masked top-k).
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from tests import exact_ref
from top_selection_fm_amd import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers
def tiny_wl(seed=0, T=2, H=4, D=8, n_entries=40, page=8, key_dtype="f32", q_dtype="f32",
            w_dtype="f32", B=None, permute=True, q_pos=None, ratio=4, w_mean=0.0):
    """Small arbitrary-shape workload (heads, dims and page size free)."""
    rng = np.random.default_rng(seed)
    B = T if B is None else B
    ppr = -(-n_entries // page)
    n_phys = B * ppr
    bt = (rng.permutation(n_phys) if permute else np.arange(n_phys)).astype(np.int32)
    bt = bt.reshape(B, ppr)
    k32 = rng.standard_normal((n_phys, page, D)).astype(np.float32) / np.float32(np.sqrt(D))
    if key_dtype == "f32":
        pool = k32
    elif key_dtype == "bf16":
        pool = W.bf16_bits(k32)
    else:
        rows = np.empty((n_phys, page, D + 4), np.uint8)
        absmax = np.abs(k32).max(-1)
        sc = (absmax / 448.0).astype("<f4")
        rows[..., :D] = W.e4m3_codes(k32 / sc[..., None])
        rows[..., D:] = sc[..., None].view(np.uint8)
        pool = rows
    q32 = rng.standard_normal((T, H, D)).astype(np.float32) / np.float32(np.sqrt(D))
    q_scale = None
    if q_dtype == "f32":
        q = q32
    elif q_dtype == "bf16":
        q = W.bf16_bits(q32)
    else:
        am = np.abs(q32.reshape(T, -1)).max(1)
        q_scale = (am / 448.0).astype(np.float32)
        q = W.e4m3_codes(q32 / q_scale[:, None, None])
    w32 = (rng.standard_normal((T, H)) * 0.125 + w_mean).astype(np.float32)
    w = w32 if w_dtype == "f32" else W.bf16_bits(w32)
    seq = np.full(B, n_entries, np.int32)
    row_req = None if B == T else np.zeros(T, np.int32)
    kv = W.KeyPool([pool], "fp8x132" if key_dtype == "fp8" else key_dtype, bt, seq)
    qq = W.Queries(q, q_dtype, w, w_dtype, q_scale=q_scale, row_req=row_req,
                   q_pos=None if q_pos is None else np.asarray(q_pos, np.int32),
                   compress_ratio=ratio)
    return W.Workload("tiny", kv, [qq])


def rel_err(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


# ----------------------------------------------------------------------------- decoding
def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                     # S.1111.111 only
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_ocp_spec_points():
    for line in open(os.path.join(GOLD, "e4m3_ocp_points.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = oracle.decode_e4m3(np.array([int(code, 16)], np.uint8))[0]
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_bf16_codes_match_torch():
    rng = np.random.default_rng(7)
    bits = np.concatenate([rng.integers(0, 1 << 16, 4096), [0, 0x8000, 0x3F80, 0x7F7F, 0x0001,
                                                             0xFF7F, 0x8001]]).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # finite codes only
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))


# ----------------------------------------------------------------------------- logits
@pytest.mark.parametrize("key_dtype,q_dtype,w_dtype", [
    ("f32", "f32", "f32"), ("bf16", "bf16", "bf16"), ("fp8", "bf16", "bf16"),
    ("fp8", "fp8", "bf16")])
def test_logits_match_exact_rationals(key_dtype, q_dtype, w_dtype):
    wl = tiny_wl(seed=3, T=3, H=4, D=8, n_entries=21, page=8, key_dtype=key_dtype,
                 q_dtype=q_dtype, w_dtype=w_dtype)
    L = oracle.logits(wl)
    ex = exact_ref.logits_logical(wl)
    n = int(wl.kv.seq_lens[0])
    assert np.all(np.isneginf(L[:, n:]))
    for t in range(3):
        for s in range(n):
            want = float(ex[t][s])
            assert rel_err(L[t, s], want) <= 1e-12 or abs(L[t, s] - want) < 1e-300, (t, s)


def test_logits_match_exact_rationals_full_width_sample():
    """64 heads x 128 dims (the indexer's shape), a sample of the tiny fp32 workload."""
    wl = W.tiny_single_query(n_entries=96)
    L = oracle.logits(wl)
    ex = exact_ref.logits_logical(wl)
    for s in range(0, 96, 7):
        assert rel_err(L[0, s], float(ex[0][s])) <= 1e-12



@pytest.mark.parametrize("key_dtype,q_dtype", [("f32", "f32"), ("fp8", "bf16"), ("fp8", "fp8")])
def test_logits_at_points_match_exact_rationals(key_dtype, q_dtype):
    """logits_at (the point-wise oracle the sampled GPU checks use) against exact rationals at
    shuffled (row, entry) points: two requests shared by five rows through row_req, causal
    positions, an unmapped page (block table -1), a page past the block table, and entries that
    are negative, past seq_len or past the causal limit all give -inf; every other point is the
    exact logit.  A wrong row-to-request map, visibility test or entry-to-page mapping fails."""
    P, N = 8, 43                                    # 6 pages a request, the last one partial
    wl = tiny_wl(seed=21, T=5, B=2, H=4, D=8, n_entries=N, page=P, key_dtype=key_dtype,
                 q_dtype=q_dtype, q_pos=[9, 400, 120, 77, 173], ratio=4)
    rr = np.array([1, 0, 1, 0, 1], np.int32)
    wl.queries[0].row_req = rr
    wl.kv.block_table[0, 2] = -1                    # request 0, entries 16..23: unmapped
    wl.kv.seq_lens[1] = 40                          # request 1 is shorter than its pages
    ex = exact_ref.logits_logical(wl)               # None where the page is unmapped
    rng = np.random.default_rng(3)
    rows, ents, want = [], [], []
    for t in range(5):
        b = int(rr[t])
        n_vis = min(int(wl.kv.seq_lens[b]), int(wl.queries[0].q_pos[t]) // 4)
        for s in list(range(-2, 52)) + [P * wl.kv.block_table.shape[1] + 5, 10 ** 6]:
            rows.append(t)
            ents.append(s)
            ok = 0 <= s < n_vis and ex[t][s] is not None
            want.append(float(ex[t][s]) if ok else -np.inf)
    perm = rng.permutation(len(rows))
    rows, ents, want = (np.asarray(rows)[perm], np.asarray(ents)[perm], np.asarray(want)[perm])
    got = oracle.logits_at(wl, rows, ents)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(np.isneginf(got[~fin]))
    assert fin.sum() > 60 and (~fin).sum() > 60
    for g, x in zip(got[fin], want[fin]):
        assert rel_err(g, x) <= 1e-12 or abs(g - x) < 1e-300
    # and the same points read out of the full logit matrix
    L = oracle.logits(wl)
    inside = (ents >= 0) & (ents < L.shape[1])
    assert np.array_equal(got[inside], L[rows[inside], ents[inside]])


def test_rank_one_closed_form():
    """k_s = a_s u and q_h = b_h u with |u| = 1 give L_s = a_s * sum_{h: a_s b_h > 0} w_h b_h."""
    H, D, N = 6, 16, 24
    wl = tiny_wl(seed=1, T=1, H=H, D=D, n_entries=N, page=8, permute=False)
    u = np.zeros(D, np.float64)
    u[[1, 4, 9, 13]] = [0.5, -0.5, 0.5, 0.5]     # unit norm, exactly representable
    a = np.array([(-1) ** s * (s + 1) / 8.0 for s in range(N)])
    b = np.array([1.5, -0.75, 0.25, -2.0, 0.5, 1.0])
    w = np.array([0.3, -0.2, 0.7, 0.1, -0.4, 0.9])
    wl.kv.pools[0][:] = (a[:, None] * u[None, :]).reshape(N // 8, 8, D).astype(np.float32)
    wl.queries[0].q[:] = (b[:, None] * u[None, :])[None].astype(np.float32)
    wl.queries[0].w[:] = w[None].astype(np.float32)
    w32 = w.astype(np.float32).astype(np.float64)
    L = oracle.logits(wl)[0]
    for s in range(N):
        sel = (b > 0) if a[s] > 0 else (b < 0)
        want = a[s] * float(np.sum(w32[sel] * b[sel]))
        assert abs(L[s] - want) <= 1e-12 * max(1.0, abs(want)), s


def test_single_head_is_matmul():
    """n_h = 1, w = 1, non-negative q and k: L = K q (numpy.matmul)."""
    D, N = 12, 40
    wl = tiny_wl(seed=2, T=1, H=1, D=D, n_entries=N, page=8, permute=False)
    rng = np.random.default_rng(5)
    K = np.abs(rng.standard_normal((N, D))).astype(np.float32)
    q = np.abs(rng.standard_normal(D)).astype(np.float32)
    wl.kv.pools[0][:] = K.reshape(N // 8, 8, D)
    wl.queries[0].q[:] = q[None, None]
    wl.queries[0].w[:] = 1.0
    L = oracle.logits(wl)[0]
    ref = np.matmul(K.astype(np.float64), q.astype(np.float64))
    assert np.allclose(L, ref, rtol=1e-13, atol=0)


def test_block_table_permutation_invariance():
    a = tiny_wl(seed=9, T=2, n_entries=64, page=8, permute=False)
    b = tiny_wl(seed=9, T=2, n_entries=64, page=8, permute=False)
    rng = np.random.default_rng(1)
    perm = rng.permutation(b.kv.n_phys_pages)
    pool = np.empty_like(b.kv.pools[0])
    pool[perm] = a.kv.pools[0]                  # physical page perm[i] now holds page i
    b.kv.pools[0][:] = pool
    b.kv.block_table[:] = perm[a.kv.block_table]
    assert np.array_equal(oracle.logits(a), oracle.logits(b))


def test_head_permutation_and_positive_rescaling():
    wl = tiny_wl(seed=4, T=2, H=6, D=8, n_entries=48, page=8)
    L0 = oracle.logits(wl)
    p = np.random.default_rng(0).permutation(6)
    wl.queries[0].q[:] = wl.queries[0].q[:, p]
    wl.queries[0].w[:] = wl.queries[0].w[:, p]
    assert np.allclose(oracle.logits(wl), L0, rtol=1e-13, atol=1e-15)
    wl.queries[0].w[:] *= np.float32(4.0)       # exact power-of-two rescale
    L4 = oracle.logits(wl)
    assert np.allclose(L4, 4.0 * L0, rtol=1e-13, atol=1e-15)
    i0, _, _ = oracle.topk(L0[0], k=5)
    i4, _, _ = oracle.topk(L4[0], k=5)
    assert np.array_equal(i0, i4)


def test_head_sum_splits_into_head_groups():
    """The score is a sum over heads, so a 128-head row's logits are the sum of its two 64-head
    halves' (each scored alone); a dropped or double-counted head group fails it."""
    wl = tiny_wl(seed=9, T=2, H=128, D=128, n_entries=70, page=64, key_dtype="fp8",
                 q_dtype="bf16", w_dtype="f32")
    L = oracle.logits(wl)
    q, w = wl.queries[0].q, wl.queries[0].w
    halves = []
    for h0 in (0, 64):
        part = W.Workload("half", wl.kv, [W.Queries(np.ascontiguousarray(q[:, h0:h0 + 64]), "bf16",
                                                    np.ascontiguousarray(w[:, h0:h0 + 64]), "f32")])
        halves.append(oracle.logits(part))
    fin = np.isfinite(L)
    assert np.array_equal(fin, np.isfinite(halves[0]))
    assert np.allclose(L[fin], (halves[0] + halves[1])[fin], rtol=1e-12, atol=1e-14)


def test_fp8_scale_factors_out():
    """Doubling every per-entry scale doubles every logit (scales are positive)."""
    wl = tiny_wl(seed=6, T=2, H=4, D=8, n_entries=32, page=8, key_dtype="fp8", q_dtype="bf16",
                 w_dtype="bf16")
    L0 = oracle.logits(wl)
    sc = wl.kv.pools[0][..., 8:].copy().view("<f4") * np.float32(2.0)
    wl.kv.pools[0][..., 8:] = sc.view(np.uint8)
    assert np.allclose(oracle.logits(wl), 2.0 * L0, rtol=1e-13, atol=1e-15)


def test_causal_visibility():
    """Row at position p sees s < floor(p / ratio); nothing else."""
    pos = [0, 3, 4, 17, 40, 123]
    wl = tiny_wl(seed=8, T=6, B=1, n_entries=30, page=8, q_pos=pos, ratio=4)
    L = oracle.logits(wl)
    for t, p in enumerate(pos):
        nv = min(30, p // 4)
        assert oracle.n_visible(wl, t) == nv
        assert np.all(np.isfinite(L[t, :nv])) and np.all(np.isneginf(L[t, nv:]))


def test_prefill_last_entry_visible_to_none():
    """Positions 131072..135167 over 33,792 entries: entry 33,791 is never visible, and row i
    sees exactly 32,768 + floor(i / 4) entries."""
    T = 4096
    kv = W.KeyPool([np.zeros((528, 64, 132), np.uint8)], "fp8x132",
                   np.arange(528, dtype=np.int32)[None], np.array([33792], np.int32))
    q = W.Queries(np.zeros((T, 1, 128), np.uint8), "fp8", np.zeros((T, 1), np.float32), "f32",
                  q_scale=np.ones(T, np.float32), row_req=np.zeros(T, np.int32),
                  q_pos=(131072 + np.arange(T)).astype(np.int32))
    wl = W.Workload("causal", kv, [q])
    nv = np.array([oracle.n_visible(wl, t) for t in range(T)])
    assert np.array_equal(nv, 32768 + np.arange(T) // 4)
    assert nv.max() == 33791 and int((nv - 32768).sum() + 32768 * T) == 136312832


# ----------------------------------------------------------------------------- threshold / union
def _three_layer_small(seed=11):
    return W.three_layer_mask_fp8(seed=seed, B=2, seq_len=2048 + 37, ragged=True)


def test_threshold_is_sigmoid_half():
    wl = _three_layer_small()
    r = oracle.resident_mask(wl, layers=[0])
    L = oracle.logits(wl, layer=0)
    for b in range(2):
        n = int(wl.kv.seq_lens[b])
        assert np.array_equal(r["mask"][b, :n].astype(bool), expit(L[b, :n]) >= 0.5)
        assert not r["mask"][b, n:].any()


@pytest.mark.parametrize("p", [0.2, 0.5, 0.7, 0.9])
def test_threshold_general_p_is_sigmoid(p):
    wl = _three_layer_small(12)
    r = oracle.resident_mask(wl, threshold=p, layers=[1])
    L = oracle.logits(wl, layer=1)
    for b in range(2):
        n = int(wl.kv.seq_lens[b])
        s = expit(L[b, :n])
        far = np.abs(s - p) > 1e-12
        assert np.array_equal(r["mask"][b, :n].astype(bool)[far], (s >= p)[far])


def test_mask_monotone_in_threshold():
    wl = _three_layer_small(13)
    prev = None
    for p in [0.05, 0.3, 0.5, 0.51, 0.8, 0.99]:
        m = oracle.resident_mask(wl, threshold=p)["mask"].astype(bool)
        if prev is not None:
            assert np.all(m <= prev)
        prev = m


def test_union_is_or_of_layers_and_max_of_sigmoids():
    wl = _three_layer_small(14)
    r = oracle.resident_mask(wl)
    per = [oracle.resident_mask(wl, layers=[l])["mask"].astype(bool) for l in range(3)]
    assert np.array_equal(r["mask"].astype(bool), per[0] | per[1] | per[2])
    Ls = [oracle.logits(wl, layer=l) for l in range(3)]
    for b in range(2):
        n = int(wl.kv.seq_lens[b])
        smax = np.max([expit(L[b, :n]) for L in Ls], axis=0)
        assert np.array_equal(r["mask"][b, :n].astype(bool), smax >= 0.5)
        assert np.array_equal(r["union"][b, :n], np.max([L[b, :n] for L in Ls], axis=0))


def test_mean_union_is_mean_of_sigmoids():
    wl = _three_layer_small(15)
    r = oracle.resident_mask(wl, mode="mean", threshold=0.4)
    Ls = [oracle.logits(wl, layer=l) for l in range(3)]
    for b in range(2):
        n = int(wl.kv.seq_lens[b])
        mean = np.mean([expit(L[b, :n]) for L in Ls], axis=0)
        assert np.allclose(r["union"][b, :n], mean, rtol=1e-14, atol=1e-15)
        far = np.abs(mean - 0.4) > 1e-12
        assert np.array_equal(r["mask"][b, :n].astype(bool)[far], (mean >= 0.4)[far])


def test_sink_and_recent_forcing():
    wl = _three_layer_small(16)
    base = oracle.resident_mask(wl)["mask"].astype(bool)
    r = oracle.resident_mask(wl, n_sink=5, n_recent=70)["mask"].astype(bool)
    for b in range(2):
        n = int(wl.kv.seq_lens[b])
        forced = np.zeros(r.shape[1], bool)
        forced[:5] = True
        forced[n - 70:n] = True
        assert np.array_equal(r[b], base[b] | forced)


def test_pages_match_numpy():
    wl = _three_layer_small(17)
    r = oracle.resident_mask(wl)
    m = r["mask"].astype(bool)
    B, ld = m.shape
    dens = m.reshape(B, -1, 64).sum(-1)
    assert np.array_equal(r["page_density"], dens)
    for b in range(B):
        nz = np.nonzero(dens[b])[0]
        assert r["page_count"][b] == nz.size
        assert np.array_equal(r["page_list"][b, :nz.size], nz)
        assert np.all(r["page_list"][b, nz.size:] == -1)


# ----------------------------------------------------------------------------- top-k
def lexsort_topk(v, k, keep=None, index=None):
    idx = np.arange(v.size) if index is None else np.asarray(index)
    ok = np.isfinite(v) | (v == np.inf)
    if keep is not None:
        ok &= keep.astype(bool)
    cand_v, cand_i = v[ok], idx[ok]
    order = np.lexsort((cand_i, -cand_v))
    return np.sort(cand_i[order[:k]])


def test_topk_matches_lexsort_prefix():
    rng = np.random.default_rng(21)
    for trial in range(20):
        n = int(rng.integers(1, 3000))
        v = np.round(rng.standard_normal(n), int(rng.integers(0, 4)))   # many duplicates
        v[rng.random(n) < 0.05] = -np.inf
        keep = (rng.random(n) < 0.8).astype(np.uint8)
        k = int(rng.integers(1, 700))
        idx, val, cnt = oracle.topk(v, keep=keep, k=k)
        want = lexsort_topk(v, k, keep)
        assert cnt == want.size
        assert np.array_equal(idx[:cnt], want) and np.all(idx[cnt:] == -1)
        assert np.array_equal(val[:cnt], v[want])


def test_topk_takes_all_when_fewer_than_k():
    v = np.array([0.5, -np.inf, -1.0, 2.0, 0.0])
    idx, _, cnt = oracle.topk(v, k=512)
    assert cnt == 4 and np.array_equal(idx[:4], [0, 2, 3, 4]) and np.all(idx[4:] == -1)


def test_topk_ties_go_to_lower_index():
    v = np.zeros(2000)
    v[[5, 900, 1500]] = 1.0
    idx, _, cnt = oracle.topk(v, k=512)
    assert cnt == 512
    assert np.array_equal(idx, np.sort(np.concatenate([[900, 1500], np.arange(510)])))


def test_topk_signed_zeros_are_equal():
    """A row whose weights are all zero scores every entry zero; -0 and +0 logits tie."""
    wl = tiny_wl(seed=22, T=1, H=4, D=8, n_entries=700, page=8)
    wl.queries[0].w[:] = np.float32(-0.0)
    L = oracle.logits(wl)[0, :700]
    assert np.all(L == 0.0)
    v = np.where(np.random.default_rng(2).random(700) < 0.5, -0.0, 0.0)
    assert np.any(np.signbit(v)) and not np.all(np.signbit(v))
    for row in (L, v):
        idx, _, cnt = oracle.topk(row, k=512)
        assert cnt == 512 and np.array_equal(idx, np.arange(512))


def test_topk_never_selects_masked_or_invisible():
    wl = tiny_wl(seed=23, T=4, B=1, n_entries=2000, page=8, q_pos=[4000, 5000, 6000, 7999],
                 ratio=4, w_mean=0.2)
    L = oracle.logits(wl)
    mask = (np.random.default_rng(3).random((1, L.shape[1])) < 0.3).astype(np.uint8)
    idx, _, cnt = oracle.topk_rows(L, k=512, mask=mask, row_req=np.zeros(4, np.int32))
    for t in range(4):
        sel = idx[t, :cnt[t]]
        assert np.all(mask[0, sel] == 1)
        assert np.all(sel < oracle.n_visible(wl, t))
        assert np.array_equal(sel, lexsort_topk(L[t], 512, mask[0]))


def test_two_level_equals_mode_a_and_gate_off():
    wl = W.two_level_resident_fp8(seed=31, B=3, seq_len=64 * 40 + 19, kmax=9, shuffled=True,
                                  poison=False, ragged=True)
    idx, val, cnt = oracle.score_resident(wl)
    L = oracle.logits(wl)
    ld = L.shape[1]
    mask = np.zeros((3, ld), np.uint8)
    for b in range(3):
        for p in wl.resident_pages[b, :wl.n_resident[b]]:
            mask[b, p * 64:(p + 1) * 64] = 1
    ia, va, ca = oracle.topk_rows(L, mask=mask)
    assert np.array_equal(idx, ia) and np.array_equal(cnt, ca)
    assert np.array_equal(val[idx >= 0], va[ia >= 0])
    # every page resident: two-level equals plain top-k over the whole history
    n_pages = -(-int(wl.kv.seq_lens.max()) // 64)
    allp = np.tile(np.arange(n_pages, dtype=np.int32), (3, 1))
    nres = np.array([-(-int(n) // 64) for n in wl.kv.seq_lens], np.int32)
    i2, _, c2 = oracle.score_resident(wl, resident_pages=allp, n_resident=nres)
    ip, _, cp = oracle.topk_rows(L)
    assert np.array_equal(i2, ip) and np.array_equal(c2, cp)


def test_two_level_never_touches_poisoned_pages():
    wl = W.two_level_resident_fp8(seed=32, B=2, seq_len=64 * 50, kmax=7, poison=True)
    idx, val, cnt = oracle.score_resident(wl)
    assert np.all(np.isfinite(val[idx >= 0]))
    for b in range(2):
        pages = set(wl.resident_pages[b, :wl.n_resident[b]].tolist())
        assert all(int(s) // 64 in pages for s in idx[b, :cnt[b]])
        assert cnt[b] == min(512, 64 * wl.n_resident[b])


def _densest_brute(d, kmax):
    """Pages with density > 0, by density descending then page ascending, first kmax, ascending."""
    out = np.full((d.shape[0], kmax), -1, np.int32)
    cnt = np.zeros(d.shape[0], np.int32)
    for b in range(d.shape[0]):
        cand = [p for p in range(d.shape[1]) if d[b, p] > 0]
        cand.sort(key=lambda p: (-int(d[b, p]), p))
        take = sorted(cand[:kmax])
        out[b, :len(take)] = take
        cnt[b] = len(take)
    return out, cnt


@pytest.mark.parametrize("kmax", [1, 7, 96, 384, 1000])
def test_densest_pages_brute_force(kmax):
    rng = np.random.default_rng(kmax)
    d = rng.integers(0, 65, (4, 300)).astype(np.int32)      # many ties among 65 levels
    d[1, rng.random(300) < 0.8] = 0                          # sparse: fewer than kmax pages
    d[2] = 0                                                 # nothing resident
    d[3, :] = 5                                              # all tied: lowest ids win
    got, cnt = oracle.densest_pages(d, kmax)
    ref, rcnt = _densest_brute(d, kmax)
    assert np.array_equal(got, ref) and np.array_equal(cnt, rcnt)
    assert cnt[2] == 0 and np.all(got[2] == -1)
    assert np.array_equal(got[3, :min(kmax, 300)], np.arange(min(kmax, 300)))


def test_densest_pages_of_the_mask_are_its_fullest_pages():
    """From a real Level-1 mask: the selected pages are resident, and no unselected page is
    denser than a selected one."""
    wl = W.three_layer_mask_fp8(seed=2003, B=2, seq_len=64 * 50 + 7, ragged=True)
    r = oracle.resident_mask(wl)
    d = r["page_density"]
    pages, cnt = oracle.densest_pages(d, 9)
    for b in range(2):
        sel = pages[b, :cnt[b]]
        assert cnt[b] == min(9, int((d[b] > 0).sum()))
        assert np.all(d[b, sel] > 0) and np.all(np.diff(sel) > 0)
        rest = np.setdiff1d(np.nonzero(d[b])[0], sel)
        if rest.size and sel.size:
            assert d[b, rest].max() <= d[b, sel].min()


@pytest.mark.parametrize("shuffled", [False, True])
def test_reserve_cells_are_the_remapped_entries(shuffled):
    """Reserve cell of entry 64 p + o = 64 j + o, j = the page's position in the resident list.
    With continuous random logits there are no exact ties, so the cell selection is the entry
    selection remapped, whatever the list order."""
    wl = W.two_level_resident_fp8(seed=33, B=3, seq_len=64 * 40 + 19, kmax=11,
                                  shuffled=shuffled, poison=False, ragged=True)
    ie, ve, ce = oracle.score_resident(wl)
    ic, vc, cc = oracle.score_resident(wl, cells=True)
    assert np.array_equal(ce, cc)
    for t in range(wl.queries[0].T):
        b = t
        lst = list(wl.resident_pages[b, :wl.n_resident[b]])
        remap = sorted(lst.index(s // 64) * 64 + s % 64 for s in ie[t, :ce[t]])
        assert np.array_equal(ic[t, :cc[t]], remap)
        assert np.all(ic[t, cc[t]:] == -1)
        # the same logits, listed by cell
        assert np.allclose(np.sort(vc[t, :cc[t]]), np.sort(ve[t, :ce[t]]), rtol=0, atol=0)


# ----------------------------------------------------------------------------- shape
def test_flop_table_slope_is_64_heads_by_128_dims():
    """The baseline column of the per-token FLOP table grows by 2 * 64 * 128 (+ ~1%) FLOP per
    compressed entry per c4 layer: the indexer's head count and head dimension."""
    rows = [list(map(float, l.split())) for l in open(os.path.join(GOLD,
            "flops_per_decode_token.txt")) if l.strip() and not l.startswith("#")]
    per = []
    for (c0, _, b0, _), (c1, _, b1, _) in zip(rows, rows[1:]):
        per.append((b1 - b0) * 1e9 / ((c1 - c0) / 4) / 21)
    for f in per:
        assert abs(f - 2 * W.HEADS * W.DIM) / (2 * W.HEADS * W.DIM) < 0.02


# ----------------------------------------------------------------------------- query encoder
from oracle import encoder as OE   # noqa: E402

PAGE_ROPE = dict(rope_dim=64, base=160000.0, factor=16.0, orig_len=65536, beta_fast=32.0,
                 beta_slow=1.0)   # the repository page's hyperparameter table


def test_encoder_hadamard_is_sylvesters_normalised():
    """Against scipy's Hadamard matrix (an independent construction), and H H = I."""
    import scipy.linalg
    rng = np.random.default_rng(41)
    for n in (2, 8, 128):
        x = rng.standard_normal((5, n))
        H = scipy.linalg.hadamard(n).astype(np.float64)
        assert np.allclose(OE.hadamard(x), x @ H / math.sqrt(n), rtol=0, atol=1e-12)
        assert np.allclose(OE.hadamard(OE.hadamard(x)), x, rtol=0, atol=1e-12)
    e0 = np.zeros(128)
    e0[0] = 1.0
    assert np.allclose(OE.hadamard(e0), np.full(128, 1 / math.sqrt(128)), rtol=0, atol=1e-15)


def test_encoder_yarn_frequencies_follow_the_wavelength_rule():
    """YaRN's definition in terms of wavelengths lambda_i = 2 pi / theta_i: a pair that turns more
    than beta_fast times over the original context keeps theta_i, one that turns fewer than
    beta_slow times is divided by the factor, and the pairs between are strictly between.  With
    factor 1 the frequencies are plain RoPE's base^(-2i/d)."""
    P = PAGE_ROPE
    d, base = P["rope_dim"], P["base"]
    theta = np.array([base ** (-2.0 * i / d) for i in range(d // 2)])
    assert np.array_equal(OE.yarn_inv_freq(d, base, 1.0, P["orig_len"], P["beta_fast"],
                                           P["beta_slow"]), theta)
    inv = OE.yarn_inv_freq(d, base, P["factor"], P["orig_len"], P["beta_fast"], P["beta_slow"])
    turns = P["orig_len"] / (2 * math.pi / theta)          # rotations over the original context
    fast, slow = turns > P["beta_fast"], turns < P["beta_slow"]
    mid = ~fast & ~slow
    assert fast.sum() == 16 and slow.sum() == 7 and mid.sum() == 9
    assert np.allclose(inv[fast], theta[fast], rtol=1e-15, atol=0)
    assert np.allclose(inv[slow], theta[slow] / P["factor"], rtol=1e-15, atol=0)
    assert np.all(inv[mid] < theta[mid]) and np.all(inv[mid] > theta[mid] / P["factor"])
    assert np.all(np.diff(inv) < 0)                         # still strictly decreasing


def test_encoder_rope_is_a_rotation_of_consecutive_pairs():
    rng = np.random.default_rng(43)
    P = PAGE_ROPE
    inv = OE.yarn_inv_freq(P["rope_dim"], P["base"], P["factor"], P["orig_len"], P["beta_fast"],
                           P["beta_slow"])
    x = rng.standard_normal((3, 64))
    assert np.array_equal(OE.rope(x, np.zeros(3), inv), x)              # position 0
    pos = np.array([7.0, 131072.0, 999999.0])
    y = OE.rope(x, pos, inv)
    n0 = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    assert np.allclose(y[:, 0::2] ** 2 + y[:, 1::2] ** 2, n0, rtol=1e-12, atol=0)
    # a unit vector on the first coordinate of pair i turns to (cos, sin) of pos * theta_i
    for i in (0, 17, 31):
        e = np.zeros((1, 64))
        e[0, 2 * i] = 1.0
        r = OE.rope(e, np.array([12345.0]), inv)
        assert np.allclose(r[0, 2 * i:2 * i + 2], [math.cos(12345 * inv[i]), math.sin(12345 * inv[i])],
                           rtol=0, atol=1e-12)
        assert np.count_nonzero(r) <= 2
    # dot products depend on the position difference only
    a, b = x[0:1], x[1:2]
    d1 = np.sum(OE.rope(a, np.array([100.0]), inv) * OE.rope(b, np.array([37.0]), inv))
    d2 = np.sum(OE.rope(a, np.array([5100.0]), inv) * OE.rope(b, np.array([5037.0]), inv))
    assert abs(d1 - d2) < 1e-9


def test_encoder_rms_norm_closed_forms():
    assert np.allclose(OE.rms_norm(np.full((1, 16), 3.0), np.ones(16), 1e-6),
                       np.full((1, 16), 3.0 / math.sqrt(9.0 + 1e-6)), rtol=1e-15, atol=0)
    rng = np.random.default_rng(47)
    a = rng.standard_normal((4, 256)) * 7.0
    r = OE.rms_norm(a, np.ones(256), 0.0)
    assert np.allclose(np.mean(r * r, axis=1), 1.0, rtol=1e-12, atol=0)
    assert np.allclose(OE.rms_norm(5.0 * a, np.ones(256), 0.0), r, rtol=1e-12, atol=0)
    g = rng.standard_normal(256)
    assert np.allclose(OE.rms_norm(a, g, 0.0), r * g, rtol=1e-12, atol=0)


def _encode_brute(h, pos, Wa, g, Wb, Wp, n_heads, head_dim, rope_dim, eps, inv):
    """The pipeline with explicit loops and math, and the Hadamard entries from their closed form
    (-1)^popcount(i & j), on tiny shapes."""
    T, D = len(h), len(h[0])
    R = len(Wa)
    q = [[[0.0] * head_dim for _ in range(n_heads)] for _ in range(T)]
    w = [[0.0] * n_heads for _ in range(T)]
    for t in range(T):
        a = [sum(h[t][k] * Wa[j][k] for k in range(D)) for j in range(R)]
        ms = sum(v * v for v in a) / R
        r = [a[j] / math.sqrt(ms + eps) * g[j] for j in range(R)]
        for hh in range(n_heads):
            x = [sum(r[k] * Wb[hh * head_dim + c][k] for k in range(R)) for c in range(head_dim)]
            off = head_dim - rope_dim
            for i in range(rope_dim // 2):
                ang = pos[t] * inv[i]
                x0, x1 = x[off + 2 * i], x[off + 2 * i + 1]
                x[off + 2 * i] = x0 * math.cos(ang) - x1 * math.sin(ang)
                x[off + 2 * i + 1] = x0 * math.sin(ang) + x1 * math.cos(ang)
            for i in range(head_dim):
                q[t][hh][i] = sum(x[j] * (-1) ** bin(i & j).count("1")
                                  for j in range(head_dim)) / math.sqrt(head_dim)
            w[t][hh] = sum(h[t][k] * Wp[hh][k] for k in range(D)) / math.sqrt(head_dim * n_heads)
    return np.array(q), np.array(w)


def test_encoder_matches_brute_force_on_tiny_shapes():
    rng = np.random.default_rng(53)
    T, D, R, NH, HD, RD = 3, 6, 4, 2, 8, 4
    h, Wa, g = rng.standard_normal((T, D)), rng.standard_normal((R, D)), rng.standard_normal(R)
    Wb, Wp = rng.standard_normal((NH * HD, R)), rng.standard_normal((NH, D))
    pos = [0, 3, 70000]
    inv = OE.yarn_inv_freq(RD, 100.0, 4.0, 64, 8.0, 1.0)
    q, w = OE.encode(h, pos, Wa, g, Wb, Wp, n_heads=NH, head_dim=HD, rope_dim=RD, eps=1e-6,
                     rope_base=100.0, rope_factor=4.0, rope_orig_len=64, beta_fast=8.0,
                     beta_slow=1.0)
    qb, wb = _encode_brute(h.tolist(), pos, Wa.tolist(), g.tolist(), Wb.tolist(), Wp.tolist(),
                           NH, HD, RD, 1e-6, inv.tolist())
    assert np.allclose(q, qb, rtol=0, atol=1e-10)
    assert np.allclose(w, wb, rtol=0, atol=1e-12)
