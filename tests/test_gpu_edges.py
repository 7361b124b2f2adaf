"""GPU edge cases and invariants of the C-ABI entry points.

Top-k on constructed logit rows (ties, signed zeros, -inf / NaN, fewer candidates than k,
k from 1 to 1024, n_valid, masks, empty rows) is compared bit-exactly with the oracle's
selection on the same float32 values.  Scoring invariants: two runs are bit-identical, a
permuted block table with the pool permuted alike gives bit-identical logits, and poisoned
pages outside the resident list never reach a result.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import gpu_util as G
from top_selection_fm_amd import api
from top_selection_fm_amd import workloads as W

pytestmark = pytest.mark.gpu


def gpu_topk(L: np.ndarray, k, n_valid=None, mask=None, row_req=None, workspace=True):
    Lt = torch.from_numpy(np.ascontiguousarray(L, np.float32)).cuda()
    nv = None if n_valid is None else torch.from_numpy(np.asarray(n_valid, np.int32)).cuda()
    mk = None if mask is None else torch.from_numpy(np.asarray(mask, np.uint8)).cuda()
    rr = None if row_req is None else torch.from_numpy(np.asarray(row_req, np.int32)).cuda()
    idx, val = G.topk(Lt, k=k, n_valid=nv, mask=mk, row_req=rr, workspace=workspace)
    return idx.cpu().numpy(), val.cpu().numpy()


def ref_topk(L, k, n_valid=None, mask=None, row_req=None):
    ri, rv, rc = oracle.topk_rows(np.asarray(L, np.float32).astype(np.float64), k=k,
                                  n_valid=n_valid, mask=mask, row_req=row_req)
    return ri, rv


def constructed_rows(rng, T, n):
    L = rng.standard_normal((T, n)).astype(np.float32)
    L[0] = 1.0                                        # all tie
    L[1] = np.where(rng.random(n) < 0.5, np.float32(-0.0), np.float32(0.0))   # signed zeros
    L[2] = np.round(L[2] * 2) / 2                     # few distinct values
    L[3, rng.random(n) < 0.3] = -np.inf
    L[4, rng.random(n) < 0.3] = np.nan
    L[5] = -np.inf                                    # no candidate at all
    L[6, :] = -np.inf
    L[6, [min(3, n - 1), n // 2, n - 1]] = [2.0, -1.0, 0.0]   # up to three candidates
    L[7] = np.float32(3.4e38) * np.sign(L[7])         # extremes
    return L


@pytest.mark.parametrize("workspace", [True, False])
@pytest.mark.parametrize("k", [1, 7, 512, 1000, 1024])
@pytest.mark.parametrize("n", [1, 600, 4096, 4097, 9000, 70000])
def test_topk_constructed_rows_bit_exact(k, n, workspace):
    rng = np.random.default_rng(k * 10007 + n)
    L = constructed_rows(rng, 12, n)
    ig, vg = gpu_topk(L, k, workspace=workspace)
    ri, rv = ref_topk(L, k)
    assert np.array_equal(ig, ri)
    sel = ri >= 0
    assert np.array_equal(vg[sel], rv[sel].astype(np.float32))
    assert np.all(np.isneginf(vg[~sel]))


@pytest.mark.parametrize("workspace", [True, False])
def test_topk_n_valid_mask_and_row_req(workspace):
    rng = np.random.default_rng(5)
    T, n = 9, 13000
    L = constructed_rows(rng, T, n)
    nv = rng.integers(0, n + 1, T).astype(np.int32)
    nv[0] = 0
    mask = (rng.random((3, n)) < 0.4).astype(np.uint8)
    row_req = (np.arange(T) % 3).astype(np.int32)
    ig, _ = gpu_topk(L, 512, n_valid=nv, mask=mask, row_req=row_req, workspace=workspace)
    ri, _ = ref_topk(L, 512, n_valid=nv, mask=mask, row_req=row_req)
    assert np.array_equal(ig, ri)
    assert np.all(ig[0] == -1)


@pytest.mark.parametrize("n", [1, 700, 4097, 20000, 34816, 34817])
def test_topk_many_rows(n):
    """520 rows, two workgroups a CU: rows of up to 34,816 entries take the 512-thread row
    kernel, 34,817 the 1,024-thread one.  Constructed rows, n_valid, a mask per request and
    row_req, bit-exact against the oracle."""
    rng = np.random.default_rng(n + 77)
    T = 520
    L = constructed_rows(rng, T, n)
    L[8:] *= rng.uniform(0.1, 10.0, (T - 8, 1)).astype(np.float32)
    ig, vg = gpu_topk(L, 512)
    ri, rv = ref_topk(L, 512)
    assert np.array_equal(ig, ri)
    sel = ri >= 0
    assert np.array_equal(vg[sel], rv[sel].astype(np.float32))
    nv = rng.integers(0, n + 1, T).astype(np.int32)
    mask = (rng.random((4, n)) < 0.6).astype(np.uint8)
    row_req = (np.arange(T) % 4).astype(np.int32)
    ig, _ = gpu_topk(L, 512, n_valid=nv, mask=mask, row_req=row_req)
    ri, _ = ref_topk(L, 512, n_valid=nv, mask=mask, row_req=row_req)
    assert np.array_equal(ig, ri)


@pytest.mark.parametrize("workspace", [True, False])
def test_topk_long_rows_262144_candidates(workspace):
    """Mode-A sized rows: 262,144 candidates, with planted duplicates of the 512th value."""
    rng = np.random.default_rng(9)
    L = rng.standard_normal((3, 262144)).astype(np.float32)
    L[1, rng.choice(262144, 5000, replace=False)] = np.float32(2.5)   # a huge tie group
    mask = (rng.random((3, 262144)) < 0.12).astype(np.uint8)
    ig, _ = gpu_topk(L, 512, workspace=workspace)
    ri, _ = ref_topk(L, 512)
    assert np.array_equal(ig, ri)
    ig, _ = gpu_topk(L, 512, mask=mask, workspace=workspace)
    ri, _ = ref_topk(L, 512, mask=mask)
    assert np.array_equal(ig, ri)


def mode_a_inputs(rng, B, layers, n, resident_frac=0.12):
    """Mode A: every layer's full-history logits of a request, one row per (request, layer),
    sharing the request's resident mask through row_req (page-clustered residency)."""
    L = rng.standard_normal((B * layers, n)).astype(np.float32)
    pages = (rng.random((B, n // 64)) < resident_frac).astype(np.uint8)
    mask = np.repeat(pages, 64, axis=1)
    row_req = np.repeat(np.arange(B, dtype=np.int32), layers)
    return L, mask, row_req


@pytest.mark.parametrize("workspace", [True, False])
def test_topk_mode_a_21_layers_shared_mask(workspace):
    """Full-history top-512 of 21 layers over 262,144 candidates, the layers of a request
    sharing its resident mask (rows 21 b .. 21 b + 20 -> request b).  Bit-exact."""
    rng = np.random.default_rng(23)
    L, mask, row_req = mode_a_inputs(rng, 2, 21, 262144)
    L[5, np.flatnonzero(mask[0])[:3000]] = np.float32(1.75)     # a tie group among residents
    ig, vg = gpu_topk(L, 512, mask=mask, row_req=row_req, workspace=workspace)
    ri, rv = ref_topk(L, 512, mask=mask, row_req=row_req)
    assert np.array_equal(ig, ri)
    assert np.array_equal(vg[ri >= 0], rv[ri >= 0].astype(np.float32))
    # nothing outside the request's resident pages is ever selected
    for t in range(L.shape[0]):
        sel = ig[t][ig[t] >= 0]
        assert mask[row_req[t], sel].all()


def test_topk_more_survivors_than_the_buffer():
    """Long rows whose sampled positions run colder than the rest: the row's cut lets about
    10% of the row through (far more than the 4,096-entry buffer, but under each chunk's
    capacity), so the final selection runs over the stage-1 survivors.  Bit-exact."""
    n = 262144
    rng = np.random.default_rng(29)
    L = rng.standard_normal((4, n)).astype(np.float32)
    runs = (np.arange(128) * (n // 128))[:, None] + np.arange(16)[None, :]   # sampled positions
    L[:, runs.ravel()] -= np.float32(1.0)
    L[2, rng.choice(n, 20000, replace=False)] = np.float32(2.0)   # ties across the boundary
    mask = (rng.random((2, n)) < 0.6).astype(np.uint8)
    row_req = np.array([0, 1, 0, 1], np.int32)
    for mk, rr in ((None, None), (mask, row_req)):
        ig, vg = gpu_topk(L, 512, mask=mk, row_req=rr, workspace=True)
        ri, rv = ref_topk(L, 512, mask=mk, row_req=rr)
        assert np.array_equal(ig, ri)
        assert np.array_equal(vg[ri >= 0], rv[ri >= 0].astype(np.float32))


@pytest.mark.parametrize("workspace", [True, False])
def test_topk_sampled_cut_and_its_fallbacks(workspace):
    """Long rows go through a sampled cut; rows where the cut cannot hold fall back to the exact
    selection over the whole row.  Every case must match the oracle bit for bit."""
    n = 65536
    stride = n // 4096                              # the sample reads every 16th entry here
    rng = np.random.default_rng(11)
    L = np.zeros((4, n), np.float32)
    L[0] = rng.standard_normal(n)                   # ordinary row: the cut holds
    L[1] = 0.25                                     # constant row: everything passes, overflow
    L[2] = 0.5                                      # sampled entries look hotter than the row:
    L[2, np.arange(100) * stride] = 1.0             # only 100 pass the cut (< k), fallback
    L[3] = rng.standard_normal(n)                   # the top values sit between sample points
    L[3, np.arange(700) * stride + 1] = 5.0 + rng.random(700)
    ig, vg = gpu_topk(L, 512, workspace=workspace)
    ri, rv = ref_topk(L, 512)
    assert np.array_equal(ig, ri)
    assert np.array_equal(vg[ri >= 0], rv[ri >= 0].astype(np.float32))


def test_topk_workspace_reused_and_dirty():
    """One workspace serves consecutive calls of different shapes and data, starting from
    arbitrary bytes: nothing in it has to be cleared between calls."""
    rng = np.random.default_rng(21)
    nb = api.fm_workspace_bytes(api.FM_OP_TOPK, 6, 70000)
    for fill in (0xFF, None, 0x00):
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        if fill is None:
            ws.copy_(torch.from_numpy(rng.integers(0, 256, nb, dtype=np.uint8)))
        else:
            ws.fill_(fill)
        for T, n in ((6, 70000), (3, 20000), (6, 70000), (5, 8193)):
            L = constructed_rows(rng, 8, n)[:T].copy()
            Lt = torch.from_numpy(L).cuda()
            idx = torch.empty((T, 512), dtype=torch.int32, device="cuda")
            need = api.fm_workspace_bytes(api.FM_OP_TOPK, T, n)
            assert need <= nb
            api.fm_topk512(Lt, n, T, None, None, 0, None, 512, idx, None, ws, nb)
            ri, _ = ref_topk(L, 512)
            assert np.array_equal(idx.cpu().numpy(), ri), (fill, T, n)


def test_scoring_is_deterministic_and_placement_invariant():
    wl = W.decode_bf16(seed=3001, B=4, seq_len=64 * 33 + 9, ragged=True)
    dw = api.DeviceWorkload(wl, "cuda:0")
    L1 = G.index_logits(dw)
    L2 = G.index_logits(dw)
    assert torch.equal(L1, L2)
    i1, v1 = G.topk(L1)
    i2, v2 = G.topk(L2)
    assert torch.equal(i1, i2) and torch.equal(v1, v2)
    # move every physical page elsewhere and remap the block table alike
    rng = np.random.default_rng(3)
    perm = rng.permutation(wl.kv.n_phys_pages)
    pool = np.empty_like(wl.kv.pools[0])
    pool[perm] = wl.kv.pools[0]
    wl2 = W.Workload(wl.name, W.KeyPool([pool], "bf16", perm[wl.kv.block_table].astype(np.int32),
                                        wl.kv.seq_lens), wl.queries)
    L3 = G.index_logits(api.DeviceWorkload(wl2, "cuda:0"))
    assert torch.equal(torch.nan_to_num(L1, nan=7.0), torch.nan_to_num(L3, nan=7.0))


def test_unmapped_pages_score_nan_and_are_never_selected():
    wl = W.decode_bf16(seed=3002, B=2, seq_len=64 * 20, ragged=False)
    bt = wl.kv.block_table.copy()
    bt[0, [2, 5]] = -1
    bt[1, 7] = 10 ** 8                        # out of range: bounds-checked on the device
    wl2 = W.Workload(wl.name, W.KeyPool(wl.kv.pools, "bf16", bt, wl.kv.seq_lens), wl.queries)
    dw = api.DeviceWorkload(wl2, "cuda:0")
    L = G.index_logits(dw).cpu().numpy()
    assert np.all(np.isnan(L[0, 2 * 64:3 * 64])) and np.all(np.isnan(L[1, 7 * 64:8 * 64]))
    assert np.isfinite(L[0, :128]).all()
    idx, _ = G.topk(torch.from_numpy(L).cuda())
    ig = idx.cpu().numpy()
    assert not np.isin(ig[0] // 64, [2, 5]).any() and not np.any(ig[1] // 64 == 7)


def test_resident_pages_out_of_range_are_skipped():
    wl = W.two_level_resident_fp8(seed=3003, B=2, seq_len=64 * 40, kmax=6, poison=True)
    rp = wl.resident_pages.copy()
    rp[1, 2] = 10 ** 6                         # not a page of this request
    dw = api.DeviceWorkload(wl, "cuda:0")
    idx, val = G.score_resident(dw, resident_pages=torch.from_numpy(rp).cuda())
    ig, vg = idx.cpu().numpy(), val.cpu().numpy()
    sel = ig[1][ig[1] >= 0]
    assert sel.size == 5 * 64 and np.all(np.isfinite(vg[1][:sel.size]))
    assert set((sel // 64).tolist()) == set(rp[1].tolist()) - {10 ** 6}


@pytest.mark.parametrize("cells", [False, True])
def test_two_level_empty_and_short_resident_lists(cells):
    """Per-request resident counts of 0 (nothing to select: all -1 / -inf), 3 pages (fewer
    entries than k: every visible entry, ascending), and 12 pages (a real top-512), with list
    positions past each count holding clean pages that must be ignored and every page outside
    the lists poisoned; entries (or reserve cells) against the oracle."""
    wl = W.two_level_resident_fp8(seed=3005, B=3, seq_len=64 * 40 + 5, kmax=12, poison=True)
    nres = np.array([0, 3, 12], np.int32)
    dw = api.DeviceWorkload(wl, "cuda:0")
    call = G.score_resident_cells if cells else G.score_resident
    idx, val = call(dw, n_resident=torch.from_numpy(nres).cuda())
    ig, vg = idx.cpu().numpy(), val.cpu().numpy()
    ri, rv, rc = oracle.score_resident(wl, n_resident=nres, cells=cells)
    assert np.all(ig[0] == -1) and np.all(np.isneginf(vg[0])), "empty list selects nothing"
    for t in (1, 2):
        sel = ig[t][ig[t] >= 0]
        assert np.all(np.isfinite(vg[t][:sel.size])), f"row {t}: a poisoned page was read"
        scale = float(np.max(np.abs(rv[t, :rc[t]])))
        of = (lambda e, t=t: oracle.logits_at(wl, np.full(len(e), t),
                                              wl.resident_pages[t][np.asarray(e) // 64] * 64
                                              + np.asarray(e) % 64)) if cells else \
             (lambda e, t=t: oracle.logits_at(wl, np.full(len(e), t), e))
        G.check_topk_row(ig[t], vg[t], ri[t], rc[t], of, scale, 512, f"row {t} cells={cells}")
        listed = wl.resident_pages[t][:nres[t]]
        if cells:
            assert np.all(sel // 64 < nres[t]), f"row {t}: a cell past the list's count"
        else:
            assert set((sel // 64).tolist()) <= set(listed.tolist()), f"row {t}: unlisted page"
    assert rc[1] < 512 and rc[2] >= 512, "the cases must cover a short and a full row"


@pytest.mark.parametrize("sink,recent", [(0, 0), (5, 100)])
def test_mask_empty_and_one_page_requests(sink, recent):
    """One fm_resident_mask call over requests of 0 entries, 37 entries (one partial page) and
    64 * 30 + 11 entries, with and without sink / recent forcing (the recent window longer
    than the short request): the empty request has no mask bit and no page, the forced
    entries are resident, and every output matches the oracle under the band rule."""
    wl = W.three_layer_mask_fp8(seed=3006, B=3, seq_len=64 * 30 + 11)
    wl.kv.seq_lens[:] = np.array([0, 37, 64 * 30 + 11], np.int32)
    dw = api.DeviceWorkload(wl, "cuda:0")
    m = G.resident_mask(dw, n_sink=sink, n_recent=recent)
    r = oracle.resident_mask(wl, n_sink=sink, n_recent=recent)
    tag = f"mask lengths 0 / 37 / 1931, sink {sink}, recent {recent}"
    mg = m["mask"].cpu().numpy()
    G.check_mask(mg, r["mask"], r["union"], 0.0, wl.kv.seq_lens, tag)
    G.check_pages(m, r, 0.0, wl.kv.seq_lens, tag)
    assert not mg[0].any() and int(m["page_count"][0]) == 0
    assert np.all(m["page_list"][0].cpu().numpy() == -1)
    if recent:
        assert mg[1, :37].all() and not mg[1, 37:].any()
        n = int(wl.kv.seq_lens[2])
        assert mg[2, :sink].all() and mg[2, n - recent:n].all() and not mg[2, n:].any()
