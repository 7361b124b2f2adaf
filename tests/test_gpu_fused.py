"""GPU parity of the fused scoring + top-k path (fm_index_topk; fm_score_resident on bf16 keys).

The fused kernel computes each logit with the same instructions as the scoring kernel of
fm_index_logits, so its selection must equal fm_topk512's over fm_index_logits' output bit for
bit (indices and values); it is also checked against the fp64 oracle under the parity rule of
tests/gpu_util.py.  Cases: ragged rows with fewer than k candidates, a row with nothing visible,
unmapped pages, a row of equal logits (the chunk selection's radix path), k from 1 to 1024, a
Mode A mask, the logits written alongside, the workspace's counters back at zero after every
call, and a shape that takes the unfused path (one long row).
"""
import numpy as np
import pytest
import torch

import oracle
from tests import gpu_util as G
from top_selection_fm_amd import api
from top_selection_fm_amd import workloads as W

pytestmark = pytest.mark.gpu


def dev(wl):
    return api.DeviceWorkload(wl, "cuda:0")


def two_call(dw, k=512, mask=None):
    """fm_index_logits then fm_topk512: the reference the fused path must reproduce exactly."""
    L = G.index_logits(dw)
    idx, val = G.topk(L, k=k, mask=mask)
    return idx, val, L


def assert_same(a, b, tag):
    ia, va = a
    ib, vb = b
    assert torch.equal(ia, ib), f"{tag}: indices differ"
    assert torch.equal(va.view(torch.int32), vb.view(torch.int32)), f"{tag}: values differ"


def oracle_parity(wl, idx, val, tag, k=512, mask=None):
    Lr = oracle.logits(wl)
    ri, rv, rc = oracle.topk_rows(Lr, k=k, mask=mask,
                                  row_req=wl.queries[0].row_req)
    ig, vg = idx.cpu().numpy(), val.cpu().numpy()
    dis = 0
    for t in range(Lr.shape[0]):
        fin = np.isfinite(Lr[t])
        scale = np.max(np.abs(Lr[t, fin])) if fin.any() else 1.0
        d, _ = G.check_topk_row(ig[t], vg[t], ri[t], rc[t], lambda e, t=t: Lr[t, e], scale, k,
                                f"{tag} row {t}")
        dis += d
        sel = ig[t][ig[t] >= 0]
        if d == 0 and sel.size:
            assert np.all(np.abs(vg[t][:sel.size] - Lr[t, sel]) <= 2e-2 * scale), f"{tag}: values"
    G.note(tag, disagreements=dis)


@pytest.fixture(scope="module")
def small():
    wl = W.decode_bf16(seed=3101, B=5, seq_len=64 * 40 + 13, ragged=True)
    wl.kv.seq_lens[3] = 100              # fewer candidates than k
    wl.kv.seq_lens[4] = 0                # nothing visible
    wl.kv.block_table[0, [2, 17]] = -1   # two unmapped pages: NaN logits, never selected
    return wl


@pytest.mark.parametrize("k", [512, 1, 7, 1000, 1024])
def test_fused_equals_two_calls_small(small, k):
    dw = dev(small)
    i2, v2, _ = two_call(dw, k=k)
    i1, v1, _ = G.index_topk(dw, k=k)
    assert_same((i1, v1), (i2, v2), f"fused k={k}")
    ig = i1.cpu().numpy()
    assert np.all(ig[4] == -1)
    assert (ig[3] >= 0).sum() == min(k, 100)
    assert not np.isin(ig[0] // 64, [2, 17]).any()
    if k == 512:
        oracle_parity(small, i1, v1, "fused small vs oracle")


def test_fused_logits_alongside(small):
    dw = dev(small)
    ld = small.kv.block_table.shape[1] * 64
    L_ref = G.index_logits(dw)
    i1, v1, L1 = G.index_topk(dw, logits_ld=ld)
    assert torch.equal(L1.view(torch.int32), L_ref.view(torch.int32))
    i2, v2 = G.topk(L_ref)
    assert_same((i1, v1), (i2, v2), "fused with logits")


def test_fused_equal_logits_take_lower_entries(small):
    """w = 0 on a row: every logit is 0, so the chunk selection meets one bin of ties (its radix
    path) and the top-k is the k lowest visible entries."""
    wl = W.Workload(small.name, small.kv, [W.Queries(small.queries[0].q.copy(), "bf16",
                                                     small.queries[0].w.copy(), "bf16")])
    wl.queries[0].w[1] = 0
    dw = dev(wl)
    i2, v2, _ = two_call(dw)
    i1, v1, _ = G.index_topk(dw)
    assert_same((i1, v1), (i2, v2), "equal logits")
    n1 = int(wl.kv.seq_lens[1])
    assert np.array_equal(i1[1].cpu().numpy(), np.arange(min(512, n1)))


def test_fused_mode_a_mask(small):
    rng = np.random.default_rng(7)
    ld = small.kv.block_table.shape[1] * 64
    mask = torch.from_numpy((rng.random((small.kv.B, ld)) < 0.12).astype(np.uint8)).cuda()
    dw = dev(small)
    i2, v2, _ = two_call(dw, mask=mask)
    i1, v1, _ = G.index_topk(dw, mask=mask)
    assert_same((i1, v1), (i2, v2), "fused masked")
    oracle_parity(small, i1, v1, "fused masked vs oracle", mask=mask.cpu().numpy())


def test_fused_repeatable_and_workspace_reuse(small, full):
    """Repeated calls give the same result, and a workspace reused across different inputs
    holds nothing that leaks into the next call (garbage-filled first)."""
    dw = dev(small)
    ws = G.index_topk_ws(dw)
    ws.fill_(0x7f)
    outs = [G.index_topk(dw, ws=ws) for _ in range(3)]
    for o in outs[1:]:
        assert_same(o[:2], outs[0][:2], "repeat")
    dwf = dev(full)
    wsf = G.index_topk_ws(dwf)
    a = G.index_topk(dwf, ws=wsf)
    b = G.index_topk(dw, ws=wsf)
    c = G.index_topk(dwf, ws=wsf)
    assert_same(b[:2], outs[0][:2], "small after full")
    assert_same(c[:2], a[:2], "full after small")


@pytest.fixture(scope="module")
def full():
    return W.decode_bf16()


def test_fused_decode_full(full):
    dw = dev(full)
    i2, v2, _ = two_call(dw)
    i1, v1, _ = G.index_topk(dw)
    assert_same((i1, v1), (i2, v2), "fused decode B32x65536")
    i3, v3, _ = G.index_topk(dw, k=1024)
    i4, v4, _ = two_call(dw, k=1024)
    assert_same((i3, v3), (i4, v4), "fused decode k=1024")
    oracle_parity(full, i1, v1, "fused decode B32x65536 vs oracle")


def test_unfused_long_row():
    """One request of 262,144 entries: too few rows to fill the chip in chunks, so the call scores
    into the workspace and selects with the staged top-k; same result as the two calls."""
    wl = W.decode_bf16(seed=3102, B=1, seq_len=262144 - 37)
    dw = dev(wl)
    L = G.index_logits(dw)
    i2, v2 = G.topk(L)
    i1, v1, _ = G.index_topk(dw)
    assert_same((i1, v1), (i2, v2), "unfused long row")


@pytest.mark.parametrize("shuffled", [False, True])
def test_two_level_bf16_fused(shuffled):
    """fm_score_resident over bf16 keys (fused): equals fm_topk512 over fm_index_logits with the
    listed pages as the mask, and the oracle's two-level top-k; cells likewise."""
    wl0 = W.decode_bf16(seed=3103 + shuffled, B=4, seq_len=64 * 60 + 21, ragged=True)
    rng = np.random.default_rng(11 + shuffled)
    kmax = 23
    res = np.full((4, kmax), -1, np.int32)
    nres = np.zeros(4, np.int32)
    for b in range(4):
        npg = -(-int(wl0.kv.seq_lens[b]) // 64)
        sel = np.sort(rng.choice(npg, min(kmax - b, npg), replace=False))
        if shuffled:
            sel = rng.permutation(sel)
        res[b, :sel.size] = sel
        nres[b] = sel.size
    wl = W.Workload(wl0.name, wl0.kv, wl0.queries, resident_pages=res, n_resident=nres)
    dw = dev(wl)
    idx, val = G.score_resident(dw)
    L = G.index_logits(dw)
    mask = torch.zeros(L.shape, dtype=torch.uint8, device="cuda")
    for b in range(4):
        for p in res[b, :nres[b]]:
            mask[b, p * 64:(p + 1) * 64] = 1
    ia, va = G.topk(L, mask=mask)
    assert_same((idx, val), (ia, va), "two-level bf16")
    ri, rv, rc = oracle.score_resident(wl)
    ig, vg = idx.cpu().numpy(), val.cpu().numpy()
    for t in range(4):
        scale = float(np.max(np.abs(rv[t, :rc[t]]))) if rc[t] else 1.0
        G.check_topk_row(ig[t], vg[t], ri[t], rc[t],
                         lambda e, t=t: oracle.logits_at(wl, np.full(len(e), t), e), scale, 512,
                         f"two-level bf16 row {t}")
    cells, cval = G.score_resident_cells(dw)
    cg = cells.cpu().numpy()
    for t in range(4):
        lst = list(res[t, :nres[t]])
        sel = ig[t][ig[t] >= 0]
        got = cg[t][cg[t] >= 0]
        want = sorted(lst.index(s // 64) * 64 + s % 64 for s in sel)
        if not shuffled:
            assert np.array_equal(got, want)
        else:   # ranked by cell, so ties may resolve differently; the cells map to valid entries
            assert got.size == sel.size


@pytest.fixture(scope="module")
def fp8_small():
    return W.three_layer_mask_fp8(seed=3110, B=4, seq_len=64 * 70 + 29, ragged=True)


@pytest.mark.parametrize("k", [512, 33, 1024])
def test_fused_fp8_keys_equals_two_calls(fp8_small, k):
    """fp8 keys with bf16 queries (the fp8 fused kernel), full rows: equal to the two calls."""
    wl = W.Workload(fp8_small.name, fp8_small.kv, fp8_small.queries[:1])
    dw = dev(wl)
    i2, v2, _ = two_call(dw, k=k)
    i1, v1, _ = G.index_topk(dw, k=k)
    assert_same((i1, v1), (i2, v2), f"fp8 fused k={k}")
    if k == 512:
        oracle_parity(wl, i1, v1, "fp8 fused vs oracle")


def test_fused_fp8_mode_a_mask(fp8_small):
    """Mode A over fp8 keys: the union mask of three encoders as the resident set of a layer's
    top-512, straight from fm_resident_mask's output."""
    wl = W.Workload(fp8_small.name, fp8_small.kv, fp8_small.queries[:1])
    dw3 = dev(fp8_small)
    m = G.resident_mask(dw3)["mask"]
    dw = dev(wl)
    i2, v2, _ = two_call(dw, mask=m)
    i1, v1, _ = G.index_topk(dw, mask=m)
    assert_same((i1, v1), (i2, v2), "fp8 fused Mode A")
    oracle_parity(wl, i1, v1, "fp8 fused Mode A vs oracle", mask=m.cpu().numpy())
