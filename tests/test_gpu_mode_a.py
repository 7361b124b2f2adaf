"""GPU parity of Mode A end to end: the Level-1 resident mask of three encoders, then the masked
top-512 of 21 layers' rows, each layer scoring its own fp8 key pool, in one fm_index_topk call
(row_pool picks a row's layer, row_req its request and mask row).

Pages: paper summary, section 6 (Mode A: full-history selection with non-resident entries at
-inf); README "Two-level recall algorithm" (Level 2 runs in every c4 layer, all of them under
the one Level-1 mask).

Checks:
  * the batched call equals one call per layer bit for bit (fm_index_logits and fm_index_topk;
    the per-layer calls take other work splits, so this also ties the fused and unfused paths);
  * 2 requests x 21 layers x 16,384 entries (ragged) against the fp64 oracle: the Level-1 mask
    and its pages, each Level-2 row's top-512 and its logits;
  * rows whose row_pool is out of range have nothing visible;
  * the two-level call (fm_score_resident) honours row_pool the same way;
  * 8 x 21 x 262,144 (the benchmarked shape and launch) on sampled rows against the oracle and,
    on every row, the properties any correct result has.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import gpu_util as G
from top_selection_fm_amd import api
from top_selection_fm_amd import workloads as W

pytestmark = pytest.mark.gpu

N_ENC = 3


def layer_view(wl, l):
    """Layer l's Level-2 rows as a one-layer workload (rows = requests) for the oracle and the
    per-layer calls."""
    B = wl.kv.B
    q2 = wl.queries[N_ENC]
    rows = slice(l * B, (l + 1) * B)
    kv = W.KeyPool([wl.kv.pools[N_ENC + l]], wl.kv.key_dtype, wl.kv.block_table,
                   wl.kv.seq_lens)
    return W.Workload(f"{wl.name}_layer{l}", kv, [W.Queries(q2.q[rows], "bf16", q2.w[rows],
                                                            "bf16")])


def encoder_view(wl):
    kv = W.KeyPool(wl.kv.pools[:N_ENC], wl.kv.key_dtype, wl.kv.block_table, wl.kv.seq_lens)
    return W.Workload(f"{wl.name}_level1", kv, wl.queries[:N_ENC])


def level2(dw, mask, k=512, logits_ld=0, query=None):
    """One fm_index_topk call over every layer's rows (all pools in the key descriptor)."""
    wl = dw.wl
    T = wl.queries[N_ENC].T
    n = max(-(-wl.kv.max_seq_len // 64) * 64, -(-logits_ld // 64) * 64)
    ws = torch.empty(api.fm_workspace_bytes(api.FM_OP_INDEX_TOPK, T, n), dtype=torch.uint8,
                     device=dw.device)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=dw.device)
    val = torch.full((T, k), -7.0, dtype=torch.float32, device=dw.device)
    L = torch.empty((T, logits_ld), dtype=torch.float32, device=dw.device) if logits_ld else None
    api.fm_index_topk(dw.query(N_ENC) if query is None else query, dw.kv(), mask,
                      0 if mask is None else mask.shape[1], k, idx, val, L, logits_ld, ws,
                      ws.numel())
    return idx, val, L


def level1(dw):
    return G.resident_mask(dw, layers=list(range(N_ENC)))


@pytest.fixture(scope="module")
def small():
    return W.mode_a_fp8(seed=3301, B=2, seq_len=16384, ragged=True)


@pytest.fixture(scope="module")
def small_dev(small):
    return api.DeviceWorkload(small, "cuda:0")


def test_row_pool_logits_equal_per_layer_calls(small, small_dev):
    dw = small_dev
    B, ld = small.kv.B, small.kv.block_table.shape[1] * 64
    T = small.queries[N_ENC].T
    out = torch.empty((T, ld), dtype=torch.float32, device=dw.device)
    api.fm_index_logits(dw.query(N_ENC), dw.kv(), out, ld)
    for l in range(T // B):
        d1 = api.DeviceWorkload(layer_view(small, l), "cuda:0")
        ref = G.index_logits(d1)
        assert torch.equal(out[l * B:(l + 1) * B].view(torch.int32), ref.view(torch.int32)), \
            f"layer {l}: batched logits differ from the per-layer call"


def test_row_pool_topk_equals_per_layer_calls(small, small_dev):
    dw = small_dev
    B = small.kv.B
    m = level1(dw)["mask"]
    idx, val, _ = level2(dw, m)
    for l in range(small.meta["n_layers"]):
        d1 = api.DeviceWorkload(layer_view(small, l), "cuda:0")
        i1, v1, _ = G.index_topk(d1, mask=m)
        assert torch.equal(idx[l * B:(l + 1) * B], i1), f"layer {l}: indices differ"
        assert torch.equal(val[l * B:(l + 1) * B].view(torch.int32), v1.view(torch.int32)), \
            f"layer {l}: values differ"


def test_mode_a_small_vs_oracle(small, small_dev):
    dw = small_dev
    B = small.kv.B
    ld = small.kv.block_table.shape[1] * 64
    # Level 1 against the oracle
    m = level1(dw)
    enc = encoder_view(small)
    r = oracle.resident_mask(enc)
    G.check_mask(m["mask"].cpu().numpy(), r["mask"], r["union"], 0.0, small.kv.seq_lens,
                 "mode A level 1")
    G.check_pages(m, r, 0.0, small.kv.seq_lens, "mode A level 1 pages")
    mask_np = m["mask"].cpu().numpy()
    # Level 2: every row of every layer against the oracle, under the GPU's own mask
    idx, val, L = level2(dw, m["mask"], logits_ld=ld)
    ig, vg, Lg = idx.cpu().numpy(), val.cpu().numpy(), L.cpu().numpy()
    dis = 0
    for l in range(small.meta["n_layers"]):
        view = layer_view(small, l)
        Lr = oracle.logits(view)
        G.check_logits(Lg[l * B:(l + 1) * B], Lr, 2e-2, f"layer {l} logits")
        ri, _, rc = oracle.topk_rows(Lr, k=512, mask=mask_np)
        for b in range(B):
            t = l * B + b
            fin = np.isfinite(Lr[b]) & (mask_np[b] != 0)
            scale = np.max(np.abs(Lr[b, fin])) if fin.any() else 1.0
            d, _ = G.check_topk_row(ig[t], vg[t], ri[b], rc[b], lambda e, b=b: Lr[b, e], scale,
                                    512, f"layer {l} request {b}")
            dis += d
            sel = ig[t][ig[t] >= 0]
            assert np.all(mask_np[b, sel] != 0), f"layer {l} request {b}: non-resident entry"
            assert np.all(np.abs(vg[t][:sel.size] - Lr[b, sel]) <= 2e-2 * scale)
    G.note("mode A small", disagreements=dis)


def test_row_pool_out_of_range_rows_are_empty(small, small_dev):
    dw = small_dev
    q2 = small.queries[N_ENC]
    T, ld = q2.T, small.kv.block_table.shape[1] * 64
    rp = q2.row_pool.copy()
    bad = [0, 5, T - 1]
    rp[bad] = [-1, len(small.kv.pools), 1000]
    d = dw.q[N_ENC]
    rp_dev = torch.from_numpy(rp.astype(np.int32)).cuda()   # held while the descriptor is used
    qd = api.query_desc(d["q"], "bf16", d["w"], "bf16", row_req=d["row_req"], row_pool=rp_dev)
    m = level1(dw)["mask"]
    idx, val, L = level2(dw, m, logits_ld=ld, query=qd)
    i0, v0, L0 = level2(dw, m, logits_ld=ld)
    good = np.setdiff1d(np.arange(T), bad)
    assert torch.equal(idx[good], i0[good]) and torch.equal(L[good].view(torch.int32),
                                                            L0[good].view(torch.int32))
    assert bool((idx[bad] == -1).all()) and bool(torch.isneginf(val[bad]).all())
    assert bool(torch.isneginf(L[bad]).all())


def test_row_pool_two_level(small, small_dev):
    """fm_score_resident over every layer's rows at once equals one call per layer."""
    dw = small_dev
    B = small.kv.B
    m = level1(dw)
    n_pages = small.kv.block_table.shape[1]
    pl, pc = m["page_list"], m["page_count"]
    T = small.queries[N_ENC].T
    nb = api.fm_workspace_bytes(api.FM_OP_SCORE_RESIDENT, T, n_pages * 64)
    ws = torch.empty(nb, dtype=torch.uint8, device=dw.device)
    idx = torch.empty((T, 512), dtype=torch.int32, device=dw.device)
    val = torch.empty((T, 512), dtype=torch.float32, device=dw.device)
    api.fm_score_resident(dw.query(N_ENC), dw.kv(), pl, pc, n_pages, 512, idx, val, ws, nb)
    for l in range(small.meta["n_layers"]):
        d1 = api.DeviceWorkload(layer_view(small, l), "cuda:0")
        i1 = torch.empty((B, 512), dtype=torch.int32, device=dw.device)
        v1 = torch.empty((B, 512), dtype=torch.float32, device=dw.device)
        nb1 = api.fm_workspace_bytes(api.FM_OP_SCORE_RESIDENT, B, n_pages * 64)
        ws1 = torch.empty(nb1, dtype=torch.uint8, device=dw.device)
        api.fm_score_resident(d1.query(0), d1.kv(), pl, pc, n_pages, 512, i1, v1, ws1, nb1)
        assert torch.equal(idx[l * B:(l + 1) * B], i1), f"layer {l}: indices differ"
        assert torch.equal(val[l * B:(l + 1) * B].view(torch.int32), v1.view(torch.int32))
    # two-level = Mode A under the page-granular mask (every entry of a resident page)
    pmask = (m["page_density"] > 0).to(torch.uint8).repeat_interleave(64, dim=1).contiguous()
    i_a, v_a, _ = level2(dw, pmask)
    assert torch.equal(idx, i_a) and torch.equal(val.view(torch.int32), v_a.view(torch.int32))


@pytest.mark.timeout(600)
def test_mode_a_full_size_sampled():
    """8 requests x 21 layers x 262,144 entries, as timed: the mask, then one fm_index_topk
    call over the 168 rows.  Every row equals fm_index_logits + fm_topk512 under the mask bit
    for bit and satisfies what any correct answer does (ascending, resident, visible, count);
    sampled rows against the oracle."""
    wl = W.mode_a_fp8()
    dw = api.DeviceWorkload(wl, "cuda:0")
    B, n_layers = wl.kv.B, wl.meta["n_layers"]
    m = level1(dw)
    G.note("mode A full", step="level 1 done")
    idx, val, _ = level2(dw, m["mask"])
    torch.cuda.synchronize()
    G.note("mode A full", step="level 2 done")
    mask_np = m["mask"].cpu().numpy()
    ig, vg = idx.cpu().numpy(), val.cpu().numpy()
    n_res = mask_np.astype(np.int64).sum(axis=1)
    for t in range(B * n_layers):
        b = t % B
        sel = ig[t][ig[t] >= 0]
        assert sel.size == min(512, n_res[b]), f"row {t}: {sel.size} selected"
        assert np.all(np.diff(sel) > 0) and np.all(ig[t][sel.size:] == -1)
        assert np.all(mask_np[b, sel] != 0) and np.all(sel < wl.kv.seq_lens[b])
        assert np.all(np.isfinite(vg[t][:sel.size])) and np.all(np.isneginf(vg[t][sel.size:]))
    # the call runs fused (24 page slots a wave, 15 chunks a row): it equals the logits written
    # by fm_index_logits and selected by fm_topk512 under the mask, bit for bit, on every row
    ld = wl.kv.block_table.shape[1] * 64
    L = torch.empty((B * n_layers, ld), dtype=torch.float32, device="cuda:0")
    api.fm_index_logits(dw.query(N_ENC), dw.kv(), L, ld)
    row_req = torch.from_numpy(np.ascontiguousarray(wl.queries[N_ENC].row_req)).to("cuda:0")
    i2, v2 = G.topk(L, k=512, mask=m["mask"], row_req=row_req)
    del L
    assert torch.equal(idx, i2), "fused and two-call indices differ"
    assert torch.equal(val.view(torch.int32), v2.view(torch.int32)), \
        "fused and two-call values differ"
    G.note("mode A full", step="fused equals two calls")
    for t in (0, 8 * 10 + 3, B * n_layers - 1):
        l, b = divmod(t, B)
        view = layer_view(wl, l)
        Lr = oracle.logits(view, rows=[b])
        ri, _, rc = oracle.topk_rows(Lr, k=512, mask=mask_np[b:b + 1])
        fin = np.isfinite(Lr[0]) & (mask_np[b] != 0)
        scale = np.max(np.abs(Lr[0, fin]))
        d, _ = G.check_topk_row(ig[t], vg[t], ri[0], rc[0], lambda e: Lr[0, e], scale, 512,
                                f"full row {t}")
        sel = ig[t][ig[t] >= 0]
        assert np.all(np.abs(vg[t][:sel.size] - Lr[0, sel]) <= 2e-2 * scale)
        G.note("mode A full", row=t, disagreements=d)
