"""GPU parity: every entry point of libfm.so, through the C ABI, against the fp64 oracle.

Small cases span several 64-entry pages with ragged tails (sizes the oracle finishes in a
second); full-size cases use the benchmark shapes: decode bf16 B=32 x 65,536, three-layer fp8
mask B=8 x 262,144, two-level fp8 B=30 x 384 resident pages, causal prefill 4,096 x 33,792
(sampled rows).  The parity rule is stated in tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import gpu_util as G
from top_selection_fm_amd import api
from top_selection_fm_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_LOW = 2e-2


def dev(wl, **kw):
    return api.DeviceWorkload(wl, "cuda:0", **kw)


def topk_parity(tag, L_ref, idx_gpu, val_gpu, rows=None, k=512, n_valid=None, mask=None,
                row_req=None):
    """Compare GPU top-k rows with the oracle's top-k of the oracle logits L_ref[rows]."""
    rows = np.arange(L_ref.shape[0]) if rows is None else np.asarray(rows)
    ri, rv, rc = oracle.topk_rows(L_ref, k=k, n_valid=n_valid, mask=mask, row_req=row_req)
    dis = band = 0
    for i, t in enumerate(rows):
        fin = np.isfinite(L_ref[i])
        scale = np.max(np.abs(L_ref[i, fin])) if fin.any() else 1.0
        d, bn = G.check_topk_row(idx_gpu[t], val_gpu[t], ri[i], rc[i],
                                 lambda e, i=i: L_ref[i, e], scale, k, f"{tag} row {t}")
        dis += d
        band += bn
        sel = idx_gpu[t][idx_gpu[t] >= 0]
        if d == 0:
            got = val_gpu[t][:len(sel)].astype(np.float64)
            ref = L_ref[i, sel]
            assert np.all(np.abs(got - ref) <= TOL_LOW * scale), f"{tag}: values"
    G.note(tag, rows=len(rows), disagreements=dis, band_entries=band)
    return dis


# ----------------------------------------------------------------------------- fp32 tiny
@pytest.mark.parametrize("n_entries", [4096, 1000, 37])
def test_tiny_fp32_logits_mask_topk(n_entries):
    wl = W.tiny_single_query(n_entries=n_entries)
    dw = dev(wl)
    ld = wl.kv.block_table.shape[1] * 64
    L = G.index_logits(dw).cpu().numpy()
    Lr = oracle.logits(wl)
    err = G.check_logits(L, Lr, TOL_F32, "tiny f32 logits")
    idx, val = G.topk(torch.from_numpy(L).cuda())
    dis = topk_parity(f"tiny f32 top-512 n={n_entries}", Lr, idx.cpu().numpy(),
                      val.cpu().numpy())
    m = G.resident_mask(dw)
    mr = oracle.resident_mask(wl)
    md, mb = G.check_mask(m["mask"].cpu().numpy(), mr["mask"], mr["union"], 0.0,
                          wl.kv.seq_lens, "tiny f32 mask")
    G.check_pages(m, mr, 0.0, wl.kv.seq_lens, "tiny f32 pages")
    G.note("tiny f32", n=n_entries, ld=ld, logit_err=err, topk_dis=dis, mask_dis=md,
           mask_band=mb, mask_true=int(mr["mask"].sum()))


# ----------------------------------------------------------------------------- decode bf16
@pytest.fixture(scope="module")
def decode_small():
    return W.decode_bf16(seed=2002, B=3, seq_len=64 * 40 + 13, ragged=True)


def test_decode_bf16_small(decode_small):
    wl = decode_small
    dw = dev(wl)
    L = G.index_logits(dw)
    Lr = oracle.logits(wl)
    err = G.check_logits(L.cpu().numpy(), Lr, TOL_LOW, "decode bf16 small")
    idx, val = G.topk(L)
    topk_parity("decode bf16 small top-512", Lr, idx.cpu().numpy(), val.cpu().numpy())
    G.note("decode bf16 small logits", err=err)


@pytest.mark.parametrize("ld", [64 * 40 + 5, 64 * 40 + 4, 64 * 39 + 12])
def test_decode_bf16_ld_not_multiple_of_page(decode_small, ld):
    # shorter than some rows: columns >= ld are not written (a stray write would land in the
    # next row, which is compared too).  ld % 4 == 0 takes the 16-byte store path, which must
    # drop the groups past ld as the 4-byte path drops single columns.
    wl = decode_small
    dw = dev(wl)
    L = G.index_logits(dw, ld=ld).cpu().numpy()
    Lr = oracle.logits(wl, s_end=ld)
    G.check_logits(L, Lr, TOL_LOW, f"decode bf16 ld={ld}")


@pytest.fixture(scope="module")
def decode_full():
    return W.decode_bf16()


def test_decode_bf16_full(decode_full):
    wl = decode_full
    dw = dev(wl)
    L = G.index_logits(dw)
    idx, val = G.topk(L)
    torch.cuda.synchronize()
    Lr = oracle.logits(wl)
    err = G.check_logits(L.cpu().numpy(), Lr, TOL_LOW, "decode bf16 B32x65536")
    dis = topk_parity("decode bf16 B32x65536 top-512", Lr, idx.cpu().numpy(), val.cpu().numpy())
    hot = wl.meta["hot_pages"]
    sel = idx.cpu().numpy()
    frac = np.mean([np.isin(sel[b] // 64, hot[b]).mean() for b in range(wl.kv.B)])
    G.note("decode bf16 full", logit_err=err, topk_dis=dis, hot_fraction_of_top512=frac)


# ----------------------------------------------------------------------------- Level-1 mask
@pytest.fixture(scope="module")
def mask_small():
    return W.three_layer_mask_fp8(seed=2003, B=3, seq_len=64 * 50 + 7, ragged=True)


@pytest.mark.parametrize("mode,p,sink,recent", [("max", 0.5, 0, 0), ("max", 0.3, 0, 0),
                                                ("max", 0.8, 3, 70), ("mean", 0.5, 0, 0),
                                                ("mean", 0.2, 1, 1)])
def test_mask_fp8_small(mask_small, mode, p, sink, recent):
    wl = mask_small
    dw = dev(wl)
    m = G.resident_mask(dw, mode=api.FM_UNION_MAX if mode == "max" else api.FM_UNION_MEAN,
                        threshold=p, n_sink=sink, n_recent=recent)
    r = oracle.resident_mask(wl, mode=mode, threshold=p, n_sink=sink, n_recent=recent)
    cut = float(np.log(p / (1 - p))) if mode == "max" else p
    mg = m["mask"].cpu().numpy()
    dis, band = G.check_mask(mg, r["mask"], r["union"], cut, wl.kv.seq_lens,
                             f"mask {mode} p={p}")
    G.check_pages(m, r, cut, wl.kv.seq_lens, f"mask {mode} p={p} pages")
    if dis == 0:
        assert np.array_equal(m["page_count"].cpu().numpy(), r["page_count"])
        assert np.array_equal(m["page_list"].cpu().numpy(), r["page_list"])
        assert np.array_equal(m["page_density"].cpu().numpy(), r["page_density"])
    u = m["union"].cpu().numpy().astype(np.float64)
    for b in range(wl.kv.B):
        n = int(wl.kv.seq_lens[b])
        ur = r["union"][b, :n]
        sc = np.max(np.abs(ur)) if mode == "max" else 1.0
        assert np.max(np.abs(u[b, :n] - ur)) <= TOL_LOW * sc
        assert np.all(np.isneginf(u[b, n:]))
    G.note(f"mask small {mode} p={p} sink={sink} recent={recent}", disagreements=dis,
           band_entries=band, resident_fraction=float(r["mask"].mean()))


def test_mask_page_compaction_matches_gpu_mask(mask_small):
    """Page outputs are a pure function of the GPU's own mask bytes."""
    wl = mask_small
    m = G.resident_mask(dev(wl))
    mg = m["mask"].cpu().numpy().astype(bool)
    dens = mg.reshape(wl.kv.B, -1, 64).sum(-1)
    assert np.array_equal(m["page_density"].cpu().numpy(), dens)
    pl = m["page_list"].cpu().numpy()
    for b in range(wl.kv.B):
        nz = np.nonzero(dens[b])[0]
        assert m["page_count"][b].item() == nz.size
        assert np.array_equal(pl[b, :nz.size], nz) and np.all(pl[b, nz.size:] == -1)


def test_mask_page_list_without_density(mask_small):
    """Without page_density the fp8 kernel stages each page's count in page_list (when it is as
    wide as the pages) and compaction turns it into the list in place; with a narrower list the
    counts come from the mask bytes.  Both equal the outputs of a call with page_density."""
    wl = mask_small
    dw = dev(wl)
    ref = G.resident_mask(dw)
    B = wl.kv.B
    ld = wl.kv.block_table.shape[1] * 64
    n_pages = ld // 64
    for width in (n_pages, n_pages + 3, 5):
        mask = torch.empty((B, ld), dtype=torch.uint8, device="cuda")
        cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        plist = torch.full((B, width), -7, dtype=torch.int32, device="cuda")
        api.fm_resident_mask([dw.query(l) for l in range(3)], dw.kv(0, [0, 1, 2]),
                             api.FM_UNION_MAX, 0.5, 0, 0, mask, ld, cnt, plist, width, None, None)
        torch.cuda.synchronize()
        assert torch.equal(mask, ref["mask"]), width
        assert torch.equal(cnt, ref["page_count"]), width
        want = ref["page_list"].cpu().numpy()
        got = plist.cpu().numpy()
        w = min(width, n_pages)
        assert np.array_equal(got[:, :w], want[:, :w]), width
        assert np.all(got[:, w:] == -1), width


def test_mask_single_layer_and_short_mask_ld(mask_small):
    wl = mask_small
    dw = dev(wl)
    ld = 64 * 20 + 9
    m = G.resident_mask(dw, layers=[1], mask_ld=ld)
    r = oracle.resident_mask(wl, layers=[1], mask_ld=ld)
    dis, _ = G.check_mask(m["mask"].cpu().numpy(), r["mask"], r["union"], 0.0,
                          np.minimum(wl.kv.seq_lens, ld), "mask layer 1, mask_ld 1289")
    G.check_pages(m, r, 0.0, np.minimum(wl.kv.seq_lens, ld), "mask_ld 1289 pages")
    if dis == 0:
        assert np.array_equal(m["page_count"].cpu().numpy(), r["page_count"])
        assert np.array_equal(m["page_list"].cpu().numpy(), r["page_list"])


@pytest.mark.parametrize("mode", ["max", "mean"])
def test_mask_two_layers(mask_small, mode):
    wl = mask_small
    dw = dev(wl)
    um = api.FM_UNION_MAX if mode == "max" else api.FM_UNION_MEAN
    m = G.resident_mask(dw, mode=um, layers=[2, 0])
    r = oracle.resident_mask(wl, mode=mode, layers=[2, 0])
    dis, _ = G.check_mask(m["mask"].cpu().numpy(), r["mask"], r["union"],
                          0.0 if mode == "max" else 0.5, wl.kv.seq_lens, f"mask layers 2,0 {mode}")
    G.check_pages(m, r, 0.0 if mode == "max" else 0.5, wl.kv.seq_lens, f"layers 2,0 {mode} pages")
    if dis == 0:
        assert np.array_equal(m["page_count"].cpu().numpy(), r["page_count"])
        assert np.array_equal(m["page_list"].cpu().numpy(), r["page_list"])


def test_mask_four_layers():
    """FM_MAX_LAYERS = 4 fp8 layers in one call: every layer takes part in the union."""
    wl = W.three_layer_mask_fp8(seed=2013, B=2, seq_len=64 * 60 + 30, n_layers=4, ragged=True,
                                cluster=2, w_bias=-0.04)
    dw = dev(wl)
    m = G.resident_mask(dw, layers=[0, 1, 2, 3])
    r = oracle.resident_mask(wl, layers=[0, 1, 2, 3])
    r3 = oracle.resident_mask(wl, layers=[0, 1, 2])
    assert not np.array_equal(r["mask"], r3["mask"]), "the fourth layer must matter here"
    dis, band = G.check_mask(m["mask"].cpu().numpy(), r["mask"], r["union"], 0.0,
                             wl.kv.seq_lens, "mask four layers")
    G.check_pages(m, r, 0.0, wl.kv.seq_lens, "mask four layers pages")
    if dis == 0:
        assert np.array_equal(m["page_count"].cpu().numpy(), r["page_count"])
    G.note("mask four layers", disagreements=dis, band_entries=band)


@pytest.fixture(scope="module")
def mask_full():
    return W.three_layer_mask_fp8()


def test_mask_fp8_full(mask_full):
    wl = mask_full
    dw = dev(wl)
    m = G.resident_mask(dw, with_union=False)      # as timed: no debug union output
    torch.cuda.synchronize()
    r = oracle.resident_mask(wl)
    dis, band = G.check_mask(m["mask"].cpu().numpy(), r["mask"], r["union"], 0.0,
                             wl.kv.seq_lens, "mask B8x262144 x3")
    pc = m["page_count"].cpu().numpy()
    banded_pages = G.check_pages(m, r, 0.0, wl.kv.seq_lens, "mask B8x262144 x3 pages")
    G.note("mask full", disagreements=dis, band_entries=band, banded_pages=banded_pages,
           resident_fraction=float(r["mask"].mean()), page_count=pc.tolist(),
           page_count_ref=r["page_count"].tolist())
    if dis == 0:
        assert np.array_equal(pc, r["page_count"])
    assert 0.08 < r["mask"].mean() < 0.16


# ----------------------------------------------------------------------------- two-level
@pytest.mark.parametrize("shuffled", [False, True])
def test_two_level_small(shuffled):
    wl = W.two_level_resident_fp8(seed=2004, B=4, seq_len=64 * 60 + 21, kmax=20,
                                  shuffled=shuffled, ragged=True)
    dw = dev(wl)
    idx, val = G.score_resident(dw)
    ri, rv, rc = oracle.score_resident(wl)
    ig, vg = idx.cpu().numpy(), val.cpu().numpy()
    dis = 0
    for t in range(wl.queries[0].T):
        sel = ig[t][ig[t] >= 0]
        allv = oracle.logits_at(wl, np.full(sel.size, t), sel)
        scale = np.max(np.abs(np.concatenate([allv, rv[t, :rc[t]]])))
        d, _ = G.check_topk_row(ig[t], vg[t], ri[t], rc[t],
                                lambda e, t=t: oracle.logits_at(wl, np.full(len(e), t), e),
                                scale, 512, f"two-level small row {t}")
        dis += d
        assert np.all(np.isfinite(vg[t][:sel.size]))
    G.note(f"two-level small shuffled={shuffled}", disagreements=dis)


def test_two_level_equals_masked_topk_and_gate_off():
    wl = W.two_level_resident_fp8(seed=2005, B=3, seq_len=64 * 30 + 3, kmax=11, shuffled=True,
                                  poison=False, ragged=True)
    dw = dev(wl)
    idx, val = G.score_resident(dw)
    L = G.index_logits(dw)
    ld = L.shape[1]
    mask = torch.zeros((3, ld), dtype=torch.uint8, device="cuda")
    for b in range(3):
        for p in wl.resident_pages[b, :wl.n_resident[b]]:
            mask[b, p * 64:(p + 1) * 64] = 1
    ia, va = G.topk(L, mask=mask)
    assert torch.equal(idx, ia) and torch.equal(val, va)
    n_pages = -(-int(wl.kv.seq_lens.max()) // 64)
    allp = torch.arange(n_pages, dtype=torch.int32, device="cuda").repeat(3, 1)
    nres = torch.tensor([-(-int(n) // 64) for n in wl.kv.seq_lens], dtype=torch.int32,
                        device="cuda")
    i2, v2 = G.score_resident(dw, resident_pages=allp, n_resident=nres)
    ip, vp = G.topk(L)
    assert torch.equal(i2, ip) and torch.equal(v2, vp)


# ----------------------------------------------------------------------------- densest pages
@pytest.mark.parametrize("kmax", [1, 96, 384, 1024])
def test_densest_pages_bit_exact(kmax):
    rng = np.random.default_rng(4000 + kmax)
    d = rng.integers(0, 65, (8, 4096)).astype(np.int32)      # page densities of 1M-entry rows
    d[1, rng.random(4096) < 0.97] = 0                        # fewer resident pages than kmax
    d[2] = 0                                                 # nothing resident
    d[3] = 64                                                # all tied
    d[4, :] = 0
    d[4, [5, 4095]] = [1, 64]                                # two pages, far apart
    dt = torch.from_numpy(d).cuda()
    pages, cnt = G.densest_pages(dt, kmax, n_pages=4000)     # the last 96 columns are ignored
    rp, rc = oracle.densest_pages(d, kmax, n_pages=4000)
    assert np.array_equal(pages.cpu().numpy(), rp)
    assert np.array_equal(cnt.cpu().numpy(), rc)


def test_mask_densest_two_level_chain():
    """Level 1 to Level 2 on the device: the GPU mask's page densities -> the KMAX densest pages
    -> two-level top-512 over them, each step compared with the oracle on the GPU's own input."""
    wl = W.three_layer_mask_fp8(seed=2006, B=3, seq_len=64 * 60 + 11, ragged=True)
    dw = dev(wl)
    m = G.resident_mask(dw)
    dens = m["page_density"]
    pages, cnt = G.densest_pages(dens, 12)
    rp, rc = oracle.densest_pages(dens.cpu().numpy(), 12)
    assert np.array_equal(pages.cpu().numpy(), rp) and np.array_equal(cnt.cpu().numpy(), rc)
    # layer 0's query row and pool score the recalled pages
    wl0 = W.Workload(wl.name, wl.kv, wl.queries[:1], resident_pages=rp, n_resident=rc,
                     meta=wl.meta)
    dw0 = dev(wl0)
    idx, val = G.score_resident(dw0, resident_pages=pages, n_resident=cnt)
    cells, cval = G.score_resident_cells(dw0, resident_pages=pages, n_resident=cnt)
    ri, rv, rcnt = oracle.score_resident(wl0)
    ig, vg = idx.cpu().numpy(), val.cpu().numpy()
    for t in range(wl0.queries[0].T):
        sel = ig[t][ig[t] >= 0]
        allv = oracle.logits_at(wl0, np.full(sel.size, t), sel)
        scale = np.max(np.abs(np.concatenate([allv, rv[t, :rcnt[t]]]))) if sel.size else 1.0
        G.check_topk_row(ig[t], vg[t], ri[t], rcnt[t],
                         lambda e, t=t: oracle.logits_at(wl0, np.full(len(e), t), e),
                         scale, 512, f"chain row {t}")
    # an ascending list: the cells are the entries remapped, the values the same
    cg, cv = cells.cpu().numpy(), cval.cpu().numpy()
    for t in range(wl0.queries[0].T):
        lst = list(rp[t, :rc[t]])
        sel = ig[t][ig[t] >= 0]
        assert np.array_equal(cg[t][cg[t] >= 0], [lst.index(s // 64) * 64 + s % 64 for s in sel])
        assert np.array_equal(cv[t], vg[t])


@pytest.mark.parametrize("shuffled", [False, True])
def test_score_resident_cells_small(shuffled):
    wl = W.two_level_resident_fp8(seed=2007, B=4, seq_len=64 * 60 + 21, kmax=20,
                                  shuffled=shuffled, ragged=True)
    dw = dev(wl)
    cells, val = G.score_resident_cells(dw)
    ri, rv, rc = oracle.score_resident(wl, cells=True)
    cg, vg = cells.cpu().numpy(), val.cpu().numpy()

    def logits_of_cells(t, cs):
        lst = wl.resident_pages[t]
        ents = np.array([int(lst[c // 64]) * 64 + c % 64 for c in cs], np.int64)
        return oracle.logits_at(wl, np.full(len(ents), t), ents)

    dis = 0
    for t in range(wl.queries[0].T):
        sel = cg[t][cg[t] >= 0]
        allv = logits_of_cells(t, sel)
        scale = np.max(np.abs(np.concatenate([allv, rv[t, :rc[t]]])))
        d, _ = G.check_topk_row(cg[t], vg[t], ri[t], rc[t], lambda cs, t=t: logits_of_cells(t, cs),
                                scale, 512, f"two-level cells row {t}")
        dis += d
    G.note(f"two-level cells shuffled={shuffled}", disagreements=dis)


@pytest.fixture(scope="module")
def two_level_full():
    return W.two_level_resident_fp8()


@pytest.mark.parametrize("shuffled", [False, True])
def test_two_level_full(two_level_full, shuffled):
    wl = two_level_full
    if shuffled:
        rng = np.random.default_rng(77)
        wl = W.Workload(wl.name, wl.kv, wl.queries,
                        resident_pages=np.stack([rng.permutation(r) for r in wl.resident_pages]),
                        n_resident=wl.n_resident, meta=wl.meta)
    dw = dev(wl)
    idx, val = G.score_resident(dw)
    torch.cuda.synchronize()
    ri, rv, rc = oracle.score_resident(wl)
    ig, vg = idx.cpu().numpy(), val.cpu().numpy()
    dis = 0
    for t in range(wl.queries[0].T):
        sel = ig[t][ig[t] >= 0]
        scale = float(np.max(np.abs(rv[t, :rc[t]])))
        d, _ = G.check_topk_row(ig[t], vg[t], ri[t], rc[t],
                                lambda e, t=t: oracle.logits_at(wl, np.full(len(e), t), e),
                                scale, 512, f"two-level full row {t}")
        dis += d
        assert np.all(np.isfinite(vg[t][:sel.size])), "poisoned page reached a result"
        pages = set(wl.resident_pages[t].tolist())
        assert all(int(s) // 64 in pages for s in sel)
    G.note(f"two-level full shuffled={shuffled}", disagreements=dis)


# ----------------------------------------------------------------------------- prefill fp8
def _prefill_rows_parity(wl, dw, rows, tag):
    L = G.index_logits(dw, ld=wl.kv.max_seq_len)
    idx, val = G.topk(L)
    torch.cuda.synchronize()
    Lr = oracle.logits(wl, rows=rows, s_end=wl.kv.max_seq_len)
    Lg = L.cpu().numpy()[rows]
    err = G.check_logits(Lg, Lr, TOL_LOW, tag)
    dis = topk_parity(tag + " top-512", Lr, idx.cpu().numpy()[rows], val.cpu().numpy()[rows],
                      rows=np.arange(len(rows)))
    return err, dis, idx


def test_prefill_small():
    wl = W.prefill_causal_fp8(seed=2006, T=100, pos0=4 * 1880, seq_len=64 * 30 + 5)
    err, dis, _ = _prefill_rows_parity(wl, dev(wl), np.arange(100), "prefill small")
    G.note("prefill small", logit_err=err, topk_dis=dis)


def test_prefill_fewer_than_k_visible():
    wl = W.prefill_causal_fp8(seed=2007, T=64, pos0=1990, seq_len=64 * 10)
    err, dis, idx = _prefill_rows_parity(wl, dev(wl), np.arange(64), "prefill short")
    nv = np.array([oracle.n_visible(wl, t) for t in range(64)])
    got = (idx.cpu().numpy() >= 0).sum(1)
    assert np.array_equal(got, np.minimum(nv, 512))


@pytest.fixture(scope="module")
def prefill_full():
    return W.prefill_causal_fp8()


def test_prefill_full_sampled_rows(prefill_full):
    """One row of every 8-row block (each block is scored by one workgroup per key chunk, and
    the chunks are dealt to the 8 XCDs), its wave position rotating with the block, plus the
    first and last rows: every workgroup of the launch is checked on every chunk it scores."""
    wl = prefill_full
    T = wl.queries[0].T
    rows = np.unique(np.concatenate([8 * np.arange(T // 8) + np.arange(T // 8) % 8,
                                     [0, 1, 2, 3, T - 4, T - 3, T - 2, T - 1]]))
    err, dis, idx = _prefill_rows_parity(wl, dev(wl), rows, "prefill 4096x33792")
    ig = idx.cpu().numpy()
    assert not np.any(ig == 33791), "entry 33,791 is visible to no row"
    assert np.all(ig < 33791)
    G.note("prefill full sampled", rows=rows.tolist(), logit_err=err, topk_dis=dis)


@pytest.mark.parametrize("code_max", [None, 1.0 / 16])
def test_prefill_small_query_codes(code_max):
    """Queries whose E4M3 codes do not fill the range: q passed unscaled (q_scale = 1, codes
    about 0.1) or with codes below 1/16.  The prefill kernel's per-row block scale keeps these
    rows as accurate as full-range ones; 15 rows (the exact float32 path) and 16 rows (the
    prefill kernel) of the same input agree."""
    wl = W.prefill_causal_fp8(seed=2040, T=16, pos0=4 * 1500, seq_len=64 * 24 + 9)
    q = wl.queries[0]
    vals = (torch.from_numpy(q.q.copy()).view(torch.float8_e4m3fn).float().numpy()
            * q.q_scale[:, None, None])
    if code_max is None:
        sc = np.ones(q.T, np.float32)
    else:
        sc = (np.abs(vals.reshape(q.T, -1)).max(1) / code_max).astype(np.float32)
    q.q[:] = W.e4m3_codes(vals / sc[:, None, None])
    q.q_scale[:] = sc
    ld = wl.kv.max_seq_len
    L16 = G.index_logits(dev(wl), ld=ld).cpu().numpy()
    q15 = W.Queries(np.ascontiguousarray(q.q[:15]), q.q_dtype, np.ascontiguousarray(q.w[:15]),
                    q.w_dtype, q_scale=np.ascontiguousarray(q.q_scale[:15]),
                    row_req=np.ascontiguousarray(q.row_req[:15]),
                    q_pos=np.ascontiguousarray(q.q_pos[:15]), compress_ratio=q.compress_ratio)
    wl15 = W.Workload(wl.name, wl.kv, [q15])
    L15 = G.index_logits(dev(wl15), ld=ld).cpu().numpy()
    Lr = oracle.logits(wl, s_end=ld)
    err16 = G.check_logits(L16, Lr, TOL_LOW, f"prefill small codes {code_max} T=16")
    err15 = G.check_logits(L15, Lr[:15], TOL_LOW, f"prefill small codes {code_max} T=15")
    fin = np.isfinite(Lr[:15])
    scale = np.max(np.abs(Lr[:15][fin]))
    assert np.max(np.abs(L16[:15][fin] - L15[fin])) <= TOL_LOW * scale
    G.note(f"prefill small codes {code_max}", err16=err16, err15=err15)


def test_prefill_topk_with_causal_lengths(prefill_full):
    """Giving the top-k each row's causal length (as a prefill caller can) selects exactly what
    the full rows select: every entry past the cut is -inf in the logits."""
    wl = prefill_full
    dw = dev(wl)
    L = G.index_logits(dw)
    ld = L.shape[1]
    nv = np.minimum(wl.queries[0].q_pos.astype(np.int64) // 4, ld).astype(np.int32)
    i_full, v_full = G.topk(L)
    i_cut, v_cut = G.topk(L, n_valid=torch.from_numpy(nv).cuda())
    assert torch.equal(i_full, i_cut) and torch.equal(v_full, v_cut)


@pytest.mark.parametrize("T,pos0,seq_len,extra_ld", [
    (16, 4 * 700, 64 * 12 + 3, 0),       # exactly one 16-row tile
    (17, 4 * 700, 64 * 12 + 3, 70),      # a ragged second tile; columns past seq_len
    (15, 4 * 700, 64 * 12 + 3, 0),       # fewer rows than a tile: one row at a time
    (40, 0, 64 * 5, 0),                  # the first rows see nothing (pos < ratio)
    (300, 4 * 9000, 64 * 140 + 17, 5),   # many tiles and chunks, no causal cut inside
])
def test_prefill_edge_shapes(T, pos0, seq_len, extra_ld):
    wl = W.prefill_causal_fp8(seed=2008 + T, T=T, pos0=pos0, seq_len=seq_len)
    dw = dev(wl)
    ld = seq_len + extra_ld
    L = G.index_logits(dw, ld=ld)
    L2 = G.index_logits(dw, ld=ld)
    assert torch.equal(L, L2), "prefill logits are not deterministic"
    idx, val = G.topk(L)
    torch.cuda.synchronize()
    rows = np.arange(T)
    Lr = oracle.logits(wl, rows=rows, s_end=ld)
    err = G.check_logits(L.cpu().numpy(), Lr, TOL_LOW, f"prefill T={T}")
    dis = topk_parity(f"prefill T={T} top-512", Lr, idx.cpu().numpy(), val.cpu().numpy())
    G.note(f"prefill edge T={T}", logit_err=err, topk_dis=dis)


def test_prefill_unmapped_pages_score_nan():
    wl = W.prefill_causal_fp8(seed=2030, T=32, pos0=4 * 1300, seq_len=64 * 20)
    bt = wl.kv.block_table.copy()
    bt[0, 3] = -1
    bt[0, 9] = 10 ** 8                       # out of range: bounds-checked on the device
    wl2 = W.Workload(wl.name, W.KeyPool(wl.kv.pools, "fp8x132", bt, wl.kv.seq_lens),
                     wl.queries)
    L = G.index_logits(dev(wl2), ld=64 * 20).cpu().numpy()
    assert np.all(np.isnan(L[:, 3 * 64:4 * 64])) and np.all(np.isnan(L[:, 9 * 64:10 * 64]))
    Lr = oracle.logits(wl, rows=np.arange(32), s_end=64 * 20)
    keep = np.ones(64 * 20, bool)
    keep[3 * 64:4 * 64] = keep[9 * 64:10 * 64] = False
    G.check_logits(L[:, keep], Lr[:, keep], TOL_LOW, "prefill unmapped")
    idx, _ = G.topk(torch.from_numpy(L).cuda())
    ig = idx.cpu().numpy()
    assert not np.isin(ig // 64, [3, 9]).any()
