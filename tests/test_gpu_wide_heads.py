"""GPU parity with 128 query heads (the retriever's head count) against the fp64 oracle.

128 heads run for fp8 keys with bf16 queries (index logits, two-level scoring, the Level-1
mask with one to four layers) and for fp32 keys with fp32 queries.  The parity rule is the one
of tests/gpu_util.py; the last test chains the query encoder (128 heads) into the mask, where
the GPU's bf16 rounding of q sets a wider band (stated there).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import encoder as OE
from tests import gpu_util as G
from top_selection_fm_amd import api
from top_selection_fm_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_LOW = 2e-2
H = 128


def dev(wl, **kw):
    return api.DeviceWorkload(wl, "cuda:0", **kw)


def topk_rows_parity(tag, L_ref, idx_gpu, val_gpu, k=512):
    ri, rv, rc = oracle.topk_rows(L_ref, k=k)
    dis = 0
    for t in range(L_ref.shape[0]):
        fin = np.isfinite(L_ref[t])
        scale = np.max(np.abs(L_ref[t, fin])) if fin.any() else 1.0
        d, _ = G.check_topk_row(idx_gpu[t], val_gpu[t], ri[t], rc[t],
                                lambda e, t=t: L_ref[t, e], scale, k, f"{tag} row {t}")
        dis += d
    return dis


@pytest.mark.parametrize("n_entries", [1000, 37])
def test_wide_fp32_logits_mask_topk(n_entries):
    wl = W.tiny_single_query(seed=2101, n_entries=n_entries, heads=H)
    dw = dev(wl)
    L = G.index_logits(dw).cpu().numpy()
    Lr = oracle.logits(wl)
    err = G.check_logits(L, Lr, TOL_F32, "h128 f32 logits")
    idx, val = G.topk(torch.from_numpy(L).cuda())
    dis = topk_rows_parity("h128 f32 top-512", Lr, idx.cpu().numpy(), val.cpu().numpy())
    m = G.resident_mask(dw)
    mr = oracle.resident_mask(wl)
    md, _ = G.check_mask(m["mask"].cpu().numpy(), mr["mask"], mr["union"], 0.0,
                         wl.kv.seq_lens, "h128 f32 mask")
    G.note("h128 f32", n=n_entries, logit_err=err, topk_dis=dis, mask_dis=md)


@pytest.fixture(scope="module")
def wide_pool():
    return W.two_level_resident_fp8(seed=2102, B=4, seq_len=64 * 70 + 19, kmax=23,
                                    shuffled=True, poison=False, ragged=True, heads=H)


def test_wide_fp8_index_logits_and_topk(wide_pool):
    wl = wide_pool
    dw = dev(wl)
    L = G.index_logits(dw)
    L2 = G.index_logits(dw)
    assert torch.equal(L, L2), "logits are not deterministic"
    Lr = oracle.logits(wl)
    err = G.check_logits(L.cpu().numpy(), Lr, TOL_LOW, "h128 fp8 logits")
    idx, val = G.topk(L)
    dis = topk_rows_parity("h128 fp8 top-512", Lr, idx.cpu().numpy(), val.cpu().numpy())
    G.note("h128 fp8 index logits", logit_err=err, topk_dis=dis)


def test_wide_fp8_two_level(wide_pool):
    wl = wide_pool
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
                                scale, 512, f"h128 two-level row {t}")
        dis += d
    G.note("h128 two-level", disagreements=dis)


@pytest.fixture(scope="module")
def wide_mask():
    return W.three_layer_mask_fp8(seed=2103, B=3, seq_len=64 * 45 + 11, n_layers=4, ragged=True,
                                  heads=H, w_bias=-0.03)


@pytest.mark.parametrize("layers,mode", [([0, 1, 2], "max"), ([0, 1, 2, 3], "max"),
                                         ([2], "max"), ([1, 3], "mean")])
def test_wide_fp8_mask(wide_mask, layers, mode):
    wl = wide_mask
    dw = dev(wl)
    um = api.FM_UNION_MAX if mode == "max" else api.FM_UNION_MEAN
    m = G.resident_mask(dw, mode=um, layers=layers)
    r = oracle.resident_mask(wl, mode=mode, layers=layers)
    dis, band = G.check_mask(m["mask"].cpu().numpy(), r["mask"], r["union"],
                             0.0 if mode == "max" else 0.5, wl.kv.seq_lens,
                             f"h128 mask layers {layers} {mode}")
    if dis == 0:
        assert np.array_equal(m["page_count"].cpu().numpy(), r["page_count"])
        assert np.array_equal(m["page_list"].cpu().numpy(), r["page_list"])
    u = m["union"].cpu().numpy().astype(np.float64)
    for b in range(wl.kv.B):
        n = int(wl.kv.seq_lens[b])
        ur = r["union"][b, :n]
        sc = np.max(np.abs(ur)) if mode == "max" else 1.0
        assert np.max(np.abs(u[b, :n] - ur)) <= TOL_LOW * sc
    G.note(f"h128 mask {layers} {mode}", disagreements=dis, band_entries=band,
           resident_fraction=float(r["mask"].mean()))


def test_wide_encoder_to_mask():
    """The retriever's Level-1 step at its head count: three 128-head query encoders
    (fm_encode_queries) feed fm_resident_mask over three fp8 pools, against the oracle encoder's
    q and w scored by the oracle.  The GPU rounds q to bf16 (relative 2^-9 per element), so the
    union logits agree to 2e-2 of each request's largest |logit| (the bf16 logit bound) and the
    mask bits agree outside that band around the cut."""
    B = 3
    base = W.three_layer_mask_fp8(seed=2104, B=B, seq_len=64 * 33 + 5, ragged=True, heads=H)
    dwk = dev(base)
    encs = [W.query_encoder(seed=2105 + l, T=B, n_heads=H, d_model=256, q_rank=128)
            for l in range(3)]
    d = "cuda:0"
    keep, qds, refs = [], [], []
    for e in encs:
        t = {k: torch.from_numpy(getattr(e, k).view(np.int16)).to(d)
             for k in ("hidden", "wq_a", "q_norm", "wq_b", "w_proj")}
        desc = api.encoder_desc(t["wq_a"], t["q_norm"], t["wq_b"], t["w_proj"], n_heads=H,
                                d_model=e.d_model, q_rank=e.q_rank)
        nb = api.fm_encode_workspace_bytes(desc, B)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=d)
        q = torch.empty((B, H, 128), dtype=torch.bfloat16, device=d)
        w = torch.empty((B, H), dtype=torch.float32, device=d)
        api.fm_encode_queries(desc, t["hidden"], B, torch.from_numpy(e.pos).to(d), q, w, ws, nb)
        keep += [t, ws, q, w]
        qds.append(api.QueryDesc(q.data_ptr(), api.FM_BF16, None, w.data_ptr(), api.FM_F32, B,
                                 H, None, None, 1))
        qr, wr = OE.encode(e.hidden, e.pos, e.wq_a, e.q_norm, e.wq_b, e.w_proj, n_heads=H)
        refs.append(W.Queries(qr.astype(np.float32), "f32", wr.astype(np.float32), "f32"))
    ld = base.kv.block_table.shape[1] * 64
    n_pages = ld // 64
    mask = torch.empty((B, ld), dtype=torch.uint8, device=d)
    cnt = torch.empty(B, dtype=torch.int32, device=d)
    union = torch.empty((B, ld), dtype=torch.float32, device=d)
    api.fm_resident_mask(qds, dwk.kv(0, [0, 1, 2]), api.FM_UNION_MAX, 0.5, 0, 0, mask, ld, cnt,
                         None, n_pages, None, union)
    torch.cuda.synchronize()
    wl_ref = W.Workload(base.name, base.kv, refs)
    r = oracle.resident_mask(wl_ref)
    mg, ug = mask.cpu().numpy(), union.cpu().numpy().astype(np.float64)
    outside = 0
    for b in range(B):
        n = int(base.kv.seq_lens[b])
        ur = r["union"][b, :n]
        sc = np.max(np.abs(ur))
        assert np.max(np.abs(ug[b, :n] - ur)) <= TOL_LOW * sc, f"request {b}: union logits"
        clear = np.abs(ur) > TOL_LOW * sc
        assert np.array_equal(mg[b, :n][clear], r["mask"][b, :n][clear]), f"request {b}: mask"
        assert not mg[b, n:].any()
        outside += int(clear.sum())
    G.note("h128 encoder -> mask", entries_outside_band=outside,
           resident_fraction=float(r["mask"].mean()))
