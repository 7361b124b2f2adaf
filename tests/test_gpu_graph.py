"""The entry points inside a captured HIP graph.

A serving loop launches the decode step (scoring + top-512), two-level scoring, the Level-1
mask and the query encoder as graphs (label construction is captured alike).  Each graph here is captured once, then replayed several times with eager work
of the library and of torch in between; every replay must reproduce the eager result bit for
bit (the kernels are deterministic).  Nothing in these calls allocates or clears memory with a
memset, so they are safe to capture.
"""
import numpy as np
import pytest
import torch

from tests import gpu_util as G
from top_selection_fm_amd import api
from top_selection_fm_amd import workloads as W

pytestmark = pytest.mark.gpu


def _replays(graph, outs, refs, disturb, n=4):
    for i in range(n):
        for o in outs:
            o.fill_(0 if o.dtype != torch.float32 else float("nan"))   # eager, outside the graph
        disturb()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r) or (o.dtype == torch.float32 and
                                         torch.equal(torch.nan_to_num(o, nan=7.0),
                                                     torch.nan_to_num(r, nan=7.0))), f"replay {i}"


def test_decode_step_graph():
    wl = W.decode_bf16(seed=3001, B=4, seq_len=64 * 300 + 17, ragged=True)
    dw = api.DeviceWorkload(wl, "cuda:0")
    B = wl.kv.B
    ld = wl.kv.block_table.shape[1] * 64
    q, kv = dw.query(), dw.kv()
    ref_l = torch.empty((B, ld), dtype=torch.float32, device="cuda")
    ref_i = torch.empty((B, 512), dtype=torch.int32, device="cuda")
    api.fm_index_logits(q, kv, ref_l, ld)
    api.fm_topk512(ref_l, ld, B, None, None, 0, None, 512, ref_i, None, None, 0)
    torch.cuda.synchronize()
    lg = torch.empty_like(ref_l)
    ix = torch.empty_like(ref_i)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.fm_index_logits(q, kv, lg, ld)
        api.fm_topk512(lg, ld, B, None, None, 0, None, 512, ix, None, None, 0)
    scratch = torch.empty_like(ref_l)

    def disturb():
        api.fm_index_logits(q, kv, scratch, ld)          # the same kernels, eagerly
        torch.randn(1 << 20, device="cuda").sum()

    _replays(g, [lg, ix], [ref_l, ref_i], disturb)


def test_two_level_graph():
    wl = W.two_level_resident_fp8(seed=3002, B=4, seq_len=64 * 60 + 21, kmax=20, ragged=True)
    dw = api.DeviceWorkload(wl, "cuda:0")
    ref_i, ref_v = G.score_resident(dw)
    torch.cuda.synchronize()
    T = wl.queries[0].T
    res_ld = dw.resident_pages.shape[1]
    nb = api.fm_workspace_bytes(api.FM_OP_SCORE_RESIDENT, T, res_ld * 64)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ix = torch.empty_like(ref_i)
    vv = torch.empty_like(ref_v)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.fm_score_resident(dw.query(0), dw.kv(0), dw.resident_pages, dw.n_resident, res_ld,
                              512, ix, vv, ws, nb)

    def disturb():
        G.score_resident(dw)

    _replays(g, [ix, vv], [ref_i, ref_v], disturb)


def test_mask_graph():
    wl = W.three_layer_mask_fp8(seed=3003, B=3, seq_len=64 * 50 + 7, ragged=True)
    dw = api.DeviceWorkload(wl, "cuda:0")
    ref = G.resident_mask(dw)
    torch.cuda.synchronize()
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    B = wl.kv.B
    mask_ld = ref["mask"].shape[1]
    n_pages = ref["page_list"].shape[1]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.fm_resident_mask([dw.query(l) for l in range(3)], dw.kv(0), api.FM_UNION_MAX, 0.5, 0,
                             0, out["mask"], mask_ld, out["page_count"], out["page_list"],
                             n_pages, out["page_density"], out["union"])

    def disturb():
        G.resident_mask(dw)

    keys = ["mask", "page_count", "page_list", "page_density", "union"]
    _replays(g, [out[k] for k in keys], [ref[k] for k in keys], disturb)


def test_encoder_graph():
    """The query encoder (four launches) captured at a decode batch and at a tiled batch."""
    for T, kw in ((32, dict(n_heads=128, d_model=512, q_rank=256)),
                  (300, dict(n_heads=64, d_model=256, q_rank=1024))):
        e = W.query_encoder(seed=3010 + T, T=T, **kw)
        t = {k: torch.from_numpy(getattr(e, k).view(np.int16)).cuda()
             for k in ("hidden", "wq_a", "q_norm", "wq_b", "w_proj")}
        pos = torch.from_numpy(e.pos).cuda()
        desc = api.encoder_desc(t["wq_a"], t["q_norm"], t["wq_b"], t["w_proj"],
                                n_heads=e.n_heads, d_model=e.d_model, q_rank=e.q_rank)
        nb = api.fm_encode_workspace_bytes(desc, T)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        q = torch.empty((T, e.n_heads, 128), dtype=torch.bfloat16, device="cuda")
        w = torch.empty((T, e.n_heads), dtype=torch.float32, device="cuda")
        api.fm_encode_queries(desc, t["hidden"], T, pos, q, w, ws, nb)
        torch.cuda.synchronize()
        ref_q, ref_w = q.clone(), w.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            api.fm_encode_queries(desc, t["hidden"], T, pos, q, w, ws, nb)
        _replays(g, [q, w], [ref_q, ref_w], lambda: ws.fill_(0))


def test_golden_labels_graph():
    g0 = W.selector_scores(seed=3020, T=12, n_layers=5, ld=3000, pool=64, per_token=16)
    T, L, ld, tau = g0.T, g0.n_layers, g0.ld, 4
    S = torch.from_numpy(g0.scores).cuda()
    nv = torch.from_numpy(g0.n_valid).cuda()
    nb = api.fm_golden_workspace_bytes(T, L, ld, tau)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ptr = torch.empty(T - tau + 2, dtype=torch.int32, device="cuda")
    cap = (T - tau + 1) * ld
    idx = torch.empty(cap, dtype=torch.int32, device="cuda")
    sc = torch.empty(cap, dtype=torch.float32, device="cuda")
    api.fm_golden_labels(S, ld, T, L, nv, 0.6, 3, tau, ptr, idx, sc, cap, ws, nb)
    torch.cuda.synchronize()
    n = int(ptr[-1].item())
    ref = (ptr.clone(), idx[:n].clone(), sc[:n].clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.fm_golden_labels(S, ld, T, L, nv, 0.6, 3, tau, ptr, idx, sc, cap, ws, nb)
    for i in range(4):
        ptr.fill_(-1)
        idx.fill_(-1)
        sc.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ptr, ref[0]) and torch.equal(idx[:n], ref[1]) and torch.equal(sc[:n], ref[2]), f"replay {i}"
