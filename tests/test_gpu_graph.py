"""The entry points inside a captured HIP graph.

A serving loop launches the decode step (scoring + top-512), two-level scoring and the Level-1
mask as graphs.  Each graph here is captured once, then replayed several times with eager work
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
