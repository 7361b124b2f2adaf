"""fm_score_resident_noalloc (the library's static workspace) against fm_score_resident (a
caller-allocated workspace): the same kernels, so the outputs must be identical, bit for bit.
Calls in a row, the second with a smaller input (the static array keeps the first call's
contents) and the third with more rows again; then a call whose workspace would not fit the
static array is refused on the host.
"""
import numpy as np
import pytest
import torch

from tests import gpu_util as G
from top_selection_fm_amd import api
from top_selection_fm_amd import workloads as W

pytestmark = pytest.mark.gpu


def _noalloc(dw, k=512, resident_pages=None, n_resident=None):
    rp = dw.resident_pages if resident_pages is None else resident_pages
    nr = dw.n_resident if n_resident is None else n_resident
    T = dw.wl.queries[0].T
    idx = torch.full((T, k), -7, dtype=torch.int32, device=dw.device)
    val = torch.full((T, k), -7.0, dtype=torch.float32, device=dw.device)
    api.fm_score_resident_noalloc(dw.query(0), dw.kv(0), rp, nr, rp.shape[1], k, idx, val)
    return idx, val


def test_noalloc_matches_score_resident_twice():
    big = W.two_level_resident_fp8(seed=2050, B=30, seq_len=64 * 2000 + 17, kmax=384,
                                   shuffled=True, ragged=True)
    small = W.two_level_resident_fp8(seed=2051, B=3, seq_len=64 * 70 + 5, kmax=21, ragged=True)
    more = W.two_level_resident_fp8(seed=2053, B=40, seq_len=64 * 300 + 3, kmax=64, ragged=True)
    for tag, wl in (("30 requests x 384 pages", big), ("3 requests x 21 pages", small),
                    ("40 requests x 64 pages", more)):
        dw = api.DeviceWorkload(wl, "cuda:0")
        i_ref, v_ref = G.score_resident(dw)
        i_na, v_na = _noalloc(dw)
        torch.cuda.synchronize()
        assert torch.equal(i_na, i_ref), tag
        assert torch.equal(v_na.view(torch.int32), v_ref.view(torch.int32)), tag
        G.note("noalloc", case=tag, selected=int((i_ref >= 0).sum().item()))


def test_noalloc_rejects_too_large_on_the_host():
    wl = W.two_level_resident_fp8(seed=2052, B=2, seq_len=64 * 40, kmax=8)
    dw = api.DeviceWorkload(wl, "cuda:0")
    res_ld = (api.STATIC_SCRATCH_BYTES // (2 * 64 * 4)) + 64      # logits alone overflow it
    rp = torch.full((2, res_ld), -1, dtype=torch.int32, device="cuda:0")
    rp[:, :8] = dw.resident_pages
    idx = torch.full((2, 512), -7, dtype=torch.int32, device="cuda:0")
    with pytest.raises(api.FmError) as e:
        api.fm_score_resident_noalloc(dw.query(0), dw.kv(0), rp, dw.n_resident, res_ld, 512, idx)
    assert e.value.status == api.FM_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(idx == -7), "nothing may be launched on error"
