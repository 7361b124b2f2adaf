"""GPU parity of the query encoder (fm_encode_queries) against the fp64 oracle.

Tolerances (derived from the arithmetic):
  * q: the GPU rounds r = RMSNorm(a) to bf16 before the second product and q to bf16 at the
    end (relative 2^-9 each), and accumulates in float32.  Both roundings act like independent
    relative errors of about 2^-9 on terms of similar size, so per (row, head) the error stays
    within 1e-2 of that head's largest |q| (the bound bf16 logits are held to);
  * w: bf16 x bf16 products are exact in float32 and only the float32 sums round, so w agrees
    to 1e-4 of the row's largest |w|.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import encoder as OE
from tests import gpu_util as G
from top_selection_fm_amd import api
from top_selection_fm_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL_Q = 1e-2
TOL_W = 1e-4


def run_encoder(e: W.EncoderInputs, **rope):
    dev = "cuda:0"
    t = {k: torch.from_numpy(getattr(e, k).view(np.int16)).to(dev)
         for k in ("hidden", "wq_a", "q_norm", "wq_b", "w_proj")}
    pos = torch.from_numpy(e.pos).to(dev)
    desc = api.encoder_desc(t["wq_a"], t["q_norm"], t["wq_b"], t["w_proj"], n_heads=e.n_heads,
                            d_model=e.d_model, q_rank=e.q_rank, **rope)
    nb = api.fm_encode_workspace_bytes(desc, e.T)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    q = torch.empty((e.T, e.n_heads, 128), dtype=torch.bfloat16, device=dev)
    w = torch.empty((e.T, e.n_heads), dtype=torch.float32, device=dev)
    api.fm_encode_queries(desc, t["hidden"], e.T, pos, q, w, ws, nb)
    torch.cuda.synchronize()
    return q.float().cpu().numpy(), w.cpu().numpy()


def oracle_encoder(e: W.EncoderInputs, rows=None, **rope):
    rows = np.arange(e.T) if rows is None else np.asarray(rows)
    kw = {k: v for k, v in rope.items()}
    if "rope_orig_len" in kw:
        kw["rope_orig_len"] = int(kw["rope_orig_len"])
    return OE.encode(e.hidden[rows], e.pos[rows], e.wq_a, e.q_norm, e.wq_b, e.w_proj,
                     n_heads=e.n_heads, **kw)


def check(tag, qg, wg, qr, wr):
    scale_q = np.max(np.abs(qr), axis=2, keepdims=True)
    err_q = np.max(np.abs(qg - qr) / np.maximum(scale_q, 1e-30))
    scale_w = np.max(np.abs(wr), axis=1, keepdims=True)
    err_w = np.max(np.abs(wg - wr) / np.maximum(scale_w, 1e-30))
    G.note(tag, q_err=err_q, w_err=err_w)
    assert err_q <= TOL_Q, f"{tag}: q error {err_q:.3g}"
    assert err_w <= TOL_W, f"{tag}: w error {err_w:.3g}"


@pytest.mark.parametrize("rope", [{}, {"rope_dim": 0}, {"rope_factor": 1.0},
                                  {"rope_dim": 128, "rope_base": 10000.0}])
def test_encoder_small_ragged(rope):
    """45 rows (two 32-row tiles, the second ragged), 32 heads, small model dims."""
    e = W.query_encoder(seed=3101, T=45, n_heads=32, d_model=96, q_rank=64)
    qg, wg = run_encoder(e, **rope)
    qr, wr = oracle_encoder(e, **rope)
    check(f"encoder small {rope}", qg, wg, qr, wr)


@pytest.mark.parametrize("n_heads", [128, 64])
def test_encoder_page_sizes(n_heads):
    """The page's sizes (d_model 4096, q_rank 2048, RoPE on 64 dims), decode-sized batch."""
    e = W.query_encoder(seed=3102, T=32, n_heads=n_heads)
    qg, wg = run_encoder(e)
    qr, wr = oracle_encoder(e)
    check(f"encoder page sizes h{n_heads}", qg, wg, qr, wr)


def test_encoder_many_rows_sampled():
    """2,080 rows (65 row tiles, a single split of K): sampled rows against the oracle, and a
    second call bit-identical to the first."""
    e = W.query_encoder(seed=3103, T=2080, n_heads=64, d_model=1024, q_rank=512)
    qg, wg = run_encoder(e)
    rows = np.array([0, 1, 31, 32, 1000, 2047, 2048, 2079])
    qr, wr = oracle_encoder(e, rows=rows)
    check("encoder 2080 rows (sampled)", qg[rows], wg[rows], qr, wr)
    qg2, wg2 = run_encoder(e)
    assert np.array_equal(qg, qg2) and np.array_equal(wg, wg2)


def test_encoder_prefill_tiled_products():
    """1,000 rows: d_model 528 leaves a 16-wide K tail, so the first product takes the
    register-staged 128 x 128 tiles (the last row tile and, with 2,112 columns, the last column
    tile partial; its columns straddle the wq_a / w_proj boundary inside a tile); the second
    (8,192 columns) takes the direct-copy 128 x 128 tiles, 512 of them."""
    e = W.query_encoder(seed=3106, T=1000, n_heads=64, d_model=528, q_rank=2048)
    qg, wg = run_encoder(e)
    rows = np.array([0, 1, 127, 128, 255, 500, 896, 999])
    qr, wr = oracle_encoder(e, rows=rows)
    check("encoder 1000 rows tiled (sampled)", qg[rows], wg[rows], qr, wr)


def test_encoder_prefill_wide_tiles():
    """600 rows x 256 heads: the second product (32,768 columns) takes the 128 x 256
    direct-copy tiles (a partial last row tile), with three LDS stages."""
    e = W.query_encoder(seed=3107, T=600, n_heads=256, d_model=256, q_rank=512)
    qg, wg = run_encoder(e)
    rows = np.array([0, 63, 64, 127, 128, 300, 511, 512, 599])
    qr, wr = oracle_encoder(e, rows=rows)
    check("encoder 600 rows x 256 heads, wide tiles (sampled)", qg[rows], wg[rows], qr, wr)


@pytest.mark.timeout(300)
def test_encoder_benchmarked_shape_sampled():
    """The benchmarked prefill call: 4,096 rows at the page's sizes (d_model 4,096, q_rank
    2,048, 128 heads), the same seeded inputs: sampled rows from every 256-row tile group
    against the oracle.  Both products take the 256 x 256 direct-copy tiles; the first has 144
    of them (2,176 columns: the last column tile holds the 128 w_proj columns and is half
    full)."""
    e = W.query_encoder(T=4096)
    qg, wg = run_encoder(e)
    rows = np.array([0, 1, 255, 256, 1000, 2047, 2048, 3071, 3072, 4094, 4095])
    qr, wr = oracle_encoder(e, rows=rows)
    check("encoder 4096 rows at the page's sizes (sampled)", qg[rows], wg[rows], qr, wr)


def test_encoder_prefill_256_tiles():
    """1,100 rows x 256 heads: the second product (32,768 columns, 640 tiles of 256 x 256) takes
    the eight-wave 256 x 256 tiles, the last row tile holding 76 rows."""
    e = W.query_encoder(seed=3109, T=1100, n_heads=256, d_model=256, q_rank=512)
    qg, wg = run_encoder(e)
    rows = np.array([0, 63, 64, 255, 256, 700, 1023, 1024, 1099])
    qr, wr = oracle_encoder(e, rows=rows)
    check("encoder 1100 rows x 256 heads, 256 x 256 tiles (sampled)", qg[rows], wg[rows], qr, wr)


@pytest.mark.parametrize("T,n_heads,d_model,q_rank", [
    (300, 64, 32, 96),      # both products 128 x 128: one k slab (the first), three (the second)
    (600, 256, 32, 32),     # one k slab each; the second product on 128 x 256 tiles
    (1100, 256, 64, 160),   # the second product on 256 x 256 tiles: one round of slabs + one
    (2100, 64, 96, 4000),   # the first on 256 x 256 tiles (3 slabs), the second on 128 x 256
])                          # (125 slabs: 41 rounds of three + two)
def test_encoder_direct_copy_slab_tails(T, n_heads, d_model, q_rank):
    """The direct-copy products when K has fewer 32-wide slabs than the kernel has LDS stages,
    or leaves a partial round of them, and when the wq_a / w_proj boundary (column q_rank)
    falls inside a column tile rather than on a tile edge; partial row and column tiles."""
    e = W.query_encoder(seed=3120 + q_rank, T=T, n_heads=n_heads, d_model=d_model, q_rank=q_rank)
    qg, wg = run_encoder(e)
    rows = np.unique(np.array([0, 1, 127, 128, 255, 256, T // 2, T - 2, T - 1]))
    qr, wr = oracle_encoder(e, rows=rows)
    check(f"encoder {T} x {n_heads} heads, d_model {d_model}, q_rank {q_rank} (sampled)",
          qg[rows], wg[rows], qr, wr)


@pytest.mark.parametrize("T", [255, 256, 257])
def test_encoder_around_the_tiled_threshold(T):
    """The second product: 255 rows take the per-32x32-tile kernel, 256 and 257 the LDS-tiled
    one; RoPE/Hadamard takes one head a wave, then 16."""
    e = W.query_encoder(seed=3108 + T, T=T, n_heads=64, d_model=256, q_rank=2048)
    qg, wg = run_encoder(e)
    rows = np.array([0, 127, 128, T - 2, T - 1])
    qr, wr = oracle_encoder(e, rows=rows)
    check(f"encoder {T} rows (sampled)", qg[rows], wg[rows], qr, wr)


def test_encoder_feeds_scoring():
    """Encoder (64 heads) -> fm_index_logits on a small bf16 pool, against the oracle encoder's
    q and w (rounded to float32) scored by the oracle: the whole per-layer path."""
    e = W.query_encoder(seed=3104, T=3, n_heads=64, d_model=256, q_rank=128)
    dev = "cuda:0"
    t = {k: torch.from_numpy(getattr(e, k).view(np.int16)).to(dev)
         for k in ("hidden", "wq_a", "q_norm", "wq_b", "w_proj")}
    desc = api.encoder_desc(t["wq_a"], t["q_norm"], t["wq_b"], t["w_proj"], n_heads=64,
                            d_model=e.d_model, q_rank=e.q_rank)
    nb = api.fm_encode_workspace_bytes(desc, e.T)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    q = torch.empty((e.T, 64, 128), dtype=torch.bfloat16, device=dev)
    w = torch.empty((e.T, 64), dtype=torch.float32, device=dev)
    api.fm_encode_queries(desc, t["hidden"], e.T, torch.from_numpy(e.pos).to(dev), q, w, ws, nb)

    wl = W.decode_bf16(seed=3105, B=3, seq_len=64 * 9 + 5, ragged=True)
    dw = api.DeviceWorkload(wl, dev)
    kv = dw.kv(0, [0])
    qd = api.QueryDesc(q.data_ptr(), api.FM_BF16, None, w.data_ptr(), api.FM_F32, e.T, 64,
                       None, None, 1)
    ld = wl.kv.block_table.shape[1] * 64
    L = torch.empty((e.T, ld), dtype=torch.float32, device=dev)
    api.fm_index_logits(qd, kv, L, ld)
    torch.cuda.synchronize()

    qr, wr = oracle_encoder(e)
    wl_ref = W.Workload(wl.name, wl.kv, [W.Queries(qr.astype(np.float32), "f32",
                                                   wr.astype(np.float32), "f32")])
    Lr = oracle.logits(wl_ref)
    err = G.check_logits(L.cpu().numpy(), Lr, 2e-2, "encoder -> scoring")
    G.note("encoder -> scoring", logit_err=err)
