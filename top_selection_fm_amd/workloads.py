"""Seeded synthetic inputs for the compressed-key indexer (scoring + selection).

Every generator draws its random numbers from NumPy's PCG64 with a fixed seed, encodes them
in the storage formats the indexer consumes, and lays the keys out as a paged pool reached
through a block table:

* bf16 values are the round-to-nearest-even upper halves of float32 draws;
* fp8 keys use the 132-byte compressed-key row of the FlashMemory-DeepSeek-V4 README
  ("compressed_k format" table): 128 OCP E4M3FN codes, then a little-endian float32
  per-entry dequantisation scale.  The generator picks scale = absmax / 448 per row, the
  E4M3FN maximum, so every code is finite;
* a page holds 64 compressed entries (README, "Key optimizations": page-granular recall,
  and "Per-decode-token FLOPs": KMAX x 64 chunks).

The module holds none of the indexer's arithmetic (no scoring, thresholding or selection):
the oracle tests and the HIP library both take their inputs from here, so it is the one
piece of code the two sides share.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

PAGE = 64          # compressed entries per page
HEADS = 64         # indexer heads (DeepSeek-V4 C4Indexer: index_n_heads)
DIM = 128          # indexer head dimension
ROW_FP8 = DIM + 4  # 132-byte compressed-key row
E4M3_MAX = 448.0
POISON_CODE = 0x7F                    # an E4M3FN NaN code
POISON_SCALE = np.uint32(0x7FC00000)  # float32 quiet NaN


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------------------- encodings
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 already scaled into [-448, 448] -> OCP E4M3FN codes (uint8), RNE."""
    x = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp8_rows(x: np.ndarray, chunk: int = 1 << 20) -> np.ndarray:
    """float32 [..., 128] -> 132-byte rows [..., 132]: E4M3 codes of x/scale, then scale."""
    x = np.asarray(x, dtype=np.float32)
    lead = x.shape[:-1]
    flat = x.reshape(-1, DIM)
    out = np.empty((flat.shape[0], ROW_FP8), np.uint8)
    for a in range(0, flat.shape[0], chunk):
        blk = flat[a:a + chunk]
        absmax = np.abs(blk).max(axis=1)
        scale = np.where(absmax > 0, absmax / np.float32(E4M3_MAX), np.float32(1.0)).astype("<f4")
        out[a:a + chunk, :DIM] = e4m3_codes(blk / scale[:, None])
        out[a:a + chunk, DIM:] = np.ascontiguousarray(scale)[:, None].view(np.uint8)
    return out.reshape(lead + (ROW_FP8,))


def fp8_tokens(x: np.ndarray):
    """float32 [T, H, D] -> (E4M3 codes [T, H, D], per-token float32 scale [T])."""
    x = np.asarray(x, dtype=np.float32)
    absmax = np.abs(x.reshape(x.shape[0], -1)).max(axis=1)
    scale = np.where(absmax > 0, absmax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    return e4m3_codes(x / scale[:, None, None]), scale


# ----------------------------------------------------------------------------- containers
@dataclass
class KeyPool:
    """Paged compressed-key pool(s); every layer's pool shares one block table."""
    pools: list                 # per layer: [n_phys_pages, PAGE, row] float32 | uint16 | uint8
    key_dtype: str              # 'f32' | 'bf16' | 'fp8x132'
    block_table: np.ndarray     # int32 [B, max_pages]; -1 marks a page that is not mapped
    seq_lens: np.ndarray        # int32 [B]

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def n_phys_pages(self) -> int:
        return int(self.pools[0].shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.B else 0

    @property
    def nbytes(self) -> int:
        return int(sum(p.nbytes for p in self.pools))


@dataclass
class Queries:
    """One layer's query rows: q [T, H, D], head weights w [T, H]."""
    q: np.ndarray               # float32 | uint16 (bf16 bits) | uint8 (E4M3 codes)
    q_dtype: str                # 'f32' | 'bf16' | 'fp8'
    w: np.ndarray               # float32 | uint16 (bf16 bits)
    w_dtype: str                # 'f32' | 'bf16'
    q_scale: np.ndarray | None = None   # float32 [T] (fp8 q only)
    row_req: np.ndarray | None = None   # int32 [T]; None: row t is request t
    q_pos: np.ndarray | None = None     # int32 [T] absolute token positions; None: no causal cut
    compress_ratio: int = 4
    row_pool: np.ndarray | None = None  # int32 [T] key layer of row t; None: layer 0

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_heads(self) -> int:
        return int(self.q.shape[1])


@dataclass
class Workload:
    name: str
    kv: KeyPool
    queries: list                               # one Queries per layer
    resident_pages: np.ndarray | None = None    # int32 [B, res_ld] logical page ids
    n_resident: np.ndarray | None = None        # int32 [B]
    meta: dict = field(default_factory=dict)


# ----------------------------------------------------------------------------- helpers
def _normal(rng, shape, mean=0.0, std=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def _keys_f32(rng, n_pages) -> np.ndarray:
    return _normal(rng, (n_pages, PAGE, DIM), std=1.0 / np.sqrt(DIM))


def _unit(v: np.ndarray) -> np.ndarray:
    n = np.linalg.norm(v, axis=-1, keepdims=True)
    return (v / np.where(n > 0, n, 1.0)).astype(np.float32)


def _ragged_lens(rng, B, seq_len, ragged) -> np.ndarray:
    if not ragged:
        return np.full(B, seq_len, np.int32)
    cut = rng.integers(0, 3 * PAGE, size=B)
    return np.maximum(seq_len - cut, 1).astype(np.int32)


def _clear_tail(pool: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray) -> None:
    """Zero the storage of entries past each request's length (never part of any result)."""
    for b, n in enumerate(seq_lens):
        p, r = divmod(int(n), PAGE)
        if r and p < block_table.shape[1] and block_table[b, p] >= 0:
            pool[block_table[b, p], r:] = 0


# ----------------------------------------------------------------------------- workloads
def tiny_single_query(seed: int = 1001, n_entries: int = 4096, heads: int = HEADS) -> Workload:
    """One fp32 query row over n_entries fp32 keys; w ~ N(-0.05, 0.125)."""
    rng = make_rng(seed)
    q = _normal(rng, (1, heads, DIM), std=1.0 / np.sqrt(DIM))
    w = _normal(rng, (1, heads), mean=-0.05, std=0.125)
    n_pages = -(-n_entries // PAGE)
    keys = _keys_f32(rng, n_pages)
    kv = KeyPool([keys], "f32", np.arange(n_pages, dtype=np.int32)[None, :],
                 np.array([n_entries], np.int32))
    _clear_tail(keys, kv.block_table, kv.seq_lens)
    return Workload("tiny_single_query_f32", kv, [Queries(q, "f32", w, "f32")],
                    meta=dict(entries=n_entries))


def decode_bf16(seed: int = 1002, B: int = 32, seq_len: int = 65536, hot_frac: float = 0.10,
                hot_offset: float = 0.5, ragged: bool = False) -> Workload:
    """B decode rows (one token each) over bf16 keys in a shared, randomly permuted pool.

    A fraction hot_frac of each request's pages is planted 'hot': their keys are shifted by
    hot_offset along the unit direction of the mean of that request's 64 query heads.
    """
    rng = make_rng(seed)
    q32 = _normal(rng, (B, HEADS, DIM), std=1.0 / np.sqrt(DIM))
    w32 = _normal(rng, (B, HEADS), mean=0.05, std=0.125)
    qb, wb = bf16_bits(q32), bf16_bits(w32)
    seq_lens = _ragged_lens(rng, B, seq_len, ragged)
    ppr = -(-seq_len // PAGE)
    n_phys = B * ppr
    bt = rng.permutation(n_phys).astype(np.int32).reshape(B, ppr)
    n_hot = int(round(hot_frac * ppr))
    hot = np.stack([np.sort(rng.choice(ppr, n_hot, replace=False)) for _ in range(B)]) \
        if n_hot else np.zeros((B, 0), np.int64)
    keys = _keys_f32(rng, n_phys)
    d = _unit(bf16_values(qb).mean(axis=1))                       # [B, D]
    for b in range(B):
        keys[bt[b, hot[b]]] += np.float32(hot_offset) * d[b]
    pool = bf16_bits(keys)
    del keys
    _clear_tail(pool, bt, seq_lens)
    kv = KeyPool([pool], "bf16", bt, seq_lens)
    return Workload(f"decode_bf16_b{B}_s{seq_len}", kv, [Queries(qb, "bf16", wb, "bf16")],
                    meta=dict(hot_pages=hot.astype(np.int32), entries=int(seq_lens.sum())))


def three_layer_mask_fp8(seed: int = 1003, B: int = 8, seq_len: int = 262144,
                         n_layers: int = 3, hot_frac: float = 0.12, cluster: int = 8,
                         hot_offset: float = 0.75, w_bias: float = -0.085,
                         shared_keys: bool = False, ragged: bool = False,
                         heads: int = HEADS) -> Workload:
    """Level-1 residency workload: n_layers query encoders over per-layer fp8 key pools.

    The pools share one permuted block table.  Each request has the same set of hot pages in
    every layer, grouped in runs of `cluster` contiguous logical pages.  Layer l's head
    weights are w0 - mean(w0) + w_bias with w0 ~ N(0, 0.125), so every row's weights sum to
    heads*w_bias; hot keys are shifted by hot_offset along the unit direction of sum_h w_h q_h
    of that layer and request.  With the defaults about 12% of entries end up resident.
    """
    rng = make_rng(seed)
    seq_lens = _ragged_lens(rng, B, seq_len, ragged)
    ppr = -(-seq_len // PAGE)
    n_phys = B * ppr
    bt = rng.permutation(n_phys).astype(np.int32).reshape(B, ppr)
    n_slots = ppr // cluster
    n_clusters = min(n_slots, int(round(hot_frac * ppr / cluster)))
    hot = []
    for _ in range(B):
        starts = np.sort(rng.choice(n_slots, n_clusters, replace=False)) * cluster
        hot.append((starts[:, None] + np.arange(cluster)[None, :]).reshape(-1))
    hot = np.stack(hot).astype(np.int32)
    queries, dirs = [], []
    for _ in range(n_layers):
        q32 = _normal(rng, (B, heads, DIM), std=1.0 / np.sqrt(DIM))
        w0 = _normal(rng, (B, heads), std=0.125)
        w32 = (w0 - w0.mean(axis=1, keepdims=True) + np.float32(w_bias)).astype(np.float32)
        qb, wb = bf16_bits(q32), bf16_bits(w32)
        queries.append(Queries(qb, "bf16", wb, "bf16"))
        dirs.append(_unit(np.einsum("bh,bhd->bd", bf16_values(wb), bf16_values(qb))))
    pools = []
    n_pools = 1 if shared_keys else n_layers
    for l in range(n_pools):
        keys = _keys_f32(rng, n_phys)
        d = _unit(sum(dirs)) if shared_keys else dirs[l]
        for b in range(B):
            keys[bt[b, hot[b]]] += np.float32(hot_offset) * d[b]
        pool = fp8_rows(keys)
        del keys
        _clear_tail(pool, bt, seq_lens)
        pools.append(pool)
    if shared_keys:
        pools = pools * n_layers
    kv = KeyPool(pools, "fp8x132", bt, seq_lens)
    return Workload(f"three_layer_mask_fp8_b{B}_s{seq_len}", kv, queries,
                    meta=dict(hot_pages=hot, shared_keys=shared_keys,
                              entries=int(seq_lens.sum())))


def mode_a_fp8(seed: int = 1009, B: int = 8, seq_len: int = 262144, n_layers: int = 21,
               ragged: bool = False) -> Workload:
    """Mode A: a Level-1 mask from three encoders, then Level-2 rows of n_layers layers.

    pools[0..2] and queries[0..2] are three_layer_mask_fp8(seed, B, seq_len) (the encoders
    that decide residency).  pools[3 + l] is layer l's own fp8 key pool: encoder pool l mod 3
    with its physical pages permuted by a seeded permutation, so each layer holds different
    keys at every entry (no hot structure is planted for Level 2).  queries[3] holds the
    n_layers * B Level-2 rows, layer-major: row l*B + b has row_req b and row_pool 3 + l;
    q ~ N(0, 1/sqrt(128)) and w ~ N(0.05, 0.125) per head, as in decode_bf16.
    """
    base = three_layer_mask_fp8(seed, B=B, seq_len=seq_len, ragged=ragged)
    rng = make_rng(seed + 7919)
    kv = base.kv
    pools = list(kv.pools)
    for l in range(n_layers):
        perm = rng.permutation(kv.n_phys_pages)
        pool = pools[l % 3][perm]
        _clear_tail(pool, kv.block_table, kv.seq_lens)
        pools.append(pool)
    T = n_layers * B
    q32 = _normal(rng, (T, HEADS, DIM), std=1.0 / np.sqrt(DIM))
    w32 = _normal(rng, (T, HEADS), mean=0.05, std=0.125)
    rows = np.arange(T, dtype=np.int32)
    level2 = Queries(bf16_bits(q32), "bf16", bf16_bits(w32), "bf16", row_req=rows % B,
                     row_pool=3 + rows // B)
    meta = dict(base.meta, n_layers=n_layers, level2_rows=T)
    return Workload(f"mode_a_fp8_b{B}_l{n_layers}_s{seq_len}",
                    KeyPool(pools, "fp8x132", kv.block_table, kv.seq_lens),
                    list(base.queries) + [level2], meta=meta)


def two_level_resident_fp8(seed: int = 1004, B: int = 30, seq_len: int = 262144,
                           kmax: int = 384, shuffled: bool = False, poison: bool = True,
                           ragged: bool = False, heads: int = HEADS) -> Workload:
    """Level-2 scoring restricted to kmax resident pages per request (fp8 keys).

    The pool holds every logical page of every request (permuted).  With poison=True the
    pages outside the resident lists hold NaN codes and NaN scales and their block-table
    entries are -1, so a result that touched one of them would show it.
    """
    rng = make_rng(seed)
    q32 = _normal(rng, (B, heads, DIM), std=1.0 / np.sqrt(DIM))
    w32 = _normal(rng, (B, heads), mean=0.05, std=0.125)
    qb, wb = bf16_bits(q32), bf16_bits(w32)
    seq_lens = _ragged_lens(rng, B, seq_len, ragged)
    ppr = -(-seq_len // PAGE)
    n_phys = B * ppr
    bt = rng.permutation(n_phys).astype(np.int32).reshape(B, ppr)
    res = np.full((B, kmax), -1, np.int32)
    n_res = np.zeros(B, np.int32)
    for b in range(B):
        n_pages_b = -(-int(seq_lens[b]) // PAGE)
        sel = np.sort(rng.choice(n_pages_b, min(kmax, n_pages_b), replace=False))
        if shuffled:
            sel = rng.permutation(sel)
        res[b, :sel.size] = sel
        n_res[b] = sel.size
    if poison:
        pool = np.full((n_phys, PAGE, ROW_FP8), POISON_CODE, np.uint8)
        pool[:, :, DIM:] = np.array([POISON_SCALE], "<u4").view(np.uint8)
    else:
        pool = np.empty((n_phys, PAGE, ROW_FP8), np.uint8)
    phys = np.concatenate([bt[b, res[b, :n_res[b]]] for b in range(B)])
    if not poison:
        phys = np.arange(n_phys)
    pool[phys] = fp8_rows(_keys_f32(rng, phys.size))
    _clear_tail(pool, bt, seq_lens)
    if poison:
        mapped = np.zeros_like(bt, dtype=bool)
        for b in range(B):
            mapped[b, res[b, :n_res[b]]] = True
        bt = np.where(mapped, bt, -1).astype(np.int32)
    kv = KeyPool([pool], "fp8x132", bt, seq_lens)
    return Workload(f"two_level_resident_fp8_b{B}_s{seq_len}_k{kmax}", kv,
                    [Queries(qb, "bf16", wb, "bf16")], resident_pages=res, n_resident=n_res,
                    meta=dict(entries=int(n_res.sum()) * PAGE, poison=poison,
                              shuffled=shuffled))


def prefill_causal_fp8(seed: int = 1005, T: int = 4096, pos0: int = 131072,
                       seq_len: int = 33792, ratio: int = 4) -> Workload:
    """T prefill rows of one request at positions pos0 + i over seq_len fp8 keys.

    Row i may use entries s < floor((pos0 + i) / ratio) (and s < seq_len).  q is E4M3 with a
    per-token scale (absmax / 448); keys are 132-byte rows; w ~ N(0.05, 0.125) in bf16.
    """
    rng = make_rng(seed)
    q32 = _normal(rng, (T, HEADS, DIM), std=1.0 / np.sqrt(DIM))
    codes, qs = fp8_tokens(q32)
    del q32
    w32 = _normal(rng, (T, HEADS), mean=0.05, std=0.125)
    n_pages = -(-seq_len // PAGE)
    pool = fp8_rows(_keys_f32(rng, n_pages))
    bt = np.arange(n_pages, dtype=np.int32)[None, :]
    seq_lens = np.array([seq_len], np.int32)
    _clear_tail(pool, bt, seq_lens)
    kv = KeyPool([pool], "fp8x132", bt, seq_lens)
    qry = Queries(codes, "fp8", bf16_bits(w32), "bf16", q_scale=qs,
                  row_req=np.zeros(T, np.int32),
                  q_pos=(pos0 + np.arange(T)).astype(np.int32), compress_ratio=ratio)
    return Workload(f"prefill_causal_fp8_t{T}_s{seq_len}", kv, [qry],
                    meta=dict(pos0=pos0))


class EncoderInputs:
    """Synthetic inputs of the retriever's query encoder (bf16 bit patterns, uint16)."""

    def __init__(self, name, hidden, pos, wq_a, q_norm, wq_b, w_proj, n_heads):
        self.name = name
        self.hidden, self.pos = hidden, pos
        self.wq_a, self.q_norm, self.wq_b, self.w_proj = wq_a, q_norm, wq_b, w_proj
        self.n_heads = n_heads
        self.T, self.d_model = hidden.shape
        self.q_rank = wq_a.shape[0]


def query_encoder(seed: int = 1007, T: int = 32, n_heads: int = 128, d_model: int = 4096,
                  q_rank: int = 2048, max_pos: int = 1 << 20) -> EncoderInputs:
    """The encoder at the page's sizes (d_model 4096, q_rank 2048, head_dim 128): random
    Linear weights with 1/sqrt(fan_in) scale, an RMSNorm weight near 1, unit-normal hidden
    states, positions uniform over a 1M-token context."""
    rng = make_rng(seed)
    hidden = bf16_bits(_normal(rng, (T, d_model)))
    wq_a = bf16_bits(_normal(rng, (q_rank, d_model), std=1.0 / np.sqrt(d_model)))
    q_norm = bf16_bits(_normal(rng, (q_rank,), mean=1.0, std=0.05))
    wq_b = bf16_bits(_normal(rng, (n_heads * DIM, q_rank), std=1.0 / np.sqrt(q_rank)))
    w_proj = bf16_bits(_normal(rng, (n_heads, d_model), std=1.0 / np.sqrt(d_model)))
    pos = rng.integers(0, max_pos, size=T).astype(np.int32)
    return EncoderInputs(f"query_encoder_t{T}_h{n_heads}_d{d_model}_r{q_rank}", hidden, pos,
                         wq_a, q_norm, wq_b, w_proj, n_heads)


class SelectorScores:
    """Future native-selector scores for golden-label construction: S [T, n_layers, ld] float32
    and n_valid [T] (token i sees the compressed entries below n_valid[i])."""

    def __init__(self, name, scores, n_valid):
        self.name = name
        self.scores = scores
        self.n_valid = n_valid

    @property
    def T(self) -> int:
        return int(self.scores.shape[0])

    @property
    def n_layers(self) -> int:
        return int(self.scores.shape[1])

    @property
    def ld(self) -> int:
        return int(self.scores.shape[2])


def selector_scores(seed: int = 1008, T: int = 128, n_layers: int = 21, ld: int = 65536,
                    pool: int = 256, per_token: int = 48, layer_frac: float = 0.7,
                    boost=(7.0, 11.0), causal: bool = True) -> SelectorScores:
    """Synthetic selector scores of T consecutive future tokens over ld compressed entries.

    Every score is N(0, 1); each token attends to per_token entries drawn from a persistent pool
    of `pool` entries, and each layer boosts a random layer_frac of those by U(boost) -- so a few
    dozen entries carry most of each token's softmax mass, the layers mostly agree, and the
    window's union stays in the hundreds.  With causal=True token i sees
    ld - (T - 1 - i) // 4 entries (one more compressed entry every 4 tokens); the scores past
    that stay in the array and are not candidates.
    """
    rng = make_rng(seed)
    S = rng.standard_normal((T, n_layers, ld), dtype=np.float32)
    hot_pool = rng.choice(ld, size=min(pool, ld), replace=False)
    for i in range(T):
        hot = rng.choice(hot_pool, size=min(per_token, hot_pool.size), replace=False)
        for l in range(n_layers):
            sel = hot[rng.random(hot.size) < layer_frac]
            S[i, l, sel] += rng.uniform(boost[0], boost[1], sel.size).astype(np.float32)
    if causal:
        n_valid = (ld - (T - 1 - np.arange(T)) // 4).astype(np.int32)
    else:
        n_valid = np.full(T, ld, np.int32)
    n_valid = np.maximum(n_valid, 0)
    return SelectorScores(f"selector_scores_t{T}_l{n_layers}_n{ld}", S, n_valid)
