"""Exact-rational brute force for tiny indexer inputs (a pin for the fp64 oracle).

Independent of the oracle's C code: element values come from torch's own float8_e4m3fn /
bfloat16 / float32 decoders, turned into exact fractions, and the logit
sum_h w_h * max(0, q_h . k) is evaluated with Python's Fraction, so it carries no rounding
at all.  Only practical for a few thousand multiply-adds.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


def _exact(values_f32: np.ndarray):
    return [Fraction(float(v)) for v in np.asarray(values_f32, np.float64).reshape(-1)]


def decoded_keys(pool: np.ndarray, key_dtype: str, head_dim: int):
    """[rows, head_dim] exact fractions of a pool given as [pages, page, row]."""
    rows = pool.reshape(-1, pool.shape[-1])
    if key_dtype == "f32":
        vals = _exact(rows.astype(np.float32))
        return [vals[i * head_dim:(i + 1) * head_dim] for i in range(rows.shape[0])]
    if key_dtype == "bf16":
        f = torch.from_numpy(rows.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
        vals = _exact(f)
        return [vals[i * head_dim:(i + 1) * head_dim] for i in range(rows.shape[0])]
    codes = torch.from_numpy(rows[:, :head_dim].copy()).view(torch.float8_e4m3fn).float().numpy()
    scales = np.ascontiguousarray(rows[:, head_dim:head_dim + 4]).view("<f4").reshape(-1)
    out = []
    for i in range(rows.shape[0]):
        sc = Fraction(float(scales[i]))
        out.append([x * sc for x in _exact(codes[i])])
    return out


def decoded_queries(q: np.ndarray, q_dtype: str, q_scale=None):
    """[T][H][D] exact fractions."""
    T, H, D = q.shape
    if q_dtype == "f32":
        f = q.astype(np.float32)
    elif q_dtype == "bf16":
        f = torch.from_numpy(q.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    else:
        f = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).float().numpy()
    out = []
    for t in range(T):
        sc = Fraction(1) if q_scale is None else Fraction(float(q_scale[t]))
        out.append([[Fraction(float(x)) * sc for x in f[t, h]] for h in range(H)])
    return out


def decoded_weights(w: np.ndarray, w_dtype: str):
    if w_dtype == "f32":
        f = w.astype(np.float32)
    else:
        f = torch.from_numpy(w.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    return [[Fraction(float(x)) for x in row] for row in f]


def logit(qt, wt, k) -> Fraction:
    total = Fraction(0)
    for h in range(len(qt)):
        dot = sum((a * b for a, b in zip(qt[h], k)), Fraction(0))
        if dot > 0:
            total += wt[h] * dot
    return total


def logits_logical(wl, layer: int = 0):
    """Exact logits [T][s] for every row over every mapped entry below seq_len (no causal
    cut: callers apply visibility themselves).  Keys are looked up page by page through the
    block table."""
    kv, qq = wl.kv, wl.queries[layer]
    P = kv.pools[layer].shape[1]
    D = qq.q.shape[2]
    keys = decoded_keys(kv.pools[layer], kv.key_dtype, D)
    Q = decoded_queries(qq.q, qq.q_dtype, qq.q_scale)
    Wt = decoded_weights(qq.w, qq.w_dtype)
    out = []
    for t in range(qq.q.shape[0]):
        b = int(qq.row_req[t]) if qq.row_req is not None else (0 if kv.B == 1 else t)
        row = []
        for s in range(int(kv.seq_lens[b])):
            phys = int(kv.block_table[b, s // P])
            row.append(None if phys < 0 else logit(Q[t], Wt[t], keys[phys * P + s % P]))
        out.append(row)
    return out
