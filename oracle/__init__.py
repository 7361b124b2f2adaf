"""fp64 CPU oracle for compressed-key indexer scoring and selection (ctypes binding).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP library
(``top_selection_fm_amd``); the two meet only in the seeded input generators
(``top_selection_fm_amd.workloads``), which hold none of the indexer's arithmetic.

The C source (``fm_oracle.c``) states, step by step, which passage of the pages each part
follows.  Every function here marshals NumPy arrays and calls it; nothing is computed in
Python except argument checks.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fm_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

O_F32, O_BF16, O_FP8, O_FP8X132 = 0, 1, 2, 3
_KEY_DT = {"f32": O_F32, "bf16": O_BF16, "fp8x132": O_FP8X132}
_Q_DT = {"f32": O_F32, "bf16": O_BF16, "fp8": O_FP8}
UNION = {"max": 0, "mean": 1}
MAX_LAYERS = 8


def build() -> str:
    """Compile fm_oracle.c with gcc (plain -O2, OpenMP over independent rows)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                           "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


class _KV(C.Structure):
    _fields_ = [("pool", C.c_void_p * MAX_LAYERS), ("n_pools", C.c_int), ("key_dtype", C.c_int),
                ("page_size", C.c_int), ("head_dim", C.c_int), ("block_table", C.c_void_p),
                ("bt_ld", C.c_int64), ("seq_lens", C.c_void_p), ("B", C.c_int),
                ("n_phys_pages", C.c_int64)]


class _Q(C.Structure):
    _fields_ = [("q", C.c_void_p), ("q_dtype", C.c_int), ("q_scale", C.c_void_p),
                ("w", C.c_void_p), ("w_dtype", C.c_int), ("T", C.c_int), ("n_heads", C.c_int),
                ("row_req", C.c_void_p), ("q_pos", C.c_void_p), ("compress_ratio", C.c_int)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = C.CDLL(_SO)
        P = C.c_void_p
        L.fmo_decode_e4m3.restype = C.c_double
        L.fmo_decode_e4m3.argtypes = [C.c_uint8]
        L.fmo_decode_bf16.restype = C.c_double
        L.fmo_decode_bf16.argtypes = [C.c_uint16]
        L.fmo_n_visible.restype = C.c_int64
        L.fmo_n_visible.argtypes = [P, P, C.c_int]
        L.fmo_logits.restype = None
        L.fmo_logits.argtypes = [P, P, C.c_int, P, C.c_int, C.c_int64, C.c_int64, P, C.c_int64]
        L.fmo_logits_at.restype = None
        L.fmo_logits_at.argtypes = [P, P, C.c_int, P, P, C.c_int64, P]
        L.fmo_topk.restype = C.c_int
        L.fmo_topk.argtypes = [P, P, P, C.c_int64, C.c_int, P, P]
        L.fmo_topk_rows.restype = None
        L.fmo_topk_rows.argtypes = [P, C.c_int64, C.c_int, P, P, C.c_int64, P, C.c_int, P, P, P]
        L.fmo_resident_mask.restype = None
        L.fmo_resident_mask.argtypes = [P, C.c_int, P, C.c_int, C.c_double, C.c_int, C.c_int, P,
                                        C.c_int64, P, P, P, C.c_int64, P]
        L.fmo_score_resident.restype = None
        L.fmo_score_resident.argtypes = [P, P, P, P, C.c_int64, C.c_int, P, P, P]
        L.fmo_score_resident_ex.restype = None
        L.fmo_score_resident_ex.argtypes = [P, P, P, P, C.c_int64, C.c_int, C.c_int, P, P, P]
        L.fmo_densest_pages.restype = None
        L.fmo_densest_pages.argtypes = [P, C.c_int64, C.c_int, C.c_int64, C.c_int, P, P]
        L.fmo_num_threads.restype = C.c_int
        L.fmo_set_num_threads.argtypes = [C.c_int]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


class _Bound:
    """Holds the C descriptors and keeps every array they point into alive."""

    def __init__(self, wl, layers=None):
        kv = wl.kv
        self.keep = []
        pools = [np.ascontiguousarray(p) for p in kv.pools]
        self.keep += pools
        bt = np.ascontiguousarray(kv.block_table, dtype=np.int32)
        sl = np.ascontiguousarray(kv.seq_lens, dtype=np.int32)
        self.keep += [bt, sl]
        self.kv = _KV()
        for i, p in enumerate(pools):
            self.kv.pool[i] = p.ctypes.data
        self.kv.n_pools = len(pools)
        self.kv.key_dtype = _KEY_DT[kv.key_dtype]
        self.kv.page_size = pools[0].shape[1]
        self.kv.head_dim = pools[0].shape[2] - (4 if kv.key_dtype == "fp8x132" else 0)
        self.kv.block_table = bt.ctypes.data
        self.kv.bt_ld = bt.shape[1]
        self.kv.seq_lens = sl.ctypes.data
        self.kv.B = sl.shape[0]
        self.kv.n_phys_pages = pools[0].shape[0]
        qs = wl.queries if layers is None else [wl.queries[i] for i in layers]
        self.q = (_Q * len(qs))()
        for i, qq in enumerate(qs):
            arrs = [np.ascontiguousarray(qq.q), np.ascontiguousarray(qq.w)]
            sc = None if qq.q_scale is None else np.ascontiguousarray(qq.q_scale, np.float32)
            rr = None if qq.row_req is None else np.ascontiguousarray(qq.row_req, np.int32)
            qp = None if qq.q_pos is None else np.ascontiguousarray(qq.q_pos, np.int32)
            self.keep += arrs + [sc, rr, qp]
            self.q[i].q = arrs[0].ctypes.data
            self.q[i].q_dtype = _Q_DT[qq.q_dtype]
            self.q[i].q_scale = _ptr(sc)
            self.q[i].w = arrs[1].ctypes.data
            self.q[i].w_dtype = _Q_DT[qq.w_dtype]
            self.q[i].T = qq.q.shape[0]
            self.q[i].n_heads = qq.q.shape[1]
            self.q[i].row_req = _ptr(rr)
            self.q[i].q_pos = _ptr(qp)
            self.q[i].compress_ratio = qq.compress_ratio

    def qref(self, i=0):
        return C.byref(self.q[i])

    def kvref(self):
        return C.byref(self.kv)


# ----------------------------------------------------------------------------- API
def decode_e4m3(codes) -> np.ndarray:
    f = lib().fmo_decode_e4m3
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([f(int(x)) for x in c.reshape(-1)], np.float64).reshape(c.shape)


def decode_bf16(bits) -> np.ndarray:
    f = lib().fmo_decode_bf16
    c = np.asarray(bits, dtype=np.uint16)
    return np.array([f(int(x)) for x in c.reshape(-1)], np.float64).reshape(c.shape)


def n_visible(wl, t: int, layer: int = 0) -> int:
    b = _Bound(wl, [layer])
    return int(lib().fmo_n_visible(b.qref(), b.kvref(), int(t)))


def logits(wl, layer: int = 0, rows=None, s_begin: int = 0, s_end: int | None = None):
    """fp64 logits [len(rows), s_end - s_begin]; -inf where an entry is not visible."""
    b = _Bound(wl, [layer])
    T = wl.queries[layer].T
    rows = np.arange(T, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    if s_end is None:
        s_end = wl.kv.block_table.shape[1] * wl.kv.pools[0].shape[1]
    out = np.empty((rows.size, s_end - s_begin), np.float64)
    kvl = _KV.from_buffer_copy(b.kv)       # layer's own pool in slot 0
    kvl.pool[0] = b.kv.pool[layer]
    lib().fmo_logits(b.qref(), C.byref(kvl), 0, rows.ctypes.data, int(rows.size),
                     int(s_begin), int(s_end), out.ctypes.data, out.shape[1])
    return out


def logits_at(wl, rows, ents, layer: int = 0):
    """fp64 logits at the listed (row, entry) points; -inf where not visible."""
    b = _Bound(wl, [layer])
    kvl = _KV.from_buffer_copy(b.kv)
    kvl.pool[0] = b.kv.pool[layer]
    r = np.ascontiguousarray(rows, np.int32).reshape(-1)
    e = np.ascontiguousarray(ents, np.int64).reshape(-1)
    out = np.empty(r.size, np.float64)
    lib().fmo_logits_at(b.qref(), C.byref(kvl), 0, r.ctypes.data, e.ctypes.data, r.size,
                        out.ctypes.data)
    return out


def topk(vals, index=None, keep=None, k: int = 512):
    v = np.ascontiguousarray(vals, np.float64)
    ix = None if index is None else np.ascontiguousarray(index, np.int64)
    kp = None if keep is None else np.ascontiguousarray(keep, np.uint8)
    oi = np.empty(k, np.int32)
    ov = np.empty(k, np.float64)
    n = lib().fmo_topk(v.ctypes.data, _ptr(ix), _ptr(kp), v.size, k, oi.ctypes.data,
                       ov.ctypes.data)
    return oi, ov, n


def topk_rows(L, k: int = 512, n_valid=None, mask=None, row_req=None):
    L = np.ascontiguousarray(L, np.float64)
    T, ld = L.shape
    nv = None if n_valid is None else np.ascontiguousarray(n_valid, np.int64)
    mk = None if mask is None else np.ascontiguousarray(mask, np.uint8)
    rr = None if row_req is None else np.ascontiguousarray(row_req, np.int32)
    oi = np.empty((T, k), np.int32)
    ov = np.empty((T, k), np.float64)
    cnt = np.empty(T, np.int32)
    lib().fmo_topk_rows(L.ctypes.data, ld, T, _ptr(nv), _ptr(mk),
                        0 if mk is None else mk.shape[1], _ptr(rr), k, oi.ctypes.data,
                        ov.ctypes.data, cnt.ctypes.data)
    return oi, ov, cnt


def resident_mask(wl, mode: str = "max", threshold: float = 0.5, n_sink: int = 0,
                  n_recent: int = 0, mask_ld: int | None = None, layers=None):
    b = _Bound(wl, layers)
    n_layers = len(wl.queries) if layers is None else len(layers)
    kv = _KV.from_buffer_copy(b.kv)
    src = list(range(len(wl.queries))) if layers is None else list(layers)
    for i, l in enumerate(src):
        kv.pool[i] = b.kv.pool[l]
    B = wl.kv.B
    if mask_ld is None:
        mask_ld = wl.kv.block_table.shape[1] * wl.kv.pools[0].shape[1]
    P = wl.kv.pools[0].shape[1]
    n_pages = -(-mask_ld // P)
    mask = np.empty((B, mask_ld), np.uint8)
    score = np.empty((B, mask_ld), np.float64)
    cnt = np.empty(B, np.int32)
    plist = np.empty((B, n_pages), np.int32)
    dens = np.empty((B, n_pages), np.int32)
    lib().fmo_resident_mask(b.q, n_layers, C.byref(kv), UNION[mode], float(threshold),
                            int(n_sink), int(n_recent), mask.ctypes.data, mask_ld,
                            score.ctypes.data, cnt.ctypes.data, plist.ctypes.data, n_pages,
                            dens.ctypes.data)
    return dict(mask=mask, union=score, page_count=cnt, page_list=plist, page_density=dens)


def score_resident(wl, k: int = 512, resident_pages=None, n_resident=None, cells: bool = False):
    """Two-level top-k over the listed resident pages.  cells=False: logical entry indices;
    cells=True: reserve cells 64 j + offset (j = the page's position in the list), ranked and
    listed by cell."""
    b = _Bound(wl, [0])
    rp = np.ascontiguousarray(wl.resident_pages if resident_pages is None else resident_pages,
                              np.int32)
    nr = np.ascontiguousarray(wl.n_resident if n_resident is None else n_resident, np.int32)
    T = wl.queries[0].T
    oi = np.empty((T, k), np.int32)
    ov = np.empty((T, k), np.float64)
    cnt = np.empty(T, np.int32)
    lib().fmo_score_resident_ex(b.qref(), b.kvref(), rp.ctypes.data, nr.ctypes.data,
                                rp.shape[1], k, int(cells), oi.ctypes.data, ov.ctypes.data,
                                cnt.ctypes.data)
    return oi, ov, cnt


def densest_pages(density, kmax: int, n_pages: int | None = None):
    """KMAX densest pages per request (density > 0 only), ties by lower page id, ascending."""
    d = np.ascontiguousarray(density, np.int32)
    B, ld = d.shape
    n_pages = ld if n_pages is None else n_pages
    out = np.empty((B, kmax), np.int32)
    cnt = np.empty(B, np.int32)
    lib().fmo_densest_pages(d.ctypes.data, ld, B, n_pages, kmax, out.ctypes.data, cnt.ctypes.data)
    return out, cnt


def num_threads() -> int:
    return int(lib().fmo_num_threads())


def set_num_threads(n: int) -> None:
    lib().fmo_set_num_threads(int(n))
