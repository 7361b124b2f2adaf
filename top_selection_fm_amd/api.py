"""ctypes binding of libfm.so (include/fm.h): marshalling only.

Every function below has the name of the C entry point it calls.  It turns torch tensors into
device pointers, passes the current HIP stream, and raises FmError when the library returns a
status other than FM_OK.  No arithmetic of the indexer happens here; if libfm.so is missing
the first call raises (there is no fallback).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfm.so")

FM_OK, FM_ERR_INVALID_ARG, FM_ERR_UNSUPPORTED, FM_ERR_WORKSPACE, FM_ERR_LAUNCH = range(5)
FM_F32, FM_BF16, FM_FP8_E4M3, FM_FP8_E4M3_SCALED132 = range(4)
FM_UNION_MAX, FM_UNION_MEAN = 0, 1
FM_OP_INDEX_LOGITS, FM_OP_TOPK, FM_OP_RESIDENT_MASK, FM_OP_SCORE_RESIDENT, FM_OP_INDEX_TOPK = range(5)
FM_MAX_LAYERS = 4
FM_MAX_POOLS = 32
PAGE = 64

KEY_DTYPES = {"f32": FM_F32, "bf16": FM_BF16, "fp8x132": FM_FP8_E4M3_SCALED132}
Q_DTYPES = {"f32": FM_F32, "bf16": FM_BF16, "fp8": FM_FP8_E4M3}

EXPORTS = ["fm_index_logits", "fm_index_topk", "fm_resident_mask", "fm_topk512", "fm_score_resident",
           "fm_score_resident_noalloc", "fm_score_resident_cells", "fm_densest_pages", "fm_workspace_bytes",
           "fm_encode_queries", "fm_encode_workspace_bytes", "fm_golden_labels",
           "fm_golden_workspace_bytes", "fm_status_string", "fm_last_error", "fm_version"]


class FmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class KvDesc(C.Structure):
    _fields_ = [("pool", C.c_void_p * FM_MAX_POOLS), ("n_pools", C.c_int),
                ("key_dtype", C.c_int), ("page_size", C.c_int), ("head_dim", C.c_int),
                ("block_table", C.c_void_p), ("bt_ld", C.c_int64), ("seq_lens", C.c_void_p),
                ("B", C.c_int), ("max_seq_len", C.c_int64), ("n_phys_pages", C.c_int64)]


class QueryDesc(C.Structure):
    _fields_ = [("q", C.c_void_p), ("q_dtype", C.c_int), ("q_scale", C.c_void_p),
                ("w", C.c_void_p), ("w_dtype", C.c_int), ("T", C.c_int), ("n_heads", C.c_int),
                ("row_req", C.c_void_p), ("q_pos", C.c_void_p), ("compress_ratio", C.c_int),
                ("row_pool", C.c_void_p)]


class EncoderDesc(C.Structure):
    _fields_ = [("wq_a", C.c_void_p), ("q_norm", C.c_void_p), ("wq_b", C.c_void_p),
                ("w_proj", C.c_void_p), ("d_model", C.c_int), ("q_rank", C.c_int),
                ("n_heads", C.c_int), ("head_dim", C.c_int), ("rope_dim", C.c_int),
                ("rms_eps", C.c_float), ("rope_base", C.c_float), ("rope_factor", C.c_float),
                ("rope_orig_len", C.c_int), ("beta_fast", C.c_float), ("beta_slow", C.c_float)]


_lib = None


def lib():
    """Open libfm.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with `python -m top_selection_fm_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I64 = C.c_void_p, C.c_int64
        L.fm_index_logits.argtypes = [P, P, P, I64, P]
        L.fm_index_topk.argtypes = [P, P, P, I64, C.c_int, P, P, P, I64, P, C.c_size_t, P]
        L.fm_resident_mask.argtypes = [P, C.c_int, P, C.c_int, C.c_float, C.c_int32, C.c_int32,
                                       P, I64, P, P, I64, P, P, P]
        L.fm_topk512.argtypes = [P, I64, C.c_int, P, P, I64, P, C.c_int, P, P, P, C.c_size_t, P]
        L.fm_score_resident.argtypes = [P, P, P, P, I64, C.c_int, P, P, P, C.c_size_t, P]
        L.fm_score_resident_cells.argtypes = [P, P, P, P, I64, C.c_int, P, P, P, C.c_size_t, P]
        L.fm_score_resident_noalloc.argtypes = [P, P, P, P, I64, C.c_int, P, P, P]
        L.fm_densest_pages.argtypes = [P, I64, C.c_int, I64, C.c_int, P, P, P]
        L.fm_encode_queries.argtypes = [P, P, C.c_int, P, P, P, P, C.c_size_t, P]
        L.fm_encode_workspace_bytes.argtypes = [P, C.c_int]
        L.fm_encode_workspace_bytes.restype = C.c_size_t
        L.fm_golden_labels.argtypes = [P, I64, C.c_int, C.c_int, P, C.c_float, C.c_int, C.c_int,
                                       P, P, P, I64, P, C.c_size_t, P]
        L.fm_golden_workspace_bytes.argtypes = [C.c_int, C.c_int, I64, C.c_int]
        L.fm_golden_workspace_bytes.restype = C.c_size_t
        for f in ("fm_index_logits", "fm_index_topk", "fm_resident_mask", "fm_topk512", "fm_score_resident",
                  "fm_score_resident_noalloc", "fm_score_resident_cells", "fm_densest_pages", "fm_encode_queries",
                  "fm_golden_labels"):
            getattr(L, f).restype = C.c_int
        L.fm_workspace_bytes.argtypes = [C.c_int, C.c_int, I64]
        L.fm_workspace_bytes.restype = C.c_size_t
        L.fm_status_string.argtypes = [C.c_int]
        L.fm_status_string.restype = C.c_char_p
        L.fm_last_error.argtypes = []
        L.fm_last_error.restype = C.c_char_p
        L.fm_version.argtypes = []
        L.fm_version.restype = C.c_int
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(status: int) -> None:
    if status != FM_OK:
        L = lib()
        raise FmError(status, f"{L.fm_status_string(status).decode()}: "
                              f"{L.fm_last_error().decode()}")


# ----------------------------------------------------------------------------- descriptors
def kv_desc(pools, key_dtype: str, block_table, seq_lens, max_seq_len: int,
            n_phys_pages: int | None = None) -> KvDesc:
    d = KvDesc()
    for i, p in enumerate(pools):
        d.pool[i] = _ptr(p)
    d.n_pools = len(pools)
    d.key_dtype = KEY_DTYPES[key_dtype]
    d.page_size = PAGE
    d.head_dim = 128
    d.block_table = _ptr(block_table)
    d.bt_ld = block_table.shape[1]
    d.seq_lens = _ptr(seq_lens)
    d.B = seq_lens.shape[0]
    d.max_seq_len = int(max_seq_len)
    d.n_phys_pages = int(pools[0].shape[0] if n_phys_pages is None else n_phys_pages)
    return d


def query_desc(q, q_dtype: str, w, w_dtype: str, q_scale=None, row_req=None, q_pos=None,
               compress_ratio: int = 4, row_pool=None) -> QueryDesc:
    d = QueryDesc()
    d.q = _ptr(q)
    d.q_dtype = Q_DTYPES[q_dtype]
    d.q_scale = _ptr(q_scale)
    d.w = _ptr(w)
    d.w_dtype = Q_DTYPES[w_dtype]
    d.T = q.shape[0]
    d.n_heads = q.shape[1]
    d.row_req = _ptr(row_req)
    d.q_pos = _ptr(q_pos)
    d.compress_ratio = compress_ratio
    d.row_pool = _ptr(row_pool)
    return d


# ----------------------------------------------------------------------------- entry points
def fm_index_logits(q: QueryDesc, kv: KvDesc, logits, ld: int, stream=None) -> None:
    _check(lib().fm_index_logits(C.byref(q), C.byref(kv), _ptr(logits), int(ld),
                                 _stream(stream)))


def fm_resident_mask(q_layers, kv: KvDesc, mode: int, threshold: float, n_sink: int,
                     n_recent: int, mask, mask_ld: int, page_count, page_list=None,
                     page_list_ld: int = 0, page_density=None, union_score=None,
                     stream=None) -> None:
    arr = (QueryDesc * len(q_layers))(*q_layers)
    _check(lib().fm_resident_mask(arr, len(q_layers), C.byref(kv), int(mode), float(threshold),
                                  int(n_sink), int(n_recent), _ptr(mask), int(mask_ld),
                                  _ptr(page_count), _ptr(page_list), int(page_list_ld),
                                  _ptr(page_density), _ptr(union_score), _stream(stream)))


def fm_index_topk(q: QueryDesc, kv: KvDesc, mask, mask_ld: int, k: int, out_idx, out_val=None,
                  logits=None, logits_ld: int = 0, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(lib().fm_index_topk(C.byref(q), C.byref(kv), _ptr(mask), int(mask_ld), int(k),
                               _ptr(out_idx), _ptr(out_val), _ptr(logits), int(logits_ld),
                               _ptr(ws), int(ws_bytes), _stream(stream)))


def fm_topk512(logits, ld: int, T: int, n_valid, mask, mask_ld: int, row_req, k: int, out_idx,
               out_val=None, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(lib().fm_topk512(_ptr(logits), int(ld), int(T), _ptr(n_valid), _ptr(mask),
                            int(mask_ld), _ptr(row_req), int(k), _ptr(out_idx), _ptr(out_val),
                            _ptr(ws), int(ws_bytes), _stream(stream)))


def fm_score_resident(q: QueryDesc, kv: KvDesc, resident_pages, n_resident, res_ld: int, k: int,
                      out_idx, out_val=None, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(lib().fm_score_resident(C.byref(q), C.byref(kv), _ptr(resident_pages),
                                   _ptr(n_resident), int(res_ld), int(k), _ptr(out_idx),
                                   _ptr(out_val), _ptr(ws), int(ws_bytes), _stream(stream)))


def fm_score_resident_noalloc(q: QueryDesc, kv: KvDesc, resident_pages, n_resident, res_ld: int,
                              k: int, out_idx, out_val=None, stream=None) -> None:
    _check(lib().fm_score_resident_noalloc(C.byref(q), C.byref(kv), _ptr(resident_pages),
                                           _ptr(n_resident), int(res_ld), int(k), _ptr(out_idx),
                                           _ptr(out_val), _stream(stream)))


STATIC_SCRATCH_BYTES = 64 << 20


def fm_score_resident_cells(q: QueryDesc, kv: KvDesc, resident_pages, n_resident, res_ld: int,
                            k: int, out_cells, out_val=None, ws=None, ws_bytes: int = 0,
                            stream=None) -> None:
    _check(lib().fm_score_resident_cells(C.byref(q), C.byref(kv), _ptr(resident_pages),
                                         _ptr(n_resident), int(res_ld), int(k), _ptr(out_cells),
                                         _ptr(out_val), _ptr(ws), int(ws_bytes), _stream(stream)))


def fm_densest_pages(density, density_ld: int, B: int, n_pages: int, kmax: int, out_pages,
                     out_count=None, stream=None) -> None:
    _check(lib().fm_densest_pages(_ptr(density), int(density_ld), int(B), int(n_pages), int(kmax),
                                  _ptr(out_pages), _ptr(out_count), _stream(stream)))


def encoder_desc(wq_a, q_norm, wq_b, w_proj, *, n_heads: int, d_model: int, q_rank: int,
                 head_dim: int = 128, rope_dim: int = 64, rms_eps: float = 1e-6,
                 rope_base: float = 160000.0, rope_factor: float = 16.0,
                 rope_orig_len: int = 65536, beta_fast: float = 32.0,
                 beta_slow: float = 1.0) -> EncoderDesc:
    """fm_encoder_desc over device tensors (bf16 bits); the defaults are the page's values."""
    return EncoderDesc(_ptr(wq_a), _ptr(q_norm), _ptr(wq_b), _ptr(w_proj), int(d_model),
                       int(q_rank), int(n_heads), int(head_dim), int(rope_dim), float(rms_eps),
                       float(rope_base), float(rope_factor), int(rope_orig_len),
                       float(beta_fast), float(beta_slow))


def fm_encode_workspace_bytes(desc: EncoderDesc, T: int) -> int:
    return int(lib().fm_encode_workspace_bytes(C.byref(desc), int(T)))


def fm_encode_queries(desc: EncoderDesc, hidden, T: int, pos, q, w, ws, ws_bytes: int,
                      stream=None) -> None:
    _check(lib().fm_encode_queries(C.byref(desc), _ptr(hidden), int(T), _ptr(pos), _ptr(q),
                                   _ptr(w), _ptr(ws), int(ws_bytes), _stream(stream)))


def fm_golden_workspace_bytes(T: int, n_layers: int, ld: int, tau: int) -> int:
    return int(lib().fm_golden_workspace_bytes(int(T), int(n_layers), int(ld), int(tau)))


def fm_golden_labels(scores, ld: int, T: int, n_layers: int, n_valid, p: float, min_votes: int,
                     tau: int, label_ptr, label_idx, label_score, cap: int, ws, ws_bytes: int,
                     stream=None) -> None:
    _check(lib().fm_golden_labels(_ptr(scores), int(ld), int(T), int(n_layers), _ptr(n_valid),
                                  float(p), int(min_votes), int(tau), _ptr(label_ptr),
                                  _ptr(label_idx), _ptr(label_score), int(cap), _ptr(ws),
                                  int(ws_bytes), _stream(stream)))


def fm_workspace_bytes(op: int, T: int, max_candidates: int) -> int:
    return int(lib().fm_workspace_bytes(int(op), int(T), int(max_candidates)))


def fm_status_string(status: int) -> str:
    return lib().fm_status_string(int(status)).decode()


def fm_last_error() -> str:
    return lib().fm_last_error().decode()


def fm_version() -> int:
    return int(lib().fm_version())


# ----------------------------------------------------------------------------- device upload
def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:          # bf16 bit patterns travel as int16 (same bytes)
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceWorkload:
    """A seeded workload (top_selection_fm_amd.workloads.Workload) copied to device memory,
    with its descriptors built.  Plumbing for tests and the benchmark."""

    def __init__(self, wl, device="cuda:0", pool_copies: int = 1):
        kv = wl.kv
        self.wl = wl
        self.device = torch.device(device)
        self.pools = [_dev(p, self.device) for p in kv.pools]
        self.block_table = _dev(kv.block_table.astype(np.int32), self.device)
        self.seq_lens = _dev(kv.seq_lens.astype(np.int32), self.device)
        self.max_seq_len = kv.max_seq_len
        self.replicas = [self.pools] + [[p.clone() for p in self.pools]
                                        for _ in range(pool_copies - 1)]
        self.q = []
        for qq in wl.queries:
            self.q.append(dict(
                q=_dev(qq.q, self.device), w=_dev(qq.w, self.device),
                q_scale=None if qq.q_scale is None else _dev(qq.q_scale.astype(np.float32),
                                                             self.device),
                row_req=None if qq.row_req is None else _dev(qq.row_req.astype(np.int32),
                                                             self.device),
                q_pos=None if qq.q_pos is None else _dev(qq.q_pos.astype(np.int32), self.device),
                row_pool=None if qq.row_pool is None else _dev(qq.row_pool.astype(np.int32),
                                                               self.device),
                q_dtype=qq.q_dtype, w_dtype=qq.w_dtype, ratio=qq.compress_ratio))
        self.resident_pages = None if wl.resident_pages is None else _dev(
            wl.resident_pages.astype(np.int32), self.device)
        self.n_resident = None if wl.n_resident is None else _dev(
            wl.n_resident.astype(np.int32), self.device)

    def kv(self, replica: int = 0, layers=None) -> KvDesc:
        pools = self.replicas[replica]
        if layers is not None:
            pools = [pools[i] for i in layers]
        return kv_desc(pools, self.wl.kv.key_dtype, self.block_table, self.seq_lens,
                       self.max_seq_len)

    def query(self, layer: int = 0) -> QueryDesc:
        d = self.q[layer]
        return query_desc(d["q"], d["q_dtype"], d["w"], d["w_dtype"], q_scale=d["q_scale"],
                          row_req=d["row_req"], q_pos=d["q_pos"], compress_ratio=d["ratio"],
                          row_pool=d["row_pool"])
