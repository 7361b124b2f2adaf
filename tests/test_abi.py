"""C-ABI checks that need no GPU: the library loads, exports what include/fm.h declares, and
rejects bad arguments on the host (status codes) before anything is launched.

Pointers passed here are fake, aligned device addresses: every call below fails validation
(or is a T = 0 no-op) and never reaches the HIP runtime.
"""
import ctypes as C
import os
import re

import pytest

from top_selection_fm_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fm.h")
FAKE = 0x10000   # 64 KiB: aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = api.lib()
    names = declared_functions()
    assert set(names) >= {"fm_index_logits", "fm_resident_mask", "fm_topk512",
                          "fm_score_resident", "fm_score_resident_cells", "fm_densest_pages"}
    for n in names:
        assert hasattr(L, n), n
    assert sorted(api.EXPORTS) == names


def test_version_and_status_strings():
    m = re.search(r"#define FM_VERSION (\d+)", open(HEADER).read())
    assert api.fm_version() == int(m.group(1))
    for s, name in enumerate(["FM_OK", "FM_ERR_INVALID_ARG", "FM_ERR_UNSUPPORTED",
                              "FM_ERR_WORKSPACE", "FM_ERR_LAUNCH"]):
        assert api.fm_status_string(s) == name
    assert api.fm_status_string(99) == "FM_ERR_UNKNOWN"


def test_workspace_bytes():
    # rows of up to 65,536 entries are selected in one pass: no top-k workspace
    assert api.fm_workspace_bytes(api.FM_OP_TOPK, 30, 384 * 64) == 0
    assert api.fm_workspace_bytes(api.FM_OP_TOPK, 30, 65536) == 0
    topk = api.fm_workspace_bytes(api.FM_OP_TOPK, 30, 65537)
    assert topk >= 30 * 9 * 1024 * 8                 # nine 8192-entry chunks per row
    assert api.fm_workspace_bytes(api.FM_OP_TOPK, 3, 262144) >= 3 * 32 * 1024 * 8
    assert api.fm_workspace_bytes(api.FM_OP_SCORE_RESIDENT, 30, 384 * 64) >= 30 * 384 * 64 * 4
    assert api.fm_workspace_bytes(api.FM_OP_SCORE_RESIDENT, 30, 2048 * 64) >= \
        30 * 2048 * 64 * 4 + api.fm_workspace_bytes(api.FM_OP_TOPK, 30, 2048 * 64)
    assert api.fm_workspace_bytes(api.FM_OP_TOPK, 30, 4096) == 0   # short rows: none
    assert api.fm_workspace_bytes(api.FM_OP_INDEX_LOGITS, 4, 100) == 0
    assert api.fm_workspace_bytes(api.FM_OP_RESIDENT_MASK, 4, 100) == 0
    assert api.fm_workspace_bytes(api.FM_OP_SCORE_RESIDENT, 0, 100) == 0


class _Shape:
    def __init__(self, *shape):
        self.shape = shape


def good_kv(key_dtype="bf16", B=2, max_seq_len=1000, n_pools=1):
    d = api.KvDesc()
    for i in range(n_pools):
        d.pool[i] = FAKE * (i + 1)
    d.n_pools = n_pools
    d.key_dtype = api.KEY_DTYPES[key_dtype]
    d.page_size = 64
    d.head_dim = 128
    d.block_table = FAKE
    d.bt_ld = (max_seq_len + 63) // 64
    d.seq_lens = FAKE
    d.B = B
    d.max_seq_len = max_seq_len
    d.n_phys_pages = 100
    return d


def good_q(q_dtype="bf16", T=2, w_dtype="bf16"):
    d = api.QueryDesc()
    d.q = FAKE
    d.q_dtype = api.Q_DTYPES[q_dtype]
    d.q_scale = FAKE if q_dtype == "fp8" else None
    d.w = FAKE
    d.w_dtype = api.Q_DTYPES[w_dtype]
    d.T = T
    d.n_heads = 64
    d.compress_ratio = 4
    return d


def status_of(fn, *args):
    with pytest.raises(api.FmError) as e:
        fn(*args)
    return e.value.status, str(e.value)


def logits_call(q, kv, ld=1000):
    return status_of(api.fm_index_logits, q, kv, FAKE, ld, 0)


@pytest.mark.parametrize("mutate,status", [
    (lambda q, kv: setattr(q, "n_heads", 128), api.FM_ERR_UNSUPPORTED),   # bf16 keys: 64 only
    (lambda q, kv: setattr(q, "n_heads", 96), api.FM_ERR_UNSUPPORTED),
    (lambda q, kv: (setattr(q, "n_heads", 128), setattr(kv, "key_dtype", api.FM_FP8_E4M3_SCALED132),
                    setattr(q, "q_dtype", api.FM_FP8_E4M3), setattr(q, "q_scale", FAKE)),
     api.FM_ERR_UNSUPPORTED),                                                 # fp8 q: 64 only
    (lambda q, kv: setattr(kv, "page_size", 32), api.FM_ERR_UNSUPPORTED),
    (lambda q, kv: setattr(kv, "head_dim", 64), api.FM_ERR_UNSUPPORTED),
    (lambda q, kv: setattr(kv, "key_dtype", api.FM_FP8_E4M3), api.FM_ERR_UNSUPPORTED),
    (lambda q, kv: setattr(q, "q_dtype", api.FM_F32), api.FM_ERR_UNSUPPORTED),
    (lambda q, kv: setattr(q, "w_dtype", api.FM_FP8_E4M3), api.FM_ERR_UNSUPPORTED),
    (lambda q, kv: kv.pool.__setitem__(0, FAKE + 4), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: kv.pool.__setitem__(0, None), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: setattr(kv, "bt_ld", 10), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: setattr(kv, "B", 0), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: setattr(kv, "max_seq_len", -1), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: setattr(kv, "n_phys_pages", 0), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: setattr(kv, "n_pools", 0), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: setattr(kv, "n_pools", api.FM_MAX_POOLS + 1), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: setattr(kv, "n_pools", 2), api.FM_ERR_INVALID_ARG),   # pool[1] NULL
    (lambda q, kv: (setattr(kv, "n_pools", 2), kv.pool.__setitem__(1, FAKE + 4)),
     api.FM_ERR_INVALID_ARG),                                              # pool[1] misaligned
    (lambda q, kv: setattr(kv, "block_table", None), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: setattr(q, "T", -1), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: setattr(q, "T", 3), api.FM_ERR_INVALID_ARG),      # T != B, no row_req
    (lambda q, kv: setattr(q, "q", FAKE + 8), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: setattr(q, "w", None), api.FM_ERR_INVALID_ARG),
    (lambda q, kv: (setattr(q, "q_pos", FAKE), setattr(q, "compress_ratio", 0)),
     api.FM_ERR_INVALID_ARG),
])
def test_index_logits_validation(mutate, status):
    q, kv = good_q(), good_kv()
    mutate(q, kv)
    got, msg = logits_call(q, kv)
    assert got == status, msg
    assert api.fm_last_error() and api.fm_last_error() in msg


def test_fp8_query_needs_scale_and_fp8_keys():
    q, kv = good_q("fp8"), good_kv("fp8x132")
    q.q_scale = None
    assert logits_call(q, kv)[0] == api.FM_ERR_INVALID_ARG
    q2, kv2 = good_q("fp8"), good_kv("bf16")
    assert logits_call(q2, kv2)[0] == api.FM_ERR_UNSUPPORTED


def test_index_logits_bad_output():
    assert status_of(api.fm_index_logits, good_q(), good_kv(), None, 1000, 0)[0] == \
        api.FM_ERR_INVALID_ARG
    assert logits_call(good_q(), good_kv(), ld=0)[0] == api.FM_ERR_INVALID_ARG
    assert status_of(api.fm_index_logits, good_q(), good_kv(), FAKE + 2, 1000, 0)[0] == \
        api.FM_ERR_INVALID_ARG


def test_zero_rows_is_a_noop():
    api.fm_index_logits(good_q(T=0), good_kv(), FAKE, 1000, 0)
    api.fm_topk512(FAKE, 100, 0, None, None, 0, None, 512, FAKE)
    assert api.fm_last_error() == ""


@pytest.mark.parametrize("args,status", [
    (dict(k=0), api.FM_ERR_UNSUPPORTED),
    (dict(k=1025), api.FM_ERR_UNSUPPORTED),
    (dict(T=-1), api.FM_ERR_INVALID_ARG),
    (dict(ld=0), api.FM_ERR_INVALID_ARG),
    (dict(logits=None), api.FM_ERR_INVALID_ARG),
    (dict(out_idx=None), api.FM_ERR_INVALID_ARG),
    (dict(mask=FAKE, mask_ld=99), api.FM_ERR_INVALID_ARG),
])
def test_topk_validation(args, status):
    a = dict(logits=FAKE, ld=100, T=2, n_valid=None, mask=None, mask_ld=0, row_req=None, k=512,
             out_idx=FAKE)
    a.update(args)
    got, _ = status_of(api.fm_topk512, a["logits"], a["ld"], a["T"], a["n_valid"], a["mask"],
                       a["mask_ld"], a["row_req"], a["k"], a["out_idx"])
    assert got == status


def test_score_resident_validation():
    q, kv = good_q(), good_kv("fp8x132")
    need = api.fm_workspace_bytes(api.FM_OP_SCORE_RESIDENT, 2, 10 * 64)
    st = lambda **kw: status_of(api.fm_score_resident, q, kv, kw.get("rp", FAKE),
                                kw.get("nr", FAKE), kw.get("res_ld", 10), kw.get("k", 512),
                                FAKE, None, kw.get("ws", FAKE), kw.get("ws_bytes", need - 4))[0]
    assert st() == api.FM_ERR_WORKSPACE
    assert st(ws=None, ws_bytes=need) == api.FM_ERR_WORKSPACE
    assert st(ws=FAKE + 16, ws_bytes=need) == api.FM_ERR_WORKSPACE   # needs 256-byte alignment
    assert st(rp=None, ws_bytes=need) == api.FM_ERR_INVALID_ARG
    assert st(res_ld=0, ws_bytes=need) == api.FM_ERR_INVALID_ARG
    assert st(k=4096, ws_bytes=need) == api.FM_ERR_UNSUPPORTED


def test_score_resident_noalloc_validation():
    """The allocation-free variant validates like fm_score_resident, and refuses (before any
    HIP call) a shape whose workspace would not fit its static array."""
    q, kv = good_q(), good_kv("fp8x132")
    st = lambda **kw: status_of(api.fm_score_resident_noalloc, q, kv, kw.get("rp", FAKE),
                                kw.get("nr", FAKE), kw.get("res_ld", 10), kw.get("k", 512),
                                FAKE, None)[0]
    assert st(rp=None) == api.FM_ERR_INVALID_ARG
    assert st(res_ld=0) == api.FM_ERR_INVALID_ARG
    assert st(k=4096) == api.FM_ERR_UNSUPPORTED
    too_big = api.STATIC_SCRATCH_BYTES // (2 * 64 * 4) + 1          # 2 rows
    assert api.fm_workspace_bytes(api.FM_OP_SCORE_RESIDENT, 2, too_big * 64) > \
        api.STATIC_SCRATCH_BYTES
    assert st(res_ld=too_big) == api.FM_ERR_WORKSPACE
    assert "static scratch" in api.fm_last_error()
    m = re.search(r"#define FM_STATIC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", open(HEADER).read())
    assert api.STATIC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))


def test_densest_pages_validation():
    st = lambda **kw: status_of(api.fm_densest_pages, kw.get("d", FAKE), kw.get("ld", 100),
                                kw.get("B", 2), kw.get("n", 100), kw.get("kmax", 96),
                                kw.get("out", FAKE), None)[0]
    assert st(kmax=0) == api.FM_ERR_UNSUPPORTED
    assert st(kmax=1025) == api.FM_ERR_UNSUPPORTED
    assert st(n=101) == api.FM_ERR_INVALID_ARG          # more pages than the row holds
    assert st(n=-1) == api.FM_ERR_INVALID_ARG
    assert st(B=-1) == api.FM_ERR_INVALID_ARG
    assert st(d=None) == api.FM_ERR_INVALID_ARG
    assert st(out=None) == api.FM_ERR_INVALID_ARG
    api.fm_densest_pages(None, 100, 0, 100, 96, None)  # B = 0: nothing to do, nothing launched


def test_score_resident_cells_validation():
    q, kv = good_q(), good_kv("fp8x132")
    need = api.fm_workspace_bytes(api.FM_OP_SCORE_RESIDENT, 2, 10 * 64)
    st = lambda **kw: status_of(api.fm_score_resident_cells, q, kv, kw.get("rp", FAKE),
                                kw.get("nr", FAKE), kw.get("res_ld", 10), kw.get("k", 512),
                                FAKE, None, kw.get("ws", FAKE), kw.get("ws_bytes", need - 4))[0]
    assert st() == api.FM_ERR_WORKSPACE
    assert st(rp=None, ws_bytes=need) == api.FM_ERR_INVALID_ARG
    assert st(k=4096, ws_bytes=need) == api.FM_ERR_UNSUPPORTED


def mask_call(qs, kv, **kw):
    arr = (api.QueryDesc * len(qs))(*qs) if qs else None
    L = api.lib()
    return L.fm_resident_mask(arr, kw.get("n_layers", len(qs)), C.byref(kv),
                              kw.get("mode", api.FM_UNION_MAX), kw.get("threshold", 0.5),
                              kw.get("n_sink", 0), kw.get("n_recent", 0),
                              kw.get("mask", FAKE), kw.get("mask_ld", 1000),
                              kw.get("page_count", FAKE), kw.get("page_list", None),
                              kw.get("page_list_ld", 0), None, None, None)


def test_resident_mask_validation():
    kv = good_kv("fp8x132", n_pools=3)
    qs = [good_q() for _ in range(3)]
    assert mask_call(qs, kv, threshold=0.0) == api.FM_ERR_INVALID_ARG
    assert mask_call(qs, kv, threshold=1.0) == api.FM_ERR_INVALID_ARG
    assert mask_call(qs, kv, n_layers=0) == api.FM_ERR_INVALID_ARG
    assert mask_call(qs, kv, n_layers=5) == api.FM_ERR_INVALID_ARG
    assert mask_call(qs, kv, mode=7) == api.FM_ERR_INVALID_ARG
    assert mask_call(qs, kv, n_sink=-1) == api.FM_ERR_INVALID_ARG
    assert mask_call(qs, kv, mask=None) == api.FM_ERR_INVALID_ARG
    assert mask_call(qs, kv, page_count=None) == api.FM_ERR_INVALID_ARG
    assert mask_call(qs, kv, page_list=FAKE, page_list_ld=0) == api.FM_ERR_INVALID_ARG
    assert mask_call(qs, good_kv("fp8x132", n_pools=2)) == api.FM_ERR_INVALID_ARG
    bad = [good_q(), good_q(T=3), good_q()]
    assert mask_call(bad, kv) == api.FM_ERR_INVALID_ARG
    fp8 = [good_q("fp8") for _ in range(3)]
    assert mask_call(fp8, kv) == api.FM_ERR_UNSUPPORTED
    mixed = [good_q() for _ in range(3)]
    mixed[1].n_heads = 128
    assert mask_call(mixed, kv) == api.FM_ERR_UNSUPPORTED
    wide_bf16 = [good_q() for _ in range(3)]
    for q in wide_bf16:
        q.n_heads = 128
    assert mask_call(wide_bf16, good_kv("bf16", n_pools=3)) == api.FM_ERR_UNSUPPORTED
    pooled = [good_q() for _ in range(3)]
    pooled[2].row_pool = FAKE                   # encoder l always scores pool[l]
    assert mask_call(pooled, kv) == api.FM_ERR_INVALID_ARG


def test_descriptor_layout_matches_header(tmp_path):
    """The ctypes descriptors have the C structs' size and field offsets (compiled with gcc
    against include/fm.h)."""
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    structs = {"fm_kv_desc": api.KvDesc, "fm_query_desc": api.QueryDesc,
               "fm_encoder_desc": api.EncoderDesc}
    lines = []
    for cname, cls in structs.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f in cls._fields_:
            lines.append(f'printf("{cname} {f[0]} %zu\\n", offsetof({cname}, {f[0]}));')
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"fm.h\"\n"
                   "int main(void) {\n" + "\n".join(lines) + "\nreturn 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = {}
    for ln in subprocess.run([str(exe)], check=True, capture_output=True,
                             text=True).stdout.split("\n"):
        if ln:
            a, b, c = ln.split()
            got[(a, b)] = int(c)
    for cname, cls in structs.items():
        assert got[(cname, "sizeof")] == C.sizeof(cls), cname
        for f in cls._fields_:
            assert got[(cname, f[0])] == getattr(cls, f[0]).offset, (cname, f[0])


def test_max_pools_pass_validation():
    """FM_MAX_POOLS pools validate (a T = 0 call returns before any launch); one more does not."""
    assert api.FM_MAX_POOLS == 32
    kv = good_kv(n_pools=api.FM_MAX_POOLS)
    api.fm_index_logits(good_q(T=0), kv, FAKE, 1000, 0)
    assert api.fm_last_error() == ""
    kv.n_pools = api.FM_MAX_POOLS + 1
    assert logits_call(good_q(T=0), kv)[0] == api.FM_ERR_INVALID_ARG


def good_enc(**kw):
    e = api.encoder_desc(FAKE, FAKE, FAKE, FAKE, n_heads=128, d_model=4096, q_rank=2048)
    for k, v in kw.items():
        setattr(e, k, v)
    return e


def test_encode_queries_validation():
    """Every bad encoder argument is refused on the host (nothing launched, no GPU needed)."""
    need = api.fm_encode_workspace_bytes(good_enc(), 32)
    assert need > 0
    assert api.fm_encode_workspace_bytes(good_enc(), 4096) > need
    assert api.fm_encode_workspace_bytes(good_enc(head_dim=64), 32) == 0
    st = lambda e=None, T=32, h=FAKE, pos=FAKE, q=FAKE, w=FAKE, ws=FAKE, nb=need: status_of(
        api.fm_encode_queries, good_enc() if e is None else e, h, T, pos, q, w, ws, nb)[0]
    assert st(e=good_enc(head_dim=64)) == api.FM_ERR_UNSUPPORTED
    assert st(e=good_enc(d_model=4100)) == api.FM_ERR_UNSUPPORTED
    assert st(e=good_enc(q_rank=2050)) == api.FM_ERR_UNSUPPORTED
    assert st(e=good_enc(n_heads=48)) == api.FM_ERR_UNSUPPORTED
    assert st(e=good_enc(q_rank=4096, n_heads=128)) == api.FM_ERR_UNSUPPORTED   # > 4096 columns
    assert st(e=good_enc(rope_dim=63)) == api.FM_ERR_INVALID_ARG
    assert st(e=good_enc(rope_dim=130)) == api.FM_ERR_INVALID_ARG
    assert st(e=good_enc(rope_factor=0.5)) == api.FM_ERR_INVALID_ARG
    assert st(e=good_enc(beta_fast=0.5)) == api.FM_ERR_INVALID_ARG
    assert st(e=good_enc(wq_b=None)) == api.FM_ERR_INVALID_ARG
    assert st(e=good_enc(wq_a=FAKE + 8)) == api.FM_ERR_INVALID_ARG     # weights 16-byte aligned
    assert st(e=good_enc(wq_b=FAKE + 8)) == api.FM_ERR_INVALID_ARG
    assert st(e=good_enc(w_proj=FAKE + 8)) == api.FM_ERR_INVALID_ARG
    assert st(T=-1) == api.FM_ERR_INVALID_ARG
    assert st(h=None) == api.FM_ERR_INVALID_ARG
    assert st(pos=None) == api.FM_ERR_INVALID_ARG
    assert st(h=FAKE + 8) == api.FM_ERR_INVALID_ARG        # hidden not 16-byte aligned
    assert st(nb=need - 1) == api.FM_ERR_WORKSPACE
    assert st(ws=FAKE + 64) == api.FM_ERR_WORKSPACE         # workspace not 256-byte aligned
    api.fm_encode_queries(good_enc(), None, 0, None, None, None, None, 0)   # T = 0: no-op


def test_golden_labels_validation():
    L = api.lib()
    need = api.fm_golden_workspace_bytes(10, 4, 1000, 3)
    assert need > 0 and api.fm_golden_workspace_bytes(10, 4, 1000, 11) == 0

    def st(**kw):
        a = dict(scores=FAKE, ld=1000, T=10, n_layers=4, n_valid=None, p=0.6, min_votes=3, tau=3,
                 ptr=FAKE, idx=FAKE, score=None, cap=100, ws=FAKE, ws_bytes=need)
        a.update(kw)
        return L.fm_golden_labels(a["scores"], a["ld"], a["T"], a["n_layers"], a["n_valid"],
                                  a["p"], a["min_votes"], a["tau"], a["ptr"], a["idx"],
                                  a["score"], a["cap"], a["ws"], a["ws_bytes"], None)
    assert st(tau=0) == api.FM_ERR_INVALID_ARG
    assert st(tau=11) == api.FM_ERR_INVALID_ARG
    assert st(ld=0) == api.FM_ERR_INVALID_ARG
    assert st(ld=65537, ws_bytes=1 << 30) == api.FM_ERR_UNSUPPORTED
    assert st(n_layers=0) == api.FM_ERR_INVALID_ARG
    assert st(n_layers=65) == api.FM_ERR_UNSUPPORTED
    assert st(min_votes=0) == api.FM_ERR_INVALID_ARG
    assert st(p=0.0) == api.FM_ERR_INVALID_ARG
    assert st(p=1.5) == api.FM_ERR_INVALID_ARG
    assert st(scores=None) == api.FM_ERR_INVALID_ARG
    assert st(scores=FAKE + 2) == api.FM_ERR_INVALID_ARG
    assert st(ptr=None) == api.FM_ERR_INVALID_ARG
    assert st(idx=None) == api.FM_ERR_INVALID_ARG
    assert st(ws_bytes=need - 1) == api.FM_ERR_WORKSPACE
    assert st(ws=FAKE + 16) == api.FM_ERR_WORKSPACE
    assert st(T=40000, tau=1, ld=65536, ws_bytes=1 << 40) == api.FM_ERR_UNSUPPORTED


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """With no built library the binding raises; there is no fallback path to compute on."""
    monkeypatch.setattr(api, "LIB_PATH", str(tmp_path / "libfm.so"))
    monkeypatch.setattr(api, "_lib", None)
    with pytest.raises(FileNotFoundError):
        api.lib()
    with pytest.raises(FileNotFoundError):
        api.fm_workspace_bytes(api.FM_OP_TOPK, 1, 100000)
