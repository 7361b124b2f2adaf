// fm_api.hip -- the C ABI of libfm.so (declared and documented in include/fm.h).
//
// Host layer only: validate every argument, fill the kernel argument blocks, enqueue the
// kernels on the caller's stream.  Nothing here allocates device memory, synchronises, or
// keeps state beyond a thread-local error message.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "fm_internal.h"

// The static workspace of fm_score_resident_noalloc: each GPU holds its own copy of this array
// (at its own address) from the library's first use on that GPU.  In host code the name is
// only a stand-in: the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[FM_STATIC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512];

fm_status fail(fm_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

fm_status ok() {
    g_err[0] = 0;
    return FM_OK;
}

#define REQUIRE(cond, status, ...)                     \
    do {                                               \
        if (!(cond)) return fail((status), __VA_ARGS__); \
    } while (0)

#define CHECK(expr)                           \
    do {                                      \
        fm_status s_ = (expr);                \
        if (s_ != FM_OK) return s_;           \
    } while (0)

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int key_fmt(fm_dtype d) {
    return d == FM_F32 ? fm::KEY_F32 : d == FM_BF16 ? fm::KEY_BF16 : fm::KEY_FP8;
}

fm_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(FM_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return FM_OK;
}

fm_status check_kv(const fm_kv_desc *kv, int n_pools_needed) {
    REQUIRE(kv, FM_ERR_INVALID_ARG, "kv descriptor is NULL");
    REQUIRE(kv->page_size == FM_PAGE_SIZE, FM_ERR_UNSUPPORTED, "page_size %d (only %d)",
            kv->page_size, FM_PAGE_SIZE);
    REQUIRE(kv->head_dim == FM_HEAD_DIM, FM_ERR_UNSUPPORTED, "head_dim %d (only %d)",
            kv->head_dim, FM_HEAD_DIM);
    REQUIRE(kv->key_dtype == FM_F32 || kv->key_dtype == FM_BF16 ||
                kv->key_dtype == FM_FP8_E4M3_SCALED132,
            FM_ERR_UNSUPPORTED, "key dtype %d", (int)kv->key_dtype);
    REQUIRE(kv->B >= 1, FM_ERR_INVALID_ARG, "B = %d", kv->B);
    REQUIRE(kv->n_pools >= n_pools_needed && kv->n_pools <= FM_MAX_POOLS, FM_ERR_INVALID_ARG,
            "n_pools = %d, need %d..%d", kv->n_pools, n_pools_needed, FM_MAX_POOLS);
    for (int l = 0; l < kv->n_pools; ++l) {
        REQUIRE(kv->pool[l], FM_ERR_INVALID_ARG, "pool[%d] is NULL", l);
        REQUIRE(aligned(kv->pool[l], 16), FM_ERR_INVALID_ARG, "pool[%d] not 16-byte aligned", l);
    }
    REQUIRE(kv->block_table && kv->seq_lens, FM_ERR_INVALID_ARG, "block_table / seq_lens NULL");
    REQUIRE(kv->max_seq_len >= 0 && kv->max_seq_len <= (int64_t)INT32_MAX, FM_ERR_INVALID_ARG,
            "max_seq_len = %lld", (long long)kv->max_seq_len);
    REQUIRE(kv->bt_ld >= 1 && kv->bt_ld >= (kv->max_seq_len + FM_PAGE_SIZE - 1) / FM_PAGE_SIZE,
            FM_ERR_INVALID_ARG, "bt_ld = %lld < ceil(max_seq_len / 64)", (long long)kv->bt_ld);
    REQUIRE(kv->n_phys_pages >= 1 && kv->n_phys_pages <= (int64_t)INT32_MAX, FM_ERR_INVALID_ARG,
            "n_phys_pages = %lld", (long long)kv->n_phys_pages);
    return FM_OK;
}

fm_status check_q(const fm_query_desc *q, const fm_kv_desc *kv, const char *name) {
    REQUIRE(q, FM_ERR_INVALID_ARG, "%s: query descriptor is NULL", name);
    REQUIRE(q->T >= 0, FM_ERR_INVALID_ARG, "%s: T = %d", name, q->T);
    REQUIRE(q->n_heads == FM_N_HEADS || q->n_heads == FM_N_HEADS_WIDE, FM_ERR_UNSUPPORTED,
            "%s: n_heads %d (%d, or %d)", name, q->n_heads, FM_N_HEADS, FM_N_HEADS_WIDE);
    REQUIRE(q->w_dtype == FM_F32 || q->w_dtype == FM_BF16, FM_ERR_UNSUPPORTED,
            "%s: w dtype %d", name, (int)q->w_dtype);
    const fm_dtype k = kv->key_dtype;
    const bool combo = (q->q_dtype == FM_F32 && k == FM_F32) ||
                       (q->q_dtype == FM_BF16 && (k == FM_BF16 || k == FM_FP8_E4M3_SCALED132)) ||
                       (q->q_dtype == FM_FP8_E4M3 && k == FM_FP8_E4M3_SCALED132);
    REQUIRE(combo, FM_ERR_UNSUPPORTED, "%s: q dtype %d with key dtype %d", name, (int)q->q_dtype,
            (int)k);
    REQUIRE(q->n_heads == FM_N_HEADS || (q->q_dtype == FM_BF16 && k == FM_FP8_E4M3_SCALED132) ||
                (q->q_dtype == FM_F32 && k == FM_F32),
            FM_ERR_UNSUPPORTED, "%s: %d heads need bf16 q with fp8 keys, or fp32 q and keys", name,
            q->n_heads);
    if (q->T == 0) return FM_OK;
    REQUIRE(q->q && q->w, FM_ERR_INVALID_ARG, "%s: q / w NULL", name);
    REQUIRE(aligned(q->q, 16), FM_ERR_INVALID_ARG, "%s: q not 16-byte aligned", name);
    REQUIRE(q->q_dtype != FM_FP8_E4M3 || q->q_scale, FM_ERR_INVALID_ARG,
            "%s: fp8 q needs q_scale", name);
    REQUIRE(q->row_req || q->T == kv->B || kv->B == 1, FM_ERR_INVALID_ARG,
            "%s: row_req NULL needs T == B or B == 1 (T = %d, B = %d)", name, q->T, kv->B);
    REQUIRE(!q->q_pos || q->compress_ratio >= 1, FM_ERR_INVALID_ARG,
            "%s: compress_ratio = %d", name, q->compress_ratio);
    return FM_OK;
}

fm::QArgs make_q(const fm_query_desc *q, const fm_kv_desc *kv) {
    fm::QArgs a;
    a.q = q->q;
    a.q_scale = q->q_scale;
    a.w = q->w;
    a.w_bf16 = q->w_dtype == FM_BF16;
    a.n_heads = q->n_heads;
    a.T = q->T;
    a.row_req = q->row_req;
    a.b_is_zero = (!q->row_req && kv->B == 1) ? 1 : 0;
    a.q_pos = q->q_pos;
    a.ratio = q->compress_ratio >= 1 ? q->compress_ratio : 1;
    a.row_pool = q->row_pool;
    return a;
}

fm::KvArgs make_kv(const fm_kv_desc *kv) {
    fm::KvArgs a;
    for (int l = 0; l < FM_MAX_POOLS; ++l)
        a.pool[l] = l < kv->n_pools ? (const uint8_t *)kv->pool[l] : nullptr;
    a.n_pools = kv->n_pools;
    a.bt = kv->block_table;
    a.bt_ld = kv->bt_ld;
    a.seq_lens = kv->seq_lens;
    a.n_phys = kv->n_phys_pages;
    a.B = kv->B;
    return a;
}

// Page slots per wave: about one round of waves (resident = the waves the kernel keeps on the
// chip at once), so each wave streams a run of pages instead of paying its start-up (query and
// page-table loads) several times; at least 1, at most 16 slots each.
#ifndef FM_F8_GENS
#define FM_F8_GENS 1    // fp8 scoring: grid generations
#endif
#ifndef FM_DEC_GENS
#define FM_DEC_GENS 1   // bf16 scoring: grid generations (resident waves x this many waves)
#endif
int pages_per_wave(int64_t total_slots, int64_t resident) {
    int64_t p = (total_slots + resident - 1) / resident;
    if (p < 1) p = 1;
    if (p > 16) p = 16;
    return (int)p;
}

fm_status run_score(const fm_query_desc *q, const fm_kv_desc *kv, const int32_t *res_pages,
                    const int32_t *n_res, int64_t res_ld, float *out, int64_t out_ld,
                    int64_t n_slots, hipStream_t st) {
    fm::ScoreArgs a;
    a.q = make_q(q, kv);
    a.kv = make_kv(kv);
    a.res_pages = res_pages;
    a.n_res = n_res;
    a.res_ld = res_ld;
    a.out = out;
    a.out_ld = out_ld;
    a.n_slots = n_slots;
    // waves resident at once: 256 CUs x 4 SIMDs x waves per SIMD of the kernel used
    const int64_t per_simd = kv->key_dtype == FM_BF16 ? 4 : kv->key_dtype == FM_FP8_E4M3_SCALED132 &&
                             q->q_dtype == FM_BF16 ? (q->n_heads == FM_N_HEADS ? FM_F8_WPE : 2) : 2;
    a.ppw = pages_per_wave((int64_t)q->T * n_slots, 1024 * per_simd *
                           (kv->key_dtype == FM_BF16 ? FM_DEC_GENS : FM_F8_GENS));
    if (kv->key_dtype == FM_F32) return launched(fm::launch_score_f32(a, st), "score_f32");
    const int qf = q->q_dtype == FM_FP8_E4M3 ? fm::Q_FP8 : fm::Q_BF16;
    return launched(fm::launch_score(a, key_fmt(kv->key_dtype), qf, st), "score");
}

// ---------------------------------------------------------------- fused scoring + top-k
// Workspace of the calls that score and select: either the fused path's chunk candidates or the
// unfused path's logits and top-k workspace.
size_t fused_region_bytes(int T) {
    return fm::align_up((size_t)T * fm::kFuseMaxChunks * 4, 256) +
           fm::align_up((size_t)T * fm::kFuseMaxChunks * 16, 256) +
           2 * fm::align_up((size_t)T * fm::kFuseMaxCand * 4, 256);
}
size_t unfused_region_bytes(int T, int64_t n) {
    return fm::align_up((size_t)T * (size_t)n * sizeof(float), 256) + fm::topk_ws_bytes(T, n);
}
size_t select_ws_bytes(int T, int64_t n) {
    return std::max(fused_region_bytes(T), unfused_region_bytes(T, n));
}

// The fused path's work split: W waves a workgroup, ppw page slots a wave, n_chunks workgroups
// a row.  It aims at one workgroup per CU (256), and gives way to the unfused path (scoring
// kernel + top-k kernel) when a row would need more than kFuseMaxChunks chunks, or when few
// workgroups would each stream long runs of pages while most of the chip idles.
struct FusePlan {
    bool fused;
    int ppw, n_chunks, ppw_pad;
};
FusePlan fuse_plan(int T, int64_t n_slots, int k, int nw, int ring, int max_ppw) {
    FusePlan p{false, 0, 0, 0};
    if (nw <= 0 || T <= 0 || n_slots <= 0) return p;
    constexpr int64_t kWgTarget = 256;
    auto clamp_ppw = [&](int64_t x) { return x < 1 ? (int64_t)1 : (x > max_ppw ? (int64_t)max_ppw : x); };
    auto chunks_of = [&](int64_t ppw) { return (n_slots + nw * ppw - 1) / (nw * ppw); };
    int64_t ppw = clamp_ppw(((int64_t)T * n_slots + kWgTarget * nw - 1) / (kWgTarget * nw));
    int64_t ch = chunks_of(ppw);
    if (ch > fm::kFuseMaxChunks) {
        ppw = clamp_ppw((n_slots + (int64_t)nw * fm::kFuseMaxChunks - 1) / ((int64_t)nw * fm::kFuseMaxChunks));
        ch = chunks_of(ppw);
    }
    int k2 = 1;
    while (k2 < k) k2 *= 2;                          // the chunk slots hold a power of two >= k
    if (ch > fm::kFuseMaxChunks || ch * k2 > fm::kFuseMaxCand) return p;
    if ((int64_t)T * ch < kWgTarget / 2 && ppw > 2) return p;
    p.fused = true;
    p.ppw = (int)ppw;
    p.n_chunks = (int)ch;
    p.ppw_pad = (int)((ppw + ring - 1) / ring * ring);
    return p;
}

// Score and select: rows of q over n_slots page slots each (the listed resident pages when
// res_pages is given, else logical pages 0 .. n_slots - 1), top-k of the visible (and, with a
// mask, resident) entries.  logits (nullable) also receives the logits.  Arguments validated.
fm_status score_select(const fm_query_desc *q, const fm_kv_desc *kv, const int32_t *res_pages,
                       const int32_t *n_res, int64_t res_ld, int64_t n_slots, const uint8_t *mask,
                       int64_t mask_ld, int k, int cells, int32_t *out_idx, float *out_val,
                       float *logits, int64_t logits_ld, void *ws, hipStream_t st) {
    const int kf = key_fmt(kv->key_dtype);
    const int qf = q->q_dtype == FM_FP8_E4M3 ? fm::Q_FP8 : q->q_dtype == FM_BF16 ? fm::Q_BF16 : fm::Q_F32;
    const fm::FuseShape fs = fm::fuse_shape(kf, qf, q->n_heads);
    const bool prefill = q->q_dtype == FM_FP8_E4M3 && kv->B == 1 && q->T >= 16 && !res_pages &&
                         !q->row_pool;
    const FusePlan p = prefill ? FusePlan{false, 0, 0, 0} : fuse_plan(q->T, n_slots, k, fs.waves, fs.round, fs.max_ppw);
    if (p.fused) {
        fm::ScoreArgs a;
        a.q = make_q(q, kv);
        a.kv = make_kv(kv);
        a.res_pages = res_pages;
        a.n_res = n_res;
        a.res_ld = res_ld;
        a.out = logits;
        a.out_ld = logits ? logits_ld : 0;
        a.n_slots = n_slots;
        a.ppw = p.ppw;
        fm::FuseArgs f;
        f.k = k;
        f.n_chunks = p.n_chunks;
        // a chunk's candidate slots: a power of two (the merge finds a slot's chunk by a
        // shift), at least k, together at most kFuseMaxCand
        auto pow2_floor = [](int x) { int p = 1; while (2 * p <= x) p *= 2; return p; };
        auto pow2_ceil = [](int x) { int p = 1; while (p < x) p *= 2; return p; };
        f.cap = std::max(pow2_ceil(k), pow2_floor(fm::kFuseMaxCand / p.n_chunks));
        f.ppw_pad = p.ppw_pad;
        f.mask = mask;
        f.mask_ld = mask ? mask_ld : 0;
        f.cells = cells;
        // entries below 2^18 are ordered through the merge's bitmap: list positions (cells),
        // or logical entries below the block table's width
        const int64_t max_entry = (!res_pages || cells) ? n_slots * FM_PAGE_SIZE : kv->bt_ld * FM_PAGE_SIZE;
        f.bit_words = max_entry <= (int64_t)1 << 18 ? (int)((max_entry + 2047) / 2048 * 64) : 0;
        uint8_t *w8 = (uint8_t *)ws;
        f.cnt = (int32_t *)w8;
        w8 += fm::align_up((size_t)q->T * fm::kFuseMaxChunks * 4, 256);
        f.cstat = (float4 *)w8;
        w8 += fm::align_up((size_t)q->T * fm::kFuseMaxChunks * 16, 256);
        f.cval = (float *)w8;
        w8 += fm::align_up((size_t)q->T * fm::kFuseMaxCand * 4, 256);
        f.cidx = (int32_t *)w8;
        f.out_idx = out_idx;
        f.out_val = out_val;
        return launched(fm::launch_score_topk(a, f, kf, qf, st), "score_topk");
    }
    // unfused: the logits (into the caller's buffer, or the workspace), then the top-k
    const int64_t ld = logits ? logits_ld : n_slots * FM_PAGE_SIZE;
    uint8_t *after = (uint8_t *)ws;
    float *wl = logits ? logits : (float *)after;
    if (!logits) after += fm::align_up((size_t)q->T * (size_t)ld * sizeof(float), 256);
    if (prefill) {
        fm::PrefillArgs a;
        a.q = make_q(q, kv);
        a.kv = make_kv(kv);
        a.out = wl;
        a.out_ld = ld;
        fm::prefill_plan(a, q->T, (ld + FM_PAGE_SIZE - 1) / FM_PAGE_SIZE);
        CHECK(launched(fm::launch_prefill(a, st), "prefill"));
    } else {
        CHECK(run_score(q, kv, res_pages, n_res, res_ld, wl, ld, n_slots, st));
    }
    fm::TopkArgs a;
    a.logits = wl;
    a.ld = ld;
    a.T = q->T;
    a.n_valid = nullptr;
    a.mask = mask;
    a.mask_ld = mask ? mask_ld : 0;
    a.row_req = q->row_req;
    a.b_is_zero = (!q->row_req && kv->B == 1) ? 1 : 0;
    a.res_pages = res_pages;
    a.n_res = n_res;
    a.res_ld = res_ld;
    a.res_cells = cells;
    a.B = kv->B;
    a.k = k;
    a.out_idx = out_idx;
    a.out_val = out_val;
    fm::TopkWs W;
    const bool staged = fm::topk_ws_bytes(q->T, ld) > 0;
    if (staged) W = fm::topk_ws_carve(after, q->T, ld);
    return launched(fm::launch_topk(a, staged ? &W : nullptr, st), "topk");
}

// Arguments of two-level scoring other than the workspace.
fm_status check_score_resident(const fm_query_desc *q, const fm_kv_desc *kv,
                               const int32_t *resident_pages, const int32_t *n_resident,
                               int64_t res_ld, int k, const int32_t *out_idx) {
    CHECK(check_kv(kv, 1));
    CHECK(check_q(q, kv, "q"));
    REQUIRE(k >= 1 && k <= FM_MAX_K, FM_ERR_UNSUPPORTED, "k = %d (1..%d)", k, FM_MAX_K);
    REQUIRE(res_ld >= 1 && res_ld * FM_PAGE_SIZE <= (int64_t)INT32_MAX / 4, FM_ERR_INVALID_ARG,
            "res_ld = %lld", (long long)res_ld);
    if (q->T == 0) return FM_OK;
    REQUIRE(resident_pages && n_resident && out_idx, FM_ERR_INVALID_ARG,
            "resident_pages / n_resident / out_idx NULL");
    return FM_OK;
}

fm_status score_resident(const fm_query_desc *q, const fm_kv_desc *kv,
                            const int32_t *resident_pages, const int32_t *n_resident,
                            int64_t res_ld, int k, int32_t *out_idx, float *out_val, void *ws,
                            size_t ws_bytes, void *stream, int cells) {
    CHECK(check_score_resident(q, kv, resident_pages, n_resident, res_ld, k, out_idx));
    if (q->T == 0) return ok();
    const size_t need = fm_workspace_bytes(FM_OP_SCORE_RESIDENT, q->T, res_ld * FM_PAGE_SIZE);
    REQUIRE(ws && ws_bytes >= need && aligned(ws, 256), FM_ERR_WORKSPACE,
            "workspace %zu bytes at %p, need %zu (256-byte aligned)", ws_bytes, ws, need);
    CHECK(score_select(q, kv, resident_pages, n_resident, res_ld, res_ld, nullptr, 0, k, cells,
                       out_idx, out_val, nullptr, 0, ws, (hipStream_t)stream));
    return ok();
}

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

fm_status scratch_address(hipStream_t st, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    REQUIRE(e == hipSuccess, FM_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    REQUIRE(dev >= 0 && dev < kMaxDevices, FM_ERR_UNSUPPORTED, "device %d (at most %d devices)",
            dev, kMaxDevices);
    if (st) {
        int sdev = -1;
        e = hipStreamGetDevice(st, &sdev);
        REQUIRE(e == hipSuccess, FM_ERR_INVALID_ARG, "hipStreamGetDevice: %s",
                hipGetErrorString(e));
        REQUIRE(sdev == dev, FM_ERR_INVALID_ARG,
                "the stream belongs to device %d, the current device is %d", sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        REQUIRE(e == hipSuccess && p, FM_ERR_LAUNCH, "hipGetSymbolAddress(scratch): %s",
                hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FM_OK;
}

// ---------------------------------------------------------------- query encoder
fm_status check_enc(const fm_encoder_desc *e) {
    REQUIRE(e, FM_ERR_INVALID_ARG, "encoder descriptor is NULL");
    REQUIRE(e->wq_a && e->q_norm && e->wq_b && e->w_proj, FM_ERR_INVALID_ARG,
            "encoder weight pointer is NULL");
    REQUIRE(aligned(e->wq_a, 16) && aligned(e->wq_b, 16) && aligned(e->w_proj, 16),
            FM_ERR_INVALID_ARG, "wq_a, wq_b and w_proj must be 16-byte aligned");
    REQUIRE(e->head_dim == FM_HEAD_DIM, FM_ERR_UNSUPPORTED, "head_dim %d (only %d)", e->head_dim,
            FM_HEAD_DIM);
    REQUIRE(e->d_model >= 16 && e->d_model % 16 == 0 && e->d_model <= (1 << 20),
            FM_ERR_UNSUPPORTED, "d_model %d (a multiple of 16, at most 2^20)", e->d_model);
    REQUIRE(e->q_rank >= 32 && e->q_rank % 32 == 0, FM_ERR_UNSUPPORTED,
            "q_rank %d (a multiple of 32)", e->q_rank);
    REQUIRE(e->n_heads >= 32 && e->n_heads % 32 == 0 && e->n_heads <= 1024, FM_ERR_UNSUPPORTED,
            "n_heads %d (a multiple of 32, at most 1024)", e->n_heads);
    REQUIRE(e->q_rank + e->n_heads <= 4096, FM_ERR_UNSUPPORTED,
            "q_rank + n_heads = %d (at most 4096)", e->q_rank + e->n_heads);
    REQUIRE(e->rope_dim >= 0 && e->rope_dim <= FM_HEAD_DIM && e->rope_dim % 2 == 0,
            FM_ERR_INVALID_ARG, "rope_dim %d (even, 0 .. %d)", e->rope_dim, FM_HEAD_DIM);
    REQUIRE(e->rms_eps >= 0.f && isfinite(e->rms_eps), FM_ERR_INVALID_ARG, "rms_eps");
    REQUIRE(e->rope_base > 1.f && isfinite(e->rope_base), FM_ERR_INVALID_ARG, "rope_base");
    REQUIRE(e->rope_factor >= 1.f && isfinite(e->rope_factor), FM_ERR_INVALID_ARG,
            "rope_factor");
    REQUIRE(e->rope_orig_len > 0, FM_ERR_INVALID_ARG, "rope_orig_len");
    REQUIRE(e->beta_slow > 0.f && e->beta_fast > e->beta_slow && isfinite(e->beta_fast),
            FM_ERR_INVALID_ARG, "beta_fast > beta_slow > 0 required");
    return FM_OK;
}

// Split-K plan of a product with `tiles` 32 x 32 output tiles over K: about FM_ENC_WAVES waves, each
// split a multiple of 128 long (the kernel's unrolled round) unless K itself is shorter.
#ifndef FM_ENC_WAVES
#define FM_ENC_WAVES 2048   // waves a product aims at
#endif
// Work split of a product with `tiles` 32 x 32 output tiles over K: S waves a workgroup (at
// most 4) and Z workgroups a tile (partial sums), about FM_ENC_WAVES waves on at least ~256
// workgroups in all when the shape allows, each wave's K range a multiple of 64 long (at least
// 128) unless K is shorter.
struct EncSplit {
    int S, Z, ksplit;
};
EncSplit enc_split(int64_t tiles, int K) {
    EncSplit p{1, 1, K};
    auto room = [&](int parts) { return K / (2 * parts) >= 128; };
    while (p.S < 4 && tiles * p.S * p.Z < FM_ENC_WAVES && room(p.S * p.Z)) p.S *= 2;
    while (p.Z < 16 && tiles * p.S * p.Z < FM_ENC_WAVES && room(p.S * p.Z)) p.Z *= 2;
    int64_t ks = (K + p.S * p.Z - 1) / (p.S * p.Z);
    ks = (ks + 63) / 64 * 64;
    if (ks >= K) ks = K;
    p.ksplit = (int)ks;
    return p;
}

struct EncPlan {
    EncSplit g1, g2;
    size_t off_r, off_c2, bytes;
};

EncPlan enc_plan(const fm_encoder_desc *e, int T) {
    EncPlan p;
    const int64_t mt = (T + 31) / 32;
    const int64_t n1 = e->q_rank + e->n_heads, n2 = (int64_t)e->n_heads * FM_HEAD_DIM;
    p.g1 = enc_split(mt * (n1 / 32), e->d_model);
    p.g2 = enc_split(mt * (n2 / 32), e->q_rank);
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t c1 = al((size_t)p.g1.Z * T * n1 * 4), r = al((size_t)T * e->q_rank * 2);
    const size_t c2 = al((size_t)p.g2.Z * T * n2 * 4);
    p.off_r = c1;
    p.off_c2 = c1 + r;
    p.bytes = c1 + r + c2;
    return p;
}

// YaRN per-pair frequencies: theta_i = base^(-2i/d), divided by the factor above the slow
// correction dim, kept below the fast one, blended linearly in between.  The correction dim of
// beta is the pair index whose wavelength fits beta times into the original context.
void yarn_freqs(const fm_encoder_desc *e, double *out) {
    const int d = e->rope_dim, half = d / 2;
    const double base = e->rope_base, f = e->rope_factor;
    auto corr = [&](double beta) {
        return d * log((double)e->rope_orig_len / (beta * 2.0 * M_PI)) / (2.0 * log(base));
    };
    double lo = floor(corr(e->beta_fast)), hi = ceil(corr(e->beta_slow));
    if (lo < 0) lo = 0;
    if (hi > half - 1) hi = half - 1;
    if (hi == lo) hi = lo + 0.001;
    for (int i = 0; i < half; ++i) {
        const double th = pow(base, -2.0 * i / d);
        if (f == 1.0) {
            out[i] = th;
            continue;
        }
        double ramp = (i - lo) / (hi - lo);
        ramp = ramp < 0 ? 0 : ramp > 1 ? 1 : ramp;
        out[i] = th / f * ramp + th * (1.0 - ramp);
    }
}

}  // namespace

extern "C" {

fm_status fm_index_logits(const fm_query_desc *q, const fm_kv_desc *kv, float *logits,
                          int64_t ld, void *stream) {
    CHECK(check_kv(kv, 1));
    CHECK(check_q(q, kv, "q"));
    REQUIRE(logits, FM_ERR_INVALID_ARG, "logits is NULL");
    REQUIRE(ld >= 1 && ld <= (int64_t)INT32_MAX / 4, FM_ERR_INVALID_ARG, "ld = %lld (1 .. 2^29)",
            (long long)ld);
    REQUIRE(aligned(logits, 4), FM_ERR_INVALID_ARG, "logits not 4-byte aligned");
    if (q->T == 0) return ok();
    const int64_t n_pages = (ld + FM_PAGE_SIZE - 1) / FM_PAGE_SIZE;
    if (q->q_dtype == FM_FP8_E4M3 && kv->B == 1 && q->T >= 16 && !q->row_pool) {
        // many rows over one request's keys (prefill): tiled for key reuse across rows
        fm::PrefillArgs a;
        a.q = make_q(q, kv);
        a.kv = make_kv(kv);
        a.out = logits;
        a.out_ld = ld;
        fm::prefill_plan(a, q->T, n_pages);
        CHECK(launched(fm::launch_prefill(a, (hipStream_t)stream), "prefill"));
        return ok();
    }
    CHECK(run_score(q, kv, nullptr, nullptr, 0, logits, ld, n_pages, (hipStream_t)stream));
    return ok();
}

fm_status fm_index_topk(const fm_query_desc *q, const fm_kv_desc *kv, const uint8_t *mask,
                        int64_t mask_ld, int k, int32_t *out_idx, float *out_val, float *logits,
                        int64_t logits_ld, void *ws, size_t ws_bytes, void *stream) {
    CHECK(check_kv(kv, 1));
    CHECK(check_q(q, kv, "q"));
    REQUIRE(k >= 1 && k <= FM_MAX_K, FM_ERR_UNSUPPORTED, "k = %d (1..%d)", k, FM_MAX_K);
    REQUIRE(!logits || (logits_ld >= 1 && logits_ld <= (int64_t)INT32_MAX / 4 && aligned(logits, 4)),
            FM_ERR_INVALID_ARG, "logits_ld = %lld (1 .. 2^29, 4-byte aligned logits)",
            (long long)logits_ld);
    const int64_t n_slots = (kv->max_seq_len + FM_PAGE_SIZE - 1) / FM_PAGE_SIZE;
    REQUIRE(n_slots >= 1, FM_ERR_INVALID_ARG, "max_seq_len = 0: nothing to score");
    REQUIRE(n_slots * FM_PAGE_SIZE <= (int64_t)INT32_MAX / 4, FM_ERR_UNSUPPORTED,
            "max_seq_len = %lld (at most 2^29)", (long long)kv->max_seq_len);
    const int64_t mask_need = std::max(n_slots * FM_PAGE_SIZE, logits ? logits_ld : (int64_t)0);
    REQUIRE(!mask || (mask_ld >= mask_need && mask_ld <= (int64_t)INT32_MAX),
            FM_ERR_INVALID_ARG, "mask_ld = %lld (%lld .. 2^31 - 1)", (long long)mask_ld,
            (long long)mask_need);
    if (q->T == 0) return ok();
    REQUIRE(out_idx, FM_ERR_INVALID_ARG, "out_idx is NULL");
    // with logits wanted, the pages up to logits_ld are covered too (past max_seq_len they are
    // invisible: -inf written, nothing read)
    const int64_t n_cover = logits ? std::max(n_slots, (logits_ld + FM_PAGE_SIZE - 1) / FM_PAGE_SIZE)
                                   : n_slots;
    const size_t need = fm_workspace_bytes(FM_OP_INDEX_TOPK, q->T, n_cover * FM_PAGE_SIZE);
    REQUIRE(ws && ws_bytes >= need && aligned(ws, 256), FM_ERR_WORKSPACE,
            "workspace %zu bytes at %p, need %zu (256-byte aligned)", ws_bytes, ws, need);
    CHECK(score_select(q, kv, nullptr, nullptr, 0, n_cover, mask, mask_ld, k, 0, out_idx, out_val,
                       logits, logits_ld, ws, (hipStream_t)stream));
    return ok();
}

fm_status fm_topk512(const float *logits, int64_t ld, int T, const int32_t *n_valid,
                     const uint8_t *mask, int64_t mask_ld, const int32_t *row_req, int k,
                     int32_t *out_idx, float *out_val, void *ws, size_t ws_bytes, void *stream) {
    REQUIRE(T >= 0, FM_ERR_INVALID_ARG, "T = %d", T);
    REQUIRE(k >= 1 && k <= FM_MAX_K, FM_ERR_UNSUPPORTED, "k = %d (1..%d)", k, FM_MAX_K);
    REQUIRE(ld >= 1 && ld <= (int64_t)INT32_MAX, FM_ERR_INVALID_ARG, "ld = %lld", (long long)ld);
    if (T == 0) return ok();
    REQUIRE(logits && out_idx, FM_ERR_INVALID_ARG, "logits / out_idx NULL");
    REQUIRE(!mask || mask_ld >= ld, FM_ERR_INVALID_ARG, "mask_ld %lld < ld %lld",
            (long long)mask_ld, (long long)ld);
    fm::TopkArgs a;
    a.logits = logits;
    a.ld = ld;
    a.T = T;
    a.n_valid = n_valid;
    a.mask = mask;
    a.mask_ld = mask_ld;
    a.row_req = row_req;
    a.b_is_zero = 0;
    a.res_pages = nullptr;
    a.res_cells = 0;
    a.n_res = nullptr;
    a.res_ld = 0;
    a.B = INT32_MAX;   // mask rows are the caller's: row_req[t] must index one
    a.k = k;
    a.out_idx = out_idx;
    a.out_val = out_val;
    // with the workspace it asks for, long rows are filtered by many workgroups first
    const size_t need = fm::topk_ws_bytes(T, ld);
    fm::TopkWs W;
    const bool staged = need > 0 && ws && aligned(ws, 256) && ws_bytes >= need;
    if (staged) W = fm::topk_ws_carve(ws, T, ld);
    CHECK(launched(fm::launch_topk(a, staged ? &W : nullptr, (hipStream_t)stream), "topk"));
    return ok();
}

fm_status fm_score_resident(const fm_query_desc *q, const fm_kv_desc *kv,
                            const int32_t *resident_pages, const int32_t *n_resident,
                            int64_t res_ld, int k, int32_t *out_idx, float *out_val, void *ws,
                            size_t ws_bytes, void *stream) {
    return score_resident(q, kv, resident_pages, n_resident, res_ld, k, out_idx, out_val, ws,
                          ws_bytes, stream, 0);
}

fm_status fm_score_resident_noalloc(const fm_query_desc *q, const fm_kv_desc *kv,
                                    const int32_t *resident_pages, const int32_t *n_resident,
                                    int64_t res_ld, int k, int32_t *out_idx, float *out_val,
                                    void *stream) {
    CHECK(check_score_resident(q, kv, resident_pages, n_resident, res_ld, k, out_idx));
    if (q->T == 0) return ok();
    const size_t need = fm_workspace_bytes(FM_OP_SCORE_RESIDENT, q->T, res_ld * FM_PAGE_SIZE);
    REQUIRE(need <= FM_STATIC_SCRATCH_BYTES, FM_ERR_WORKSPACE,
            "T = %d rows x res_ld = %lld pages need %zu bytes of workspace; the static scratch "
            "holds %llu",
            q->T, (long long)res_ld, need, (unsigned long long)FM_STATIC_SCRATCH_BYTES);
    void *ws = nullptr;
    CHECK(scratch_address((hipStream_t)stream, &ws));
    return score_resident(q, kv, resident_pages, n_resident, res_ld, k, out_idx, out_val, ws,
                          FM_STATIC_SCRATCH_BYTES, stream, 0);
}

fm_status fm_score_resident_cells(const fm_query_desc *q, const fm_kv_desc *kv,
                                  const int32_t *resident_pages, const int32_t *n_resident,
                                  int64_t res_ld, int k, int32_t *out_cells, float *out_val,
                                  void *ws, size_t ws_bytes, void *stream) {
    return score_resident(q, kv, resident_pages, n_resident, res_ld, k, out_cells, out_val, ws,
                          ws_bytes, stream, 1);
}

fm_status fm_densest_pages(const int32_t *density, int64_t density_ld, int B, int64_t n_pages,
                           int kmax, int32_t *out_pages, int32_t *out_count, void *stream) {
    REQUIRE(B >= 0, FM_ERR_INVALID_ARG, "B = %d", B);
    REQUIRE(kmax >= 1 && kmax <= FM_MAX_K, FM_ERR_UNSUPPORTED, "kmax = %d (1..%d)", kmax, FM_MAX_K);
    REQUIRE(n_pages >= 0 && n_pages <= density_ld && n_pages <= (int64_t)INT32_MAX,
            FM_ERR_INVALID_ARG, "n_pages = %lld, density_ld = %lld", (long long)n_pages,
            (long long)density_ld);
    if (B == 0) return ok();
    REQUIRE(density && out_pages, FM_ERR_INVALID_ARG, "density / out_pages NULL");
    fm::DensestArgs a;
    a.density = density;
    a.ld = density_ld;
    a.n_pages = n_pages;
    a.kmax = kmax;
    a.out_pages = out_pages;
    a.out_count = out_count;
    CHECK(launched(fm::launch_densest(a, B, (hipStream_t)stream), "densest_pages"));
    return ok();
}

fm_status fm_resident_mask(const fm_query_desc *q_layers, int n_layers, const fm_kv_desc *kv,
                           fm_union_mode mode, float threshold, int32_t n_sink,
                           int32_t n_recent, uint8_t *mask, int64_t mask_ld,
                           int32_t *page_count, int32_t *page_list, int64_t page_list_ld,
                           int32_t *page_density, float *union_score, void *stream) {
    REQUIRE(n_layers >= 1 && n_layers <= FM_MAX_LAYERS, FM_ERR_INVALID_ARG, "n_layers = %d",
            n_layers);
    CHECK(check_kv(kv, n_layers));
    REQUIRE(q_layers, FM_ERR_INVALID_ARG, "q_layers is NULL");
    for (int l = 0; l < n_layers; ++l) {
        CHECK(check_q(&q_layers[l], kv, "q_layers[l]"));
        REQUIRE(!q_layers[l].row_pool, FM_ERR_INVALID_ARG,
                "q_layers[%d].row_pool must be NULL (encoder l scores pool[l])", l);
        REQUIRE(q_layers[l].T == kv->B, FM_ERR_INVALID_ARG,
                "q_layers[%d].T = %d, must equal B = %d (one row per request)", l,
                q_layers[l].T, kv->B);
        REQUIRE(q_layers[l].q_dtype == q_layers[0].q_dtype, FM_ERR_UNSUPPORTED,
                "layers mix q dtypes");
        REQUIRE(q_layers[l].n_heads == q_layers[0].n_heads, FM_ERR_UNSUPPORTED,
                "layers mix head counts");
        REQUIRE(q_layers[l].q_dtype != FM_FP8_E4M3, FM_ERR_UNSUPPORTED,
                "fp8 queries are not supported for the resident mask");
    }
    REQUIRE(mode == FM_UNION_MAX || mode == FM_UNION_MEAN, FM_ERR_INVALID_ARG, "mode = %d",
            (int)mode);
    REQUIRE(threshold > 0.f && threshold < 1.f, FM_ERR_INVALID_ARG,
            "threshold %g outside (0, 1)", (double)threshold);
    REQUIRE(n_sink >= 0 && n_recent >= 0, FM_ERR_INVALID_ARG, "n_sink / n_recent negative");
    REQUIRE(mask && page_count, FM_ERR_INVALID_ARG, "mask / page_count NULL");
    REQUIRE(mask_ld >= 1 && mask_ld <= (int64_t)INT32_MAX, FM_ERR_INVALID_ARG, "mask_ld = %lld",
            (long long)mask_ld);
    REQUIRE(!page_list || page_list_ld >= 1, FM_ERR_INVALID_ARG, "page_list_ld = %lld",
            (long long)page_list_ld);
    hipStream_t st = (hipStream_t)stream;
    fm::MaskArgs a;
    for (int l = 0; l < FM_MAX_LAYERS; ++l)
        a.q[l] = l < n_layers ? make_q(&q_layers[l], kv) : fm::QArgs{};
    a.kv = make_kv(kv);
    a.n_layers = n_layers;
    a.mean_mode = mode == FM_UNION_MEAN;
    const double p = (double)threshold;
    a.cut = mode == FM_UNION_MEAN ? threshold : (p == 0.5 ? 0.0f : (float)log(p / (1.0 - p)));
    a.n_sink = n_sink;
    a.n_recent = n_recent;
    a.mask = mask;
    a.mask_ld = mask_ld;
    a.union_score = union_score;
    a.n_pages = (mask_ld + FM_PAGE_SIZE - 1) / FM_PAGE_SIZE;
    // one pool passed for every encoder (fp8 keys, bf16 queries of 64 heads): read it once
    a.shared_keys = 0;
    if (n_layers >= 2 && kv->key_dtype == FM_FP8_E4M3_SCALED132 &&
        q_layers[0].q_dtype == FM_BF16 && q_layers[0].n_heads == FM_N_HEADS) {
        a.shared_keys = 1;
        for (int l = 1; l < n_layers; ++l)
            if (kv->pool[l] != kv->pool[0]) a.shared_keys = 0;
    }
    // fp8 pools: the scoring kernel leaves each page's resident count in page_density (or, as
    // scratch, in page_list when that is wide enough), so compaction reads one word a page
    a.dens_out = nullptr;
    a.dens_ld = 0;
    if (kv->key_dtype == FM_FP8_E4M3_SCALED132) {
        if (page_density) {
            a.dens_out = page_density;
            a.dens_ld = a.n_pages;
        } else if (page_list && page_list_ld >= a.n_pages) {
            a.dens_out = page_list;
            a.dens_ld = page_list_ld;
        }
    }
    CHECK(launched(fm::launch_mask(a, key_fmt(kv->key_dtype), kv->B, st), "resident_mask"));
    fm::CompactArgs c;
    c.mask = mask;
    c.mask_ld = mask_ld;
    c.dens_in = a.dens_out;
    c.dens_ld = a.dens_ld;
    c.n_pages = a.n_pages;
    c.page_count = page_count;
    c.page_list = page_list;
    c.page_list_ld = page_list_ld;
    c.page_density = page_density;
    CHECK(launched(fm::launch_compact(c, kv->B, st), "page_compact"));
    return ok();
}

size_t fm_encode_workspace_bytes(const fm_encoder_desc *e, int T) {
    if (T <= 0 || T > (1 << 22) || check_enc(e) != FM_OK) return 0;
    return enc_plan(e, T).bytes;
}

fm_status fm_encode_queries(const fm_encoder_desc *e, const void *hidden, int T,
                            const int32_t *pos, void *q, float *w, void *ws, size_t ws_bytes,
                            void *stream) {
    CHECK(check_enc(e));
    REQUIRE(T >= 0 && T <= (1 << 22), FM_ERR_INVALID_ARG, "T = %d (0 .. 2^22)", T);
    if (T == 0) return ok();
    REQUIRE(hidden && pos && q && w, FM_ERR_INVALID_ARG, "hidden, pos, q and w must be non-NULL");
    REQUIRE(aligned(hidden, 16), FM_ERR_INVALID_ARG, "hidden must be 16-byte aligned");
    REQUIRE(aligned(q, 4) && aligned(w, 4), FM_ERR_INVALID_ARG, "q and w must be 4-byte aligned");
    const EncPlan p = enc_plan(e, T);
    REQUIRE(ws && aligned(ws, 256) && ws_bytes >= p.bytes, FM_ERR_WORKSPACE,
            "workspace: need %zu bytes, 256-byte aligned", p.bytes);
    hipStream_t st = (hipStream_t)stream;
    uint8_t *base = (uint8_t *)ws;
    float *c1 = (float *)base;
    uint16_t *r = (uint16_t *)(base + p.off_r);
    float *c2 = (float *)(base + p.off_c2);

    fm::EncGemmArgs g1;
    g1.A = (const uint16_t *)hidden;
    g1.lda = e->d_model;
    g1.M = T;
    g1.W0 = (const uint16_t *)e->wq_a;
    g1.N0 = e->q_rank;
    g1.W1 = (const uint16_t *)e->w_proj;
    g1.N1 = e->n_heads;
    g1.K = e->d_model;
    g1.ksplit = p.g1.ksplit;
    g1.S = p.g1.S;
    g1.Z = p.g1.Z;
    g1.C = c1;
    CHECK(launched(fm::launch_enc_gemm(g1, st), "encoder wq_a / w_proj"));

    fm::EncNormArgs na;
    na.C = c1;
    na.Z = p.g1.Z;
    na.M = T;
    na.rank = e->q_rank;
    na.n_heads = e->n_heads;
    na.g = (const uint16_t *)e->q_norm;
    na.eps = e->rms_eps;
    na.w_scale = (float)(1.0 / sqrt((double)e->head_dim * (double)e->n_heads));
    na.r = r;
    na.w = w;
    CHECK(launched(fm::launch_enc_norm(na, st), "encoder RMSNorm"));

    fm::EncGemmArgs g2;
    g2.A = r;
    g2.lda = e->q_rank;
    g2.M = T;
    g2.W0 = (const uint16_t *)e->wq_b;
    g2.N0 = e->n_heads * FM_HEAD_DIM;
    g2.W1 = nullptr;
    g2.N1 = 0;
    g2.K = e->q_rank;
    g2.ksplit = p.g2.ksplit;
    g2.S = p.g2.S;
    g2.Z = p.g2.Z;
    g2.C = c2;
    CHECK(launched(fm::launch_enc_gemm(g2, st), "encoder wq_b"));

    fm::EncRopeArgs ra;
    ra.C = c2;
    ra.Z = p.g2.Z;
    ra.M = T;
    ra.n_heads = e->n_heads;
    ra.rope_dim = e->rope_dim;
    ra.pos = pos;
    for (int i = 0; i < fm::kEncMaxPairs; ++i) ra.inv_freq[i] = 0.0;
    yarn_freqs(e, ra.inv_freq);
    ra.q = (uint16_t *)q;
    CHECK(launched(fm::launch_enc_rope_had(ra, st), "encoder RoPE / Hadamard"));
    return ok();
}

size_t fm_golden_workspace_bytes(int T, int n_layers, int64_t ld, int tau) {
    if (T <= 0 || n_layers <= 0 || ld <= 0 || tau <= 0 || tau > T) return 0;
    return fm::labels_ws_bytes(T, n_layers, ld, tau);
}

fm_status fm_golden_labels(const float *scores, int64_t ld, int T, int n_layers,
                           const int32_t *n_valid, float p, int min_votes, int tau,
                           int32_t *label_ptr, int32_t *label_idx, float *label_score,
                           int64_t cap, void *ws, size_t ws_bytes, void *stream) {
    REQUIRE(T >= 1 && tau >= 1 && tau <= T, FM_ERR_INVALID_ARG, "T = %d, tau = %d (1 <= tau <= T)",
            T, tau);
    REQUIRE(ld >= 1, FM_ERR_INVALID_ARG, "ld = %lld", (long long)ld);
    REQUIRE(ld <= fm::kLabelMaxLd, FM_ERR_UNSUPPORTED, "ld = %lld (at most %d)", (long long)ld,
            fm::kLabelMaxLd);
    REQUIRE(n_layers >= 1, FM_ERR_INVALID_ARG, "n_layers = %d", n_layers);
    REQUIRE(n_layers <= 64, FM_ERR_UNSUPPORTED, "n_layers = %d (at most 64)", n_layers);
    REQUIRE((int64_t)(T - tau + 1) * ld < (int64_t)INT32_MAX, FM_ERR_UNSUPPORTED,
            "(T - tau + 1) * ld = %lld labels could overflow int32 pointers",
            (long long)((int64_t)(T - tau + 1) * ld));
    REQUIRE(min_votes >= 1, FM_ERR_INVALID_ARG, "min_votes = %d", min_votes);
    REQUIRE(p > 0.f && p <= 1.f, FM_ERR_INVALID_ARG, "p = %g outside (0, 1]", (double)p);
    REQUIRE(scores && aligned(scores, 4), FM_ERR_INVALID_ARG, "scores NULL or not 4-byte aligned");
    REQUIRE(label_ptr, FM_ERR_INVALID_ARG, "label_ptr is NULL");
    REQUIRE(cap >= 0 && (cap == 0 || label_idx), FM_ERR_INVALID_ARG,
            "cap = %lld needs label_idx", (long long)cap);
    const size_t need = fm::labels_ws_bytes(T, n_layers, ld, tau);
    REQUIRE(ws && aligned(ws, 256) && ws_bytes >= need, FM_ERR_WORKSPACE,
            "workspace %zu bytes at %p, need %zu (256-byte aligned)", ws_bytes, ws, need);
    fm::LabelArgs a;
    a.scores = scores;
    a.ld = ld;
    a.T = T;
    a.n_layers = n_layers;
    a.n_valid = n_valid;
    a.p = p;
    a.min_votes = min_votes;
    a.tau = tau;
    a.words = (int)((ld + 31) / 32);
    a.label_ptr = label_ptr;
    a.label_idx = label_idx;
    a.label_score = cap ? label_score : nullptr;
    a.cap = cap;
    fm::labels_ws_carve(a, ws);
    CHECK(launched(fm::launch_labels(a, (hipStream_t)stream), "golden labels"));
    return ok();
}

size_t fm_workspace_bytes(fm_op op, int T, int64_t max_candidates) {
    if (T <= 0 || max_candidates <= 0) return 0;
    if (op == FM_OP_TOPK) return fm::topk_ws_bytes(T, max_candidates);
    if (op == FM_OP_SCORE_RESIDENT || op == FM_OP_INDEX_TOPK) return select_ws_bytes(T, max_candidates);
    return 0;
}

const char *fm_status_string(fm_status s) {
    switch (s) {
    case FM_OK: return "FM_OK";
    case FM_ERR_INVALID_ARG: return "FM_ERR_INVALID_ARG";
    case FM_ERR_UNSUPPORTED: return "FM_ERR_UNSUPPORTED";
    case FM_ERR_WORKSPACE: return "FM_ERR_WORKSPACE";
    case FM_ERR_LAUNCH: return "FM_ERR_LAUNCH";
    }
    return "FM_ERR_UNKNOWN";
}

const char *fm_last_error(void) { return g_err; }

int fm_version(void) { return FM_VERSION; }

}  // extern "C"
