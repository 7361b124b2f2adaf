// score.hip -- index-logit kernels for gfx950.
//
// L[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . k[s,:]) over 64 heads of dimension 128
// (FlashMemory-DeepSeek-V4 paper summary, section 3, the Memory-Indexer score; DeepSeek-V4 CSA
// page, section 3, formula CSA-1).  All 64 heads of a query row share one key row, so a page of
// 64 entries is a dense [64 heads x 128] . [128 x 64 entries] contraction: it runs on MFMA.
//
// Operand layout (v_mfma_f32_16x16x32_bf16, wave64): lane l = 16 g + r holds row r of the A
// tile (a head) and column r of the B tile (an entry), eight k-values each; the accumulator
// lane holds rows 4 g .. 4 g + 3 of column r.  A dot product does not depend on the order of
// its terms, so the eight dimensions a lane carries are chosen per key format to make its
// loads contiguous; queries are loaded with the same assignment:
//   bf16 keys: lane group g, k-step kk -> dims (4 kk + g) * 8 .. +8   (16 B of the 256-B row)
//   fp8  keys: lane group g, k-step kk -> dims 32 g + 8 kk .. +8      (32 B of the 132-B row)
// fp8 keys are widened to bf16 with v_cvt_scalef32_pk_bf16_fp8 (exact: every E4M3 value is a
// bf16 value); the per-entry scale is applied after the head sum, which is valid because the
// scale is positive (ReLU(c x) = c ReLU(x) for c > 0).  fp8 queries against fp8 keys use the
// gfx950 v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales.
//
// The head sum: each lane weights and sums its 16 accumulator values (4 head tiles x 4 rows),
// then two cross-lane adds (lane xor 16, xor 32) complete the 64-head sum for its column.
//
// Streaming: keys are read once, straight from HBM into MFMA operand registers in the layout
// above; the query fragments stay in registers.  A decode call is HBM-bound, so what matters is
// the number of bytes in flight per CU: every wave keeps the next page (bf16) or two (fp8)
// loading while it scores one, with loads and stores that never sit behind a branch, so the
// wait before a page covers that page's loads only.
#include <math.h>

#include <type_traits>

#include "fm_internal.h"
#include "select_dev.h"

#ifndef FM_BF16_RING
#define FM_BF16_RING 4
#endif
#ifndef FM_F8_RING
#define FM_F8_RING 4
#endif
#ifndef FM_DECODE_WAVES
#define FM_DECODE_WAVES 4
#endif
#ifndef FM_WAVES_PER_EU
#define FM_WAVES_PER_EU 2
#endif
#ifndef FM_QLDS_AHEAD
#define FM_QLDS_AHEAD 2   // two-level: A fragments read ahead from LDS
#endif
#ifndef FM_MASK_AHEAD
#define FM_MASK_AHEAD 6   // fp8 mask: A fragments read ahead from LDS
#endif
#ifndef FM_MASK_RESIDENT
#define FM_MASK_RESIDENT 2048   // fp8 mask: waves to spread the pages over (2 a SIMD)
#endif
#ifndef FM_MASK_RING
#define FM_MASK_RING 4    // fp8 mask: tiles in the load ring
#endif
#ifndef FM_MASK_WPE
#define FM_MASK_WPE 2     // fp8 mask: waves per SIMD the registers are sized for
#endif
#ifndef FM_MASK_MAXPPW
#define FM_MASK_MAXPPW 16
#endif
#ifndef FM_MASK_F8
#define FM_MASK_F8 1   // fp8 mask: layers-per-wave kernel (0: one wave per layer)
#endif
#ifndef FM_SHARED_AHEAD
#define FM_SHARED_AHEAD 2  // fp8 mask over one shared pool: rounds a wave's tile loads run ahead
#endif
#ifndef FM_SHARED_WPE
#define FM_SHARED_WPE 3    // fp8 mask over one shared pool: waves per SIMD the registers are sized for
#endif
#ifndef FM_SHARED_PPW
#define FM_SHARED_PPW 8    // fp8 mask over one shared pool: pages a workgroup, at most
#endif
#ifndef FM_SHARED_WG
#define FM_SHARED_WG 512   // fp8 mask over one shared pool: workgroups to spread the pages over
#endif

namespace fm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// page-slot states (wave-uniform), besides a non-negative physical page id
constexpr int kSlotInvisible = -1;  // every entry of the page is past the visible length
constexpr int kSlotUnmapped = -2;   // the block table (or resident list) points nowhere valid
constexpr int kSlotEmpty = -3;      // resident-list slot beyond n_resident: nothing to write
constexpr int kMaxPpw = 16;         // page slots per wave, at most
constexpr int kF8FuseMaxPpw = 24;   // ... in the fused fp8 kernel, so that Mode A's 4,096-page
                                    // rows fit 16 chunks (12 waves x 22 slots)
constexpr int kStorePolicy = 0;     // logit stores: default cache policy (see store_wave_logits)
constexpr int kMaskPpw = FM_MASK_MAXPPW;   // pages per wave of the fp8 mask kernel, at most

__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// request of row t; -1 when row_req points outside [0, B) or row_pool outside [0, n_pools)
__device__ __forceinline__ int row_request(const QArgs &q, const KvArgs &kv, int t) {
    const int b = q.row_req ? q.row_req[t] : (q.b_is_zero ? 0 : t);
    if (q.row_pool) {
        const int l = q.row_pool[t];
        if (l < 0 || l >= kv.n_pools) return -1;
    }
    return (b >= 0 && b < kv.B) ? b : -1;
}

// key pool of row t (rows are wave-uniform); pool 0 for a row that row_request rejects
__device__ __forceinline__ const uint8_t *row_pool(const QArgs &q, const KvArgs &kv, int t) {
    if (!q.row_pool) return kv.pool[0];
    const int l = __builtin_amdgcn_readfirstlane(q.row_pool[t]);
    return kv.pool[(l >= 0 && l < kv.n_pools) ? l : 0];
}

// entries row t may use (0 for a row whose request is out of range)
__device__ __forceinline__ int64_t n_visible(const QArgs &q, const KvArgs &kv, int t, int b) {
    if (b < 0) return 0;
    int64_t n = kv.seq_lens[b];
    if (q.q_pos) {
        int64_t c = (int64_t)q.q_pos[t] / q.ratio;
        n = c < n ? c : n;
    }
    return n < 0 ? 0 : n;
}

template <int KF>
__device__ __forceinline__ int dim_base(int g, int kk) {
    return KF == KEY_BF16 ? (kk * 4 + g) * 8 : g * 32 + kk * 8;
}

// ---------------------------------------------------------------- query operands (A)
// bf16 q: fragment (m, kk) = 8 bf16 of head 16 m + r at dims dim_base(g, kk)
// fp8  q: fragment m      = 32 E4M3 codes of head 16 m + r at dims 32 g .. 32 g + 31
template <int KF>
__device__ __forceinline__ u32x4 q_frag_bf16(const uint8_t *qrow, int m, int kk, int r, int g) {
    const uint16_t *q = (const uint16_t *)qrow;
    return *(const u32x4 *)(q + (16 * m + r) * kDim + dim_base<KF>(g, kk));
}

__device__ __forceinline__ i32x8 q_frag_fp8(const uint8_t *qrow, int m, int r, int g) {
    return *(const i32x8 *)(qrow + (16 * m + r) * kDim + g * 32);
}

struct QRegBf16 {
    u32x4 a[4][4];
    __device__ __forceinline__ u32x4 get(int m, int kk) const { return a[m][kk]; }
};
struct QRegFp8 {
    i32x8 a[4];
    __device__ __forceinline__ i32x8 get(int m) const { return a[m]; }
};
// w[t, 16 m + 4 g + i] for the accumulator rows this lane holds
__device__ __forceinline__ void load_w(float (&wv)[16], const void *w, int w_bf16, int t, int g) {
    const int64_t base = (int64_t)t * kHeads + 4 * g;
    if (w_bf16) {
        const uint16_t *w16 = (const uint16_t *)w + base;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[m * 4 + i] = bf16f(w16[16 * m + i]);
    } else {
        const float *w32 = (const float *)w + base;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[m * 4 + i] = w32[16 * m + i];
    }
}

// ---------------------------------------------------------------- key pages in registers
struct PgBf16 { u32x4 b[4][4]; };              // [entry tile j][k-step kk]
struct PgFp8 { u32x4 b[4][2]; float scale; };  // [entry tile j][half]: 16 codes; own-row scale

__device__ __forceinline__ u32x4 load16(const uint8_t *p) {  // 4-byte aligned
    const uint32_t *w = (const uint32_t *)p;
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Page loads go through a buffer descriptor spanning exactly the page, so no lane can read past
// it; a page that is not to be read (unmapped, invisible, or padding) gets a zero-size
// descriptor, for which the loads return zeros without touching memory.  That keeps every load
// unconditional (no branches around memory operations, exact wait counts) while an invalid
// page is never dereferenced.  phys is wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t *pool, int phys, int bytes) {
    const bool ok = phys >= 0;
    return __builtin_amdgcn_make_buffer_rsrc((void *)(pool + (int64_t)(ok ? phys : 0) * bytes),
                                             (short)0, ok ? bytes : 0, 0x00020000);
}

// bf16 page: one VGPR offset per lane (row r, 16-byte chunk g), entry tile j in the scalar
// offset, k-step kk in the immediate offset.
__device__ __forceinline__ void load_page(PgBf16 &P, const uint8_t *pool, int phys, int r, int g, int) {
    const __amdgpu_buffer_rsrc_t rs = page_rsrc(pool, phys, kPage * kRowBf16);
    const uint32_t off = (uint32_t)(r * kRowBf16 + g * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            P.b[j][kk] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + kk * 64, j * 16 * kRowBf16, 0);
}

// fp8 page: 132-byte rows, so the 16-byte loads are 4-byte aligned (as plain global loads of the
// same rows are); the lane's own row scale comes along.
__device__ __forceinline__ void load_page(PgFp8 &P, const uint8_t *pool, int phys, int r, int g, int ln) {
    const __amdgpu_buffer_rsrc_t rs = page_rsrc(pool, phys, kPage * kRowFp8);
    const uint32_t off = (uint32_t)(r * kRowFp8 + g * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            P.b[j][h] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + h * 16, j * 16 * kRowFp8, 0);
    P.scale = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(ln * kRowFp8 + kDim), 0, 0));
}

__device__ __forceinline__ u32x4 b_operand(const PgBf16 &P, int j, int kk) { return P.b[j][kk]; }

__device__ __forceinline__ u32x4 b_operand(const PgFp8 &P, int j, int kk) {
    u32x4 v = P.b[j][kk >> 1];
    uint32_t d0 = (kk & 1) ? v[2] : v[0];
    uint32_t d1 = (kk & 1) ? v[3] : v[1];
    u32x4 o;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true));
    return o;
}

__device__ __forceinline__ float page_scale(const PgBf16 &) { return 1.0f; }
__device__ __forceinline__ float page_scale(const PgFp8 &P) { return P.scale; }

// weighted ReLU head sum of one 16-entry tile; every lane of column r returns the total.
// The four lane groups (rows of 16 lanes) are combined with the gfx950 row swaps: after
// permlane16_swap each row holds its pair's two partials, after permlane32_swap the two pair
// sums; both operands are the same register, and every lane adds in the same order.
__device__ __forceinline__ float head_sum(const f32x4 (&acc)[4], const float (&wv)[16]) {
    float p = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) p = fmaf(wv[m * 4 + i], fmaxf(acc[m][i], 0.f), p);
    const uint32_t u = __float_as_uint(p);
    const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    p = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    const uint32_t v = __float_as_uint(p);
    const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// logit (before key/query scales) of page entry `lane` for one bf16 query row
template <class QS, class Pg>
__device__ __forceinline__ float page_logit_bf16q(const QS &Q, const float (&wv)[16], const Pg &P, int g) {
    float tot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x4 acc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 bk = __builtin_bit_cast(bf16x8, b_operand(P, j, kk));
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, Q.get(m, kk)), bk, acc[m], 0, 0, 0);
        }
        tot[j] = head_sum(acc, wv);
    }
    return g == 0 ? tot[0] : g == 1 ? tot[1] : g == 2 ? tot[2] : tot[3];
}

// same for an fp8 query row against fp8 keys (one 16x16x128 MFMA per head tile)
template <class QS>
__device__ __forceinline__ float page_logit_fp8q(const QS &Q, const float (&wv)[16], const PgFp8 &P, int g) {
    float tot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        i32x8 bk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bk[e] = (int)P.b[j][0][e];
            bk[4 + e] = (int)P.b[j][1][e];
        }
        f32x4 acc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
            acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                Q.get(m), bk, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        tot[j] = head_sum(acc, wv);
    }
    return g == 0 ? tot[0] : g == 1 ? tot[1] : g == 2 ? tot[2] : tot[3];
}

template <int KF> struct PageOf;
template <> struct PageOf<KEY_BF16> { typedef PgBf16 T; static constexpr int row = kRowBf16, nbuf = 2; };
template <> struct PageOf<KEY_FP8> { typedef PgFp8 T; static constexpr int row = kRowFp8, nbuf = 3; };

// Query operand source of one row: registers, or the workgroup's LDS copy.
// Query operand source of one row, in registers.
template <int KF, int QF> struct QSource;

template <int KF> struct QSource<KF, Q_BF16> {
    QRegBf16 q;
    __device__ void init(const uint8_t *qrow, int r, int g) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) q.a[m][kk] = q_frag_bf16<KF>(qrow, m, kk, r, g);
    }
    template <class Pg>
    __device__ float logit(const float (&wv)[16], const Pg &P, int g) const {
        return page_logit_bf16q(q, wv, P, g);
    }
};

template <int KF> struct QSource<KF, Q_FP8> {
    QRegFp8 q;
    __device__ void init(const uint8_t *qrow, int r, int g) {
#pragma unroll
        for (int m = 0; m < 4; ++m) q.a[m] = q_frag_fp8(qrow, m, r, g);
    }
    __device__ float logit(const float (&wv)[16], const PgFp8 &P, int g) const {
        return page_logit_fp8q(q, wv, P, g);
    }
};

// Resolve a page slot to a physical page id or a slot state.
__device__ __forceinline__ int resolve_slot(const ScoreArgs &A, int b, int64_t nvis, int64_t nres,
                                            int64_t j, int &lp_out) {
    int64_t lp;
    if (A.res_pages) {
        if (j >= nres) { lp_out = -1; return kSlotEmpty; }
        lp = A.res_pages[(int64_t)b * A.res_ld + j];
    } else {
        lp = j;
    }
    lp_out = (int)lp;
    if (lp < 0 || lp >= A.kv.bt_ld) return lp * kPage >= nvis && lp >= 0 ? kSlotInvisible : kSlotUnmapped;
    if (lp * kPage >= nvis) return kSlotInvisible;
    int phys = A.kv.bt[(int64_t)b * A.kv.bt_ld + lp];
    if (phys < 0 || phys >= A.kv.n_phys) return kSlotUnmapped;
    return phys;
}

// Page stream of one wave: take(P, i) for i = 0 .. n - 1 in order, with the loads of the next
// NBUF - 1 pages in flight.  fetch(P, i) must be valid (a zero-size load) for i up to
// n + NBUF - 2, and take(P, i) harmless for i up to the next multiple of NBUF: the loop runs in
// whole rounds of NBUF so every buffer index is a compile-time constant and the body has no
// branches around memory operations.
template <int NBUF, class Pg, class Fetch, class Take>
__device__ __forceinline__ void stream_pages(int n, Pg (&P)[NBUF], Fetch fetch, Take take) {
#pragma unroll
    for (int v = 0; v < NBUF - 1; ++v) fetch(P[v], v);
    for (int i0 = 0; i0 < n; i0 += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
            fetch(P[(u + NBUF - 1) % NBUF], i0 + u + NBUF - 1);
            take(P[u], i0 + u);
        }
    }
}

// A wave's logits, staged in LDS as res[slot][entry], out to row orsrc.  Slot i of the wave is
// output columns (slot0 + i) * 64 .. + 63 in both modes (its logical page, or its place in the
// resident list), so the wave's logits are one contiguous run: with 16-byte aligned columns
// (out_ld % 4 == 0) it goes out as 16-byte stores, lane ln taking entries 4 (ln % 16) .. + 3 of
// slot 4 p + ln / 16, four slots an instruction (res must have 4 ceil(nslot / 4) rows, 16-byte
// aligned).  Unmapped slots give NaN, invisible entries -inf, empty slots nothing.  The stores
// keep the default cache policy: the top-k that follows reads the logits, and finds part of
// them still in the caches (a decode step measured ~2 us faster than with non-temporal stores).
__device__ __forceinline__ void store_wave_logits(const ScoreArgs &A, __amdgpu_buffer_rsrc_t orsrc,
                                                  const float (*res)[64], int phys_l, int lp_l,
                                                  int64_t slot0, int nslot, int64_t nvis, int ln) {
    if ((A.out_ld & 3) == 0) {
        const int c = 4 * (ln & 15);
        for (int p = 0; 4 * p < nslot; ++p) {
            const int i = 4 * p + (ln >> 4);          // < 16: slots past nslot are empty
            const int phys = __shfl(phys_l, i);
            const int lp = __shfl(lp_l, i);
            const int64_t col = phys == kSlotEmpty ? A.out_ld : (slot0 + i) * kPage + c;
            const f32x4 got = *(const f32x4 *)&res[i][c];
            const float bad = phys == kSlotUnmapped ? __builtin_nanf("") : -INFINITY;
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x = phys >= 0 ? got[e] : bad;
                if ((int64_t)lp * kPage + c + e >= nvis) x = -INFINITY;
                v[e] = __float_as_uint(x);
            }
            const uint32_t voff = (uint32_t)(min(col, A.out_ld) * 4);   // out_ld * 4: dropped
            __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, voff, 0, kStorePolicy);
        }
        return;
    }
    for (int i = 0; i < nslot; ++i) {
        const int phys = __builtin_amdgcn_readlane(phys_l, i);
        const int lp = __builtin_amdgcn_readlane(lp_l, i);
        const int64_t col = phys == kSlotEmpty ? A.out_ld : (slot0 + i) * kPage + ln;
        float v = phys >= 0 ? res[i][ln] : (phys == kSlotUnmapped ? __builtin_nanf("") : -INFINITY);
        if ((int64_t)lp * kPage + ln >= nvis) v = -INFINITY;
        const uint32_t voff = (uint32_t)(min(col, A.out_ld) * 4);   // out_ld * 4: dropped
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), orsrc, voff, 0, kStorePolicy);
    }
}

// ---------------------------------------------------------------- row scoring kernel
// grid (ceil(n_slots / (4 ppw)), T), 4 waves per workgroup, all on row blockIdx.y; wave w of
// workgroup x scores slots [(4 x + w) ppw, +ppw).  The query fragments stay in registers; pages
// stream from HBM straight into MFMA operand registers, the next NBUF - 1 pages loading while
// one is scored (NBUF = 2 for 16-KB bf16 pages, 3 for 8.25-KB fp8 pages).  Slots past the
// wave's own are empty (nothing read, nothing written); outputs go through a buffer descriptor
// spanning the output row, so a column past out_ld (or an empty slot's) is dropped by the
// hardware.
template <int KF, int QF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FM_WAVES_PER_EU)))
void score_kernel(ScoreArgs A) {
    typedef typename PageOf<KF>::T Pg;
    __shared__ __align__(16) float s_res[4][kMaxPpw + 4][64];   // logits until the wave's loads are done
    const int t = blockIdx.y;
    const int ln = __lane_id(), r = ln & 15, g = ln >> 4;
    const int wave = threadIdx.x >> 6;
    const int64_t slot0 = ((int64_t)blockIdx.x * 4 + wave) * A.ppw;
    if (slot0 >= A.n_slots) return;
    const int nslot = (int)min((int64_t)A.ppw, A.n_slots - slot0);
    const int braw = row_request(A.q, A.kv, t);
    const int64_t nvis = n_visible(A.q, A.kv, t, braw);
    const int b = braw < 0 ? 0 : braw;
    const int64_t nres = (A.res_pages && braw >= 0) ? A.n_res[b] : 0;
    const uint8_t *pool = row_pool(A.q, A.kv, t);
    const uint8_t *qrow = (const uint8_t *)A.q.q + (int64_t)t * kHeads * kDim * (QF == Q_FP8 ? 1 : 2);
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A.out + (int64_t)t * A.out_ld), (short)0, (int)(A.out_ld * 4), 0x00020000);

    QSource<KF, QF> Q;
    Q.init(qrow, r, g);

    // lane i describes slot i of this wave: physical page (or slot state) and logical page
    int lp_l = -1, phys_l = kSlotEmpty;
    if (ln < nslot) phys_l = resolve_slot(A, b, nvis, nres, slot0 + ln, lp_l);

    float wv[16];
    load_w(wv, A.q.w, A.q.w_bf16, t, g);
    const float qscale = (QF == Q_FP8) ? A.q.q_scale[t] : 1.0f;

    auto fetch = [&](Pg &P, int i) {   // i < 64: ppw <= 16, padded by at most NBUF
        const int phys = __builtin_amdgcn_readlane(phys_l, i);
        load_page(P, pool, phys, r, g, ln);
    };
    auto emit = [&](const Pg &P, int i) {    // logits to LDS; stored after the last load
        s_res[wave][i][ln] = Q.logit(wv, P, g) * page_scale(P) * qscale;
    };
    Pg P[PageOf<KF>::nbuf];
    stream_pages(nslot, P, fetch, emit);
    store_wave_logits(A, orsrc, s_res[wave], phys_l, lp_l, slot0, nslot, nvis, ln);
}

// ---------------------------------------------------------------- bf16 decode: tile ring
// bf16 keys x bf16 queries, the decode shape.  Same work split and output as score_kernel, but
// built for occupancy, which is what an HBM-bound gather needs: the query fragments (the MFMA A
// operands, 16 KB per row) sit in LDS, written once by the four waves of the workgroup (they
// score the same row) and read back per k-step, so a wave needs about 120 VGPRs and four waves
// share each SIMD.  The unit of the load pipeline is a 16-entry tile (4 KB per wave, 16 VGPRs):
// a ring of RING tiles keeps RING - 1 tiles loading at every moment, each tile's loads going
// out as soon as its registers are free.
struct TileBf16 { u32x4 b[4]; };   // [k-step kk]

template <int RING>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FM_DECODE_WAVES)))
void score_bf16_ring_kernel(ScoreArgs A) {
    __shared__ u32x4 s_q[16][64];        // fragment (m, kk) = 4 m + kk, lane-contiguous
    __shared__ __align__(16) float s_res[4][kMaxPpw][64];   // each wave's logits until its loads are done
    const int t = blockIdx.y;
    const int ln = __lane_id(), r = ln & 15, g = ln >> 4;
    const int wave = threadIdx.x >> 6;
    // The page list is resolved first and the first key tiles are requested before the query
    // fragments are staged: every wave of the grid starts at once, so the latency of these
    // dependent reads is paid once per launch and is better overlapped than serialised.
    const int64_t slot0 = ((int64_t)blockIdx.x * 4 + wave) * A.ppw;
    const int nslot = (int)max((int64_t)0, min((int64_t)A.ppw, A.n_slots - slot0));
    const int braw = row_request(A.q, A.kv, t);
    const int64_t nvis = n_visible(A.q, A.kv, t, braw);
    const int b = braw < 0 ? 0 : braw;
    const int64_t nres = (A.res_pages && braw >= 0) ? A.n_res[b] : 0;
    const uint8_t *pool = row_pool(A.q, A.kv, t);
    int lp_l = -1, phys_l = kSlotEmpty;
    if (ln < nslot) phys_l = resolve_slot(A, b, nvis, nres, slot0 + ln, lp_l);
    u32x4 qf[4];
    {
        const uint8_t *qrow = (const uint8_t *)A.q.q + (int64_t)t * kHeads * kDim * 2;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int fi = wave * 4 + f;
            qf[f] = q_frag_bf16<KEY_BF16>(qrow, fi >> 2, fi & 3, r, g);
        }
    }
    float wv[16];
    load_w(wv, A.q.w, A.q.w_bf16, t, g);
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A.out + (int64_t)t * A.out_ld), (short)0, (int)(A.out_ld * 4), 0x00020000);

    const uint32_t off = (uint32_t)(r * kRowBf16 + g * 16);
    auto fetch = [&](TileBf16 &T, int x) {       // tile x: page x / 4, entry tile x % 4
        const __amdgpu_buffer_rsrc_t rs =
            page_rsrc(pool, __builtin_amdgcn_readlane(phys_l, x >> 2), kPage * kRowBf16);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            T.b[kk] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + kk * 64, (x & 3) * 16 * kRowBf16, 0);
    };
    auto tile_logit = [&](const TileBf16 &T) {
        // a zero the compiler cannot see through: the query fragments are read from LDS for
        // every tile instead of being hoisted into registers, which would cost occupancy
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        const u32x4 *qs = &s_q[0][ln + z];
        f32x4 acc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 bk = __builtin_bit_cast(bf16x8, T.b[kk]);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, qs[(4 * m + kk) * 64]), bk, acc[m], 0, 0, 0);
        }
        return head_sum(acc, wv);
    };
    // A page's logits go to LDS; the global stores wait until every load of the wave has been
    // issued and consumed.  (Vector memory operations complete in issue order, so a store among
    // the loads would make each later wait for a key tile wait for the store as well.)
    auto emit = [&](const f32x4 &tot, int i) {   // page slot i: lane = entry, tile g
        s_res[wave][i][ln] = g == 0 ? tot[0] : g == 1 ? tot[1] : g == 2 ? tot[2] : tot[3];
    };

    // tiles 0 .. 4 nslot - 1 in order; slots past nslot are empty (zero-size loads)
    TileBf16 T[RING];
#pragma unroll
    for (int v = 0; v < RING - 1; ++v) {
        fetch(T[v], v);
        __builtin_amdgcn_sched_barrier(0);     // tiles issue in ring order, as the loop refills them
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) s_q[wave * 4 + f][ln] = qf[f];
    __syncthreads();
    if (nslot == 0) return;
    f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int x0 = 0; x0 < 4 * nslot; x0 += 4 * RING) {
#pragma unroll
        for (int u = 0; u < 4 * RING; ++u) {
            fetch(T[(u + RING - 1) % RING], x0 + u + RING - 1);
            tot[u & 3] = tile_logit(T[u % RING]);
            if ((u & 3) == 3) emit(tot, (x0 + u) >> 2);
        }
    }
    store_wave_logits(A, orsrc, s_res[wave], phys_l, lp_l, slot0, nslot, nvis, ln);
}

// ---------------------------------------------------------------- fused scoring + top-k
// The top-k of a row (paper summary, section 3: the native selector keeps the top-k inside the
// resident set; CSA page, section 3: index_topk = 512) without the row's logits reaching
// memory.  Two kernels:
//   1. workgroup (c, t) scores its chunk of row t into LDS and keeps a superset of the chunk's
//      top-k (the entries of the chunk's highest value bins, at most `cap` of them; exactly the
//      chunk's top-k when that superset would not fit).  Every member of the row's top-k is in
//      its own chunk's top-k, because the order (value descending, entry ascending) is total.
//      The candidates, their number and two bounds (the smallest candidate value, the chunk's
//      largest value) go to the workspace.
//   2. one workgroup per row selects the row's top-k exactly from its chunks' candidates and
//      writes it in ascending entry order.  A chunk that kept at least k candidates proves
//      that the row's k-th value is at least its smallest candidate, so candidates below the
//      largest such bound are dropped on loading and the value bins span only what is left.

template <int NT>
struct FuseLds {
    uint32_t hist[kBins];
    uint32_t sh[NT / 64 + 1];
    uint32_t misc[4];
    float shf[NT / 64];
    float shf2[NT / 64];
    uint32_t shc[NT / 64];
    uint32_t wsum[NT / 64];
    int32_t bnd[kBnd];
    uint32_t n_out, n_bnd;
};

// the candidates of a chunk in LDS (value j and its entry entry_of(j)), as a radix_rule source
template <class EntryOf>
struct ChunkSrc {
    const float *v;
    int n;
    EntryOf entry_of;
    template <int NT, class F>
    __device__ void each(F f) const {
        for (int j = (int)threadIdx.x; j < n; j += NT) {
            const float x = v[j];
            if (x > -INFINITY) f(x, (int64_t)entry_of(j));   // -inf and NaN are not candidates
        }
    }
};

// The bin holding the r-th largest of hist (r >= 1, r <= total): S.misc[0] = the bin,
// S.misc[1] = the count in higher bins; with r2 > 0 also the bin of the r2-th largest in
// S.misc[2] (0 when r2 exceeds the total).  Wave w owns BPW bins from the top, lane l BPL of
// them (bins below 0 hold nothing); two barriers.
template <int NT, class Lds>
__device__ void top_bin(uint32_t r, Lds &S, uint32_t r2 = 0) {
    constexpr int NWv = NT / 64;
    constexpr int BPL = (kBins + NT - 1) / NT, BPW = 64 * BPL;
    const int w = threadIdx.x >> 6, ln = __lane_id();
    const int top = kBins - 1 - BPW * w - BPL * ln;      // this lane's bins: top, top - 1, ...
    uint32_t h[BPL], sum = 0;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
        h[i] = top - i >= 0 ? S.hist[top - i] : 0u;
        sum += h[i];
    }
    const uint32_t incl = wave_incl_scan<NT>(sum);
    if (ln == 63) S.wsum[w] = incl;
    __syncthreads();
    uint32_t above = 0;
    for (int v = 0; v < w; ++v) above += S.wsum[v];
    above += incl - sum;                                  // count in bins above this lane's
    if (w == 0 && ln == 0 && r2) S.misc[2] = 0u;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
        if (above < r && r <= above + h[i]) {
            S.misc[0] = (uint32_t)(top - i);
            S.misc[1] = above;
        }
        if (r2 && above < r2 && r2 <= above + h[i]) S.misc[2] = (uint32_t)(top - i);
        above += h[i];
    }
    __syncthreads();
}

// Keep the candidates of the chunk's n values in LDS (-inf and NaN are not candidates) that
// can be in the top-k: all of them when they fit in cap; else those of the value bins from
// the top down to the bin holding the chunk's k-th largest, when they fit; else exactly the
// chunk's top-k (boundary bin ranked by the full key, or the radix selection).  Writes them to
// cval / cidx (any order), their number to *cnt_out and to *stat_out: x = a value at or below
// every kept one, y = the chunk maximum, z = a value with at least `share` candidates at or
// above it (-inf when unknown or fewer exist).  On entry: the per-wave candidate counts,
// minima and maxima in S.shc / shf / shf2, S.hist zero, S.n_out = S.n_bnd = 0, followed by a
// barrier.  NV = n / NT values a thread (n a multiple of NT).
template <int NT, int NV, class EntryOf>
__device__ void chunk_select(const float *vals, uint32_t k, uint32_t cap, uint32_t share,
                             EntryOf entry_of, float *cval, int32_t *cidx, int32_t *cnt_out,
                             float4 *stat_out, FuseLds<NT> &S) {
    constexpr int NWv = NT / 64;
    constexpr int n = NV * NT;
    const int tid = threadIdx.x, ln = __lane_id();
    const uint64_t lt = ln == 0 ? 0ull : (~0ull >> (64 - ln));
    uint32_t total = 0;
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int i = 0; i < NWv; ++i) {
        total += S.shc[i];
        lo = fminf(lo, S.shf[i]);
        hi = fmaxf(hi, S.shf2[i]);
    }
    float v[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) v[u] = vals[u * NT + tid];
    // keep the values whose flag is set: per group of four values a thread, one slot
    // reservation for the wave, then the stores
    static_assert(NV % 4 == 0, "groups of four");
    auto emit_all = [&](auto &&flag) {
#pragma unroll
        for (int u0 = 0; u0 < NV; u0 += 4) {
            uint64_t ms[4];
            uint32_t wtot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                ms[q] = __ballot(flag(u0 + q));
                wtot += (uint32_t)__popcll(ms[q]);
            }
            if (wtot == 0) continue;
            uint32_t base = 0;
            if (ln == 0) base = atomicAdd(&S.n_out, wtot);
            base = __shfl(base, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if ((ms[q] >> ln) & 1ull) {
                    const uint32_t p = base + (uint32_t)__popcll(ms[q] & lt);
                    if (p < cap) {
                        cval[p] = v[u0 + q];
                        cidx[p] = (int32_t)entry_of((u0 + q) * NT + tid);
                    }
                }
                base += (uint32_t)__popcll(ms[q]);
            }
        }
    };
    const float width = hi - lo;
    uint32_t kept;
    float bound = lo, zshare = -INFINITY;
    if (total <= cap) {
        kept = total;
        emit_all([&](int u) { return v[u] > -INFINITY; });
    } else {
        bool radix = !(width < INFINITY);
        LinBins bins{lo, 0.f, !(hi > lo)};
        bins.inv_w = bins.flat || radix ? 0.f : (float)kBins / width;
        kept = k;
        if (!radix) {
#pragma unroll
            for (int u = 0; u < NV; ++u)
                if (v[u] > -INFINITY) atomicAdd(&S.hist[bins(v[u])], 1u);
            __syncthreads();
            top_bin<NT>(k, S, share <= total ? share : 0u);
            const int bstar = (int)S.misc[0];
            const uint32_t above = S.misc[1], nb = S.hist[bstar];
            // a value at or below every member of bins >= b: the lower edge of the bin below
            auto edge = [&](int b) {
                return !bins.flat && b > 0 ? lo + (float)(b - 1) * (width / (float)kBins) : lo;
            };
            bound = edge(bstar);
            if (share <= total) zshare = edge((int)S.misc[2]);
            if (above + nb <= cap) {
                kept = above + nb;              // the bins from the top down to bstar, whole
                emit_all([&](int u) { return v[u] > -INFINITY && bins(v[u]) >= bstar; });
            } else if (nb <= (uint32_t)kBnd) {
                // higher bins whole, the boundary bin ranked by the full key
                const uint32_t need = k - above;
                emit_all([&](int u) { return v[u] > -INFINITY && bins(v[u]) > bstar; });
#pragma unroll
                for (int u = 0; u < NV; ++u)
                    if (v[u] > -INFINITY && bins(v[u]) == bstar) S.bnd[atomicAdd(&S.n_bnd, 1u)] = u * NT + tid;
                __syncthreads();
                for (uint32_t a0 = 0; a0 < nb; a0 += NT) {
                    const uint32_t a = a0 + tid;
                    bool keep = false;
                    int ja = 0;
                    if (a < nb) {
                        ja = S.bnd[a];
                        const uint64_t ka = full_key(vals[ja], entry_of(ja));
                        uint32_t rank = 0;
                        for (uint32_t cc = 0; cc < nb; ++cc) {
                            const int jc = S.bnd[cc];
                            rank += full_key(vals[jc], entry_of(jc)) > ka;
                        }
                        keep = rank < need;
                    }
                    const uint64_t mk = __ballot(keep);
                    if (mk) {
                        uint32_t b0 = 0;
                        if (ln == 0) b0 = atomicAdd(&S.n_out, (uint32_t)__popcll(mk));
                        b0 = __shfl(b0, 0);
                        if (keep) {
                            const uint32_t p = b0 + (uint32_t)__popcll(mk & lt);
                            cval[p] = vals[ja];
                            cidx[p] = (int32_t)entry_of(ja);
                        }
                    }
                }
            } else {
                radix = true;
                bound = lo;
                __syncthreads();                   // hist is read before the radix clears it
            }
        }
        if (radix) {
            const ChunkSrc<EntryOf> src{vals, n, entry_of};
            const Rule rule = radix_rule<NT>(src, k, S.hist, S.sh, S.misc);
            __syncthreads();
            emit_all([&](int u) {
                return v[u] > -INFINITY && (full_key(v[u], entry_of(u * NT + tid)) & rule.M) >= rule.P;
            });
        }
    }
    if (tid == 0) {
        *cnt_out = (int32_t)min(kept, cap);
        *stat_out = make_float4(bound, hi, zshare, 0.f);
    }
}

// The candidates of a wave's page slots: entries of empty slots, of unmapped pages, past the
// visible length or (Mode A) outside the resident mask become -inf in LDS; the wave's candidate
// count, minimum and maximum go to S (lane 0).
template <int NT>
__device__ __forceinline__ void mark_candidates(const FuseArgs &F, float (*res)[64], int ppw_pad,
                                                int phys_l, int lp_l, int nslot, int64_t nvis,
                                                int b, int ln, int wave, FuseLds<NT> &S) {
    const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(F.mask ? F.mask + (int64_t)b * F.mask_ld : nullptr), (short)0,
        F.mask ? (int)F.mask_ld : 0, 0x00020000);
    uint32_t c = 0;
    float lo = INFINITY, hi = -INFINITY;
    for (int i = 0; i < ppw_pad; ++i) {
        const int phys = __builtin_amdgcn_readlane(phys_l, i);
        const int lp = __builtin_amdgcn_readlane(lp_l, i);
        const int64_t s = (int64_t)lp * kPage + ln;
        bool ok = i < nslot && phys >= 0 && s < nvis;
        if (F.mask && ok) ok = __builtin_amdgcn_raw_buffer_load_b8(mr, (uint32_t)s, 0, 0) != 0;
        const float v = res[i][ln];
        if (!ok) {
            res[i][ln] = -INFINITY;
        } else if (v > -INFINITY) {
            ++c;
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        c += __shfl_xor(c, o);
        lo = fminf(lo, __shfl_xor(lo, o));
        hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    if (ln == 0) {
        S.shc[wave] = c;
        S.shf[wave] = lo;
        S.shf2[wave] = hi;
    }
}

// LDS of the row merge
constexpr int kMergeWords = 8192;         // output-order bitmap: entries below 2^18
template <int NT>
struct MergeLds {
    uint32_t hist[kBins];
    uint32_t bits[kMergeWords];           // selected entries below 2^18, one bit each
    uint32_t pref[kMergeWords];           // selected entries in lower words
    uint32_t sh[NT / 64 + 1];
    uint32_t wsum[NT / 64];
    uint32_t misc[4];
    float bnd_v[kBnd];                    // the boundary bin's candidates
    int32_t bnd_e[kBnd];
    alignas(16) int32_t sel_e[FM_MAX_K];  // selected (entry, value), unordered
    float sel_v[FM_MAX_K];
    int32_t ccnt[kFuseMaxChunks];         // the chunks' kept counts and bounds
    float4 cst[kFuseMaxChunks];
    uint32_t m, n_sel, n_bnd;
};

// the merge's candidates in registers (SPT a thread), as a radix_rule source
template <int SPT>
struct RegSrc {
    const float *v;
    const int32_t *e;
    const bool *ok;
    template <int NT, class F>
    __device__ void each(F f) const {
#pragma unroll
        for (int u = 0; u < SPT; ++u)
            if (ok[u]) f(v[u], (int64_t)e[u]);
    }
};

// One workgroup per row: the row's top-k from its chunks' candidates, in ascending entry order.
// Every thread reads its share of all candidate slots (and one chunk's count and bounds) in one
// round of loads and keeps them in registers; candidates below the row's proven lower bound on
// its k-th value are dropped, the rest binned over [bound, row maximum].  Then the boundary
// bin, the exact rank of its entries, and the output order from a bitmap of the selected
// entries (entries below 32 bit_words) or from counts of smaller selected entries.
template <int NT, int SPT>
__global__ __launch_bounds__(NT) void merge_chunks_kernel(FuseArgs F) {
    __shared__ MergeLds<NT> S;
    const int t = blockIdx.x, tid = threadIdx.x, ln = __lane_id();
    const int nc = F.n_chunks, cap = F.cap, cap_log2 = __builtin_ctz((unsigned)F.cap);
    const uint32_t k = (uint32_t)F.k;
    const int64_t row_c = (int64_t)t * nc;
    const int cand = nc * cap;
    const uint64_t lt = ln == 0 ? 0ull : (~0ull >> (64 - ln));
    for (int i = tid; i < kBins; i += NT) S.hist[i] = 0u;
    for (int i = tid; i < F.bit_words; i += NT) S.bits[i] = 0u;
    if (tid == 0) {
        S.m = 0u;
        S.n_sel = 0u;
        S.n_bnd = 0u;
    }
    if (tid < nc) {
        S.ccnt[tid] = min(F.cnt[row_c + tid], cap);
        S.cst[tid] = F.cstat[row_c + tid];
    }
    float v[SPT];
    int32_t e[SPT];
    bool ok[SPT];
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const int i = u * NT + tid;
        v[u] = -INFINITY;
        e[u] = 0;
        if (i < cand) {
            v[u] = F.cval[row_c * cap + i];
            e[u] = F.cidx[row_c * cap + i];
        }
    }
    __syncthreads();                                         // LDS cleared, counts staged
    // Lower bounds on the row's k-th value: a chunk that kept k candidates has k values at or
    // above its x; and every chunk has ceil(k / chunks) values at or above its z, so together k
    // at or above the smallest z.  Candidates below the larger bound cannot be selected.
    float lo = -INFINITY, hi = -INFINITY, lo_any = INFINITY, zmin = INFINITY;
    for (int c = 0; c < nc; ++c) {
        const int cnt = S.ccnt[c];
        const float4 st = S.cst[c];
        if (cnt >= F.k) lo = fmaxf(lo, st.x);
        zmin = fminf(zmin, st.z);
        if (cnt > 0) {
            hi = fmaxf(hi, st.y);
            lo_any = fminf(lo_any, st.x);
        }
    }
    if (zmin < INFINITY) lo = fmaxf(lo, zmin);
    const float blo = lo > -INFINITY ? lo : lo_any;         // the bins' lower end
    const float width = hi - blo;
    bool radix = !(width < INFINITY) || !(hi >= blo);
    LinBins bins{blo, 0.f, !(hi > blo)};
    bins.inv_w = bins.flat || radix ? 0.f : (float)kBins / width;
    int bn[SPT];
    uint32_t mine = 0;
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const int i = u * NT + tid;
        const int c = i >> cap_log2;                         // cap is a power of two
        ok[u] = i < cand && (i & (cap - 1)) < S.ccnt[c] && v[u] >= lo;
        mine += ok[u] ? 1u : 0u;
        bn[u] = ok[u] && !radix ? bins(v[u]) : -1;
        if (bn[u] >= 0) atomicAdd(&S.hist[bn[u]], 1u);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mine += __shfl_xor(mine, o);
    if (ln == 0 && mine) atomicAdd(&S.m, mine);
    __syncthreads();
    const uint32_t m = S.m;
    // append (x, en) where `take` holds, one slot reservation per wave (every lane calls it)
    auto append = [&](bool take, float x, int32_t en, uint32_t *counter, float *xs, int32_t *es,
                      uint32_t cap_n, bool sel) {
        const uint64_t mk = __ballot(take);
        if (!mk) return;
        uint32_t b0 = 0;
        if (ln == 0) b0 = atomicAdd(counter, (uint32_t)__popcll(mk));
        b0 = __shfl(b0, 0);
        if (take) {
            const uint32_t p = b0 + (uint32_t)__popcll(mk & lt);
            if (p < cap_n) {
                es[p] = en;
                xs[p] = x;
            }
            if (sel && (uint32_t)en < 32u * (uint32_t)F.bit_words)
                atomicOr(&S.bits[en >> 5], 1u << (en & 31));
        }
    };
    auto select = [&](bool take, float x, int32_t en) {
        append(take, x, en, &S.n_sel, S.sel_v, S.sel_e, (uint32_t)FM_MAX_K, true);
    };
    // append this thread's slots u with take(u) set, one slot reservation per wave for all of
    // them (the reservations are serial LDS round trips)
    auto append_all = [&](auto &&take, uint32_t *counter, float *xs, int32_t *es, uint32_t cap_n,
                          bool sel) {
        uint64_t mk[SPT];
        uint32_t tot = 0;
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            mk[u] = __ballot(take(u));
            tot += (uint32_t)__popcll(mk[u]);
        }
        if (tot == 0) return;
        uint32_t b0 = 0;
        if (ln == 0) b0 = atomicAdd(counter, tot);
        b0 = __shfl(b0, 0);
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            if ((mk[u] >> ln) & 1ull) {
                const uint32_t p = b0 + (uint32_t)__popcll(mk[u] & lt);
                if (p < cap_n) {
                    es[p] = e[u];
                    xs[p] = v[u];
                }
                if (sel && (uint32_t)e[u] < 32u * (uint32_t)F.bit_words)
                    atomicOr(&S.bits[e[u] >> 5], 1u << (e[u] & 31));
            }
            b0 += (uint32_t)__popcll(mk[u]);
        }
    };
    auto select_all = [&](auto &&take) {
        append_all(take, &S.n_sel, S.sel_v, S.sel_e, (uint32_t)FM_MAX_K, true);
    };
    if (m <= k) {
        select_all([&](int u) { return ok[u]; });
    } else {
        if (!radix) {
            top_bin<NT>(k, S);
            const int bstar = (int)S.misc[0];
            const uint32_t need = k - S.misc[1], nb = S.hist[bstar];
            if (nb <= (uint32_t)kBnd) {
                select_all([&](int u) { return bn[u] > bstar; });
                append_all([&](int u) { return bn[u] == bstar; }, &S.n_bnd, S.bnd_v, S.bnd_e,
                           (uint32_t)kBnd, false);
                __syncthreads();
                for (uint32_t a0 = 0; a0 < nb; a0 += NT) {
                    const uint32_t a = a0 + tid;
                    bool take = false;
                    float x = 0.f;
                    int32_t en = 0;
                    if (a < nb) {
                        x = S.bnd_v[a];
                        en = S.bnd_e[a];
                        const uint64_t ka = full_key(x, en);
                        uint32_t rank = 0;
                        for (uint32_t c = 0; c < nb; ++c) rank += full_key(S.bnd_v[c], S.bnd_e[c]) > ka;
                        take = rank < need;
                    }
                    select(take, x, en);
                }
            } else {
                radix = true;
                __syncthreads();                   // hist is read before the radix clears it
            }
        }
        if (radix) {
            const RegSrc<SPT> src{v, e, ok};
            const Rule rule = radix_rule<NT>(src, k, S.hist, S.sh, S.misc);
            __syncthreads();
            select_all([&](int u) { return ok[u] && (full_key(v[u], e[u]) & rule.M) >= rule.P; });
        }
    }
    __syncthreads();
    const uint32_t cnt = min(S.n_sel, k);
    int32_t *oi = F.out_idx + (int64_t)t * F.k;
    float *ov = F.out_val ? F.out_val + (int64_t)t * F.k : nullptr;
    if (F.bit_words > 0) {
        // positions from the bitmap: prefix popcounts of the words, then within the word
        constexpr int WPT = kMergeWords / NT;                // words a thread, at most
        const int nw = F.bit_words;
        uint32_t wd[WPT], c = 0;
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int w = WPT * tid + i;
            wd[i] = w < nw ? S.bits[w] : 0u;
            c += (uint32_t)__popc(wd[i]);
        }
        const uint32_t incl = wave_incl_scan<NT>(c);
        if (ln == 63) S.wsum[tid >> 6] = incl;
        __syncthreads();
        uint32_t pre = incl - c;
        for (int w = 0; w < (tid >> 6); ++w) pre += S.wsum[w];
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int w = WPT * tid + i;
            if (w < nw) S.pref[w] = pre;
            pre += (uint32_t)__popc(wd[i]);
        }
        __syncthreads();
        for (uint32_t i = tid; i < cnt; i += NT) {
            const int32_t en = S.sel_e[i];
            const uint32_t w = ((uint32_t)en >> 5) & (kMergeWords - 1);
            const uint32_t pos = S.pref[w] + (uint32_t)__popc(S.bits[w] & ((1u << (en & 31)) - 1u));
            oi[pos] = en;
            if (ov) ov[pos] = S.sel_v[i];
        }
    } else {
        // positions from counts of smaller selected entries (the list padded to a multiple of
        // 16 with INT32_MAX, read four at a time)
        const uint32_t cnt16 = (cnt + 15u) & ~15u;
        for (uint32_t i = cnt + tid; i < cnt16; i += NT) S.sel_e[i] = 0x7fffffff;
        __syncthreads();
        for (uint32_t i = tid; i < cnt; i += NT) {
            const int32_t en = S.sel_e[i];
            uint32_t pos = 0;
            for (uint32_t c = 0; c < cnt16; c += 16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int4 x = *(const int4 *)&S.sel_e[c + 4 * q];
                    pos += (x.x < en) + (x.y < en) + (x.z < en) + (x.w < en);
                }
            }
            oi[pos] = en;
            if (ov) ov[pos] = S.sel_v[i];
        }
    }
    for (int i = (int)cnt + tid; i < F.k; i += NT) {
        oi[i] = -1;
        if (ov) ov[i] = -INFINITY;
    }
}

// bf16 keys x bf16 queries (the decode shape), NW waves a workgroup scoring one row's chunk:
// the tile ring of score_bf16_ring_kernel, logits into LDS, then the fused selection.
template <int RING, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(FM_DECODE_WAVES)))
void score_topk_bf16_kernel(ScoreArgs A, FuseArgs F) {
    constexpr int NT = 64 * NW;
    static_assert(16 % NW == 0 || NW % 16 == 0, "query fragments a wave");
    extern __shared__ __align__(16) float s_dyn[];          // [NW][ppw_pad][64] logits
    __shared__ u32x4 s_q[16][64];
    __shared__ int32_t s_base[NW * kMaxPpw];                // entry of a slot's first column
    __shared__ FuseLds<NT> S;
    // workgroup (chunk, row) = (id / T8, id % T8), T8 = T rounded up to 8: the workgroups go to
    // the 8 XCDs in turn, so every chunk of row t runs on the XCD of the merge workgroup t
    const int t8 = (int)(gridDim.x / (unsigned)F.n_chunks);
    const int t = (int)(blockIdx.x % (unsigned)t8), chunk = (int)(blockIdx.x / (unsigned)t8);
    if (t >= A.q.T) return;
    const int tid = threadIdx.x, ln = __lane_id(), r = ln & 15, g = ln >> 4;
    const int wave = tid >> 6;
    const int ppw_pad = F.ppw_pad;
    const int64_t slot0 = ((int64_t)chunk * NW + wave) * A.ppw;
    const int nslot = (int)max((int64_t)0, min((int64_t)A.ppw, A.n_slots - slot0));
    const int braw = row_request(A.q, A.kv, t);
    const int64_t nvis = n_visible(A.q, A.kv, t, braw);
    const int b = braw < 0 ? 0 : braw;
    const int64_t nres = (A.res_pages && braw >= 0) ? A.n_res[b] : 0;
    const uint8_t *pool = row_pool(A.q, A.kv, t);
    int lp_l = -1, phys_l = kSlotEmpty;
    if (ln < nslot) phys_l = resolve_slot(A, b, nvis, nres, slot0 + ln, lp_l);
    constexpr int QPW = NW >= 16 ? 1 : 16 / NW;             // query fragments a wave stages
    u32x4 qf[QPW];
    {
        const uint8_t *qrow = (const uint8_t *)A.q.q + (int64_t)t * kHeads * kDim * 2;
#pragma unroll
        for (int f = 0; f < QPW; ++f) {
            const int fi = wave * QPW + f;
            if (fi < 16) qf[f] = q_frag_bf16<KEY_BF16>(qrow, fi >> 2, fi & 3, r, g);
        }
    }
    float wv[16];
    load_w(wv, A.q.w, A.q.w_bf16, t, g);
    float (*res)[64] = (float (*)[64])(s_dyn + (int64_t)wave * ppw_pad * 64);

    const uint32_t off = (uint32_t)(r * kRowBf16 + g * 16);
    auto fetch = [&](TileBf16 &T, int x) {       // tile x: page x / 4, entry tile x % 4
        const __amdgpu_buffer_rsrc_t rs =
            page_rsrc(pool, __builtin_amdgcn_readlane(phys_l, x >> 2), kPage * kRowBf16);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            T.b[kk] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + kk * 64, (x & 3) * 16 * kRowBf16, 0);
    };
    auto tile_logit = [&](const TileBf16 &T) {
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        const u32x4 *qs = &s_q[0][ln + z];
        f32x4 acc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 bk = __builtin_bit_cast(bf16x8, T.b[kk]);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, qs[(4 * m + kk) * 64]), bk, acc[m], 0, 0, 0);
        }
        return head_sum(acc, wv);
    };

    TileBf16 T[RING];
#pragma unroll
    for (int v = 0; v < RING - 1; ++v) {
        fetch(T[v], v);
        __builtin_amdgcn_sched_barrier(0);     // tiles issue in ring order, as the loop refills them
    }
#pragma unroll
    for (int f = 0; f < QPW; ++f) {
        const int fi = wave * QPW + f;
        if (fi < 16) s_q[fi][ln] = qf[f];
    }
    for (int i = tid; i < kBins; i += NT) S.hist[i] = 0u;
    if (tid == 0) {
        S.n_out = 0u;
        S.n_bnd = 0u;
    }
    if (ln < ppw_pad)
        s_base[wave * ppw_pad + ln] = (int32_t)((F.cells ? slot0 + ln : (int64_t)lp_l) * kPage);
    __syncthreads();
    f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int x0 = 0; x0 < 4 * nslot; x0 += 4 * RING) {
#pragma unroll
        for (int u = 0; u < 4 * RING; ++u) {
            fetch(T[(u + RING - 1) % RING], x0 + u + RING - 1);
            tot[u & 3] = tile_logit(T[u % RING]);
            if ((u & 3) == 3)
                res[(x0 + u) >> 2][ln] = g == 0 ? tot[0] : g == 1 ? tot[1] : g == 2 ? tot[2] : tot[3];
        }
    }
    if (A.out) {
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(A.out + (int64_t)t * A.out_ld), (short)0, (int)(A.out_ld * 4), 0x00020000);
        store_wave_logits(A, orsrc, res, phys_l, lp_l, slot0, nslot, nvis, ln);
    }
    mark_candidates<NT>(F, res, ppw_pad, phys_l, lp_l, nslot, nvis, b, ln, wave, S);
    __syncthreads();
    const int64_t slot = (int64_t)t * F.n_chunks + chunk;
    auto entry_of = [&](int j) { return s_base[j >> 6] + (j & 63); };
    auto sel = [&](auto nv) {
        chunk_select<NT, decltype(nv)::value>(s_dyn, (uint32_t)F.k, (uint32_t)F.cap,
                                              (uint32_t)((F.k + F.n_chunks - 1) / F.n_chunks),
                                              entry_of, F.cval + slot * F.cap,
                                              F.cidx + slot * F.cap, F.cnt + slot,
                                              F.cstat + slot, S);
    };
    // values a thread: NW ppw_pad 64 / NT = ppw_pad (a multiple of the ring, at most 16)
    if (ppw_pad <= 4) sel(std::integral_constant<int, 4>());
    else if (ppw_pad <= 8) sel(std::integral_constant<int, 8>());
    else if (ppw_pad <= 12) sel(std::integral_constant<int, 12>());
    else sel(std::integral_constant<int, 16>());
}

// ---------------------------------------------------------------- fp8 keys x bf16 queries
// 32-entry tiles on v_mfma_f32_32x32x16_bf16 (the 16x16x32 bf16 MFMA of gfx950 runs at half
// that rate, and fp8 pages carry twice the entries per byte of bf16 ones, so here the matrix
// core time matters).  Lane l = j + 32 h of a tile holds key entry j's codes 64 h .. 64 h + 63
// (four 16-byte loads; 132-byte rows are 4-byte aligned) and its scale; k-step s takes the
// 8 codes 8 s .. 8 s + 7 of that half, widened to bf16 (exact), against query dims
// 64 h + 8 s .. + 8 of head 32 m + j (A operand, head tile m = 0, 1).  The accumulator register
// v of lane j + 32 h is head 32 m + 8 (v / 4) + 4 h + v % 4 for entry j, so a lane sums its 32
// heads with their weights and one row swap with lane j + 32 (1 - h) completes the 64.
struct TileF8 { u32x4 c[4]; float scale; };

// one query row's head weights for the 32x32 accumulator layout: w[m][v] is head
// 32 m + 8 (v / 4) + 4 h + v % 4 of lane j + 32 h
__device__ __forceinline__ void load_w32(float (&w)[2][16], const void *wp, int w_bf16, int t, int ln) {
    const int64_t base = (int64_t)t * kHeads + 4 * (ln >> 5);
    if (w_bf16) {
        const uint16_t *w16 = (const uint16_t *)wp + base;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v) w[m][v] = bf16f(w16[32 * m + 8 * (v >> 2) + (v & 3)]);
    } else {
        const float *w32 = (const float *)wp + base;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v) w[m][v] = w32[32 * m + 8 * (v >> 2) + (v & 3)];
    }
}

// A operand (m, k-step s) of lane j + 32 h: dims 64 h + 8 s .. + 8 of head 32 m + j
__device__ __forceinline__ u32x4 qa_frag(const uint8_t *qrow, int m, int st, int ln) {
    return *(const u32x4 *)((const uint16_t *)qrow + (32 * m + (ln & 31)) * kDim + 64 * (ln >> 5) + 8 * st);
}

// One query row with its A operands in LDS, shared by the four waves of a workgroup that
// score the same row (each wave writes 4 of the 16 fragments; the caller synchronises the
// workgroup before the first use), and its weights in registers.
struct QF8Lds {
    const u32x4 *a;                 // [8 m + s][lane]
    float w[2][16];
    __device__ void init(u32x4 *lds, const uint8_t *qrow, const void *wp, int w_bf16, int t, int ln) {
        const int wave = threadIdx.x >> 6;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int fi = 4 * wave + f;
            lds[fi * 64 + ln] = qa_frag(qrow, fi >> 3, fi & 7, ln);
        }
        a = lds;
        load_w32(w, wp, w_bf16, t, ln);
    }
    // fragments of one tile; the opaque zero keeps them from being hoisted into registers
    // across tiles, which would cost occupancy
    __device__ __forceinline__ const u32x4 *frags() const {
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        return a + __lane_id() + z;
    }
    __device__ __forceinline__ u32x4 get(const u32x4 *f, int m, int st) const { return f[(8 * m + st) * 64]; }
    __device__ __forceinline__ const f32x4 *weights() const { return (const f32x4 *)&w[0][0]; }
    static constexpr int kMT = 2;
    static constexpr bool kLds = true;
    static constexpr int kAhead = FM_QLDS_AHEAD;
};

// The same with the A operands in registers (one wave per row).
struct QF8Reg {
    u32x4 a[2][8];
    float w[2][16];
    __device__ void init(const uint8_t *qrow, const void *wp, int w_bf16, int t, int ln) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int st = 0; st < 8; ++st) a[m][st] = qa_frag(qrow, m, st, ln);
        load_w32(w, wp, w_bf16, t, ln);
    }
    __device__ __forceinline__ const u32x4 *frags() const { return nullptr; }
    __device__ __forceinline__ u32x4 get(const u32x4 *, int m, int st) const { return a[m][st]; }
    __device__ __forceinline__ const f32x4 *weights() const { return (const f32x4 *)&w[0][0]; }
    static constexpr int kMT = 2;
    static constexpr bool kLds = false;
    static constexpr int kAhead = 4;
};

// The A operands in registers, the head weights in LDS ([lane half][16 m + v], as QWideLds lays
// them out; every lane of a half reads the same words): 32 fewer registers than QF8Reg.
struct QF8RegW {
    u32x4 a[2][8];
    const f32x4 *w;
    // wave-wide: lane l writes one weight of the row into lds_w[64] (the caller synchronises
    // the workgroup before the first use)
    __device__ void init(const uint8_t *qrow, float *lds_w, const void *wp, int w_bf16, int t, int ln) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int st = 0; st < 8; ++st) a[m][st] = qa_frag(qrow, m, st, ln);
        const int h = ln >> 5, m = (ln >> 4) & 1, v = ln & 15;
        const int64_t head = (int64_t)t * kHeads + 32 * m + 8 * (v >> 2) + 4 * h + (v & 3);
        lds_w[ln] = w_bf16 ? bf16f(((const uint16_t *)wp)[head]) : ((const float *)wp)[head];
        w = (const f32x4 *)lds_w;
    }
    __device__ __forceinline__ const u32x4 *frags() const { return nullptr; }
    __device__ __forceinline__ u32x4 get(const u32x4 *, int m, int st) const { return a[m][st]; }
    __device__ __forceinline__ const f32x4 *weights() const {
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        return w + 8 * (__lane_id() >> 5) + z;
    }
    static constexpr int kMT = 2;
    static constexpr bool kLds = false;
    static constexpr int kAhead = 4;
};

// One query row's A operands and head weights for 32 MT heads, both in LDS, staged by the whole
// workgroup (its waves all score that row): fragment (m, s) at a[(8 m + s) * 64 + lane] as
// qa_frag lays it out, weights as [lane half h][16 m + v] = head 32 m + 8 (v / 4) + 4 h + v % 4,
// the accumulator layout of tile_logit_f8.  The wide-head (128) kernels use it.
template <int MT>
struct QWideLds {
    const u32x4 *a;
    const f32x4 *w;
    // every thread of the workgroup calls this; the caller synchronises before the first use
    __device__ void stage(u32x4 *lds_a, float *lds_w, const uint8_t *qrow, const void *wp, int w_bf16,
                          int64_t wrow) {
        const int ln = __lane_id(), nw = (int)(blockDim.x >> 6);
        for (int fi = (int)(threadIdx.x >> 6); fi < 8 * MT; fi += nw)
            lds_a[fi * 64 + ln] = qa_frag(qrow, fi >> 3, fi & 7, ln);
        for (int i = (int)threadIdx.x; i < 32 * MT; i += (int)blockDim.x) {
            const int h = i / (16 * MT), m = (i % (16 * MT)) >> 4, v = i & 15;
            const int64_t head = wrow * 32 * MT + 32 * m + 8 * (v >> 2) + 4 * h + (v & 3);
            lds_w[i] = w_bf16 ? bf16f(((const uint16_t *)wp)[head]) : ((const float *)wp)[head];
        }
        a = lds_a;
        w = (const f32x4 *)lds_w;
    }
    __device__ __forceinline__ const u32x4 *frags() const {
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        return a + __lane_id() + z;
    }
    __device__ __forceinline__ u32x4 get(const u32x4 *f, int m, int st) const { return f[(8 * m + st) * 64]; }
    __device__ __forceinline__ const f32x4 *weights() const {
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        return w + 4 * MT * (__lane_id() >> 5) + z;
    }
    static constexpr int kMT = MT;
    static constexpr bool kLds = true;
    static constexpr int kAhead = FM_MASK_AHEAD;
};

// tile (page slot, half) of a page through its buffer descriptor (zero-size: nothing read)
__device__ __forceinline__ void load_tile_f8(TileF8 &T, const __amdgpu_buffer_rsrc_t &rs, int half, int ln) {
    const uint32_t row = (uint32_t)((32 * half + (ln & 31)) * kRowFp8);
    const uint32_t off = row + 64 * (ln >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) T.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, 0, 0);
    T.scale = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, row + kDim, 0, 0));
}

// max(x, 0) for a float through its bit pattern: every negative float (and -0) is a negative
// int.  One integer max instead of the quieting max pair a float max needs in IEEE mode.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Coalesced variant for tiles that pass through LDS: instruction k of lane ln reads code bytes
// 16 (ln % 8) .. + 15 of row 32 half + 8 k + ln / 8 (eight lanes cover a row's 128 code bytes);
// half 0 also reads the scale of row ln of the page.  tile_to_mma_layout() then moves the codes
// through the wave's LDS buffer (144-byte rows: aligned, no bank conflicts) into the layout
// load_tile_f8 produces.  Row-contiguous 128-byte reads stream markedly faster from HBM than
// sixteen-byte pieces of 64 different rows.
constexpr int kTileLdsRow = 144;
__device__ __forceinline__ void load_tile_rows(TileF8 &T, const __amdgpu_buffer_rsrc_t &rs, int half, int ln) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t row = (uint32_t)(32 * half + 8 * k + (ln >> 3));
        T.c[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, row * kRowFp8 + 16 * (ln & 7), 0, 0);
    }
    if (half == 0) T.scale = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)ln * kRowFp8 + kDim, 0, 0));
}
__device__ __forceinline__ void tile_to_mma_layout(TileF8 &T, uint8_t *buf, int ln) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
        *(u32x4 *)(buf + (8 * k + (ln >> 3)) * kTileLdsRow + 16 * (ln & 7)) = T.c[k];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        T.c[k] = *(const u32x4 *)(buf + (ln & 31) * kTileLdsRow + 64 * (ln >> 5) + 16 * k);
}

// logit of entry (lane % 32) of the tile, scale applied; both lane halves return it.  The A
// fragments are fetched QF::kAhead MFMAs ahead of their use (from LDS for the LDS sources).
template <class QF>
__device__ __forceinline__ float tile_logit_f8(const QF &Q, const TileF8 &T) {
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    constexpr int MT = QF::kMT;                   // head tiles of 32
    const u32x4 *qf = Q.frags();
    f32x16 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][v] = 0.f;
    constexpr int D = QF::kAhead;                 // fragments in flight (fragment k = MT st + m)
    u32x4 a[D];
#pragma unroll
    for (int k = 0; k < D; ++k) a[k] = Q.get(qf, k % MT, k / MT);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        const uint32_t d0 = T.c[st >> 1][(st & 1) * 2], d1 = T.c[st >> 1][(st & 1) * 2 + 1];
        u32x4 bw;
        bw[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false));
        bw[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true));
        bw[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false));
        bw[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true));
        const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int k = MT * st + m;
            acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[k % D]), b, acc[m], 0, 0, 0);
            if (k + D < 8 * MT) a[k % D] = Q.get(qf, (k + D) % MT, (k + D) / MT);
            if (QF::kLds) __builtin_amdgcn_sched_barrier(0);
        }
    }
    const f32x4 *wt = Q.weights();
    float p = 0.f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const f32x4 w4 = wt[4 * m + v4];
#pragma unroll
            for (int e = 0; e < 4; ++e) p = fmaf(w4[e], relu_bits(acc[m][4 * v4 + e]), p);
        }
    const uint32_t u = __float_as_uint(p);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * T.scale;
}

// Tile stream of one wave over page slots 0 .. n - 1 (two tiles a page): fetch(T, x) loads
// tile x, take(tot0, tot1, i) receives page slot i's two tile results.  A ring of RING tiles
// keeps RING - 1 loading; fetch must be a valid (zero-size) load past the wave's pages.
template <int RING, class QF, class Fetch, class Take>
__device__ __forceinline__ void stream_tiles_f8(int n, const QF &Q, Fetch fetch, Take take) {
    static_assert(RING % 2 == 0, "the ring holds whole pages");
    TileF8 T[RING];
#pragma unroll
    for (int v = 0; v < RING - 1; ++v) {
        fetch(T[v], v);
        __builtin_amdgcn_sched_barrier(0);     // tiles issue in ring order, as the loop refills them
    }
    float t0 = 0.f;
    for (int x0 = 0; x0 < 2 * n; x0 += 2 * RING) {
#pragma unroll
        for (int u = 0; u < 2 * RING; ++u) {
            fetch(T[(u + RING - 1) % RING], x0 + u + RING - 1);
            const float tl = tile_logit_f8(Q, T[u % RING]);
            if (u & 1) take(t0, tl, (x0 + u) >> 1);
            else t0 = tl;
        }
    }
}

// Two-level (and any bf16-query) scoring over fp8 pages: the work split, slot states and
// deferred stores of score_kernel, with the tile stream above.  One wave's page slots of row
// blockIdx.y, with the row's query source Q already staged.
template <int RING, class QF>
__device__ __forceinline__ void score_f8_slots(const ScoreArgs &A, const QF &Q, float (*res)[64], int t,
                                               int ln, int wave) {
    const int64_t slot0 = ((int64_t)blockIdx.x * 4 + wave) * A.ppw;
    if (slot0 >= A.n_slots) return;
    const int nslot = (int)min((int64_t)A.ppw, A.n_slots - slot0);
    const int braw = row_request(A.q, A.kv, t);
    const int64_t nvis = n_visible(A.q, A.kv, t, braw);
    const int b = braw < 0 ? 0 : braw;
    const int64_t nres = (A.res_pages && braw >= 0) ? A.n_res[b] : 0;
    const uint8_t *pool = row_pool(A.q, A.kv, t);
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A.out + (int64_t)t * A.out_ld), (short)0, (int)(A.out_ld * 4), 0x00020000);
    int lp_l = -1, phys_l = kSlotEmpty;
    if (ln < nslot) phys_l = resolve_slot(A, b, nvis, nres, slot0 + ln, lp_l);

    auto fetch = [&](TileF8 &T, int x) {
        load_tile_f8(T, page_rsrc(pool, __builtin_amdgcn_readlane(phys_l, x >> 1), kPage * kRowFp8), x & 1, ln);
    };
    auto take = [&](float t0, float t1, int i) { res[i][ln] = (ln >> 5) ? t1 : t0; };
    stream_tiles_f8<RING>(nslot, Q, fetch, take);
    store_wave_logits(A, orsrc, res, phys_l, lp_l, slot0, nslot, nvis, ln);
}

// 32 MT heads: MT = 2 keeps the query fragments in LDS and the head weights in registers
// (QF8Lds); MT = 4 (128 heads) keeps both in LDS (QWideLds), at two waves a SIMD.
template <int RING, int MT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT == 2 ? FM_F8_WPE : 2)))
void score_f8_kernel(ScoreArgs A) {
    __shared__ __align__(16) float s_res[4][kMaxPpw + RING][64];
    __shared__ u32x4 s_qa[8 * MT * 64];
    const int t = blockIdx.y;
    const int ln = __lane_id();
    const int wave = threadIdx.x >> 6;
    const uint8_t *qrow = (const uint8_t *)A.q.q + (int64_t)t * (32 * MT) * kDim * 2;
    if constexpr (MT == 2) {
        QF8Lds Q;
        Q.init(s_qa, qrow, A.q.w, A.q.w_bf16, t, ln);
        __syncthreads();
        score_f8_slots<RING>(A, Q, s_res[wave], t, ln, wave);
    } else {
        __shared__ __align__(16) float s_w[32 * MT];
        QWideLds<MT> Q;
        Q.stage(s_qa, s_w, qrow, A.q.w, A.q.w_bf16, t);
        __syncthreads();
        score_f8_slots<RING>(A, Q, s_res[wave], t, ln, wave);
    }
}

// fp8 keys x bf16 queries, 64 heads (two-level scoring, Mode A over fp8 pools), NW waves a
// workgroup scoring one row's chunk: the 32-entry tile stream of score_f8_kernel with the
// query fragments staged in LDS for the workgroup, logits into LDS, then the fused selection.
template <int RING, int NW, int MAXPPW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(FM_F8_WPE)))
void score_topk_f8_kernel(ScoreArgs A, FuseArgs F) {
    constexpr int NT = 64 * NW;
    extern __shared__ __align__(16) float s_dyn[];          // [NW][ppw_pad][64] logits
    __shared__ u32x4 s_qa[16 * 64];                          // fragment (m, s) at (8 m + s) 64
    __shared__ int32_t s_base[NW * MAXPPW];
    __shared__ FuseLds<NT> S;
    // workgroup (chunk, row) = (id / T8, id % T8), T8 = T rounded up to 8: the workgroups go to
    // the 8 XCDs in turn, so every chunk of row t runs on the XCD of the merge workgroup t
    const int t8 = (int)(gridDim.x / (unsigned)F.n_chunks);
    const int t = (int)(blockIdx.x % (unsigned)t8), chunk = (int)(blockIdx.x / (unsigned)t8);
    if (t >= A.q.T) return;
    const int tid = threadIdx.x, ln = __lane_id();
    const int wave = tid >> 6;
    const int ppw_pad = F.ppw_pad;
    const uint8_t *qrow = (const uint8_t *)A.q.q + (int64_t)t * kHeads * kDim * 2;
    for (int fi = wave; fi < 16; fi += NW) s_qa[fi * 64 + ln] = qa_frag(qrow, fi >> 3, fi & 7, ln);
    QF8Lds Q;
    Q.a = s_qa;
    load_w32(Q.w, A.q.w, A.q.w_bf16, t, ln);
    const int64_t slot0 = ((int64_t)chunk * NW + wave) * A.ppw;
    const int nslot = (int)max((int64_t)0, min((int64_t)A.ppw, A.n_slots - slot0));
    const int braw = row_request(A.q, A.kv, t);
    const int64_t nvis = n_visible(A.q, A.kv, t, braw);
    const int b = braw < 0 ? 0 : braw;
    const int64_t nres = (A.res_pages && braw >= 0) ? A.n_res[b] : 0;
    const uint8_t *pool = row_pool(A.q, A.kv, t);
    int lp_l = -1, phys_l = kSlotEmpty;
    if (ln < nslot) phys_l = resolve_slot(A, b, nvis, nres, slot0 + ln, lp_l);
    for (int i = tid; i < kBins; i += NT) S.hist[i] = 0u;
    if (tid == 0) {
        S.n_out = 0u;
        S.n_bnd = 0u;
    }
    if (ln < ppw_pad)
        s_base[wave * ppw_pad + ln] = (int32_t)((F.cells ? slot0 + ln : (int64_t)lp_l) * kPage);
    __syncthreads();
    float (*res)[64] = (float (*)[64])(s_dyn + (int64_t)wave * ppw_pad * 64);
    auto fetch = [&](TileF8 &T, int x) {
        load_tile_f8(T, page_rsrc(pool, __builtin_amdgcn_readlane(phys_l, x >> 1), kPage * kRowFp8), x & 1, ln);
    };
    auto take = [&](float t0, float t1, int i) { res[i][ln] = (ln >> 5) ? t1 : t0; };
    stream_tiles_f8<RING>(nslot, Q, fetch, take);
    if (A.out) {
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(A.out + (int64_t)t * A.out_ld), (short)0, (int)(A.out_ld * 4), 0x00020000);
        store_wave_logits(A, orsrc, res, phys_l, lp_l, slot0, nslot, nvis, ln);
    }
    mark_candidates<NT>(F, res, ppw_pad, phys_l, lp_l, nslot, nvis, b, ln, wave, S);
    __syncthreads();
    const int64_t slot = (int64_t)t * F.n_chunks + chunk;
    auto entry_of = [&](int j) { return s_base[j >> 6] + (j & 63); };
    auto sel = [&](auto nv) {
        chunk_select<NT, decltype(nv)::value>(s_dyn, (uint32_t)F.k, (uint32_t)F.cap,
                                              (uint32_t)((F.k + F.n_chunks - 1) / F.n_chunks),
                                              entry_of, F.cval + slot * F.cap,
                                              F.cidx + slot * F.cap, F.cnt + slot,
                                              F.cstat + slot, S);
    };
    if (ppw_pad <= 4) sel(std::integral_constant<int, 4>());
    else if (ppw_pad <= 8) sel(std::integral_constant<int, 8>());
    else if (ppw_pad <= 12) sel(std::integral_constant<int, 12>());
    else if (MAXPPW <= 16 || ppw_pad <= 16) sel(std::integral_constant<int, 16>());
    else sel(std::integral_constant<int, MAXPPW>());
}

// ---------------------------------------------------------------- fp32 path (VALU)
// One thread per output column; fp32 products and sums.  For fp32 inputs only; NH heads.
template <int NH>
__global__ __launch_bounds__(256) void score_f32_kernel(ScoreArgs A) {
    __shared__ float qs[NH * kDim];
    __shared__ float wsm[NH];
    const int t = blockIdx.y;
    const float *qrow = (const float *)A.q.q + (int64_t)t * NH * kDim;
    for (int i = threadIdx.x; i < NH * kDim; i += blockDim.x) qs[i] = qrow[i];
    for (int i = threadIdx.x; i < NH; i += blockDim.x)
        wsm[i] = A.q.w_bf16 ? bf16f(((const uint16_t *)A.q.w)[(int64_t)t * NH + i])
                            : ((const float *)A.q.w)[(int64_t)t * NH + i];
    __syncthreads();
    const int64_t col = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (col >= A.n_slots * kPage || col >= A.out_ld) return;
    const int braw = row_request(A.q, A.kv, t);
    const int64_t nvis = n_visible(A.q, A.kv, t, braw);
    const int b = braw < 0 ? 0 : braw;
    const int64_t nres = (A.res_pages && braw >= 0) ? A.n_res[b] : 0;
    int lp;
    int phys = resolve_slot(A, b, nvis, nres, col / kPage, lp);
    if (phys == kSlotEmpty) return;
    const int64_t s = (int64_t)lp * kPage + col % kPage;
    float v;
    if (phys >= 0 && s < nvis) {
        const float *k = (const float *)row_pool(A.q, A.kv, t) +
                         ((int64_t)phys * kPage + col % kPage) * kDim;
        float kr[kDim];
#pragma unroll
        for (int d = 0; d < kDim; ++d) kr[d] = k[d];
        v = 0.f;
        for (int h = 0; h < NH; ++h) {
            float x = 0.f;
#pragma unroll
            for (int d = 0; d < kDim; ++d) x = fmaf(qs[h * kDim + d], kr[d], x);
            v = fmaf(wsm[h], fmaxf(x, 0.f), v);
        }
    } else if (phys == kSlotUnmapped && s < nvis) {
        v = __builtin_nanf("");
    } else {
        v = -INFINITY;
    }
    A.out[(int64_t)t * A.out_ld + col] = v;
}

// ---------------------------------------------------------------- Level-1 mask
// Union of n_layers encoders per entry (paper summary, section 3, R_t equation; README "Joint
// checkpoint + ensemble": max or mean of the per-layer sigmoids).  Grid (ceil(n_pages / PPW),
// B), one wave per layer (blockDim = 64 n_layers): wave l streams PPW consecutive pages of
// request blockIdx.y from pool l with layer l's query fragments in registers, and leaves its
// logits in LDS; then the workgroup forms the union, the decision and the mask bytes.
template <int KF, int PPW>
__global__ __launch_bounds__(64 * FM_MAX_LAYERS) __attribute__((amdgpu_waves_per_eu(FM_WAVES_PER_EU)))
void mask_kernel(MaskArgs A) {
    typedef typename PageOf<KF>::T Pg;
    constexpr int NB = PageOf<KF>::nbuf;
    __shared__ float s_u[FM_MAX_LAYERS][PPW + FM_F8_RING][kPage];
    const int b = blockIdx.y;
    const int ln = __lane_id(), r = ln & 15, g = ln >> 4;
    const int l = threadIdx.x >> 6;              // this wave's layer
    const int64_t page0 = (int64_t)blockIdx.x * PPW;
    const int np = (int)min((int64_t)PPW, A.n_pages - page0);
    const int64_t seq = A.kv.seq_lens[b];

    // lane i describes page page0 + i (i < np): physical page or state; past np: invisible
    int phys_l = kSlotInvisible;
    if (ln < np) {
        const int64_t lp = page0 + ln;
        if (lp * kPage >= seq) phys_l = kSlotInvisible;
        else if (lp >= A.kv.bt_ld) phys_l = kSlotUnmapped;
        else {
            const int p = A.kv.bt[(int64_t)b * A.kv.bt_ld + lp];
            phys_l = (p < 0 || p >= A.kv.n_phys) ? kSlotUnmapped : p;
        }
    }

    if constexpr (KF == KEY_FP8) {
        const QArgs &QA = A.q[l];
        const uint8_t *pool = A.kv.pool[l];
        QF8Reg Q;
        Q.init((const uint8_t *)QA.q + (int64_t)b * kHeads * kDim * 2, QA.w, QA.w_bf16, b, ln);
        auto fetch = [&](TileF8 &T, int x) {
            load_tile_f8(T, page_rsrc(pool, __builtin_amdgcn_readlane(phys_l, x >> 1), kPage * kRowFp8), x & 1, ln);
        };
        auto take = [&](float t0, float t1, int i) {
            const int phys = __builtin_amdgcn_readlane(phys_l, i);
            const float L = (ln >> 5) ? t1 : t0;
            s_u[l][i][ln] = phys >= 0 ? L : (phys == kSlotUnmapped ? __builtin_nanf("") : -INFINITY);
        };
        stream_tiles_f8<FM_F8_RING>(np, Q, fetch, take);
    } else {
        const QArgs &QA = A.q[l];
        float wv[16];
        load_w(wv, QA.w, QA.w_bf16, b, g);
        const uint8_t *pool = A.kv.pool[l];
        QSource<KF, Q_BF16> Q;
        Q.init((const uint8_t *)QA.q + (int64_t)b * kHeads * kDim * 2, r, g);
        auto fetch = [&](Pg &P, int i) {
            load_page(P, pool, __builtin_amdgcn_readlane(phys_l, i), r, g, ln);
        };
        auto take = [&](const Pg &P, int i) {
            const int phys = __builtin_amdgcn_readlane(phys_l, i);
            const float L = Q.logit(wv, P, g) * page_scale(P);
            s_u[l][i][ln] = phys >= 0 ? L : (phys == kSlotUnmapped ? __builtin_nanf("") : -INFINITY);
        };
        Pg P[NB];
        stream_pages(np, P, fetch, take);
    }
    __syncthreads();

    const float inv_n = 1.0f / (float)A.n_layers;
    uint8_t *mrow = A.mask + (int64_t)b * A.mask_ld;
    for (int e = threadIdx.x; e < np * kPage; e += blockDim.x) {
        const int i = e >> 6, x = e & 63;
        const int64_t s = (page0 + i) * kPage + x;
        if (s >= A.mask_ld) continue;
        float u = A.mean_mode ? 0.f : -INFINITY;
        for (int k = 0; k < A.n_layers; ++k) {
            const float L = s_u[k][i][x];
            u = A.mean_mode ? u + inv_n / (1.0f + expf(-L))
                            : ((L != L || u != u) ? __builtin_nanf("") : fmaxf(u, L));
        }
        const bool valid = s < seq;
        const bool m = valid && (u >= A.cut || s < A.n_sink || s >= seq - A.n_recent);
        mrow[s] = m ? 1 : 0;
        if (A.union_score) A.union_score[(int64_t)b * A.mask_ld + s] = valid ? u : -INFINITY;
    }
}

// Tile stream over page slots 0 .. n - 1 with coalesced row loads (load_tile_rows) moved to the
// MFMA layout through the wave's LDS buffer: take(t0, t1, sc, i) receives page slot i's two tile
// results and the scale of entry (lane) of the page.
template <int RING, class QF, class Fetch, class Take>
__device__ __forceinline__ void stream_tiles_rows(int n, const QF &Q, uint8_t *buf, Fetch fetch, Take take) {
    static_assert(RING % 2 == 0, "the ring holds whole pages");
    const int ln = __lane_id();
    TileF8 T[RING];
#pragma unroll
    for (int v = 0; v < RING - 1; ++v) {
        fetch(T[v], v);
        __builtin_amdgcn_sched_barrier(0);     // tiles issue in ring order, as the loop refills them
    }
    float t0 = 0.f, sc = 1.f;
    for (int x0 = 0; x0 < 2 * n; x0 += 2 * RING) {
#pragma unroll
        for (int u = 0; u < 2 * RING; ++u) {
            fetch(T[(u + RING - 1) % RING], x0 + u + RING - 1);
            TileF8 &Tu = T[u % RING];
            if ((u & 1) == 0) sc = Tu.scale;
            tile_to_mma_layout(Tu, buf, ln);
            Tu.scale = 1.f;
            const float tl = tile_logit_f8(Q, Tu);
            if (u & 1) take(t0, tl, sc, (x0 + u) >> 1);
            else t0 = tl;
        }
    }
}

// The same union over fp8 pools with bf16 queries, four waves a workgroup, every wave on its own
// ppw pages of request blockIdx.y for all NL layers in turn: layer l's query operands and head
// weights sit in the wave's registers while it streams its pages of pool l, and the running
// union of each entry waits in LDS.  After the last layer the wave forms the decisions and
// writes its pages' mask bytes.  32 MT heads: with MT = 4 (128 heads) a layer's query would not
// fit the registers, so the workgroup stages each layer's fragments and weights in LDS
// (QWideLds) in turn, and every wave stays to the last barrier (one without pages streams
// nothing).
template <int NL, int MT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FM_MASK_WPE)))
void mask_f8_kernel(MaskArgs A) {
    constexpr int RING = FM_MASK_RING;
    __shared__ float s_u[4][kMaskPpw][kPage];                                      // unions
    __shared__ __attribute__((aligned(16))) uint8_t s_tile[4][32 * kTileLdsRow];   // transposes
    const int b = blockIdx.y;
    const int ln = __lane_id(), wave = threadIdx.x >> 6;
    const int64_t page0 = ((int64_t)blockIdx.x * 4 + wave) * A.ppw;
    if (MT == 2 && page0 >= A.n_pages) return;
    const int np = (int)max((int64_t)0, min((int64_t)A.ppw, A.n_pages - page0));
    const int64_t seq = A.kv.seq_lens[b];

    // lane i describes page page0 + i (i < np): physical page or state; past np: invisible
    int phys_l = kSlotInvisible;
    if (ln < np) {
        const int64_t lp = page0 + ln;
        if (lp * kPage >= seq) phys_l = kSlotInvisible;
        else if (lp >= A.kv.bt_ld) phys_l = kSlotUnmapped;
        else {
            const int p = A.kv.bt[(int64_t)b * A.kv.bt_ld + lp];
            phys_l = (p < 0 || p >= A.kv.n_phys) ? kSlotUnmapped : p;
        }
    }
    const float inv_n = 1.0f / (float)NL;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        const uint8_t *qrow = (const uint8_t *)A.q[l].q + (int64_t)b * (32 * MT) * kDim * 2;
        const uint8_t *pool = A.kv.pool[l];
        auto fetch = [&](TileF8 &T, int x) {
            load_tile_rows(T, page_rsrc(pool, __builtin_amdgcn_readlane(phys_l, x >> 1), kPage * kRowFp8), x & 1, ln);
        };
        auto take = [&](float t0, float t1, float sc, int i) {
            if (i >= np) return;
            const int phys = __builtin_amdgcn_readlane(phys_l, i);
            float L = ((ln >> 5) ? t1 : t0) * sc;
            L = phys >= 0 ? L : (phys == kSlotUnmapped ? __builtin_nanf("") : -INFINITY);
            float &u = s_u[wave][i][ln];
            if (A.mean_mode) {
                const float p = inv_n / (1.0f + expf(-L));
                u = l == 0 ? p : u + p;
            } else {
                u = l == 0 ? L : ((L != L || u != u) ? __builtin_nanf("") : fmaxf(u, L));
            }
        };
        if constexpr (MT == 2) {
            QF8Reg Q;
            Q.init(qrow, A.q[l].w, A.q[l].w_bf16, b, ln);
            // the query loads complete before the tile ring starts, so that the stream's waits
            // count ring loads only (otherwise each pass of its loop waits for every load)
            __builtin_amdgcn_s_waitcnt(0);
            stream_tiles_rows<RING>(np, Q, s_tile[wave], fetch, take);
        } else {
            __shared__ u32x4 s_qa[8 * MT * 64];
            __shared__ __align__(16) float s_w[32 * MT];
            if (l > 0) __syncthreads();     // every wave is done with the previous layer
            QWideLds<MT> Q;
            Q.stage(s_qa, s_w, qrow, A.q[l].w, A.q[l].w_bf16, b);
            __syncthreads();
            stream_tiles_rows<RING>(np, Q, s_tile[wave], fetch, take);
        }
    }

    // decisions and mask bytes (0 / 1): 16-byte chunks when the span is whole and aligned, else
    // one by one.  Chunk c covers entries 16 (c % 4) .. + 15 of page c / 4.
    uint8_t *mrow = A.mask + (int64_t)b * A.mask_ld;
    const int64_t s0 = page0 * kPage;
    const int nb = (int)min((int64_t)np * kPage, A.mask_ld - s0);
    auto decide = [&](int e) -> bool {     // entry s0 + e of the wave's span
        const int64_t s = s0 + e;
        const float u = s_u[wave][e >> 6][e & 63];
        if (A.union_score) A.union_score[(int64_t)b * A.mask_ld + s] = s < seq ? u : -INFINITY;
        return s < seq && (u >= A.cut || s < A.n_sink || s >= seq - A.n_recent);
    };
    if (A.dens_out) {
        // the page flags of compaction: resident entries of each page, one ballot a page
        for (int i = 0; i < np; ++i) {
            const int e = i * kPage + ln;
            const int64_t s = s0 + e;
            const float u = s_u[wave][i][ln];
            const bool d = e < nb && s < seq && (u >= A.cut || s < A.n_sink || s >= seq - A.n_recent);
            const uint64_t m = __ballot(d);
            if (ln == 0) A.dens_out[(int64_t)b * A.dens_ld + page0 + i] = (int32_t)__popcll(m);
        }
    }
    if (nb % 16 == 0 && ((uintptr_t)(mrow + s0) % 16) == 0) {
        for (int c = ln; 16 * c < nb; c += 64) {
            u32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t w = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) w |= (decide(16 * c + 4 * q + k) ? 1u : 0u) << (8 * k);
                v[q] = w;
            }
            *(u32x4 *)(mrow + s0 + 16 * c) = v;
        }
    } else {
        for (int e = ln; e < nb; e += 64) mrow[s0 + e] = decide(e) ? 1 : 0;
    }
}

// The union over NL encoders that all score one pool (the pools are the same array), fp8 keys,
// bf16 queries, 64 heads.  A workgroup of NL waves streams up to FM_SHARED_PPW pages of request
// blockIdx.y, and each key tile leaves HBM once for all encoders: in round r wave w loads tile
// NL r + w (coalesced rows, FM_SHARED_AHEAD rounds ahead in registers) and writes it to the
// workgroup's LDS (double-buffered by round); after the round's barrier every wave scores all NL
// tiles of the round with its own encoder's query operands and head weights (wave l = encoder
// l, held in registers).  Each logit is the same float the per-layer kernel computes, and the
// union is formed in the same layer order, so the result equals mask_f8_kernel's.
template <int NL>
__global__ __launch_bounds__(64 * NL) __attribute__((amdgpu_waves_per_eu(FM_SHARED_WPE)))
void mask_f8_shared_kernel(MaskArgs A) {
    constexpr int D = FM_SHARED_AHEAD;
    constexpr int PPW = FM_SHARED_PPW;
    constexpr int NT = 64 * NL;
    __shared__ float s_l[NL][PPW][kPage];                                   // logits, then union
    __shared__ float s_sc[PPW][kPage];                                      // entry scales
    __shared__ __attribute__((aligned(16))) uint8_t s_t[2][NL][32 * kTileLdsRow];   // tiles
    __shared__ __align__(16) float s_w[NL][64];                             // head weights
    const int b = blockIdx.y;
    const int tid = threadIdx.x, ln = __lane_id();
    const int l = __builtin_amdgcn_readfirstlane(tid >> 6);                // this wave's encoder
    const int64_t page0 = (int64_t)blockIdx.x * A.ppw;
    const int np = (int)max((int64_t)0, min((int64_t)A.ppw, A.n_pages - page0));
    const int64_t seq = A.kv.seq_lens[b];
    int phys_l = kSlotInvisible;            // lane i: page page0 + i (as in mask_f8_kernel)
    if (ln < np) {
        const int64_t lp = page0 + ln;
        if (lp * kPage >= seq) phys_l = kSlotInvisible;
        else if (lp >= A.kv.bt_ld) phys_l = kSlotUnmapped;
        else {
            const int p = A.kv.bt[(int64_t)b * A.kv.bt_ld + lp];
            phys_l = (p < 0 || p >= A.kv.n_phys) ? kSlotUnmapped : p;
        }
    }
    const uint8_t *pool = A.kv.pool[0];
    // tile x of the workgroup's pages (past the last page: a zero-size load), as load_tile_rows
    // loads it, except that every tile issues the scale load (the second half's through a
    // zero-size descriptor): the same number of loads per tile keeps the loop's waits exact
    auto fetch = [&](TileF8 &T, int x) {
        const int phys = __builtin_amdgcn_readlane(phys_l, x >> 1);
        const __amdgpu_buffer_rsrc_t rs = page_rsrc(pool, phys, kPage * kRowFp8);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t row = (uint32_t)(32 * (x & 1) + 8 * k + (ln >> 3));
            T.c[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, row * kRowFp8 + 16 * (ln & 7), 0, 0);
        }
        const __amdgpu_buffer_rsrc_t rsc = page_rsrc(pool, (x & 1) ? -1 : phys, kPage * kRowFp8);
        T.scale = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsc, (uint32_t)ln * kRowFp8 + kDim, 0, 0));
    };
    const int ntile = 2 * np;
    const int nround = (ntile + NL - 1) / NL;
    QF8RegW Q;
    Q.init((const uint8_t *)A.q[l].q + (int64_t)b * kHeads * kDim * 2, s_w[l], A.q[l].w,
           A.q[l].w_bf16, b, ln);
    // the query loads complete before the tile ring starts, so that the loop's waits count
    // ring loads only (otherwise every round waits for all loads in flight)
    __builtin_amdgcn_s_waitcnt(0);
    TileF8 T[D];
#pragma unroll
    for (int u = 0; u < D; ++u) {
        fetch(T[u], NL * u + l);
        __builtin_amdgcn_sched_barrier(0);     // tiles issue in ring order, as the loop refills them
    }
    // every pass of the loop refills all D ring slots (rounds past the last one load nothing),
    // so the loads in flight at its head are the same on every pass
    for (int r0 = 0; r0 < nround; r0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int r = r0 + u;
            const bool live = r < nround;
            const int x = NL * r + l;
            if (live && x < ntile) {
                uint8_t *buf = s_t[r & 1][l];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    *(u32x4 *)(buf + (8 * k + (ln >> 3)) * kTileLdsRow + 16 * (ln & 7)) = T[u].c[k];
                if ((x & 1) == 0) s_sc[x >> 1][ln] = T[u].scale;
            }
            fetch(T[u], NL * (r + D) + l);
            if (!live) continue;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                const int xj = NL * r + j;
                if (xj >= ntile) break;
                const uint8_t *src = s_t[r & 1][j];
                TileF8 B;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    B.c[k] = *(const u32x4 *)(src + (ln & 31) * kTileLdsRow + 64 * (ln >> 5) + 16 * k);
                B.scale = 1.f;
                const float tl = tile_logit_f8(Q, B);
                const int e = 32 * (xj & 1) + (ln & 31);
                if (ln < 32) s_l[l][xj >> 1][e] = tl * s_sc[xj >> 1][e];
            }
        }
    }
    __syncthreads();
    // union of each entry over the encoders, in layer order, into s_l[0]
    const float inv_n = 1.0f / (float)NL;
    for (int e = tid; e < np * kPage; e += NT) {
        const int i = __builtin_amdgcn_readfirstlane(e >> 6), x = e & 63;
        const int phys = __builtin_amdgcn_readlane(phys_l, i);
        float u = 0.f;
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const float L = phys >= 0 ? s_l[k][i][x] : (phys == kSlotUnmapped ? __builtin_nanf("") : -INFINITY);
            if (A.mean_mode) {
                const float p = inv_n / (1.0f + expf(-L));
                u = k == 0 ? p : u + p;
            } else {
                u = k == 0 ? L : ((L != L || u != u) ? __builtin_nanf("") : fmaxf(u, L));
            }
        }
        s_l[0][i][x] = u;
    }
    __syncthreads();
    uint8_t *mrow = A.mask + (int64_t)b * A.mask_ld;
    const int64_t s0 = page0 * kPage;
    const int nb = (int)max((int64_t)0, min((int64_t)np * kPage, A.mask_ld - s0));
    auto decide = [&](int e) -> bool {     // entry s0 + e of the workgroup's span
        const int64_t s = s0 + e;
        const float u = s_l[0][e >> 6][e & 63];
        return s < seq && (u >= A.cut || s < A.n_sink || s >= seq - A.n_recent);
    };
    if (A.dens_out) {
        for (int i = l; i < np; i += NL) {
            const int e = i * kPage + ln;
            const uint64_t m = __ballot(e < nb && decide(e));
            if (ln == 0) A.dens_out[(int64_t)b * A.dens_ld + page0 + i] = (int32_t)__popcll(m);
        }
    }
    if (A.union_score)
        for (int e = tid; e < nb; e += NT) {
            const int64_t s = s0 + e;
            A.union_score[(int64_t)b * A.mask_ld + s] = s < seq ? s_l[0][e >> 6][e & 63] : -INFINITY;
        }
    if (nb % 16 == 0 && ((uintptr_t)(mrow + s0) % 16) == 0) {
        for (int c = tid; 16 * c < nb; c += NT) {
            u32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t w = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) w |= (decide(16 * c + 4 * q + k) ? 1u : 0u) << (8 * k);
                v[q] = w;
            }
            *(u32x4 *)(mrow + s0 + 16 * c) = v;
        }
    } else {
        for (int e = tid; e < nb; e += NT) mrow[s0 + e] = decide(e) ? 1 : 0;
    }
}

// fp32 keys: one thread per entry, fp32 VALU arithmetic; NH heads.
template <int NH>
__global__ __launch_bounds__(256) void mask_f32_kernel(MaskArgs A) {
    __shared__ float qs[NH * kDim];
    __shared__ float wsm[NH];
    const int b = blockIdx.y;
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t seq = A.kv.seq_lens[b];
    const float inv_n = 1.0f / (float)A.n_layers;
    float u = A.mean_mode ? 0.f : -INFINITY;
    for (int l = 0; l < A.n_layers; ++l) {
        __syncthreads();
        const float *qrow = (const float *)A.q[l].q + (int64_t)b * NH * kDim;
        for (int i = threadIdx.x; i < NH * kDim; i += blockDim.x) qs[i] = qrow[i];
        for (int i = threadIdx.x; i < NH; i += blockDim.x)
            wsm[i] = A.q[l].w_bf16 ? bf16f(((const uint16_t *)A.q[l].w)[(int64_t)b * NH + i])
                                   : ((const float *)A.q[l].w)[(int64_t)b * NH + i];
        __syncthreads();
        if (s >= seq || s >= A.mask_ld) continue;
        int64_t lp = s / kPage;
        int phys = lp < A.kv.bt_ld ? A.kv.bt[(int64_t)b * A.kv.bt_ld + lp] : -1;
        float L;
        if (phys < 0 || phys >= A.kv.n_phys) {
            L = __builtin_nanf("");
        } else {
            const float *k = (const float *)A.kv.pool[l] + ((int64_t)phys * kPage + s % kPage) * kDim;
            float kr[kDim];
#pragma unroll
            for (int d = 0; d < kDim; ++d) kr[d] = k[d];
            L = 0.f;
            for (int h = 0; h < NH; ++h) {
                float x = 0.f;
#pragma unroll
                for (int d = 0; d < kDim; ++d) x = fmaf(qs[h * kDim + d], kr[d], x);
                L = fmaf(wsm[h], fmaxf(x, 0.f), L);
            }
        }
        u = A.mean_mode ? u + inv_n / (1.0f + expf(-L))
                        : ((L != L || u != u) ? __builtin_nanf("") : fmaxf(u, L));
    }
    if (s >= A.mask_ld) return;
    bool valid = s < seq;
    bool m = valid && (u >= A.cut || s < A.n_sink || s >= seq - A.n_recent);
    A.mask[(int64_t)b * A.mask_ld + s] = m ? 1 : 0;
    if (A.union_score) A.union_score[(int64_t)b * A.mask_ld + s] = valid ? u : -INFINITY;
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_score(const ScoreArgs &a, int key_fmt, int q_fmt, hipStream_t s) {
    dim3 grid((unsigned)((a.n_slots + 4 * a.ppw - 1) / (4 * a.ppw)), (unsigned)a.q.T);
    if (key_fmt == KEY_BF16 && q_fmt == Q_BF16) {
        if (FM_BF16_RING)
            score_bf16_ring_kernel<FM_BF16_RING ? FM_BF16_RING : 4><<<grid, 256, 0, s>>>(a);
        else
            score_kernel<KEY_BF16, Q_BF16><<<grid, 256, 0, s>>>(a);
    }
    else if (key_fmt == KEY_FP8 && q_fmt == Q_BF16 && a.q.n_heads == 128)
        score_f8_kernel<FM_F8_RING, 4><<<grid, 256, 0, s>>>(a);
    else if (key_fmt == KEY_FP8 && q_fmt == Q_BF16)
        score_f8_kernel<FM_F8_RING, 2><<<grid, 256, 0, s>>>(a);
    else if (key_fmt == KEY_FP8 && q_fmt == Q_FP8)
        score_kernel<KEY_FP8, Q_FP8><<<grid, 256, 0, s>>>(a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

#ifndef FM_FUSE_F8_WAVES
#define FM_FUSE_F8_WAVES 12   // fp8 fused scoring: waves a workgroup (3 a SIMD)
#endif
FuseShape fuse_shape(int key_fmt, int q_fmt, int n_heads) {
    if (key_fmt == KEY_BF16 && q_fmt == Q_BF16 && n_heads == kHeads)
        return FuseShape{16, FM_BF16_RING ? FM_BF16_RING : 4, kMaxPpw};
    if (key_fmt == KEY_FP8 && q_fmt == Q_BF16 && n_heads == kHeads)
        return FuseShape{FM_FUSE_F8_WAVES, 4, kF8FuseMaxPpw};
    return FuseShape{0, 1, 1};                       // no fused kernel for this format
}

hipError_t launch_score_topk(const ScoreArgs &a, const FuseArgs &f, int key_fmt, int q_fmt,
                             hipStream_t s) {
    const unsigned grid = (unsigned)(f.n_chunks * ((a.q.T + 7) / 8 * 8));
    if (key_fmt == KEY_BF16 && q_fmt == Q_BF16 && a.q.n_heads == kHeads) {
        constexpr int NW = 16;
        score_topk_bf16_kernel<FM_BF16_RING ? FM_BF16_RING : 4, NW>
            <<<grid, 64 * NW, (size_t)NW * f.ppw_pad * 64 * 4, s>>>(a, f);
    } else if (key_fmt == KEY_FP8 && q_fmt == Q_BF16 && a.q.n_heads == kHeads) {
        // rows longer than 16 slots a wave (Mode A's 4,096-page rows) take their own
        // instantiation, so the shorter rows' kernel keeps its registers
        constexpr int NW = FM_FUSE_F8_WAVES;
        if (f.ppw_pad <= kMaxPpw)
            score_topk_f8_kernel<FM_F8_RING, NW, kMaxPpw><<<grid, 64 * NW, (size_t)NW * f.ppw_pad * 64 * 4, s>>>(a, f);
        else
            score_topk_f8_kernel<FM_F8_RING, NW, kF8FuseMaxPpw><<<grid, 64 * NW, (size_t)NW * f.ppw_pad * 64 * 4, s>>>(a, f);
    } else {
        return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    merge_chunks_kernel<1024, kFuseMaxCand / 1024><<<(unsigned)a.q.T, 1024, 0, s>>>(f);
    return hipGetLastError();
}

hipError_t launch_score_f32(const ScoreArgs &a, hipStream_t s) {
    dim3 grid((unsigned)((a.n_slots * kPage + 255) / 256), (unsigned)a.q.T);
    if (a.q.n_heads == 128)
        score_f32_kernel<128><<<grid, 256, 0, s>>>(a);
    else
        score_f32_kernel<kHeads><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_mask(const MaskArgs &a0, int key_fmt, int B, hipStream_t s) {
    constexpr int PPW = 16;
    MaskArgs a = a0;
    // fp8 layers-per-wave kernel: spread the pages over FM_MASK_RESIDENT waves, at most
    // kMaskPpw pages a wave
    const int64_t total = a.n_pages * (int64_t)B;
    a.ppw = (int)std::min<int64_t>(kMaskPpw, std::max<int64_t>(1, (total + FM_MASK_RESIDENT - 1) / FM_MASK_RESIDENT));
    if (key_fmt == KEY_F32) {
        dim3 grid((unsigned)((a.mask_ld + 255) / 256), (unsigned)B);
        if (a.q[0].n_heads == 128)
            mask_f32_kernel<128><<<grid, 256, 0, s>>>(a);
        else
            mask_f32_kernel<kHeads><<<grid, 256, 0, s>>>(a);
    } else if (key_fmt == KEY_FP8 && a.q[0].n_heads == 128) {
        dim3 grid((unsigned)((a.n_pages + 4 * a.ppw - 1) / (4 * a.ppw)), (unsigned)B);
        if (a.n_layers == 1) mask_f8_kernel<1, 4><<<grid, 256, 0, s>>>(a);
        else if (a.n_layers == 2) mask_f8_kernel<2, 4><<<grid, 256, 0, s>>>(a);
        else if (a.n_layers == 3) mask_f8_kernel<3, 4><<<grid, 256, 0, s>>>(a);
        else mask_f8_kernel<4, 4><<<grid, 256, 0, s>>>(a);
    } else if (key_fmt == KEY_FP8 && a.shared_keys && a.n_layers >= 2) {
        // one pool for every encoder: workgroups of n_layers waves, each key tile read once
        a.ppw = (int)std::min<int64_t>(FM_SHARED_PPW, std::max<int64_t>(1, (total + FM_SHARED_WG - 1) / FM_SHARED_WG));
        dim3 grid((unsigned)((a.n_pages + a.ppw - 1) / a.ppw), (unsigned)B);
        if (a.n_layers == 2) mask_f8_shared_kernel<2><<<grid, 128, 0, s>>>(a);
        else if (a.n_layers == 3) mask_f8_shared_kernel<3><<<grid, 192, 0, s>>>(a);
        else mask_f8_shared_kernel<4><<<grid, 256, 0, s>>>(a);
    } else if (key_fmt == KEY_FP8 && FM_MASK_F8) {
        dim3 grid((unsigned)((a.n_pages + 4 * a.ppw - 1) / (4 * a.ppw)), (unsigned)B);
        if (a.n_layers == 1) mask_f8_kernel<1, 2><<<grid, 256, 0, s>>>(a);
        else if (a.n_layers == 2) mask_f8_kernel<2, 2><<<grid, 256, 0, s>>>(a);
        else if (a.n_layers == 3) mask_f8_kernel<3, 2><<<grid, 256, 0, s>>>(a);
        else mask_f8_kernel<4, 2><<<grid, 256, 0, s>>>(a);
    } else {
        dim3 grid((unsigned)((a.n_pages + PPW - 1) / PPW), (unsigned)B);
        const unsigned threads = 64u * (unsigned)a.n_layers;
        if (key_fmt == KEY_BF16)
            mask_kernel<KEY_BF16, PPW><<<grid, threads, 0, s>>>(a);
        else
            mask_kernel<KEY_FP8, PPW><<<grid, threads, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace fm
