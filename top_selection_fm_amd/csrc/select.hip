// select.hip -- selection kernels for gfx950: per-row top-k and resident-page compaction.
//
// Top-k (paper summary, section 3: the native selector keeps the top-k inside the resident
// set; README "Two-level recall": non-resident logits are -inf before the native top-512;
// DeepSeek-V4 CSA page, section 8: with fewer than 512 entries every entry is kept).
// The order is "logit descending, then entry index ascending".  Each candidate gets a unique
// 64-bit key: the order-preserving uint32 image of its logit (-0 folded onto +0) above the
// bitwise complement of its entry index.  An exact radix selection finds the k-th largest
// key: six digits (11/11/10 bits of the logit word, then of the index word), most significant
// first, with an LDS histogram per digit; a level stops early when the bin holding the k-th
// key contains exactly the number still needed.  The result is a rule "decided key prefix >=
// P", which selects exactly min(k, |C|) candidates.  Selected entries are gathered in LDS and
// bitonic-sorted by index, so the output is ascending and deterministic.
//
// One workgroup per row.  Rows longer than the LDS candidate buffer are first cut down: a
// strided sample of 4,096 entries is binned linearly in value (2,048 bins over the sample's
// range), and the bin at which the sample's count from the top reaches about 1.3 k n / 4096
// becomes the cut.  One pass over the row appends every candidate whose bin is at or above the
// cut to the LDS buffer; the exact selection then runs on the buffer.  Binning is monotone in
// the value, so when at least k candidates pass, every member of the row's top-k passed too
// (a candidate in a lower bin has k larger ones above it) and the result is exact.  If fewer
// than k pass, or the buffer overflows, the exact selection runs over the whole row instead.
//
// Compaction (README, page-granular recall): a page of 64 entries is resident when any entry
// of the mask is; a block-wide exclusive scan of the page flags yields the ascending list.
#include <float.h>
#include <math.h>

#include "fm_internal.h"

#ifndef FM_TOPK_U
#define FM_TOPK_U 4
#endif
#ifndef FM_TOPK_ROW
#define FM_TOPK_ROW 1   // rows of up to 65,536 entries: single-pass row kernel
#endif
#ifndef FM_TOPK_NT
#define FM_TOPK_NT 1024  // threads of the single-pass row kernel
#endif
#ifndef FM_TOPK_SHORT_VEC
#define FM_TOPK_SHORT_VEC 17   // float4 blocks a thread of the 512-thread row kernel
#endif
#ifndef FM_TOPK_STAGE_MIN
#define FM_TOPK_STAGE_MIN 4096
#endif

#include "select_dev.h"

namespace fm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTopkLdsThreads = 1024; // largest workgroup sharing TopkLds

// ---------------------------------------------------------------- element sources
// each<NT>(f) calls f(value, entry) for every candidate this thread owns.

struct RowSrc {   // one row of a logit matrix (optionally through a resident-page map / mask)
    const float *row;
    int64_t n;
    const int32_t *rp;     // resident pages of the row's request (two-level), or null
    const uint8_t *mrow;   // mask row, or null
    __device__ int64_t entry(int64_t j) const {
        return rp ? (int64_t)rp[j >> 6] * kPage + (j & 63) : j;
    }
    __device__ bool cand(int64_t j, float &v, int64_t &s) const {
        v = row[j];
        if (!(v > -INFINITY)) return false;           // -inf and NaN are never candidates
        s = entry(j);
        return !(mrow && !mrow[s]);
    }
    template <int NT, class F>
    __device__ void each(F f) const {
        for (int64_t j0 = threadIdx.x; j0 < n; j0 += 4 * NT) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = (j0 + u * NT < n) ? row[j0 + u * NT] : -INFINITY;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (!(v[u] > -INFINITY)) continue;     // -inf and NaN are never candidates
                const int64_t s = entry(j0 + u * NT);
                if (mrow && !mrow[s]) continue;
                f(v[u], s);
            }
        }
    }
};

// Sort the cnt gathered entries by index (bitonic, in LDS) and write the output row.
template <int NT>
__device__ void sort_and_write(int32_t *sel_idx, float *sel_val, int cnt, int k, int32_t *oi,
                               float *ov) {
    const int tid = threadIdx.x;
    int npow = 1;
    while (npow < cnt) npow <<= 1;
    for (int i = cnt + tid; i < npow; i += NT) {
        sel_idx[i] = 0x7fffffff;
        sel_val[i] = -INFINITY;
    }
    __syncthreads();
    for (int size = 2; size <= npow; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (npow >> 1); i += NT) {
                const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
                const bool asc = (lo & size) == 0;
                const int32_t a = sel_idx[lo], c = sel_idx[hi];
                if ((a > c) == asc) {
                    sel_idx[lo] = c;
                    sel_idx[hi] = a;
                    const float x = sel_val[lo];
                    sel_val[lo] = sel_val[hi];
                    sel_val[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < k; i += NT) {
        oi[i] = i < cnt ? sel_idx[i] : -1;
        if (ov) ov[i] = i < cnt ? sel_val[i] : -INFINITY;
    }
}

__device__ RowSrc row_source(const TopkArgs &A, int t) {
    const int b = A.row_req ? A.row_req[t] : (A.b_is_zero ? 0 : t);
    const bool b_ok = b >= 0 && b < A.B;
    RowSrc R;
    R.row = A.logits + (int64_t)t * A.ld;
    R.rp = (A.res_pages && !A.res_cells) ? A.res_pages + (int64_t)(b_ok ? b : 0) * A.res_ld : nullptr;
    R.mrow = A.mask ? A.mask + (int64_t)(b_ok ? b : 0) * A.mask_ld : nullptr;
    int64_t n = b_ok ? A.ld : 0;
    if (A.res_pages && b_ok) n = min(n, (int64_t)A.n_res[b] * kPage);
    if (A.n_valid) n = min(n, (int64_t)A.n_valid[t]);
    R.n = n < 0 ? 0 : n;
    return R;
}

// ---------------------------------------------------------------- top-k kernel
// The cut of a row: candidates with bins(v) >= b pass.  b < 0 means "no cut" (all pass).
struct Cut {
    LinBins bins;
    int b;
};

// Sample position i (of M) of a row of n > kBuf entries: M / 16 runs of 16 contiguous entries
// spread evenly over the row (few cache lines, many pages).
template <int M>
__device__ __forceinline__ int64_t sample_pos(int i, int64_t n) {
    return (int64_t)(i >> 4) * n / (M / 16) + (i & 15);
}

// Cut of row R from its sample (block-uniform).  Aims at the sample's (2 k m / n + 16)-th
// largest value (m = sample size), i.e. about 2 k + 16 n / m candidates of the row passing:
// comfortably more than k, far fewer than the buffer holds.
template <int NT, int M>
__device__ Cut row_cut(const RowSrc &R, uint32_t k, float *sval, uint32_t *hist, uint32_t *sh,
                       uint32_t *misc, float *shf) {
    const int tid = threadIdx.x;
    Cut c;
    c.bins = LinBins{-INFINITY, 0.f, true};
    c.b = -1;
    if (R.n <= kBuf) return c;
    float lo = INFINITY, hi = -INFINITY;
    static_assert(M % NT == 0, "sample layout");
    constexpr int PER = M / NT;
    // every sampled value in flight at once, then every mask byte (read unconditionally)
    float sv[PER];
    int64_t se[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int64_t j = sample_pos<M>(tid + q * NT, R.n);
        sv[q] = R.row[j];
        se[q] = R.entry(j);
    }
    uint8_t sm[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) sm[q] = R.mrow ? R.mrow[se[q]] : (uint8_t)1;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const float v = sv[q];
        const bool ok = v > -INFINITY && sm[q] != 0;     // -inf and NaN are never candidates
        sval[tid + q * NT] = ok ? v : __builtin_nanf("");
        if (ok) {
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
        }
    }
    lo = block_reduce<NT>(lo, false, shf);
    hi = block_reduce<NT>(hi, true, shf);
    if (!(lo <= hi)) return c;                               // no sampled candidate
    const uint32_t r = 2u * (uint32_t)(((uint64_t)k * M + R.n - 1) / R.n) + 16u;
    LinBins bins{lo, 0.f, !(hi > lo)};
    bins.inv_w = bins.flat ? 0.f : (float)kBins / (hi - lo);
    for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < M; i += NT) {
        const float v = sval[i];
        if (v == v) atomicAdd(&hist[bins(v)], 1u);
    }
    __syncthreads();
    constexpr int BPT = kBins / NT;
    const int top = kBins - 1 - BPT * tid;
    uint32_t h[BPT], sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        h[i] = hist[top - i];
        sum += h[i];
    }
    uint32_t total;
    uint32_t above = block_excl_scan<NT>(sum, sh, total);
    if (total < r) return c;                                 // too few sampled to cut: all pass
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        if (above < r && r <= above + h[i]) misc[0] = (uint32_t)(top - i);
        above += h[i];
    }
    __syncthreads();
    c.bins = bins;
    c.b = (int)misc[0];
    __syncthreads();
    return c;
}

// Append the candidates of entries [j0, j1) that pass the cut to (bv, be), keeping the first
// `cap`; returns how many passed.  Each thread has 16 values in flight per step (four 16-byte
// loads; element j = base + 4 (u NT + tid) + c, so every load instruction covers 8 KB).
template <int NT>
__device__ uint32_t filter_range(const RowSrc &R, int64_t j0, int64_t j1, const Cut &cut,
                                 float *bv, int32_t *be, uint32_t cap, uint32_t *s_count) {
    const int tid = threadIdx.x, ln = __lane_id();
    if (tid == 0) *s_count = 0u;
    __syncthreads();
    const uint64_t lt = (ln == 0) ? 0ull : (~0ull >> (64 - ln));
    const bool vec = !R.rp && ((uintptr_t)(R.row + j0) % 16 == 0);
    constexpr int U = FM_TOPK_U;
    for (int64_t base = j0; base < j1; base += (int64_t)NT * U * 4) {
        float v[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base + 4 * ((int64_t)u * NT + tid);
            if (vec && j + 4 <= j1) {
                const float4 x = *(const float4 *)(R.row + j);
                v[u][0] = x.x; v[u][1] = x.y; v[u][2] = x.z; v[u][3] = x.w;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) v[u][c] = (j + c < j1) ? R.row[j + c] : -INFINITY;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t j = base + 4 * ((int64_t)u * NT + tid) + c;
                const float x = v[u][c];
                int64_t s = 0;
                bool hit = x > -INFINITY && cut.bins(x) >= cut.b;
                if (hit) {
                    s = R.entry(j);
                    hit = !(R.mrow && !R.mrow[s]);
                }
                const uint64_t mask = __ballot(hit);
                if (mask) {
                    const int leader = (int)__builtin_ctzll(mask);
                    uint32_t b0 = 0;
                    if (ln == leader) b0 = atomicAdd(s_count, (uint32_t)__popcll(mask));
                    b0 = __shfl(b0, leader);
                    const uint32_t pos = b0 + (uint32_t)__popcll(mask & lt);
                    if (hit && pos < cap) {
                        bv[pos] = x;
                        be[pos] = (int32_t)s;
                    }
                }
            }
    }
    __syncthreads();
    const uint32_t n = *s_count;
    __syncthreads();
    return n;
}

// Shared memory of a row cut and a chunk filter (the sample, the cut's histogram, reductions).
struct CutLds {
    float sample[kLongSample];
    uint32_t hist[kBins];
    uint32_t sh[kTopkThreads / 64 + 1];
    uint32_t misc[2];
    float shf[kTopkThreads / 64];
    uint32_t s_count;
};

// Shared memory of a final selection.  The cut's sample aliases bval, which is filled only
// after the cut is known.
struct TopkLds {
    float bval[kBuf];
    int32_t bent[kBuf];
    uint32_t hist[kBins];
    uint32_t sh[kTopkLdsThreads / 64 + 1];
    uint32_t misc[2];
    float shf[kTopkLdsThreads / 64];
    uint32_t s_count;
    alignas(16) int32_t sel_idx[FM_MAX_K];
    float sel_val[FM_MAX_K];
    int32_t bnd[kBnd];
    uint32_t cnt2[2];
    uint32_t offs[kTopkMaxChunks + 1];
};
static_assert(kSample <= kBuf, "the sample fits the candidate buffer");

// ---------------------------------------------------------------- single-pass row top-k
// Rows of up to 4 NT VEC entries: one workgroup of NT threads per row loads the whole row
// into registers at once (every load in flight together), takes the cut's sample from those
// registers (a few values a thread, spread over the row), keeps the candidates
// at or above the cut in the LDS buffer and selects exactly from it (select_buffer).  One read
// of the row, no workspace, no second launch.  When the cut does not hold (fewer than k pass,
// or more than the buffer holds) the exact radix selection runs over the row instead.
// Two shapes: 512 threads for rows of up to 34,816 entries, two rows a CU, so that one row's
// loads overlap the other's selection (4,096 rows of 33,792: 300 -> 181 us against one row a
// CU); 1,024 threads for rows of up to 65,536 entries.
constexpr int kRowNT = FM_TOPK_NT;
constexpr int kRowMax = 65536;
constexpr int kRowVec = kRowMax / (4 * kRowNT);
constexpr int kShortNT = 512;
constexpr int kShortVec = FM_TOPK_SHORT_VEC;
constexpr int kShortMax = 4 * kShortNT * kShortVec;

// WPE: waves a SIMD the registers are sized for (4: at most 128 VGPRs)
template <int NT, int VEC, int WPE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE)))
void topk_row_kernel(TopkArgs A) {
    constexpr int NW = NT / 64;
    constexpr int SPT = kSample / NT;               // sampled values a thread
    static_assert(SPT * NT == kSample && SPT <= 4, "sample layout");
    static_assert(NT <= kTopkLdsThreads, "TopkLds sized for the workgroup");
    __shared__ TopkLds L;
    __shared__ float s_max[NW];
    const int t = blockIdx.x, tid = threadIdx.x, ln = __lane_id(), w = tid >> 6;
    const RowSrc R = row_source(A, t);
    const int64_t n = R.n;
    const uint32_t k = (uint32_t)A.k;
    for (int i = tid; i < kBins; i += NT) L.hist[i] = 0u;   // ordered by the barriers below

    // the row, every non-candidate (-inf, NaN, masked, past n) as -inf.  Buffer loads bounded
    // by the row (4-byte alignment suffices; dwords past n read as 0 and are replaced)
    float v[VEC][4];
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)R.row, (short)0, (int)(n * 4), 0x00020000);
    const int n32 = (int)n;                           // n <= 4 NT VEC here
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
        const int j = 4 * (u * NT + tid);
        const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)j * 4u, 0, 0));
#pragma unroll
        for (int c = 0; c < 4; ++c) v[u][c] = (j + c < n32) ? x[c] : -INFINITY;
    }
    if (R.mrow) {
        // a masked row has no resident-page map (fm_topk512): mask byte j covers position j
        const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)R.mrow, (short)0, n32, 0x00020000);
#pragma unroll
        for (int u = 0; u < VEC; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t j = (uint32_t)(4 * (u * NT + tid) + c);
                if (!__builtin_amdgcn_raw_buffer_load_b8(mr, j, 0, 0)) v[u][c] = -INFINITY;
            }
    }

    // The cut: candidates x >= tau pass.  -FLT_MAX (no cut) passes every candidate and no -inf
    // or NaN.  For rows > kBuf the cut comes from a sample of SPT register values a thread,
    // v[(SPT tid + q) % un][q] (q < SPT), un the number of float4 blocks a thread holds that
    // reach into the row: the sample spreads over the row's entries only, whatever its length,
    // aiming at about 2 k + 16 n / kSample candidates passing.
    float tau = -FLT_MAX, smax = 0.f;
    if (n > kBuf) {
        float lo = INFINITY, hi = -INFINITY;
        const int un = min(VEC, (n32 + 4 * NT - 1) / (4 * NT));
        int uq = (int)((uint32_t)(SPT * tid) % (uint32_t)un);
#pragma unroll
        for (int q = 0; q < SPT; ++q, uq = uq + 1 == un ? 0 : uq + 1) {
            float sq = -INFINITY;
#pragma unroll
            for (int u = 0; u < VEC; ++u) sq = u == uq ? v[u][q] : sq;
            L.bval[q * NT + tid] = sq > -INFINITY ? sq : __builtin_nanf("");
            lo = sq > -INFINITY ? fminf(lo, sq) : lo;
            hi = fmaxf(hi, sq);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            lo = fminf(lo, __shfl_xor(lo, o));
            hi = fmaxf(hi, __shfl_xor(hi, o));
        }
        if (ln == 0) {
            L.shf[w] = lo;
            s_max[w] = hi;
        }
        __syncthreads();
        lo = INFINITY;
        hi = -INFINITY;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            lo = fminf(lo, L.shf[i]);
            hi = fmaxf(hi, s_max[i]);
        }
        const float width = hi - lo;
        if (lo <= hi && width < INFINITY) {           // some sampled candidate, a finite range
            const uint32_t r = 2u * (uint32_t)(((uint64_t)k * kSample + n - 1) / n) + 16u;
            LinBins bins{lo, 0.f, !(hi > lo)};
            bins.inv_w = bins.flat ? 0.f : (float)kBins / width;
#pragma unroll
            for (int q = 0; q < SPT; ++q) {
                const float x = L.bval[q * NT + tid];
                if (x == x) atomicAdd(&L.hist[bins(x)], 1u);
            }
            __syncthreads();
            constexpr int BPT = kBins / NT;
            const int top = kBins - 1 - BPT * tid;
            uint32_t h[BPT], sum = 0;
#pragma unroll
            for (int i = 0; i < BPT; ++i) {
                h[i] = L.hist[top - i];
                sum += h[i];
            }
            uint32_t total;
            uint32_t above = block_excl_scan<NT>(sum, L.sh, total);
            if (total >= r) {
#pragma unroll
                for (int i = 0; i < BPT; ++i) {
                    if (above < r && r <= above + h[i]) L.misc[0] = (uint32_t)(top - i);
                    above += h[i];
                }
                __syncthreads();
                // the lower edge of the cut bin; any threshold is exact once k candidates pass
                const float e = bins.flat ? lo : lo + (float)L.misc[0] * (width / (float)kBins);
                tau = e > -FLT_MAX ? e : -FLT_MAX;
                smax = hi;
            }
        }
    }

    // candidates x >= tau into the LDS buffer: a counting pass, one scan of the wave counts,
    // then a writing pass at exact positions (row positions first, turned into
    // entries afterwards, so a resident-page lookup never sits inside the loop)
    uint32_t wcount = 0;
#pragma unroll
    for (int u = 0; u < VEC; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) wcount += v[u][c] >= tau ? 1u : 0u;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wcount += __shfl_xor(wcount, o);
    __syncthreads();                                  // the sample's reads of sh are done
    if (ln == 0) L.sh[w] = wcount;
    __syncthreads();
    uint32_t base = 0, passed = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t ci = L.sh[i];
        base += i < w ? ci : 0u;
        passed += ci;
    }
    bool asc = false;

    if (passed <= (uint32_t)kBuf) {
        // a copy of tau the compiler cannot see through: the first pass's 64 compare masks
        // are not kept alive for this one
        float tw;
        asm volatile("v_mov_b32 %0, %1" : "=v"(tw) : "v"(tau));
        uint32_t run = base;
#pragma unroll
        for (int u = 0; u < VEC; ++u) {
            if (4 * u * NT >= n32) continue;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float x = v[u][c];
                const uint64_t m = __ballot(x >= tw);
                if (m) {
                    if (x >= tw) {
                        const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                        const uint32_t p = run + below;
                        L.bval[p] = x;
                        L.bent[p] = 4 * (u * NT + tid) + c;
                    }
                    run += (uint32_t)__popcll(m);
                }
            }
        }
        // a resident-page row whose page list is ascending: positions and entries are in the
        // same order, so the row is selected by position and mapped to entries when written
        if (R.rp) {
            const int npg = (n32 + kPage - 1) / kPage;
            int ok = 1;
            for (int i = tid; i + 1 < npg; i += NT) ok &= R.rp[i] < R.rp[i + 1] ? 1 : 0;
            asc = __syncthreads_and(ok) != 0;
        }
        if (R.rp && !asc) {
            // row positions to entries through the resident-page list, every lookup in flight
            constexpr int EPT = kBuf / NT;
            __syncthreads();
            int32_t pg[EPT];
#pragma unroll
            for (int q = 0; q < EPT; ++q) {
                const uint32_t i = q * NT + tid;
                pg[q] = i < passed ? R.rp[L.bent[i] >> 6] : 0;
            }
#pragma unroll
            for (int q = 0; q < EPT; ++q) {
                const uint32_t i = q * NT + tid;
                if (i < passed) L.bent[i] = pg[q] * kPage + (L.bent[i] & 63);
            }
        }
    }
    __syncthreads();

    int32_t *oi = A.out_idx + (int64_t)t * A.k;
    float *ov = A.out_val ? A.out_val + (int64_t)t * A.k : nullptr;
    if (passed <= (uint32_t)kBuf && !(tau > -FLT_MAX && passed < k)) {
        // bins over [tau, sample max]: every buffered value is >= tau, and the binning clamps
        // values above the sample's maximum into the top bin (monotone, so still exact)
        select_buffer<NT>(L.bval, L.bent, (int)passed, k, L.hist, L.sh, L.misc, L.shf, L.bnd,
                          L.sel_idx, L.sel_val, L.cnt2, oi, ov, A.k, tau > -FLT_MAX, tau, smax,
                          (!R.rp || asc) && n <= (int64_t)kOrderBits, asc ? R.rp : nullptr);
    } else {
        const Rule rule = radix_rule<NT>(R, k, L.hist, L.sh, L.misc);
        if (tid == 0) L.s_count = 0u;
        __syncthreads();
        gather<NT>(R, rule, L.sel_val, L.sel_idx, &L.s_count, FM_MAX_K);
        __syncthreads();
        sort_and_write<NT>(L.sel_idx, L.sel_val, (int)min(L.s_count, k), A.k, oi, ov);
    }
}

// Filter one kTopkChunk-entry chunk of row t into its workspace slot with the row's cut, which
// the cut kernel computed once for the row from its sample.
__device__ void filter_chunk(const TopkArgs &A, const TopkWs &W, const RowSrc &R, int c, int t,
                             uint32_t &s_count) {
    constexpr int NT = kTopkThreads;
    constexpr int U = kTopkChunk / (4 * NT);      // float4 loads a thread
    static_assert(U * 4 * NT == kTopkChunk, "chunk layout");
    const int tid = threadIdx.x, ln = __lane_id();
    const int64_t slot = (int64_t)t * W.n_chunks + c;
    // the chunk's values (4 U a thread) are requested first and stay in flight while the row's
    // cut is read (element j = j0 + 4 (u NT + tid) + e)
    const int64_t j0 = (int64_t)c * kTopkChunk, j1 = min(j0 + kTopkChunk, R.n);
    const bool vec = !R.rp && ((uintptr_t)(R.row + j0) % 16 == 0);
    float v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t j = j0 + 4 * ((int64_t)u * NT + tid);
        if (vec && j + 4 <= j1) {
            const float4 x = *(const float4 *)(R.row + j);
            v[u][0] = x.x; v[u][1] = x.y; v[u][2] = x.z; v[u][3] = x.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[u][e] = (j + e < j1) ? R.row[j + e] : -INFINITY;
        }
    }
    // a mask row without a page map: the chunk's mask bytes come with the values (bounded by the
    // row: bytes past n read as 0), so no hit waits on a dependent load
    const bool pre = R.mrow && !R.rp;
    uint8_t mb[U][4];
    if (pre) {
        const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)R.mrow, (short)0, (int)R.n, 0x00020000);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mb[u][e] = __builtin_amdgcn_raw_buffer_load_b8(
                    mr, (uint32_t)(j0 + 4 * ((int64_t)u * NT + tid) + e), 0, 0);
    }
    Cut cut;
    {
        const float4 cw = W.cut[t];
        cut.bins = LinBins{cw.x, cw.y, cw.z != 0.f};
        cut.b = __float_as_int(cw.w);
    }
    if (tid == 0) s_count = 0u;
    __syncthreads();
    float *bv = W.val + slot * kTopkCap;
    int32_t *be = W.idx + slot * kTopkCap;
    const uint64_t lt = (ln == 0) ? 0ull : (~0ull >> (64 - ln));
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t j = j0 + 4 * ((int64_t)u * NT + tid) + e;
            const float x = v[u][e];
            int64_t sidx = 0;
            bool hit = x > -INFINITY && cut.bins(x) >= cut.b;
            if (hit) {
                sidx = R.entry(j);
                hit = pre ? mb[u][e] != 0 : !(R.mrow && !R.mrow[sidx]);
            }
            const uint64_t mask = __ballot(hit);
            if (mask) {
                const int leader = (int)__builtin_ctzll(mask);
                uint32_t b0 = 0;
                if (ln == leader) b0 = atomicAdd(&s_count, (uint32_t)__popcll(mask));
                b0 = __shfl(b0, leader);
                const uint32_t pos = b0 + (uint32_t)__popcll(mask & lt);
                if (hit && pos < (uint32_t)kTopkCap) {
                    bv[pos] = x;
                    be[pos] = (int32_t)sidx;
                }
            }
        }
    __syncthreads();
    if (tid == 0) W.cnt[slot] = cut.b < 0 ? (int32_t)(kTopkCap + 1) : (int32_t)s_count;
}

// The stage-1 survivors of a row in the workspace, chunk c's at slot base + c (offs in LDS: chunk
// c holds survivors offs[c] .. offs[c + 1] - 1 of the row).
struct WsSrc {
    const float *val;
    const int32_t *idx;
    const uint32_t *offs;
    int n_chunks;
    int64_t base;
    template <int NT, class F>
    __device__ void each(F f) const {
        const uint32_t total = offs[n_chunks];
        for (uint32_t g = threadIdx.x; g < total; g += NT) {
            int lo = 0, hi = n_chunks;                      // offs[lo] <= g < offs[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (offs[mid] <= g) lo = mid; else hi = mid;
            }
            const int64_t at = (base + lo) * kTopkCap + (g - offs[lo]);
            f(val[at], (int64_t)idx[at]);
        }
    }
};

// Final selection of row t.  With stage-1 survivors (staged) the buffer is filled from the
// workspace; otherwise the workgroup cuts and filters the row itself.  More survivors than the
// buffer holds (but at least k, none dropped) are selected exactly from the workspace; when the
// cut did not hold (fewer than k passed, or a chunk overflowed) the exact selection runs over the
// whole row.
__device__ void select_row(const TopkArgs &A, const TopkWs &W, bool staged, const RowSrc &R, int t,
                           TopkLds &L) {
    constexpr int NT = kTopkThreads;
    const int tid = threadIdx.x;
    const uint32_t k = (uint32_t)A.k;
    bool from_buf, from_ws = false;
    uint32_t total = 0;
    if (staged) {
        // survivors of the row's chunks: offsets first, then one round of loads
        const int64_t base = (int64_t)t * W.n_chunks;
        if (tid == 0) {
            uint32_t acc = 0, over = 0;
            for (int c = 0; c < W.n_chunks; ++c) {
                const uint32_t n = (uint32_t)W.cnt[base + c];
                L.offs[c] = acc;
                over |= n > (uint32_t)kTopkCap;
                acc += n;
            }
            L.offs[W.n_chunks] = acc;
            L.misc[0] = over;
        }
        __syncthreads();
        total = L.offs[W.n_chunks];
        from_buf = !L.misc[0] && total >= k && total <= (uint32_t)kBuf;
        from_ws = !L.misc[0] && total > (uint32_t)kBuf;
        __syncthreads();
        if (from_buf) {
            constexpr int U = kBuf / NT;
            float xv[U];
            int32_t xe[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t g = tid + u * NT;
                if (g < total) {
                    int lo = 0, hi = W.n_chunks;            // offs[lo] <= g < offs[hi]
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (L.offs[mid] <= g) lo = mid; else hi = mid;
                    }
                    const int64_t at = (base + lo) * kTopkCap + (g - L.offs[lo]);
                    xv[u] = W.val[at];
                    xe[u] = W.idx[at];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t g = tid + u * NT;
                if (g < total) {
                    L.bval[g] = xv[u];
                    L.bent[g] = xe[u];
                }
            }
        }
        __syncthreads();
    } else {
        const Cut cut = row_cut<NT, kSample>(R, k, L.bval, L.hist, L.sh, L.misc, L.shf);
        total = filter_range<NT>(R, 0, R.n, cut, L.bval, L.bent, kBuf, &L.s_count);
        from_buf = total <= (uint32_t)kBuf && !(cut.b >= 0 && total < k);
    }

    int32_t *oi = A.out_idx + (int64_t)t * A.k;
    float *ov = A.out_val ? A.out_val + (int64_t)t * A.k : nullptr;
    if (from_buf) {
        select_buffer<NT>(L.bval, L.bent, (int)total, k, L.hist, L.sh, L.misc, L.shf, L.bnd,
                          L.sel_idx, L.sel_val, L.cnt2, oi, ov, A.k);
    } else if (from_ws) {
        const WsSrc S{W.val, W.idx, L.offs, W.n_chunks, (int64_t)t * W.n_chunks};
        const Rule rule = radix_rule<NT>(S, k, L.hist, L.sh, L.misc);
        if (tid == 0) L.s_count = 0u;
        __syncthreads();
        gather<NT>(S, rule, L.sel_val, L.sel_idx, &L.s_count, FM_MAX_K);
        __syncthreads();
        sort_and_write<NT>(L.sel_idx, L.sel_val, (int)min(L.s_count, k), A.k, oi, ov);
    } else {
        const Rule rule = radix_rule<NT>(R, k, L.hist, L.sh, L.misc);
        if (tid == 0) L.s_count = 0u;
        __syncthreads();
        gather<NT>(R, rule, L.sel_val, L.sel_idx, &L.s_count, FM_MAX_K);
        __syncthreads();
        sort_and_write<NT>(L.sel_idx, L.sel_val, (int)min(L.s_count, k), A.k, oi, ov);
    }
}

// Stage 0 of the workspace path: grid T, the cut of each long row from its sample, once.
__global__ __launch_bounds__(kTopkThreads) void topk_cut_kernel(TopkArgs A, TopkWs W) {
    __shared__ CutLds L;
    const int t = blockIdx.x;
    const RowSrc R = row_source(A, t);
    if (R.n <= kBuf) return;                 // short rows: stage 2 selects them directly
    const Cut c = row_cut<kTopkThreads, kLongSample>(R, (uint32_t)A.k, L.sample, L.hist, L.sh,
                                                     L.misc, L.shf);
    if (threadIdx.x == 0)
        W.cut[t] = make_float4(c.bins.lo, c.bins.inv_w, c.bins.flat ? 1.f : 0.f, __int_as_float(c.b));
}

// Stage 1 of the workspace path: grid (n_chunks, T), one workgroup per kTopkChunk-entry chunk
// of a long row.  A chunk past its row's end records no survivors.
__global__ __launch_bounds__(kTopkThreads) void topk_filter_kernel(TopkArgs A, TopkWs W) {
    __shared__ uint32_t s_count;
    const int c = blockIdx.x, t = blockIdx.y;
    const RowSrc R = row_source(A, t);
    if (R.n <= kBuf) return;                 // short rows: stage 2 selects them directly
    if ((int64_t)c * kTopkChunk >= R.n) {
        if (threadIdx.x == 0) W.cnt[(int64_t)t * W.n_chunks + c] = 0;
        return;
    }
    filter_chunk(A, W, R, c, t, s_count);
}

// Stage 2: one workgroup per row selects from the chunks' survivors (rows longer than kBuf
// with a workspace) or from the row itself.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs A, TopkWs W, int staged) {
    __shared__ TopkLds L;
    const int t = blockIdx.x;
    const RowSrc R = row_source(A, t);
    select_row(A, W, staged && R.n > kBuf, R, t, L);
}

// ---------------------------------------------------------------- page compaction
// number of nonzero bytes of a 32-bit word
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
    x |= x >> 4;
    x |= x >> 2;
    x |= x >> 1;
    return __popc(x & 0x01010101u);
}

// One workgroup per request, rounds of 4 kRowThreads pages.  The round's mask bytes are read
// coalesced (16-byte chunk i kRowThreads + tid of the round; four consecutive lanes share a
// page) with every load in flight at once, the per-page counts go to LDS, and thread t then
// takes pages 4 t .. 4 t + 3 for one block scan that places the resident pages in order.
__global__ __launch_bounds__(kRowThreads) void compact_kernel(CompactArgs A) {
    constexpr int PPT = 4;
    constexpr int RP = PPT * kRowThreads;                 // pages a round
    __shared__ uint32_t sh[kRowThreads / 64 + 1];
    __shared__ uint32_t s_d[RP];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const uint8_t *mrow = A.mask + (int64_t)b * A.mask_ld;
    const bool wide = ((uintptr_t)mrow % 16 == 0);
    uint32_t running = 0;
    for (int64_t base = 0; base < A.n_pages; base += RP) {
        const int np = (int)min((int64_t)RP, A.n_pages - base);
        if (A.dens_in) {
            // the scoring kernel's page densities (the list may be this same array: every
            // density of the round is read before the barriers of the scan below, and list
            // positions never pass the page they come from)
            for (int p = tid; p < np; p += kRowThreads)
                s_d[p] = (uint32_t)A.dens_in[(int64_t)b * A.dens_ld + base + p];
        } else if (wide && (base + np) * kPage <= A.mask_ld) {
            uint4 x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int q = i * kRowThreads + tid;          // chunk of the round
                x[i] = q < 4 * np ? ((const uint4 *)(mrow + base * kPage))[q] : uint4{0, 0, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t d = nonzero_bytes(x[i].x) + nonzero_bytes(x[i].y) + nonzero_bytes(x[i].z) +
                             nonzero_bytes(x[i].w);
                d += __shfl_xor(d, 1);
                d += __shfl_xor(d, 2);
                if ((tid & 3) == 0) s_d[(i * kRowThreads + tid) >> 2] = d;
            }
        } else {
            for (int p = tid; p < np; p += kRowThreads) {
                const int64_t s0 = (base + p) * kPage, s1 = min(s0 + kPage, A.mask_ld);
                uint32_t d = 0;
                for (int64_t s = s0; s < s1; ++s) d += mrow[s] != 0;
                s_d[p] = d;
            }
        }
        __syncthreads();
        uint32_t dens[PPT], cnt = 0;
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = PPT * tid + i;
            dens[i] = p < np ? s_d[p] : 0u;
            if (p < np && A.page_density && A.page_density != A.dens_in)
                A.page_density[(int64_t)b * A.n_pages + base + p] = (int32_t)dens[i];
            cnt += dens[i] > 0 ? 1u : 0u;
        }
        uint32_t tot;
        uint32_t pos = running + block_excl_scan<kRowThreads>(cnt, sh, tot);
        if (A.page_list) {
#pragma unroll
            for (int i = 0; i < PPT; ++i)
                if (dens[i] > 0) {
                    if (pos < A.page_list_ld) A.page_list[(int64_t)b * A.page_list_ld + pos] = (int32_t)(base + PPT * tid + i);
                    ++pos;
                }
        }
        running += tot;
    }
    if (tid == 0) A.page_count[b] = (int32_t)running;
    if (A.page_list)
        for (int64_t i = running + tid; i < A.page_list_ld; i += kRowThreads)
            A.page_list[(int64_t)b * A.page_list_ld + i] = -1;
}

// ---------------------------------------------------------------- densest pages
// One request's page densities as top-k candidates: page p with density d > 0 is a candidate
// of value d (exact in float for d <= 2^24); the radix selection ranks them by (d, lower p).
struct DensSrc {
    const int32_t *d;
    int64_t n;
    template <int NT, class F>
    __device__ void each(F f) const {
        for (int64_t p = threadIdx.x; p < n; p += NT) {
            const int32_t x = d[p];
            if (x > 0) f((float)x, p);
        }
    }
};

// One workgroup per request: the kmax densest pages, ascending page id, -1 padded.
__global__ __launch_bounds__(kRowNT) void densest_kernel(DensestArgs A) {
    constexpr int NT = kRowNT;
    __shared__ TopkLds L;
    const int b = blockIdx.x, tid = threadIdx.x;
    const DensSrc src{A.density + (int64_t)b * A.ld, A.n_pages};
    const Rule rule = radix_rule<NT>(src, (uint32_t)A.kmax, L.hist, L.sh, L.misc);
    if (tid == 0) L.s_count = 0u;
    __syncthreads();
    gather<NT>(src, rule, L.sel_val, L.sel_idx, &L.s_count, FM_MAX_K);
    __syncthreads();
    const int cnt = (int)min(L.s_count, (uint32_t)A.kmax);
    sort_and_write<NT>(L.sel_idx, L.sel_val, cnt, A.kmax, A.out_pages + (int64_t)b * A.kmax, nullptr);
    if (tid == 0 && A.out_count) A.out_count[b] = cnt;
}

}  // namespace

size_t topk_ws_bytes(int T, int64_t n) {
    if (T <= 0 || n <= FM_TOPK_STAGE_MIN || n <= (int64_t)kRowMax ||
        n > (int64_t)kTopkMaxChunks * kTopkChunk)
        return 0;
    const size_t slots = (size_t)T * (size_t)((n + kTopkChunk - 1) / kTopkChunk);
    return align_up(slots * kTopkCap * sizeof(float), 256) +
           align_up(slots * kTopkCap * sizeof(int32_t), 256) + align_up(slots * sizeof(int32_t), 256) +
           align_up((size_t)T * sizeof(float4), 256);
}

TopkWs topk_ws_carve(void *ws, int T, int64_t n) {
    const int64_t chunks = (n + kTopkChunk - 1) / kTopkChunk;
    const size_t slots = (size_t)T * (size_t)chunks;
    uint8_t *p = (uint8_t *)ws;
    TopkWs W;
    W.n_chunks = (int)chunks;
    W.val = (float *)p;
    p += align_up(slots * kTopkCap * sizeof(float), 256);
    W.idx = (int32_t *)p;
    p += align_up(slots * kTopkCap * sizeof(int32_t), 256);
    W.cnt = (int32_t *)p;
    p += align_up(slots * sizeof(int32_t), 256);
    W.cut = (float4 *)p;
    return W;
}

hipError_t launch_topk(const TopkArgs &a, const TopkWs *ws, hipStream_t s) {
    if (a.ld <= (int64_t)kShortMax && FM_TOPK_ROW) {
        topk_row_kernel<kShortNT, kShortVec, 4><<<dim3((unsigned)a.T), dim3(kShortNT), 0, s>>>(a);
        return hipGetLastError();
    }
    if (a.ld <= (int64_t)kRowMax && FM_TOPK_ROW) {
        topk_row_kernel<kRowNT, kRowVec, 4><<<dim3((unsigned)a.T), dim3(kRowNT), 0, s>>>(a);
        return hipGetLastError();
    }
    if (ws) {
        topk_cut_kernel<<<dim3((unsigned)a.T), dim3(kTopkThreads), 0, s>>>(a, *ws);
        const hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
        topk_filter_kernel<<<dim3((unsigned)ws->n_chunks, (unsigned)a.T), dim3(kTopkThreads), 0, s>>>(a, *ws);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    topk_kernel<<<dim3((unsigned)a.T), dim3(kTopkThreads), 0, s>>>(a, ws ? *ws : TopkWs{}, ws ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_densest(const DensestArgs &a, int B, hipStream_t s) {
    densest_kernel<<<dim3((unsigned)B), dim3(kRowNT), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs &a, int B, hipStream_t s) {
    compact_kernel<<<dim3((unsigned)B), dim3(kRowThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fm
