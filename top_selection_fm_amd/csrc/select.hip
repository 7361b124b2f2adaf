// select.hip -- selection kernels for gfx950: per-row top-k and resident-page compaction.
//
// Top-k (paper summary, section 3: the native selector keeps the top-k inside the resident
// set; README "Two-level recall": non-resident logits are -inf before the native top-512;
// DeepSeek-V4 CSA page, section 8: with fewer than 512 entries every entry is kept).
// The order is "logit descending, then entry index ascending".  Each candidate gets a unique
// 64-bit key: the order-preserving uint32 image of its logit (-0 folded onto +0) above the
// bitwise complement of its entry index.  The k-th largest key is found by radix selection,
// six digits (11/11/10 bits of the logit word, then of the index word), most significant
// first, with an LDS histogram per digit; a level stops early when the bin holding the k-th
// key contains exactly the number still needed.  The result is a rule "decided key prefix >=
// P", which selects exactly min(k, |C|) candidates.  Selected entries are gathered in LDS and
// bitonic-sorted by index, so the output is ascending and deterministic.
//
// Two paths:
//   * single pass (no workspace): one 1024-thread workgroup per row runs the digit passes
//     over the row in global memory;
//   * two stages (workspace): stage 1 cuts every row into 4,096-entry chunks, one 256-thread
//     workgroup per chunk stages its chunk in LDS and keeps the chunk's own top-k (every
//     element of the row's top-k is in the top-k of its chunk, so nothing is lost); stage 2
//     runs one workgroup per row over the <= ceil(n / 4096) * k survivors.
//
// Compaction (README, page-granular recall): a page of 64 entries is resident when any entry
// of the mask is; a block-wide exclusive scan of the page flags yields the ascending list.
#include <math.h>

#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kBins = 2048;
constexpr int kRowThreads = 1024;
constexpr int kChunkThreads = 256;

template <int NT>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    const int ln = __lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (ln >= o) x += y;
    }
    return x;
}

// Exclusive prefix sum over a block of NT threads; `total` gets the sum.  sh: NT/64 + 1 words.
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t x, uint32_t *sh, uint32_t &total) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, ln = __lane_id();
    uint32_t inc = wave_incl_scan<NT>(x);
    if (ln == 63) sh[w] = inc;
    __syncthreads();
    if (w == 0) {
        uint32_t v = ln < NW ? sh[ln] : 0u;
        uint32_t vi = wave_incl_scan<NT>(v);
        if (ln < NW) sh[ln] = vi - v;
        if (ln == NW - 1) sh[NW] = vi;
    }
    __syncthreads();
    uint32_t res = sh[w] + inc - x;
    total = sh[NW];
    __syncthreads();
    return res;
}

__device__ __forceinline__ uint32_t ordered_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;   // -0.0 ties with +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t full_key(float v, int64_t s) {
    return ((uint64_t)ordered_key(v) << 32) | (uint32_t)~(uint32_t)s;
}

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
    template <int NT, class F>
    __device__ void each(F f) const {
        for (int64_t j = threadIdx.x; j < n; j += NT) {
            const float v = row[j];
            if (!(v > -INFINITY)) continue;          // -inf and NaN are never candidates
            const int64_t s = entry(j);
            if (mrow && !mrow[s]) continue;
            f(v, s);
        }
    }
};

struct LdsChunk {  // a staged chunk: non-candidates already turned into NaN
    const float *v;
    const int32_t *e;
    int m;
    template <int NT, class F>
    __device__ void each(F f) const {
        for (int i = threadIdx.x; i < m; i += NT) {
            const float x = v[i];
            if (x > -INFINITY) f(x, (int64_t)e[i]);
        }
    }
};

struct ChunkList {  // stage-1 survivors of one row: n_chunks lists of up to k entries
    const float *V;
    const int32_t *E;
    const int32_t *C;
    int n_chunks, k;
    template <int NT, class F>
    __device__ void each(F f) const {
        for (int c = 0; c < n_chunks; ++c) {
            const int cnt = C[c];
            for (int i = threadIdx.x; i < cnt; i += NT) f(V[(int64_t)c * k + i], (int64_t)E[(int64_t)c * k + i]);
        }
    }
};

struct Rule {
    uint64_t P, M;   // selected iff (key & M) >= P
};

// Radix selection of the k largest keys among the candidates of `src` (block of NT threads).
template <int NT, class Src>
__device__ Rule radix_rule(const Src &src, uint32_t k, uint32_t *hist, uint32_t *sh,
                           uint32_t *misc) {
    constexpr int BPT = kBins / NT;   // histogram bins owned by each thread in the scan
    const int tid = threadIdx.x;
    uint32_t pre_hi = 0, msk_hi = 0, pre_lo = 0, msk_lo = 0;
    uint32_t remaining = k;
    for (int level = 0; level < 6; ++level) {
        const int sub = level % 3;
        const int shift = sub == 0 ? 21 : sub == 1 ? 10 : 0;
        const int width = sub == 2 ? 10 : 11;
        const uint32_t dmask = ((1u << width) - 1u) << shift;
        for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
        __syncthreads();
        src.template each<NT>([&](float v, int64_t s) {
            const uint32_t kh = ordered_key(v), kl = ~(uint32_t)s;
            if ((kh & msk_hi) != pre_hi || (kl & msk_lo) != pre_lo) return;
            atomicAdd(&hist[((level < 3 ? kh : kl) & dmask) >> shift], 1u);
        });
        __syncthreads();
        // thread tid owns bins top, top - 1, ..., top - BPT + 1; the scan runs from the top down
        const int top = kBins - 1 - BPT * tid;
        uint32_t h[BPT];
        uint32_t sum = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            h[i] = hist[top - i];
            sum += h[i];
        }
        uint32_t total;
        uint32_t above = block_excl_scan<NT>(sum, sh, total);
        if (total <= remaining) break;               // fewer candidates than needed: all
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            if (above < remaining && remaining <= above + h[i]) {
                misc[0] = (uint32_t)(top - i);
                misc[1] = above;
            }
            above += h[i];
        }
        __syncthreads();
        const uint32_t bin = misc[0], cnt = hist[bin];
        remaining -= misc[1];
        if (level < 3) {
            pre_hi |= bin << shift;
            msk_hi |= dmask;
        } else {
            pre_lo |= bin << shift;
            msk_lo |= dmask;
        }
        __syncthreads();
        if (cnt == remaining) break;                 // the whole bin is selected
    }
    return Rule{((uint64_t)pre_hi << 32) | pre_lo, ((uint64_t)msk_hi << 32) | msk_lo};
}

// Append every selected candidate to (val, idx) through an LDS counter (unordered).
template <int NT, class Src>
__device__ void gather(const Src &src, const Rule &rule, float *val, int32_t *idx,
                       uint32_t *counter, uint32_t cap) {
    src.template each<NT>([&](float v, int64_t s) {
        if ((full_key(v, s) & rule.M) >= rule.P) {
            const uint32_t pos = atomicAdd(counter, 1u);
            if (pos < cap) {
                val[pos] = v;
                idx[pos] = (int32_t)s;
            }
        }
    });
}

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
    R.rp = A.res_pages ? A.res_pages + (int64_t)(b_ok ? b : 0) * A.res_ld : nullptr;
    R.mrow = A.mask ? A.mask + (int64_t)(b_ok ? b : 0) * A.mask_ld : nullptr;
    int64_t n = b_ok ? A.ld : 0;
    if (R.rp && b_ok) n = min(n, (int64_t)A.n_res[b] * kPage);
    if (A.n_valid) n = min(n, (int64_t)A.n_valid[t]);
    R.n = n < 0 ? 0 : n;
    return R;
}

// ---------------------------------------------------------------- single pass
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(TopkArgs A) {
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t sh[kRowThreads / 64 + 1];
    __shared__ uint32_t misc[2];
    __shared__ uint32_t s_count;
    __shared__ int32_t sel_idx[FM_MAX_K];
    __shared__ float sel_val[FM_MAX_K];
    const int t = blockIdx.x;
    const RowSrc src = row_source(A, t);
    const Rule rule = radix_rule<kRowThreads>(src, (uint32_t)A.k, hist, sh, misc);
    if (threadIdx.x == 0) s_count = 0u;
    __syncthreads();
    gather<kRowThreads>(src, rule, sel_val, sel_idx, &s_count, FM_MAX_K);
    __syncthreads();
    sort_and_write<kRowThreads>(sel_idx, sel_val, (int)min(s_count, (uint32_t)A.k), A.k,
                                A.out_idx + (int64_t)t * A.k,
                                A.out_val ? A.out_val + (int64_t)t * A.k : nullptr);
}

// ---------------------------------------------------------------- two stages
__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(TopkArgs A, TopkWs W) {
    __shared__ float cv[kTopkChunk];
    __shared__ int32_t ce[kTopkChunk];
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t sh[kChunkThreads / 64 + 1];
    __shared__ uint32_t misc[2];
    __shared__ uint32_t s_count;
    const int c = blockIdx.x, t = blockIdx.y;
    const RowSrc R = row_source(A, t);
    const int64_t j0 = (int64_t)c * kTopkChunk;
    const int m = (int)max((int64_t)0, min((int64_t)kTopkChunk, R.n - j0));
    for (int i = threadIdx.x; i < m; i += kChunkThreads) {
        const int64_t j = j0 + i;
        float v = R.row[j];
        const int64_t s = R.entry(j);
        if (R.mrow && !R.mrow[s]) v = __builtin_nanf("");
        cv[i] = v;
        ce[i] = (int32_t)s;
    }
    __syncthreads();
    const LdsChunk src{cv, ce, m};
    const Rule rule = radix_rule<kChunkThreads>(src, (uint32_t)A.k, hist, sh, misc);
    if (threadIdx.x == 0) s_count = 0u;
    __syncthreads();
    const int64_t slot = (int64_t)t * W.n_chunks + c;
    gather<kChunkThreads>(src, rule, W.val + slot * A.k, W.idx + slot * A.k, &s_count,
                          (uint32_t)A.k);
    __syncthreads();
    if (threadIdx.x == 0) W.cnt[slot] = (int32_t)min(s_count, (uint32_t)A.k);
}

__global__ __launch_bounds__(kRowThreads) void topk_merge_kernel(TopkArgs A, TopkWs W) {
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t sh[kRowThreads / 64 + 1];
    __shared__ uint32_t misc[2];
    __shared__ uint32_t s_count;
    __shared__ int32_t sel_idx[FM_MAX_K];
    __shared__ float sel_val[FM_MAX_K];
    const int t = blockIdx.x;
    const int64_t base = (int64_t)t * W.n_chunks;
    const ChunkList src{W.val + base * A.k, W.idx + base * A.k, W.cnt + base, W.n_chunks, A.k};
    const Rule rule = radix_rule<kRowThreads>(src, (uint32_t)A.k, hist, sh, misc);
    if (threadIdx.x == 0) s_count = 0u;
    __syncthreads();
    gather<kRowThreads>(src, rule, sel_val, sel_idx, &s_count, FM_MAX_K);
    __syncthreads();
    sort_and_write<kRowThreads>(sel_idx, sel_val, (int)min(s_count, (uint32_t)A.k), A.k,
                                A.out_idx + (int64_t)t * A.k,
                                A.out_val ? A.out_val + (int64_t)t * A.k : nullptr);
}

// ---------------------------------------------------------------- page compaction
// number of nonzero bytes of a 32-bit word
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
    x |= x >> 4;
    x |= x >> 2;
    x |= x >> 1;
    return __popc(x & 0x01010101u);
}

__global__ __launch_bounds__(kRowThreads) void compact_kernel(CompactArgs A) {
    __shared__ uint32_t sh[kRowThreads / 64 + 1];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const uint8_t *mrow = A.mask + (int64_t)b * A.mask_ld;
    const bool wide = ((uintptr_t)mrow % 16 == 0);
    uint32_t running = 0;
    for (int64_t base = 0; base < A.n_pages; base += kRowThreads) {
        const int64_t p = base + tid;
        uint32_t dens = 0;
        if (p < A.n_pages) {
            const int64_t s0 = p * kPage, s1 = min(s0 + kPage, A.mask_ld);
            if (wide && s1 - s0 == kPage) {
                const uint4 *m4 = (const uint4 *)(mrow + s0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint4 v = m4[i];
                    dens += nonzero_bytes(v.x) + nonzero_bytes(v.y) + nonzero_bytes(v.z) +
                            nonzero_bytes(v.w);
                }
            } else {
                for (int64_t s = s0; s < s1; ++s) dens += mrow[s] != 0;
            }
            if (A.page_density) A.page_density[(int64_t)b * A.n_pages + p] = (int32_t)dens;
        }
        const uint32_t flag = dens > 0 ? 1u : 0u;
        uint32_t tot;
        const uint32_t pos = running + block_excl_scan<kRowThreads>(flag, sh, tot);
        if (flag && A.page_list && pos < A.page_list_ld)
            A.page_list[(int64_t)b * A.page_list_ld + pos] = (int32_t)p;
        running += tot;
    }
    if (tid == 0) A.page_count[b] = (int32_t)running;
    if (A.page_list)
        for (int64_t i = running + tid; i < A.page_list_ld; i += kRowThreads)
            A.page_list[(int64_t)b * A.page_list_ld + i] = -1;
}

}  // namespace

size_t topk_ws_bytes(int T, int64_t n) {
    if (T <= 0 || n <= 0) return 0;
    const int64_t chunks = (n + kTopkChunk - 1) / kTopkChunk;
    const size_t slots = (size_t)T * (size_t)chunks;
    return align_up(slots * kTopkWsK * sizeof(float), 256) +
           align_up(slots * kTopkWsK * sizeof(int32_t), 256) +
           align_up(slots * sizeof(int32_t), 256);
}

TopkWs topk_ws_carve(void *ws, int T, int64_t n) {
    const int64_t chunks = (n + kTopkChunk - 1) / kTopkChunk;
    const size_t slots = (size_t)T * (size_t)chunks;
    uint8_t *p = (uint8_t *)ws;
    TopkWs W;
    W.n_chunks = (int)chunks;
    W.val = (float *)p;
    p += align_up(slots * kTopkWsK * sizeof(float), 256);
    W.idx = (int32_t *)p;
    p += align_up(slots * kTopkWsK * sizeof(int32_t), 256);
    W.cnt = (int32_t *)p;
    return W;
}

hipError_t launch_topk(const TopkArgs &a, const TopkWs *ws, hipStream_t s) {
    if (ws && a.k <= kTopkWsK) {
        topk_chunk_kernel<<<dim3((unsigned)ws->n_chunks, (unsigned)a.T), dim3(kChunkThreads), 0, s>>>(a, *ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        topk_merge_kernel<<<dim3((unsigned)a.T), dim3(kRowThreads), 0, s>>>(a, *ws);
    } else {
        topk_row_kernel<<<dim3((unsigned)a.T), dim3(kRowThreads), 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs &a, int B, hipStream_t s) {
    compact_kernel<<<dim3((unsigned)B), dim3(kRowThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fm
