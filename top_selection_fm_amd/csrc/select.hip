// select.hip -- selection kernels for gfx950: per-row top-k and resident-page compaction.
//
// Top-k (paper summary, section 3: the native selector keeps the top-k inside the resident
// set; README "Two-level recall": non-resident logits are -inf before the native top-512;
// DeepSeek-V4 CSA page, section 8: with fewer than 512 entries every entry is kept).
// The order is "logit descending, then entry index ascending".  Each candidate gets a unique
// 64-bit key: the order-preserving uint32 image of its logit (-0 folded onto +0) above the
// bitwise complement of its entry index.  The k-th largest key is found by radix selection,
// six digits (11/11/10 bits of the logit word, then of the index word), most significant
// first, with an LDS histogram per digit.  A digit level stops early when the bin holding the
// k-th key contains exactly the number still needed: then every key whose decided prefix is
// >= the prefix found is selected.  Selected entries are gathered in LDS and bitonic-sorted by
// index, so the output is ascending and deterministic.  One 1024-thread workgroup per row.
//
// Compaction (README, page-granular recall): a page of 64 entries is resident when any entry
// of the mask is; a block-wide exclusive scan of the page flags yields the ascending list.
#include <math.h>

#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kWaves = kTopkThreads / 64;
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    const int ln = __lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (ln >= o) x += y;
    }
    return x;
}

// Exclusive prefix sum over the block (blockDim.x == kTopkThreads); `total` gets the sum.
__device__ uint32_t block_excl_scan(uint32_t x, uint32_t *sh, uint32_t &total) {
    const int w = threadIdx.x >> 6, ln = __lane_id();
    uint32_t inc = wave_incl_scan(x);
    if (ln == 63) sh[w] = inc;
    __syncthreads();
    if (w == 0) {
        uint32_t v = ln < kWaves ? sh[ln] : 0u;
        uint32_t vi = wave_incl_scan(v);
        if (ln < kWaves) sh[ln] = vi - v;
        if (ln == kWaves - 1) sh[kWaves] = vi;
    }
    __syncthreads();
    uint32_t res = sh[w] + inc - x;
    total = sh[kWaves];
    __syncthreads();
    return res;
}

__device__ __forceinline__ uint32_t ordered_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;   // -0.0 ties with +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs A) {
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t scan_sh[kWaves + 1];
    __shared__ int32_t sel_idx[FM_MAX_K];
    __shared__ float sel_val[FM_MAX_K];
    __shared__ uint32_t s_count, s_bin, s_above;

    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int b = A.row_req ? A.row_req[t] : (A.b_is_zero ? 0 : t);
    const bool b_ok = b >= 0 && b < A.B;
    const float *row = A.logits + (int64_t)t * A.ld;
    const int32_t *rp = A.res_pages ? A.res_pages + (int64_t)(b_ok ? b : 0) * A.res_ld : nullptr;
    const uint8_t *mrow = A.mask ? A.mask + (int64_t)(b_ok ? b : 0) * A.mask_ld : nullptr;
    int64_t n = b_ok ? A.ld : 0;
    if (rp && b_ok) n = min(n, (int64_t)A.n_res[b] * kPage);
    if (A.n_valid) n = min(n, (int64_t)A.n_valid[t]);
    if (n < 0) n = 0;

    auto entry = [&](int64_t j) -> int64_t { return rp ? (int64_t)rp[j >> 6] * kPage + (j & 63) : j; };
    auto candidate = [&](int64_t j, float &v) -> bool {
        v = row[j];
        if (!(v > -INFINITY)) return false;          // -inf and NaN are never candidates
        if (mrow && !mrow[entry(j)]) return false;
        return true;
    };

    uint32_t pre_hi = 0, msk_hi = 0, pre_lo = 0, msk_lo = 0;
    uint32_t remaining = (uint32_t)A.k;
    for (int level = 0; level < 6; ++level) {
        const int sub = level % 3;
        const int shift = sub == 0 ? 21 : sub == 1 ? 10 : 0;
        const int width = sub == 2 ? 10 : 11;
        const uint32_t dmask = ((1u << width) - 1u) << shift;
        for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0u;
        __syncthreads();
        for (int64_t j = tid; j < n; j += kTopkThreads) {
            float v;
            if (!candidate(j, v)) continue;
            uint32_t kh = ordered_key(v), kl = ~(uint32_t)entry(j);
            if ((kh & msk_hi) != pre_hi || (kl & msk_lo) != pre_lo) continue;
            uint32_t d = ((level < 3 ? kh : kl) & dmask) >> shift;
            atomicAdd(&hist[d], 1u);
        }
        __syncthreads();
        // thread tid owns bins hb = 2047 - 2 tid and hb - 1; the scan runs from the top bin down
        const uint32_t hb = kBins - 1 - 2 * tid;
        const uint32_t h_hi = hist[hb], h_lo = hist[hb - 1];
        uint32_t total;
        const uint32_t above = block_excl_scan(h_hi + h_lo, scan_sh, total);
        if (total <= remaining) break;                // fewer candidates than k: take them all
        if (above < remaining && remaining <= above + h_hi) {
            s_bin = hb;
            s_above = above;
        } else if (above + h_hi < remaining && remaining <= above + h_hi + h_lo) {
            s_bin = hb - 1;
            s_above = above + h_hi;
        }
        __syncthreads();
        const uint32_t bin = s_bin, cnt = hist[bin];
        remaining -= s_above;
        if (level < 3) {
            pre_hi |= bin << shift;
            msk_hi |= dmask;
        } else {
            pre_lo |= bin << shift;
            msk_lo |= dmask;
        }
        __syncthreads();
        if (cnt == remaining) break;                  // the whole bin is selected
    }

    // every candidate whose decided key prefix is >= the prefix found
    if (tid == 0) s_count = 0u;
    __syncthreads();
    const uint64_t P = ((uint64_t)pre_hi << 32) | pre_lo;
    const uint64_t M = ((uint64_t)msk_hi << 32) | msk_lo;
    for (int64_t j = tid; j < n; j += kTopkThreads) {
        float v;
        if (!candidate(j, v)) continue;
        const int64_t s = entry(j);
        const uint64_t key = ((uint64_t)ordered_key(v) << 32) | (uint32_t)~(uint32_t)s;
        if ((key & M) >= P) {
            uint32_t pos = atomicAdd(&s_count, 1u);
            if (pos < FM_MAX_K) {
                sel_idx[pos] = (int32_t)s;
                sel_val[pos] = v;
            }
        }
    }
    __syncthreads();
    const int cnt = (int)min(s_count, (uint32_t)A.k);
    int npow = 1;
    while (npow < cnt) npow <<= 1;
    for (int i = cnt + tid; i < npow; i += kTopkThreads) {
        sel_idx[i] = 0x7fffffff;
        sel_val[i] = -INFINITY;
    }
    __syncthreads();
    for (int size = 2; size <= npow; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (npow >> 1); i += kTopkThreads) {
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
    int32_t *oi = A.out_idx + (int64_t)t * A.k;
    float *ov = A.out_val ? A.out_val + (int64_t)t * A.k : nullptr;
    for (int i = tid; i < A.k; i += kTopkThreads) {
        oi[i] = i < cnt ? sel_idx[i] : -1;
        if (ov) ov[i] = i < cnt ? sel_val[i] : -INFINITY;
    }
}

// number of nonzero bytes of a 32-bit word
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
    x |= x >> 4;
    x |= x >> 2;
    x |= x >> 1;
    return __popc(x & 0x01010101u);
}

__global__ __launch_bounds__(kTopkThreads) void compact_kernel(CompactArgs A) {
    __shared__ uint32_t sh[kWaves + 1];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const uint8_t *mrow = A.mask + (int64_t)b * A.mask_ld;
    const bool wide = ((uintptr_t)mrow % 16 == 0);
    uint32_t running = 0;
    for (int64_t base = 0; base < A.n_pages; base += kTopkThreads) {
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
        const uint32_t pos = running + block_excl_scan(flag, sh, tot);
        if (flag && A.page_list && pos < A.page_list_ld)
            A.page_list[(int64_t)b * A.page_list_ld + pos] = (int32_t)p;
        running += tot;
    }
    if (tid == 0) A.page_count[b] = (int32_t)running;
    if (A.page_list)
        for (int64_t i = running + tid; i < A.page_list_ld; i += kTopkThreads)
            A.page_list[(int64_t)b * A.page_list_ld + i] = -1;
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    topk_kernel<<<dim3((unsigned)a.T), dim3(kTopkThreads), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs &a, int B, hipStream_t s) {
    compact_kernel<<<dim3((unsigned)B), dim3(kTopkThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fm
