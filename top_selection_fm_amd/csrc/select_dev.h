// select_dev.h -- device building blocks of exact top-k selection, shared by the selection
// kernels (select.hip) and the fused scoring + selection kernels (score.hip).
//
// The order is "value descending, then entry index ascending" (paper summary, section 3: the
// native selector keeps the top-k inside the resident set; the tie rule is not on the pages and
// is this library's: the lower entry wins).  Each candidate gets a unique 64-bit key: the
// order-preserving uint32 image of its value (-0 folded onto +0) above the bitwise complement
// of its entry index.
#pragma once

#include <math.h>

#include "fm_internal.h"

namespace fm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBins = 2048;
constexpr int kRowThreads = 1024;     // page compaction
constexpr int kTopkThreads = 512;
constexpr int kSample = 2048;         // sampled entries of a long row
constexpr int kLongSample = 8192;     // sampled entries of a row cut by its own kernel
constexpr int kBnd = 1024;            // boundary-bin capacity of the final selection
constexpr int kBuf = 4096;            // LDS candidate buffer

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

struct LdsBuf {     // candidates already filtered into LDS
    const float *v;
    const int32_t *e;
    int m;
    template <int NT, class F>
    __device__ void each(F f) const {
        for (int i = threadIdx.x; i < m; i += NT) f(v[i], (int64_t)e[i]);
    }
};

// Monotone linear binning of values over [lo, hi] into kBins bins (-1 below lo).
struct LinBins {
    float lo, inv_w;
    bool flat;
    __device__ int operator()(float v) const {
        if (v < lo) return -1;
        if (flat) return v > lo ? kBins - 1 : 0;
        const float x = (v - lo) * inv_w;
        return x >= (float)(kBins - 1) ? kBins - 1 : (int)x;
    }
};

struct Rule {
    uint64_t P, M;   // selected iff (key & M) >= P
};

// Radix selection of the k largest keys among the candidates of `src` (block of NT threads).
template <int NT, class Src>
__device__ Rule radix_rule(const Src &src, uint32_t k, uint32_t *hist, uint32_t *sh,
                           uint32_t *misc) {
    constexpr int BPT = (kBins + NT - 1) / NT;   // histogram bins a thread owns in the scan
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
            h[i] = top - i >= 0 ? hist[top - i] : 0u;     // bins below 0 hold nothing
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

template <int NT>
__device__ float block_reduce(float x, bool take_max, float *shf) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float y = __shfl_xor(x, o);
        x = take_max ? fmaxf(x, y) : fminf(x, y);
    }
    const int w = threadIdx.x >> 6;
    if (__lane_id() == 0) shf[w] = x;
    __syncthreads();
    x = shf[0];
    for (int i = 1; i < NT / 64; ++i) x = take_max ? fmaxf(x, shf[i]) : fminf(x, shf[i]);
    __syncthreads();
    return x;
}

// Final selection of the top-k among m buffered candidates (values bval, entries bent), written
// to the output row in ascending entry order.  One linear-bin histogram over the buffer's value
// range finds the bin holding the k-th largest value; the entries of higher bins are all
// selected, and the few in that bin are ranked exactly by the full key.  When that bin holds
// more than kBnd entries (many near-equal values) the radix selection takes over.
//
// have_range: [rlo, rhi] bounds the buffer's values (the caller knows them; skips a reduction).
// The output order: when every entry is below kOrderBits (small_entries), from a bitmap of the
// selected entries and prefix popcounts; otherwise from counts of smaller entries.  out_rp
// (small_entries only): the buffered indices are row positions of a resident-page row with an
// ascending page list, written out as entries out_rp[j / 64] * 64 + j % 64.
constexpr int kOrderBits = kBins * 32;
template <int NT>
__device__ void select_buffer(const float *bval, const int32_t *bent, int m, uint32_t k,
                              uint32_t *hist, uint32_t *sh, uint32_t *misc, float *shf,
                              int32_t *bnd, int32_t *sel_idx, float *sel_val, uint32_t *cnt2,
                              int32_t *oi, float *ov, int k_out, bool have_range = false,
                              float rlo = 0.f, float rhi = 0.f, bool small_entries = false,
                              const int32_t *out_rp = nullptr) {
    const int tid = threadIdx.x;
    if (tid == 0) {
        cnt2[0] = 0u;
        cnt2[1] = 0u;
    }
    if ((uint32_t)m <= k) {
        for (int i = tid; i < m; i += NT) {
            sel_idx[i] = bent[i];
            sel_val[i] = bval[i];
        }
        if (tid == 0) cnt2[0] = (uint32_t)m;
        __syncthreads();
    } else {
        float lo, hi;
        if (have_range) {
            lo = rlo;
            hi = rhi;
        } else {
            lo = INFINITY;
            hi = -INFINITY;
            for (int i = tid; i < m; i += NT) {
                lo = fminf(lo, bval[i]);
                hi = fmaxf(hi, bval[i]);
            }
            lo = block_reduce<NT>(lo, false, shf);
            hi = block_reduce<NT>(hi, true, shf);
        }
        LinBins bins{lo, 0.f, !(hi > lo)};
        bins.inv_w = bins.flat ? 0.f : (float)kBins / (hi - lo);
        for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < m; i += NT) atomicAdd(&hist[bins(bval[i])], 1u);
        __syncthreads();
        constexpr int BPT = (kBins + NT - 1) / NT;
        const int top = kBins - 1 - BPT * tid;
        uint32_t h[BPT], sum = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            h[i] = top - i >= 0 ? hist[top - i] : 0u;
            sum += h[i];
        }
        uint32_t total;
        uint32_t above = block_excl_scan<NT>(sum, sh, total);
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            if (above < k && k <= above + h[i]) {
                misc[0] = (uint32_t)(top - i);
                misc[1] = above;
            }
            above += h[i];
        }
        __syncthreads();
        const int bstar = (int)misc[0];
        const uint32_t need = k - misc[1];
        const uint32_t nb = hist[bstar];
        __syncthreads();            // every thread has nb before the radix path clears hist
        if (nb <= (uint32_t)kBnd) {
            for (int i = tid; i < m; i += NT) {
                const int b = bins(bval[i]);
                if (b > bstar) {
                    const uint32_t p = atomicAdd(&cnt2[0], 1u);
                    sel_idx[p] = bent[i];
                    sel_val[p] = bval[i];
                } else if (b == bstar) {
                    bnd[atomicAdd(&cnt2[1], 1u)] = i;
                }
            }
            __syncthreads();
            for (uint32_t a = tid; a < nb; a += NT) {
                const int ia = bnd[a];
                const uint64_t ka = full_key(bval[ia], bent[ia]);
                uint32_t rank = 0;
                for (uint32_t c = 0; c < nb; ++c) rank += full_key(bval[bnd[c]], bent[bnd[c]]) > ka;
                if (rank < need) {
                    const uint32_t p = atomicAdd(&cnt2[0], 1u);
                    sel_idx[p] = bent[ia];
                    sel_val[p] = bval[ia];
                }
            }
            __syncthreads();
        } else {
            const LdsBuf src{bval, bent, m};
            const Rule rule = radix_rule<NT>(src, k, hist, sh, misc);
            __syncthreads();
            gather<NT>(src, rule, sel_val, sel_idx, &cnt2[0], FM_MAX_K);
            __syncthreads();
        }
    }
    const int cnt = (int)min(cnt2[0], k);
    if constexpr (kBins % NT != 0) small_entries = false;   // the bitmap layout needs it
    if (small_entries) {
        // ascending entry order from a bitmap of the selected entries (kBins words, in hist)
        // and the prefix popcount of each word (16-bit, in bnd)
        static_assert(kBnd * 2 >= kBins, "bitmap layout");
        constexpr int WPT = kBins % NT == 0 ? kBins / NT : 1;
        __syncthreads();
        for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < cnt; i += NT) atomicOr(&hist[sel_idx[i] >> 5], 1u << (sel_idx[i] & 31));
        __syncthreads();
        uint32_t wd[WPT], c = 0;
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            wd[i] = hist[WPT * tid + i];
            c += (uint32_t)__popc(wd[i]);
        }
        uint32_t tot;
        uint32_t pre = block_excl_scan<NT>(c, sh, tot);
        uint16_t *pref = (uint16_t *)bnd;
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            pref[WPT * tid + i] = (uint16_t)pre;
            pre += (uint32_t)__popc(wd[i]);
        }
        __syncthreads();
        for (int i = tid; i < cnt; i += NT) {
            const int32_t e = sel_idx[i];
            const uint32_t wv = hist[e >> 5];
            const int pos = (int)pref[e >> 5] + __popc(wv & ((1u << (e & 31)) - 1u));
            oi[pos] = out_rp ? out_rp[e >> 6] * kPage + (e & 63) : e;
            if (ov) ov[pos] = sel_val[i];
        }
    } else {
        // ascending entry order: each selected entry's position is the number of smaller
        // entries (sel_idx padded to a multiple of 16 with INT32_MAX, read four at a time)
        const int cnt16 = (cnt + 15) & ~15;
        for (int i = cnt + tid; i < cnt16; i += NT) sel_idx[i] = 0x7fffffff;
        __syncthreads();
        for (int i = tid; i < cnt; i += NT) {
            const int32_t e = sel_idx[i];
            int pos = 0;
            for (int c = 0; c < cnt16; c += 16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int4 x = *(const int4 *)&sel_idx[c + 4 * q];
                    pos += (x.x < e) + (x.y < e) + (x.z < e) + (x.w < e);
                }
            }
            oi[pos] = e;
            if (ov) ov[pos] = sel_val[i];
        }
    }
    for (int i = cnt + tid; i < k_out; i += NT) {
        oi[i] = -1;
        if (ov) ov[i] = -INFINITY;
    }
}


}  // namespace
}  // namespace fm
