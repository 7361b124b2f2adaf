// labels.hip -- golden labels for training the retriever, built from the future native
// selector's scores (FlashMemory-DeepSeek-V4 paper summary, section 4, label construction):
//   P[i,l,:] = softmax of S[i,l,:] over token i's candidates;
//   M[i,l]   = the candidates sorted by score (descending, lower entry first) up to the last one
//              whose cumulative mass is at most p;
//   V[i,s]   = the number of layers whose nucleus holds s;  A[i] = {s : V[i,s] >= min_votes};
//   Y[t]     = the union of A[i] over the lookahead window i = t .. t + tau - 1, as CSR.
//
// Three steps (the last one four kernels):
//   nucleus_kernel  one workgroup per (token, layer) row holds the row in registers and finds
//                   the nucleus boundary exactly: softmax masses in 2^-44 fixed point summed
//                   as integers (so the sums, and with them every decision, are independent of
//                   the summation order), a mass histogram over linear score bins to find the
//                   boundary bin, then the boundary score among that bin's scores (gathered in
//                   LDS): by one wave comparing every pair when they are at most 64, else by a
//                   32-bit radix search.  Equal scores at the boundary are taken by lower entry.
//                   Membership goes out as one bit per entry.  The kernel is bound by vector
//                   instruction issue (a wave64 instruction takes four cycles), so every pass
//                   over the row is branch-free or skips its rare work behind one compare.
//   golden_kernel   votes across layers, one thread per 32-entry word (bit-sliced counts):
//                   the golden bits A[i].
//   window kernels  prefix and suffix ORs of the golden words within blocks of tau tokens;
//                   per (window t, 256-word chunk): the window's OR from one suffix and one
//                   prefix and its count, an exclusive scan of the counts into label_ptr and
//                   chunk positions, then the ascending indices with their scores, the
//                   fraction of the window's tokens whose golden set holds the entry.
#include <float.h>
#include <math.h>

#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kNucNT = 1024;                 // threads of a nucleus row
constexpr int kNucVec = kLabelMaxLd / (4 * kNucNT);   // float4 blocks a thread
constexpr int kNucBins = 2048;
constexpr float kNucSpan = 32.0f;            // linear bins over scores in [max - 32, max]
constexpr int kWinNT = 256;                  // threads of a window kernel

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

template <class U>
__device__ __forceinline__ U wave_incl_scan_t(U x) {
    const int ln = __lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const U y = __shfl_up(x, o);
        if (ln >= o) x += y;
    }
    return x;
}

// exclusive prefix sum over the NT threads of the block; sh holds NT / 64 + 1 values
template <class U, int NT>
__device__ U block_excl_scan_t(U x, U *sh, U &total) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, ln = __lane_id();
    const U inc = wave_incl_scan_t<U>(x);
    if (ln == 63) sh[w] = inc;
    __syncthreads();
    if (w == 0) {
        const U v = ln < NW ? sh[ln] : (U)0;
        const U vi = wave_incl_scan_t<U>(v);
        if (ln < NW) sh[ln] = vi - v;
        if (ln == NW - 1) sh[NW] = vi;
    }
    __syncthreads();
    const U res = sh[w] + inc - x;
    total = sh[NW];
    __syncthreads();
    return res;
}

// order-preserving key of a score: a larger score has a larger key; -0 and +0 are one key
__device__ __forceinline__ uint32_t score_key(float x) {
    const uint32_t u = __float_as_uint(x == 0.f ? 0.f : x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr float kLog2e = 1.44269504088896341f;
constexpr float kBinsPerUnit = (float)kNucBins / kNucSpan;
constexpr int kNucList = 4096;               // boundary-bin entries gathered in LDS, at most

// Per-row constants: the row maximum mx, and cb placing x = mx - kNucSpan at bin 0.
struct RowConst {
    float mx, cb;
};

// Softmax masses in fixed point: exp(x - mx) in units of 2^-44, rounded to nearest.  The
// exponential's argument (x - mx) log2(e) is small for the heavy entries, so its rounding
// costs them about 2^-23 |x - mx| relative; the fixed-point rounding adds at most 2^-45 of the
// largest mass per entry.  A mass is at most 2^44 and a row at most 2^16 entries, so the
// 64-bit sums cannot overflow.
constexpr int kMassBits = 44;

__device__ __forceinline__ u64 mass_fx(float x, const RowConst &k) {
    const float m = __builtin_amdgcn_exp2f((x - k.mx) * kLog2e);
    return (u64)__builtin_rintf(__builtin_ldexpf(m, kMassBits));
}

// linear bin of a score over [mx - kNucSpan, mx]: monotone in x, so every score of a higher
// bin is larger than every score of a lower one
__device__ __forceinline__ int score_bin(float x, const RowConst &k) {
    const int b = (int)fmaf(x, kBinsPerUnit, k.cb);
    return b < 0 ? 0 : (b > kNucBins - 1 ? kNucBins - 1 : b);
}

// the score of an order-preserving key (score_key's inverse)
__device__ __forceinline__ float key_score(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// the largest float below a finite x: y > float_below(x) exactly when y >= x, for every non-NaN
// y (-0 and +0 count as equal)
__device__ __forceinline__ float float_below(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) == 0u) return -__uint_as_float(1u);     // below +-0: -(smallest denormal)
    return __uint_as_float((u & 0x80000000u) ? u + 1u : u - 1u);
}

// The row's registers pass through an empty asm statement before each sweep over them, so the
// compiler cannot keep per-entry results (keys, bins, masses) of one sweep alive for the next:
// 64 values a thread already fill half the registers.
template <int VEC>
__device__ __forceinline__ void opaque_row(float (&v)[VEC][4]) {
#pragma unroll
    for (int u = 0; u < VEC; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(v[u][c]));
}

struct NucLds {
    u64 hm[kNucBins];                   // mass per bin
    uint32_t hc[kNucBins];              // entries per bin (radix passes)
    float lx[kNucList];                 // scores of the boundary bin
    u64 sh64[kNucNT / 64 + 1];
    uint32_t sh32[kNucNT / 64 + 1];
    float shf[kNucNT / 64];
    u64 m64[2];
    uint32_t m32[2];
    uint32_t list_n;
};

// Bins [0, nb) are walked from the top (largest scores first): find the bin where the running
// mass, starting at 0, first exceeds `room`; its index goes to m32[0] and the mass of the bins
// above it to m64[0].  The caller guarantees that the bins' total exceeds room.
template <int NT>
__device__ void find_boundary_bin(NucLds &L, int nb, u64 room) {
    const int tid = threadIdx.x;
    constexpr int BPT = kNucBins / NT;
    const int top = nb - 1 - BPT * tid;
    u64 h[BPT], sum = 0;
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        h[k] = top - k >= 0 ? L.hm[top - k] : 0ull;
        sum += h[k];
    }
    u64 total;
    u64 above = block_excl_scan_t<u64, NT>(sum, L.sh64, total);
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        if (above <= room && room < above + h[k]) {
            L.m32[0] = (uint32_t)(top - k);
            L.m64[0] = above;
        }
        above += h[k];
    }
    __syncthreads();
}

// OR of x over each group of eight neighbouring lanes (every lane of the group gets it): two
// quad permutations and a mirror within each half row, all on the DPP path
__device__ __forceinline__ uint32_t or8(uint32_t x) {
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // lanes ^ 1
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // lanes ^ 2
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);  // 7 - lane
    return x;
}

__global__ __launch_bounds__(kNucNT) void nucleus_kernel(LabelArgs A) {
    constexpr int NT = kNucNT, NW = NT / 64, VEC = kNucVec;
    __shared__ NucLds L;
    const int l = blockIdx.x, i = blockIdx.y, tid = threadIdx.x, ln = __lane_id(), w = tid >> 6;
    const float *row = A.scores + ((int64_t)i * A.n_layers + l) * A.ld;
    uint32_t *mout = A.mbits + ((int64_t)i * A.n_layers + l) * A.words;
    int n = A.n_valid ? A.n_valid[i] : (int)A.ld;
    n = n < 0 ? 0 : (n > (int)A.ld ? (int)A.ld : n);
    for (int b = tid; b < kNucBins; b += NT) L.hm[b] = 0ull;
    if (tid == 0) L.list_n = 0u;

    // the row, every load issued before any is used; entries past n, -inf and NaN are not
    // candidates (-inf here)
    float v[VEC][4];
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)row, (short)0, n * 4, 0x00020000);
    {
        f32x4 raw[VEC];
#pragma unroll
        for (int u = 0; u < VEC; ++u)
            raw[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rs, (uint32_t)(4 * (u * NT + tid)) * 4u, 0, 0));
#pragma unroll
        for (int u = 0; u < VEC; ++u) {
            const int j = 4 * (u * NT + tid);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float x = raw[u][c];
                v[u][c] = ((j + c < n) & (x == x)) ? x : -INFINITY;
            }
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < VEC; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) mx = fmaxf(mx, v[u][c]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (ln == 0) L.shf[w] = mx;
    __syncthreads();
    mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < NW; ++k) mx = fmaxf(mx, L.shf[k]);
    if (mx == -INFINITY) {                      // no candidate: an empty nucleus
        for (int wd = tid; wd < A.words; wd += NT) mout[wd] = 0u;
        return;
    }
    const RowConst K{mx, (kNucSpan - mx) * kBinsPerUnit};

    // masses, their total and the mass histogram over linear score bins, branch-free: a
    // non-candidate's mass is exp2(-inf) = 0 and adds nothing to the bin it lands in
    u64 zt = 0;
#pragma unroll
    for (int u = 0; u < VEC; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float x = v[u][c];
            const u64 q = mass_fx(x, K);
            zt += q;
            atomicAdd(&L.hm[score_bin(x, K)], q);
        }
    u64 Z;
    (void)block_excl_scan_t<u64, NT>(zt, L.sh64, Z);   // also orders the histogram's atomics
    // room for the members: cumulative mass <= p Z, in the same fixed point
    const u64 room = (u64)((double)A.p * (double)Z);
    const bool all = room >= Z;                 // p = 1 (or above): every candidate
    float xstar = INFINITY;
    uint32_t r = 0u, g = 0u;
    if (!all) {
        find_boundary_bin<NT>(L, kNucBins, room);
        const int b1 = (int)L.m32[0];
        u64 above = L.m64[0];
        // the boundary bin's scores, gathered in LDS (few: the bins are narrow).  A score of
        // bin b1 is at least the bin's lower edge; one compare against the edge less a bin
        // (far wider than the rounding of the bin arithmetic for scores below 2^13) skips the
        // bin arithmetic for nearly every entry.
        const float xe = (b1 > 0 && fabsf(mx) < 8192.f) ? mx - kNucSpan + (float)(b1 - 1) / kBinsPerUnit
                                                         : -FLT_MAX;
        opaque_row<VEC>(v);
#pragma unroll
        for (int u = 0; u < VEC; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float x = v[u][c];
                if (x >= xe) {
                    if ((x > -INFINITY) & (score_bin(x, K) == b1)) {
                        const uint32_t e = atomicAdd(&L.list_n, 1u);
                        if (e < (uint32_t)kNucList) L.lx[e] = x;
                    }
                }
            }
        __syncthreads();
        const uint32_t nlist = (uint32_t)__builtin_amdgcn_readfirstlane((int)L.list_n);
        bool resolved = false;
        if (nlist <= 64u) {
            // One wave, a gathered score a lane: the mass of larger scores and of equal ones
            // (exact sums), and the lane whose score holds the boundary: gt <= room - above
            // < gt + eq.  Its score is the boundary score, every entry of it weighs eq / cnt.
            if (w == 0) {
                const bool has = (uint32_t)ln < nlist;
                const float x = has ? L.lx[ln] : -INFINITY;
                const uint32_t key = has ? score_key(x) : 0u;
                const u64 q = has ? mass_fx(x, K) : 0ull;
                u64 gt = 0, eq = 0;
                uint32_t cnt = 0;
                for (int j = 0; j < (int)nlist; ++j) {
                    const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)key, j);
                    const u64 qj = ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(q >> 32), j) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)q, j);
                    gt += kj > key ? qj : 0ull;
                    eq += kj == key ? qj : 0ull;
                    cnt += kj == key ? 1u : 0u;
                }
                const u64 rp = room - above;
                const uint64_t bm = __ballot(has && gt <= rp && rp < gt + eq);
                if (ln == 0) L.m32[1] = bm ? 1u : 0u;
                if (bm && ln == __ffsll((long long)bm) - 1) {
                    // r = floor((rp - gt) / (eq / cnt)) of the cnt equal entries, below cnt as
                    // rp - gt < eq; a single entry (the usual case) leaves r = 0
                    uint32_t rr = 0u;
                    if (cnt > 1u) {
                        const u64 wq = eq / cnt;
                        const u64 q = (rp - gt) / (wq ? wq : 1ull);
                        rr = (uint32_t)(q < (u64)cnt ? q : (u64)cnt);
                    }
                    L.m32[0] = key;
                    L.hc[0] = cnt;
                    L.hc[1] = rr;
                }
            }
            __syncthreads();
            if (L.m32[1]) {
                resolved = true;
                xstar = key_score(L.m32[0]);
                g = L.hc[0];
                r = L.hc[1];
            }
            __syncthreads();                    // L.m32 / L.hc are read before reuse
        }
        if (!resolved) {
            // the exact boundary score inside bin b1: radix over the 32-bit key, 11 + 11 + 10
            // bits, over the gathered scores (or, if the bin overflowed the list, over the row
            // in memory)
            uint32_t prefix = 0u, pmask = 0u, dig = 0u;
            auto radix_pass = [&](int pass, auto &&sweep) {
                const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
                const int nb = pass == 2 ? 1024 : 2048;
                for (int b = tid; b < kNucBins; b += NT) {
                    L.hm[b] = 0ull;
                    L.hc[b] = 0u;
                }
                __syncthreads();
                sweep([&](float x) {
                    const uint32_t key = score_key(x);
                    if ((key & pmask) == prefix) {
                        const uint32_t d = (key >> shift) & (uint32_t)(nb - 1);
                        atomicAdd(&L.hm[d], mass_fx(x, K));
                        atomicAdd(&L.hc[d], 1u);
                    }
                });
                __syncthreads();
                find_boundary_bin<NT>(L, nb, room - above);
                dig = L.m32[0];
                above += L.m64[0];
                prefix |= dig << shift;
                pmask |= (uint32_t)(nb - 1) << shift;
            };
            if (nlist <= (uint32_t)kNucList) {
#pragma unroll 1
                for (int pass = 0; pass < 3; ++pass)
                    radix_pass(pass, [&](auto &&add) {
                        for (uint32_t e = tid; e < nlist; e += NT) add(L.lx[e]);
                    });
            } else {
#pragma unroll 1
                for (int pass = 0; pass < 3; ++pass)
                    radix_pass(pass, [&](auto &&add) {
                        // the row again from memory (the bin overflowed the list: many equal or
                        // nearly equal scores), so the registers stay as they are
                        for (int j = 4 * tid; j < n; j += 4 * NT) {
                            const f32x4 x4 = __builtin_bit_cast(
                                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)j * 4u, 0, 0));
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                const float x = x4[c];
                                if (j + c < n && x == x && x > -INFINITY && score_bin(x, K) == b1) add(x);
                            }
                        }
                    });
            }
            // every entry of the boundary score has the same mass wq; r of its g entries are
            // members
            xstar = key_score(prefix);
            g = L.hc[dig];
            const u64 wq = g ? L.hm[dig] / g : 1ull;   // g > 0 and wq > 0: the bin holds the boundary
            const u64 rr = (room - above) / (wq ? wq : 1ull);
            r = (uint32_t)(rr < (u64)g ? rr : (u64)g);
            __syncthreads();                    // L.hc / L.hm are read before anything reuses them
        }
    }

    // membership bits: score > xstar, or score == xstar among the first r of those by entry
    // index (lower entries first).  Entry 4 (u NT + tid) + c is bit 4 (tid % 8) + c of word
    // (u NT + tid) / 8: eight neighbouring lanes assemble a word.
    const bool split = !all && r > 0u && r < g;  // workgroup-uniform
    const bool take_eq = all || r == g;
    opaque_row<VEC>(v);
    if (!split) {
        // one compare an entry: x > thr, with thr = -inf (every candidate), the float below
        // xstar (ties taken) or xstar
        const float thr = all ? -INFINITY : (take_eq ? float_below(xstar) : xstar);
#pragma unroll
        for (int u = 0; u < VEC; ++u) {
            uint32_t nib = 0u;
#pragma unroll
            for (int c = 0; c < 4; ++c) nib |= (v[u][c] > thr ? 1u : 0u) << c;
            const uint32_t word = or8(nib << (4 * (tid & 7)));
            const int wd = (u * NT + tid) >> 3;
            if ((tid & 7) == 0 && wd < A.words) mout[wd] = word;
        }
        return;
    }
    uint32_t run = 0u;                          // boundary entries in earlier slabs
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
        uint32_t nib = 0u, eq_mask = 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float x = v[u][c];
            nib |= (x > xstar ? 1u : 0u) << c;
            eq_mask |= (x == xstar ? 1u : 0u) << c;
        }
        uint32_t tot;
        const uint32_t before = run + block_excl_scan_t<uint32_t, NT>((uint32_t)__popc(eq_mask), L.sh32, tot);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if ((eq_mask >> c) & 1u) {
                const uint32_t rank = before + (uint32_t)__popc(eq_mask & ((1u << c) - 1u));
                nib |= (rank < r ? 1u : 0u) << c;
            }
        run += tot;
        const uint32_t word = or8(nib << (4 * (tid & 7)));
        const int wd = (u * NT + tid) >> 3;
        if ((tid & 7) == 0 && wd < A.words) mout[wd] = word;
    }
}

// votes of token blockIdx.y across layers, one thread per 32-entry word.  The 32 entries' vote
// counts are kept as seven bit planes (at most 64 layers): a layer's word enters through a
// ripple of half adders, and count >= min_votes is the absence of a borrow out of
// count - min_votes, taken plane by plane.
__global__ __launch_bounds__(256) void golden_kernel(LabelArgs A) {
    const int wd = blockIdx.x * 256 + threadIdx.x, i = blockIdx.y;
    if (wd >= A.words) return;
    const uint32_t *m = A.mbits + (int64_t)i * A.n_layers * A.words + wd;
    uint32_t c[7] = {0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll 8
    for (int l = 0; l < A.n_layers; ++l) {
        uint32_t carry = m[(int64_t)l * A.words];
#pragma unroll
        for (int q = 0; q < 7; ++q) {
            const uint32_t t = c[q] & carry;
            c[q] ^= carry;
            carry = t;
        }
    }
    uint32_t gw = 0u;
    if (A.min_votes < 128) {
        uint32_t borrow = 0u;
#pragma unroll
        for (int q = 0; q < 7; ++q) {
            const uint32_t mb = ((A.min_votes >> q) & 1) ? ~0u : 0u;
            borrow = (~c[q] & (mb | borrow)) | (mb & borrow);
        }
        gw = ~borrow;
    }
    A.gbits[(int64_t)i * A.words + wd] = gw;
}

// Prefix and suffix ORs of the golden words within blocks of tau consecutive tokens (block b
// is tokens b tau .. b tau + tau - 1, the last one possibly shorter): P[i] = OR of the block's
// tokens up to i, S[i] = OR of its tokens from i.  Thread: one word of one block.
__global__ __launch_bounds__(256) void window_ps_kernel(LabelArgs A) {
    const int wd = blockIdx.x * 256 + threadIdx.x, blk = blockIdx.y;
    if (wd >= A.words) return;
    const int i0 = blk * A.tau, i1 = min(A.T, i0 + A.tau);
    const uint32_t *g = A.gbits + wd;
    // sixteen tokens' words are loaded before any of their ORs is stored (the stores could
    // alias the loads as far as the compiler knows)
    constexpr int kB = 16;
    uint32_t x = 0u;
    for (int b0 = i0; b0 < i1; b0 += kB) {
        uint32_t v[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) v[u] = b0 + u < i1 ? g[(int64_t)(b0 + u) * A.words] : 0u;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            x |= v[u];
            if (b0 + u < i1) A.pbits[(int64_t)(b0 + u) * A.words + wd] = x;
        }
    }
    x = 0u;
    for (int b1 = i1; b1 > i0; b1 -= kB) {
        uint32_t v[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) v[u] = b1 - 1 - u >= i0 ? g[(int64_t)(b1 - 1 - u) * A.words] : 0u;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            x |= v[u];
            if (b1 - 1 - u >= i0) A.sbits[(int64_t)(b1 - 1 - u) * A.words + wd] = x;
        }
    }
}

// Window t = blockIdx.x, words [256 c, 256 c + 256) with c = blockIdx.y: the label words (the
// OR of the window's tau golden words) to the workspace, and their label count.  Tokens t ..
// t + tau - 1 span the end of t's block and the start of the next, so the OR is S[t] |
// P[t + tau - 1] (both S[t] when t starts a block).
__global__ __launch_bounds__(kWinNT) void window_or_kernel(LabelArgs A) {
    __shared__ uint32_t sh[kWinNT / 64 + 1];
    const int t = blockIdx.x, c = blockIdx.y, wd = c * kWinNT + (int)threadIdx.x;
    uint32_t y = 0u;
    if (wd < A.words) {
        y = A.sbits[(int64_t)t * A.words + wd] | A.pbits[(int64_t)(t + A.tau - 1) * A.words + wd];
        A.ybits[(int64_t)t * A.words + wd] = y;
    }
    uint32_t tot;
    (void)block_excl_scan_t<uint32_t, kWinNT>((uint32_t)__popc(y), sh, tot);
    if (threadIdx.x == 0) A.counts[(int64_t)t * A.chunks + c] = (int32_t)tot;
}

// exclusive prefix sum of the (window, chunk) counts in window-major order (one workgroup):
// the chunks' first positions, and label_ptr
__global__ __launch_bounds__(1024) void window_scan_kernel(LabelArgs A) {
    __shared__ uint32_t sh[1024 / 64 + 1];
    const int windows = A.T - A.tau + 1;
    const int64_t n = (int64_t)windows * A.chunks;
    uint32_t carry = 0u;
    for (int64_t b = 0; b < n; b += 1024) {
        const int64_t e = b + threadIdx.x;
        uint32_t tot;
        const uint32_t ex = block_excl_scan_t<uint32_t, 1024>(e < n ? (uint32_t)A.counts[e] : 0u, sh, tot);
        if (e < n) {
            A.counts[e] = (int32_t)(carry + ex);
            if (e % A.chunks == 0) A.label_ptr[e / A.chunks] = (int32_t)(carry + ex);
        }
        carry += tot;
    }
    if (threadIdx.x == 0) A.label_ptr[windows] = (int32_t)carry;
}

// window t = blockIdx.x, chunk c = blockIdx.y: the chunk's labels in ascending entry order
// (thread order is word order), each with the fraction of the window's tokens whose golden set
// holds it.  Positions at or past cap are not written.
__global__ __launch_bounds__(kWinNT) void window_write_kernel(LabelArgs A) {
    __shared__ uint32_t sh[kWinNT / 64 + 1];
    const int t = blockIdx.x, c = blockIdx.y, wd = c * kWinNT + (int)threadIdx.x;
    const uint32_t y = wd < A.words ? A.ybits[(int64_t)t * A.words + wd] : 0u;
    uint32_t tot;
    int64_t pos = (int64_t)A.counts[(int64_t)t * A.chunks + c] +
                  block_excl_scan_t<uint32_t, kWinNT>((uint32_t)__popc(y), sh, tot);
    const uint32_t *gb = A.gbits + (int64_t)t * A.words + wd;
    uint32_t bits = y;
    while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1u;
        if (pos < A.cap) {
            A.label_idx[pos] = 32 * wd + b;
            if (A.label_score) {
                int hits = 0;
#pragma unroll 16
                for (int k = 0; k < A.tau; ++k) hits += (gb[(int64_t)k * A.words] >> b) & 1u;
                A.label_score[pos] = (float)hits / (float)A.tau;
            }
        }
        ++pos;
    }
}

}  // namespace

size_t labels_ws_bytes(int T, int n_layers, int64_t ld, int tau) {
    const size_t words = (size_t)((ld + 31) / 32), windows = (size_t)(T - tau + 1);
    const size_t chunks = (words + kWinNT - 1) / kWinNT;
    return align_up((size_t)T * n_layers * words * 4, 256) + 3 * align_up((size_t)T * words * 4, 256) +
           align_up(windows * words * 4, 256) + align_up(windows * chunks * 4, 256);
}

void labels_ws_carve(LabelArgs &a, void *ws) {
    uint8_t *p = (uint8_t *)ws;
    const size_t words = (size_t)a.words, windows = (size_t)(a.T - a.tau + 1);
    a.chunks = (int)((words + kWinNT - 1) / kWinNT);
    a.mbits = (uint32_t *)p;
    p += align_up((size_t)a.T * a.n_layers * words * 4, 256);
    a.gbits = (uint32_t *)p;
    p += align_up((size_t)a.T * words * 4, 256);
    a.pbits = (uint32_t *)p;
    p += align_up((size_t)a.T * words * 4, 256);
    a.sbits = (uint32_t *)p;
    p += align_up((size_t)a.T * words * 4, 256);
    a.ybits = (uint32_t *)p;
    p += align_up(windows * words * 4, 256);
    a.counts = (int32_t *)p;
}

hipError_t launch_labels(const LabelArgs &a, hipStream_t s) {
    nucleus_kernel<<<dim3((unsigned)a.n_layers, (unsigned)a.T), dim3(kNucNT), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    golden_kernel<<<dim3((unsigned)((a.words + 255) / 256), (unsigned)a.T), dim3(256), 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    window_ps_kernel<<<dim3((unsigned)((a.words + 255) / 256), (unsigned)((a.T + a.tau - 1) / a.tau)), dim3(256), 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 wgrid((unsigned)(a.T - a.tau + 1), (unsigned)a.chunks);
    window_or_kernel<<<wgrid, dim3(kWinNT), 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    window_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    window_write_kernel<<<wgrid, dim3(kWinNT), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fm
