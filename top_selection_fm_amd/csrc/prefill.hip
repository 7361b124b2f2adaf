// prefill.hip -- index logits for many query rows of one request: fp8 queries x fp8 keys.
//
// L[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . k[s,:]) over 64 heads of dimension 128
// (FlashMemory-DeepSeek-V4 paper summary, section 3, the Memory-Indexer score; DeepSeek-V4 CSA
// page, section 3, formula CSA-1), with the causal cut s < floor(pos_t / ratio) (CSA page,
// section 10).  Prefill has thousands of rows over the same keys, so the work is a real dense
// contraction: it is tiled for operand reuse and runs on the fp8 MFMA.
//
// Tiling.  A workgroup (8 waves) owns 8 consecutive query rows, one per wave, and a chunk of
// key pages.  Each wave keeps the fp8 queries of its row in registers; the key pages stream
// through a ring of three LDS buffers (one page of 64 entries per step) and every key fragment
// read from LDS feeds 4 MFMAs.  A page's global loads go out two steps before it is scored.
// The workgroup's linear id is split as (chunk = id % n_chunks, row block = id / n_chunks):
// workgroups are dealt to the 8 XCDs round-robin, so with n_chunks a multiple of 8 each XCD
// only ever reads the key chunks that belong to it, and they stay in its L2.
//
// MFMA layout (v_mfma_scale_f32_16x16x128_f8f6f4, wave64).  Row i of fragment n of the A tile
// is head 16 n + i of the wave's query row, so the accumulator lane 16 g + j holds heads
// 16 n + 4 g + 0..3 for key entry j of a 16-entry block; the head sum is 16 in-lane terms per
// block, and one reduce-scatter over the four lane groups finishes a page's four blocks.  The K dimension (128 head dims) is split the same
// way for queries and keys (32 consecutive bytes per lane), so the dot products are exact
// whatever order the hardware walks K in.  The MFMAs of block u + 1 are issued between the
// epilogue steps of block u, across page boundaries too.
//
// Epilogue.  The MFMA's power-of-two block scale multiplies every dot product of E4M3 codes by
// 2^-e, with e chosen per query row from the largest exponent field E of the row's codes: a
// code is below 2^(E-6) in magnitude (2^-6 for E = 0), a key code at most 448 < 2^9, so
// |S| < 128 * 2^(E-6) * 2^9 = 2^(E+10) and e = max(E, 1) + 10 puts every dot product strictly
// inside (-1, 1) (e = 25 for codes that fill the E4M3 range).  Each pair of head results is
// rounded to f16 with the conversion's clamp to [0, 1] (packed), which on that range is exactly
// ReLU, and multiplied by the head weights with v_dot2c_f32_f16 into float accumulators: two
// VALU instructions per four head results.  The weights are scaled per row by a power of two
// into [2^14, 2^15) first, so a bf16 weight converts to f16 exactly.  The only rounding beyond
// float accumulation is the f16 rounding of each ReLU(S) term: relative 2^-11 for terms of at
// least 2^(e-14) code-product units, else absolute 2^(e-25) units (one unit for full-range
// query codes, 2^-10 units for codes below 1, as when q is passed unscaled).  The per-token
// query scale, the per-entry key scale and the powers of two are applied to the sum, which is
// valid because the scales are positive.
#include <math.h>

#include "fm_internal.h"

#ifndef FM_PF_WAVES
#define FM_PF_WAVES 8   // query rows (waves) of a workgroup
#endif

namespace fm {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kLdsRow = 144;                       // a key row's 128 codes, padded (bank spread)
constexpr int kMaxChunkPages = 128;                // pages of one workgroup's key chunk, at most
constexpr int kWaves = FM_PF_WAVES;                // one query row per wave
constexpr int kStageParts = 512 / (64 * kWaves);    // 16-byte parts of a page each thread stages
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ int row_request(const QArgs &q, const KvArgs &kv, int t) {
    const int b = q.row_req ? q.row_req[t] : (q.b_is_zero ? 0 : t);
    return (b >= 0 && b < kv.B) ? b : -1;
}

__device__ __forceinline__ int64_t n_visible(const QArgs &q, const KvArgs &kv, int t, int b) {
    if (b < 0) return 0;
    int64_t n = kv.seq_lens[b];
    if (q.q_pos) {
        const int64_t c = (int64_t)q.q_pos[t] / q.ratio;
        n = c < n ? c : n;
    }
    return n < 0 ? 0 : n;
}

// Physical page of logical page p of request 0, or -1 when it is not mapped.
__device__ __forceinline__ int page_phys(const KvArgs &kv, int64_t p) {
    if (p >= kv.bt_ld) return -1;
    const int phys = kv.bt[p];
    return (phys < 0 || phys >= kv.n_phys) ? -1 : phys;
}

// ReLU(f16(x)), x in (-1, 1): the clamp to [0, 1] folds into the conversion instruction
__device__ __forceinline__ h2 relu16(float a, float b) {
    const h2 x = __builtin_convertvector(f32x2{a, b}, h2);
    return __builtin_elementwise_min(__builtin_elementwise_max(x, h2{0, 0}), h2{1, 1});
}

// One fp8 accumulator tile of the epilogue: heads 16 n + 4 g + 0..3 of this lane's row.
__device__ __forceinline__ float epi_step(const f32x4 &c, h2 w01, h2 w23, float a) {
    a = __builtin_amdgcn_fdot2(relu16(c[0], c[1]), w01, a, false);
    return __builtin_amdgcn_fdot2(relu16(c[2], c[3]), w23, a, false);
}

// The four 16-entry blocks of a page as partial head sums p[u] (lane 16 g + j: heads 4 g + 0..3
// of each fragment, entry j of block u) become totals by one reduce-scatter over the four
// 16-lane rows: a 16-lane row swap and add leaves rows 0 + 1 and 2 + 3 of one block in the even
// rows and of the other in the odd rows, and a 32-lane swap and add then leaves block g's total
// (entry j) in row g.  Six instructions for the page.
__device__ __forceinline__ float block_totals(float p0, float p1, float p2, float p3) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
    const float q01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const float q23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(q01), __float_as_uint(q23), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void prefill_fp8_kernel(PrefillArgs A) {
    __shared__ __attribute__((aligned(16))) uint8_t s_codes[3][kPage * kLdsRow];
    __shared__ float s_scale[3][kPage];
    __shared__ int s_phys[kMaxChunkPages];

    const int tid = threadIdx.x, ln = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);                    // uniform
    const int j = ln & 15, g = ln >> 4;
    const int chunk = (int)(blockIdx.x % (unsigned)A.n_chunks);
    const int rblk = (int)(blockIdx.x / (unsigned)A.n_chunks);
    const int t0 = rblk * kWaves;
    const int T = A.q.T;

    int nv8 = 0;
    if (j < kWaves && t0 + j < T)
        nv8 = (int)n_visible(A.q, A.kv, t0 + j, row_request(A.q, A.kv, t0 + j));
    int tile_nvis = nv8;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) tile_nvis = max(tile_nvis, __shfl_xor(tile_nvis, o));
    const int t = t0 + wave;
    const bool row_ok = t < T;
    const int nvis_t = __shfl(nv8, wave);
    float *orow = A.out + (int64_t)(row_ok ? t : 0) * A.out_ld;

    // queries: fragment n, A row i = head 16 n + i, bytes 32 g .. 32 g + 31
    i32x8 qf[4];
    {
        const uint8_t *qb = (const uint8_t *)A.q.q + (int64_t)(row_ok ? t : 0) * kHeads * kDim;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const uint8_t *p = qb + (16 * n + j) * kDim + 32 * g;
            const u32x4 a = row_ok ? *(const u32x4 *)p : u32x4{0u, 0u, 0u, 0u};
            const u32x4 b = row_ok ? *(const u32x4 *)(p + 16) : u32x4{0u, 0u, 0u, 0u};
            qf[n] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                          (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
        }
    }
    // the row's largest exponent field sets the block scale 2^-sexp of its dot products
    int sexp;
    {
        uint32_t em = 0;
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const uint32_t x = (uint32_t)qf[n][v];
#pragma unroll
                for (int by = 0; by < 4; ++by) em = max(em, (x >> (8 * by + 3)) & 15u);
            }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) em = max(em, (uint32_t)__shfl_xor((int)em, o));
        sexp = __builtin_amdgcn_readfirstlane((int)max(em, 1u) + 10);
    }
    const int scale_a = 127 - sexp;                    // E8M0 block scale of the A operand
    // this lane's 16 head weights (heads 16 n + 4 g + 0..3) as f16 pairs scaled by 2^ew
    h2 wp[8];
    float row_factor;
    {
        const int64_t base = (int64_t)(row_ok ? t : 0) * kHeads + 4 * g;
        float wl[4][4];
        if (A.q.w_bf16) {
            const uint16_t *w16 = (const uint16_t *)A.q.w + base;
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int v = 0; v < 4; ++v) wl[n][v] = bf16f(w16[16 * n + v]);
        } else {
            const float *w32 = (const float *)A.q.w + base;
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int v = 0; v < 4; ++v) wl[n][v] = w32[16 * n + v];
        }
        float m = 0.f;
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int v = 0; v < 4; ++v) m = fmaxf(m, fabsf(wl[n][v]));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        int ex = 0;
        if (m > 0.f) (void)frexpf(m, &ex);
        const int ew = m > 0.f ? 15 - ex : 0;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            wp[2 * n] = __builtin_convertvector(f32x2{ldexpf(wl[n][0], ew), ldexpf(wl[n][1], ew)}, h2);
            wp[2 * n + 1] = __builtin_convertvector(f32x2{ldexpf(wl[n][2], ew), ldexpf(wl[n][3], ew)}, h2);
        }
        const float qs = row_ok ? A.q.q_scale[t] : 0.f;
        row_factor = ldexpf(qs, sexp - ew);
    }

    const int64_t p_begin = (int64_t)chunk * A.chunk_pages;
    const int64_t p_end = min(p_begin + A.chunk_pages, A.n_pages);
    const int64_t p_vis = min(p_end, ((int64_t)tile_nvis + kPage - 1) / kPage);
    for (int i = tid; i < A.chunk_pages; i += kThreads)
        s_phys[i] = p_begin + i < p_end ? page_phys(A.kv, p_begin + i) : -1;
    __syncthreads();

    // staging: thread tid carries entry tid / 8, code bytes 16 (tid % 8) .. + 15, and the scale,
    // through a buffer descriptor of the page (scalar setup, 32-bit offsets)
    // (kStageParts parts a thread: entries se + i kThreads / 8)
    const int se = tid >> 3, sp = tid & 7;
    const uint32_t soff = (uint32_t)(se * kRowFp8);
    u32x4 Rc[kStageParts];
    float Rs[kStageParts];
#pragma unroll
    for (int i = 0; i < kStageParts; ++i) {
        Rc[i] = u32x4{0u, 0u, 0u, 0u};
        Rs[i] = 0.f;
    }
    auto stage = [&](int64_t p) {
        const int64_t pc = min(p, p_vis - 1);
        const int phys = __builtin_amdgcn_readfirstlane(max(s_phys[pc - p_begin], 0));   // uniform
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(A.kv.pool[0] + (int64_t)phys * (kPage * kRowFp8)), (short)0, kPage * kRowFp8,
            0x00020000);
#pragma unroll
        for (int i = 0; i < kStageParts; ++i) {
            const uint32_t o = soff + (uint32_t)(i * (kThreads / 8) * kRowFp8);
            Rc[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, o + 16 * sp, 0, 0);
            Rs[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, o + kDim, 0, 0));
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kStageParts; ++i) {
            const int e = se + i * (kThreads / 8);
            *(u32x4 *)&s_codes[buf][e * kLdsRow + 16 * sp] = Rc[i];
            if (sp == 0) s_scale[buf][e] = Rs[i];
        }
    };
    auto kfrag = [&](int buf, int u) {
        const uint8_t *kp = s_codes[buf] + (16 * u + j) * kLdsRow + 32 * g;
        const u32x4 k0 = *(const u32x4 *)kp;
        const u32x4 k1 = *(const u32x4 *)(kp + 16);
        return i32x8{(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3],
                     (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
    };
    // the row's logits through a buffer descriptor: a store at or past out_ld is dropped
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)orow, (short)0, row_ok ? (int)(A.out_ld * 4) : 0, 0x00020000);
    const int out_ld32 = (int)A.out_ld;                  // out_ld * 4 < 2^31 (checked on the host)
    int pend_s = out_ld32;
    float pend_v = 0.f;
    auto flush = [&]() {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend_v), orsrc,
                                              (uint32_t)min(pend_s, out_ld32) * 4u, 0, 0);
    };
    // the fp8 MFMAs of the next block into `nxt`, the current block's epilogue on the vector
    // unit: this lane's partial head sum of the current block
    auto phase = [&](f32x4 (&nxt)[4], const i32x8 &kn, const f32x4 (&cur)[4]) {
        float a = 0.f;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            nxt[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                qf[n], kn, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, scale_a, 0, 127);
            a = epi_step(cur[n], wp[2 * n], wp[2 * n + 1], a);
            if (n & 1) __builtin_amdgcn_sched_barrier(0);
        }
        return a;
    };

    if (p_begin < p_vis) {
        stage(p_begin);
        commit(0);
        stage(p_begin + 1);
        commit(1);
        stage(p_begin + 2);
        __syncthreads();
        f32x4 ca[4], cb[4];
#pragma unroll
        for (int n = 0; n < 4; ++n)
            ca[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                qf[n], kfrag(0, 0), f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, scale_a, 0, 127);
        i32x8 k1 = kfrag(0, 1);
        int b0 = 0;
        for (int64_t p = p_begin; p < p_vis; ++p) {
            const int b1 = b0 == 2 ? 0 : b0 + 1, b2 = b1 == 2 ? 0 : b1 + 1;
            commit(b2);
            stage(p + 3);
            flush();
            f32x4 tot;
            const i32x8 k2 = kfrag(b0, 2);
            tot[0] = phase(cb, k1, ca);
            const i32x8 k3 = kfrag(b0, 3);
            tot[1] = phase(ca, k2, cb);
            const i32x8 kn = kfrag(b1, 0);
            tot[2] = phase(cb, k3, ca);
            k1 = kfrag(b1, 1);
            tot[3] = phase(ca, kn, cb);
            // lane group g holds block g's totals and stores them
            const int e = 16 * g + j;
            const int s = (int)p * kPage + e;
            const float tt = block_totals(tot[0], tot[1], tot[2], tot[3]);
            const float v = s_phys[p - p_begin] >= 0 ? tt * row_factor * s_scale[b0][e]
                                                     : __builtin_nanf("");
            pend_s = s;
            pend_v = s < nvis_t ? v : -INFINITY;
            __syncthreads();
            b0 = b1;
        }
        flush();
    }
    for (int64_t p = max(p_vis, p_begin); p < p_end; ++p) {
        const int64_t s = p * kPage + 16 * g + j;
        if (row_ok && s < A.out_ld) orow[s] = -INFINITY;
    }
}

}  // namespace

void prefill_plan(PrefillArgs &a, int T, int64_t n_pages) {
    const int64_t rblocks = (T + kWaves - 1) / kWaves;
    int64_t chunks = (4096 + rblocks - 1) / rblocks;         // about 16 workgroups per CU
    const int64_t max_chunks = n_pages / 8 > 1 ? n_pages / 8 : 1;   // >= 8 pages per chunk
    if (chunks > max_chunks) chunks = max_chunks;
    if (chunks >= 8) chunks = chunks / 8 * 8;                 // one chunk set per XCD
    const int64_t min_chunks = (n_pages + kMaxChunkPages - 1) / kMaxChunkPages;
    if (chunks < min_chunks) chunks = min_chunks;             // the chunk's table fits in LDS
    if (chunks < 1) chunks = 1;
    a.n_pages = n_pages;
    a.n_chunks = (int)chunks;
    a.chunk_pages = (n_pages + chunks - 1) / chunks;
    a.n_rowblocks = (int)rblocks;
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
    const unsigned grid = (unsigned)((int64_t)a.n_chunks * a.n_rowblocks);
    prefill_fp8_kernel<<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fm
