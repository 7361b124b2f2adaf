// encoder.hip -- the retriever's query encoder: hidden states -> indexer queries q and weights w.
//
// The per-layer pipeline of the FlashMemory-DeepSeek-V4 repository page (section "Retriever
// architecture", with its "Hyperparameters" table):
//   a = hidden . wq_a^T,  r = RMSNorm(a) * q_norm,  x = r . wq_b^T as [n_heads, head_dim],
//   YaRN RoPE on the last rope_dim dims of each head, normalised Walsh-Hadamard over head_dim;
//   w = hidden . w_proj^T * head_dim^-0.5 * n_heads^-0.5.
//
// Four launches, all streaming their weights once from HBM:
//   1. enc_gemm_kernel: [a | w_raw] = hidden . [wq_a ; w_proj]^T (float32, Z partial sums);
//   2. enc_norm_kernel: RMSNorm -> r (bf16, the next product's operand), and the scaled head
//      weights w;
//   3. enc_gemm_kernel: x = r . wq_b^T (float32);
//   4. enc_rope_had_kernel: per (row, head), the partials' sum, YaRN RoPE, Walsh-Hadamard.
//
// The products run on v_mfma_f32_32x32x16_bf16.  Weights are Linear weights ([out, in],
// K-contiguous), so both MFMA operands are read straight from memory in their register layout:
// lane j + 32 h of a wave holds row j's 8 values k0 + 8 h .. + 7 of a 16-wide k step, for the
// activation (A) and the weight (B) alike, and the 32x32 accumulator register v of lane j + 32 h
// is output row 8 (v / 4) + 4 h + v % 4, column j.  Decode-sized inputs (tens of rows) make
// the products weight-bandwidth bound: Z workgroups of S waves share a 32 x 32 output tile, each
// wave a K range, so that enough waves on enough CUs stream the weight matrix at once.  From
// FM_ENC_TILED_MIN_ROWS rows the products are MFMA-bound and take LDS-tiled kernels (below):
// enc_gemm_dma_kernel, whose operands are copied from memory straight into LDS, when K is a
// multiple of 32 and the operands are 16-byte aligned, else enc_gemm_tiled_kernel, which
// stages them through registers.
#include <math.h>

#include <type_traits>

#include "fm_internal.h"

#ifndef FM_ENC_TILED_MIN_ROWS
#define FM_ENC_TILED_MIN_ROWS 256   // rows from which a product (without split K) is LDS-tiled
#endif

namespace fm {
namespace {

constexpr int kTiledMinRows = FM_ENC_TILED_MIN_ROWS;
constexpr int kRopeHeadsPerWave = 16;   // heads of one row a RoPE / Hadamard wave takes, from
                                        // 256 rows (n_heads % 32 == 0); one below

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t bf16_rne(float x) {   // finite inputs
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ f32x16 mma(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Workgroup (nt, mt, z) of S waves computes partial z of the 32 x 32 output tile (nt, mt):
// wave w takes the K range [c ksplit, (c + 1) ksplit), c = z S + w, and the S accumulators are
// summed through LDS into C[z].  Rows of A past M read as zeros through the buffer
// descriptor's bounds.
template <int S>
__global__ __launch_bounds__(64 * S) void enc_gemm_kernel(EncGemmArgs G) {
    const int ln = __lane_id(), j = ln & 31, h = ln >> 5;
    const int w = threadIdx.x >> 6;
    const int nt = blockIdx.x, mt = blockIdx.y, z = blockIdx.z;
    const int N = G.N0 + G.N1;
    const int n0 = nt * 32;
    const uint16_t *W = n0 < G.N0 ? G.W0 + (int64_t)n0 * G.K : G.W1 + (int64_t)(n0 - G.N0) * G.K;
    const int rows = min(32, G.M - mt * 32);
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(G.A + (int64_t)mt * 32 * G.lda), (short)0, rows * (int)G.lda * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)W, (short)0, 32 * G.K * 2, 0x00020000);
    const int kb = min(G.K, (z * S + w) * G.ksplit), ke = min(G.K, kb + G.ksplit);
    const uint32_t arow = (uint32_t)(j * G.lda * 2 + 16 * h), wrow = (uint32_t)(j * G.K * 2 + 16 * h);
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    // rounds of four 16-wide k steps; the next round's loads are issued before this round's
    // MFMAs, so two rounds are in flight.  Only whole rounds inside [kb, ke) are fetched; the
    // tail takes one 16-wide step at a time.
    constexpr int RS = 4;
    int k0 = kb;
    const int rounds = (ke - kb) / (16 * RS);
    if (rounds > 0) {
        u32x4 a[2][RS], b[2][RS];
        auto fetch = [&](u32x4 (&ra)[RS], u32x4 (&rb)[RS], int k) {
#pragma unroll
            for (int u = 0; u < RS; ++u) {
                ra[u] = __builtin_amdgcn_raw_buffer_load_b128(ar, arow + (uint32_t)(k + 16 * u) * 2, 0, 0);
                rb[u] = __builtin_amdgcn_raw_buffer_load_b128(wr, wrow + (uint32_t)(k + 16 * u) * 2, 0, 0);
            }
        };
        fetch(a[0], b[0], k0);
        for (int i = 0; i < rounds; i += 2) {
            if (i + 1 < rounds) fetch(a[1], b[1], k0 + 16 * RS * (i + 1));
#pragma unroll
            for (int u = 0; u < RS; ++u) acc = mma(a[0][u], b[0][u], acc);
            if (i + 1 < rounds) {
                if (i + 2 < rounds) fetch(a[0], b[0], k0 + 16 * RS * (i + 2));
#pragma unroll
                for (int u = 0; u < RS; ++u) acc = mma(a[1][u], b[1][u], acc);
            }
        }
        k0 += 16 * RS * rounds;
    }
    for (; k0 < ke; k0 += 16) {
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(ar, arow + (uint32_t)k0 * 2, 0, 0);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(wr, wrow + (uint32_t)k0 * 2, 0, 0);
        acc = mma(a, b, acc);
    }
    // accumulator register v of lane l is output row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
    auto put = [&](int v, int l, float x) {
        const int r = mt * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        if (r < G.M) G.C[((int64_t)z * G.M + r) * N + n0 + (l & 31)] = x;
    };
    if constexpr (S == 1) {
#pragma unroll
        for (int v = 0; v < 16; ++v) put(v, ln, acc[v]);
    } else {
        __shared__ float red[S][16][64];
#pragma unroll
        for (int v = 0; v < 16; ++v) red[w][v][ln] = acc[v];
        __syncthreads();
        for (int e = threadIdx.x; e < 16 * 64; e += 64 * S) {
            const int v = e >> 6, l = e & 63;
            float x = 0.f;
#pragma unroll
            for (int q = 0; q < S; ++q) x += red[q][v][l];
            put(v, l, x);
        }
    }
}

template <int NT>
__device__ float block_sum(float x, float *sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    if (__lane_id() == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t += sh[i];
    __syncthreads();
    return t;
}

// One workgroup per row: a = the sum of the Z partials of hidden . wq_a^T, r = a / sqrt(mean(a^2)
// + eps) * q_norm (bf16), w = the projected weights * weight scale.  Thread tid owns columns
// tid + i NT of the row.
constexpr int kNormNT = 1024;
constexpr int kNormCols = 4;       // rank + n_heads <= kNormCols * kNormNT
constexpr int kNormZ = 8;          // partials requested together
__global__ __launch_bounds__(kNormNT) void enc_norm_kernel(EncNormArgs E) {
    __shared__ float sh[kNormNT / 64];
    const int m = blockIdx.x, tid = threadIdx.x;
    const int N = E.rank + E.n_heads;
    // every partial of the thread's columns requested at once (columns past N read column
    // N - 1 and are not used), then summed
    float a[kNormCols];
#pragma unroll
    for (int i = 0; i < kNormCols; ++i) a[i] = 0.f;
    for (int z0 = 0; z0 < E.Z; z0 += kNormZ) {
        float p[kNormZ][kNormCols];
#pragma unroll
        for (int dz = 0; dz < kNormZ; ++dz) {
            const int z = min(z0 + dz, E.Z - 1);
            const float *row = E.C + ((int64_t)z * E.M + m) * N;
#pragma unroll
            for (int i = 0; i < kNormCols; ++i) p[dz][i] = row[min(tid + i * kNormNT, N - 1)];
        }
#pragma unroll
        for (int dz = 0; dz < kNormZ; ++dz)
#pragma unroll
            for (int i = 0; i < kNormCols; ++i) a[i] += z0 + dz < E.Z ? p[dz][i] : 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kNormCols; ++i) {
        const int n = tid + i * kNormNT;
        if (n < E.rank) ss = fmaf(a[i], a[i], ss);
    }
    const float ms = block_sum<kNormNT>(ss, sh) / (float)E.rank;
    const float inv = 1.0f / sqrtf(ms + E.eps);
#pragma unroll
    for (int i = 0; i < kNormCols; ++i) {
        const int n = tid + i * kNormNT;
        if (n < E.rank) {
            const float g = __uint_as_float((uint32_t)E.g[n] << 16);
            E.r[(int64_t)m * E.rank + n] = bf16_rne(a[i] * inv * g);
        } else if (n < N) {
            E.w[(int64_t)m * E.n_heads + (n - E.rank)] = a[i] * E.w_scale;
        }
    }
}

// One wave per (row, HPW heads), four waves a workgroup: lane l holds dims 2 l, 2 l + 1 of each
// head in turn.  Every load of the wave's heads is issued before the first head is turned.  The
// RoPE angle pos * theta_i is formed and reduced in fp64 (positions reach millions of radians),
// once per row and pair: every head of the row turns by the same angles.
template <int HPW>
__global__ __launch_bounds__(256) void enc_rope_had_kernel(EncRopeArgs E) {
    const int ln = __lane_id();
    const int groups = E.n_heads / HPW;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (int64_t)E.M * groups) return;
    const int m = (int)(item / groups), h0 = (int)(item % groups) * HPW;
    const int N = E.n_heads * kDim;
    float2 xv[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) xv[hh] = make_float2(0.f, 0.f);
    for (int z = 0; z < E.Z; ++z) {
        const float *row = E.C + ((int64_t)z * E.M + m) * N + h0 * kDim + 2 * ln;
        float2 p[HPW];
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) p[hh] = *(const float2 *)&row[hh * kDim];
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            xv[hh].x += p[hh].x;
            xv[hh].y += p[hh].y;
        }
    }
    // the rotation of pair ln at this row's position: the same for every head of the row
    const int first = (kDim - E.rope_dim) / 2;          // the first rotated pair
    float c = 1.f, sn = 0.f;
    if (ln >= first) {
        const double ang = (double)E.pos[m] * E.inv_freq[ln - first];
        c = (float)cos(ang);
        sn = (float)sin(ang);
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        float x0 = xv[hh].x, x1 = xv[hh].y;
        if (ln >= first) {
            const float y0 = x0 * c - x1 * sn, y1 = x0 * sn + x1 * c;
            x0 = y0;
            x1 = y1;
        }
        // Walsh-Hadamard butterflies (Sylvester order): dims 2 l and 2 l + 1 in the lane, then
        // lanes l and l ^ s for s = 1 .. 32 (dims 2 l + c and 2 (l ^ s) + c)
        {
            const float a = x0, b = x1;
            x0 = a + b;
            x1 = a - b;
        }
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) {
            const float o0 = __shfl_xor(x0, s), o1 = __shfl_xor(x1, s);
            const bool up = (ln & s) != 0;
            x0 = up ? o0 - x0 : x0 + o0;
            x1 = up ? o1 - x1 : x1 + o1;
        }
        const float nrm = 0.08838834764831845f;              // 1 / sqrt(128)
        const uint32_t packed = (uint32_t)bf16_rne(x0 * nrm) | ((uint32_t)bf16_rne(x1 * nrm) << 16);
        *(uint32_t *)&E.q[((int64_t)m * E.n_heads + h0 + hh) * kDim + 2 * ln] = packed;
    }
}

// Prefill-sized products (hundreds of rows and more): a BM x BN output tile a workgroup
// (256 x 256 with eight waves of 64 x 128, 128 x 256 with four of 64 x 128, or 128 x 128 with
// four of 64 x 64), staged through LDS 32 k-values at a time, so each A row and each weight row
// is read from memory once per tile instead of once per 32 x 32 tile.  This kernel (128 x 128,
// for K not a multiple of 32) runs the global loads two k-slabs ahead in two register stages
// while the current slab is multiplied from one of two LDS buffers, zeroing the pieces past K.
// LDS rows are padded to 40 bf16 (80 B), which keeps the 16-byte operand reads of a wave
// conflict-free.  Z = 1 (no partial sums).
#ifndef FM_ENC_TK
#define FM_ENC_TK 32
#endif
constexpr int kTK = FM_ENC_TK, kTLd = kTK + 8;
#ifndef FM_ENC_WIDE_TILES
#define FM_ENC_WIDE_TILES 512
#endif
constexpr int kWideTiles = FM_ENC_WIDE_TILES;
#ifndef FM_ENC_BIG_TILES_MIN
#define FM_ENC_BIG_TILES_MIN 128
#endif
constexpr int kBigTilesMin = FM_ENC_BIG_TILES_MIN;
#ifndef FM_ENC_GROUP_M
#define FM_ENC_GROUP_M 4
#endif
constexpr int kTGroupM = FM_ENC_GROUP_M;

template <int BM, int BN, int WGM, int WGN, int WPE>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(WPE)))
void enc_gemm_tiled_kernel(EncGemmArgs G) {
    // NT threads in WGM x WGN waves, each BM / WGM x BN / WGN of the tile (TI x TJ MFMA tiles);
    // PR 16-byte pieces a row of a k-slab; PA / PW pieces a thread loads of A / W
    constexpr int NW = WGM * WGN, NT = 64 * NW, TI = BM / WGM / 32, TJ = BN / WGN / 32;
    constexpr int PR = kTK / 8, PA = BM * PR / NT, PW = BN * PR / NT;
    static_assert(TI >= 1 && TJ >= 1 && BM % (WGM * 32) == 0 && BN % (WGN * 32) == 0, "wave grid");
    static_assert(PA >= 1 && PW >= 1 && BM * PR % NT == 0 && BN * PR % NT == 0, "slab layout");
    __shared__ __align__(16) uint16_t sA[2][BM * kTLd];
    __shared__ __align__(16) uint16_t sW[2][BN * kTLd];
    const int tid = threadIdx.x, ln = __lane_id(), j = ln & 31, h = ln >> 5, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int N = G.N0 + G.N1;
    // Tile order: the chip's 8 XCDs (each with its own L2) take consecutive workgroup ids in
    // turn, so workgroup b runs on XCD b % 8; each XCD is given a contiguous run of tiles, and
    // within it tiles go in groups of kTGroupM row tiles by every column tile, so the
    // workgroups an L2 serves at once share their activation rows and weight rows.
    const int mT = (G.M + BM - 1) / BM, nTl = (N + BN - 1) / BN, total = mT * nTl;
    const int b = blockIdx.x, x = b % 8, per = total / 8, rem = total % 8;
    const int t = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + b / 8;
    const int grp = t / (kTGroupM * nTl), fm = grp * kTGroupM, gs = min(kTGroupM, mT - fm);
    const int within = t - grp * kTGroupM * nTl;
    const int m0 = (fm + within % gs) * BM, n0 = (within / gs) * BN;
    // this thread's slab pieces: piece p = tid P + e is row p / PR, k values 8 (p % PR) .. + 7
    const uint16_t *ap[PA];
    const uint16_t *wp[PW];
    int aofs[PA], wofs[PW], akp[PA], wkp[PW];
#pragma unroll
    for (int e = 0; e < PA; ++e) {
        const int p = tid * PA + e, r = p / PR, kp = 8 * (p % PR);
        ap[e] = G.A + (int64_t)min(m0 + r, G.M - 1) * G.lda;
        aofs[e] = r * kTLd + kp;
        akp[e] = kp;
    }
#pragma unroll
    for (int e = 0; e < PW; ++e) {
        const int p = tid * PW + e, r = p / PR, kp = 8 * (p % PR);
        const int n = min(n0 + r, N - 1);
        wp[e] = n < G.N0 ? G.W0 + (int64_t)n * G.K : G.W1 + (int64_t)(n - G.N0) * G.K;
        wofs[e] = r * kTLd + kp;
        wkp[e] = kp;
    }
    // Two register stages: the loads of slab kt + 2 are issued while slab kt is multiplied and
    // slab kt + 1, loaded a step earlier, waits to be written to LDS.  Every load is issued
    // (a piece past K reads the row's last piece and is zeroed when written), so the wait
    // before a stage's LDS write covers only that stage's loads.
    u32x4 ra[2][PA], rw[2][PW];
    auto load = [&](int st, int k0) {   // K is a multiple of 16, so a piece is wholly in or out
#pragma unroll
        for (int e = 0; e < PA; ++e) ra[st][e] = *(const u32x4 *)(ap[e] + min(k0 + akp[e], G.K - 8));
#pragma unroll
        for (int e = 0; e < PW; ++e) rw[st][e] = *(const u32x4 *)(wp[e] + min(k0 + wkp[e], G.K - 8));
    };
    auto stash = [&](int st, int buf, int k0) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < PA; ++e) *(u32x4 *)&sA[buf][aofs[e]] = k0 + akp[e] < G.K ? ra[st][e] : zero;
#pragma unroll
        for (int e = 0; e < PW; ++e) *(u32x4 *)&sW[buf][wofs[e]] = k0 + wkp[e] < G.K ? rw[st][e] : zero;
    };
    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int jj = 0; jj < TJ; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;
    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < kTK / 16; ++ks) {
            u32x4 a[TI], bw[TJ];
#pragma unroll
            for (int i = 0; i < TI; ++i)
                a[i] = *(const u32x4 *)&sA[buf][(wm * (BM / WGM) + 32 * i + j) * kTLd + 16 * ks + 8 * h];
#pragma unroll
            for (int jj = 0; jj < TJ; ++jj)
                bw[jj] = *(const u32x4 *)&sW[buf][(wn * (BN / WGN) + 32 * jj + j) * kTLd + 16 * ks + 8 * h];
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int jj = 0; jj < TJ; ++jj) acc[i][jj] = mma(a[i], bw[jj], acc[i][jj]);
        }
    };
    const int nk = (G.K + kTK - 1) / kTK;
    // Slab kt is in LDS buffer kt & 1; slab kt + 1 is in register stage s1; stage s0 is free.
    // The loads are issued unconditionally (past the last slab they read the last piece of
    // each row and are never written), and the loop runs whole pairs of steps, so that every
    // path reaching a stage's LDS write has the same loads in flight.
    auto step = [&](int kt, int s1, int s0) {
        load(s0, (kt + 2) * kTK);
        __builtin_amdgcn_sched_barrier(0);     // the loads go out before the step's MFMAs
        compute(kt & 1);
        if (kt + 1 < nk) stash(s1, (kt + 1) & 1, (kt + 1) * kTK);
        __syncthreads();
    };
    load(0, 0);
    load(1, kTK);
    stash(0, 0, 0);
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        step(kt, 1, 0);
        step(kt + 1, 0, 1);
    }
    if (kt < nk) step(kt, 1, 0);
    // accumulator v of lane j + 32 h: row 8 (v / 4) + 4 h + v % 4, column j of its MFMA tile
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int jj = 0; jj < TJ; ++jj) {
            const int col = n0 + wn * (BN / WGN) + 32 * jj + j;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * (BM / WGM) + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (row < G.M && col < N) G.C[(int64_t)row * N + col] = acc[i][jj][v];
            }
        }
}


// Prefill-sized products with the operands copied straight from memory into LDS: each wave
// instruction of global_load_lds_dwordx4 lands 64 pieces of 16 bytes contiguously in LDS, so
// no register staging is needed and S - 1 slabs of 32 k values stay in flight while one is
// multiplied.  Tiles and waves as in enc_gemm_tiled_kernel.  A slab row is 64 bytes; its four
// 16-byte pieces are stored in the order piece ^ dma_swz(row), which puts the 16-byte operand
// reads of any 8 or 16 consecutive rows on distinct bank groups.  Each stage is an LDS array
// of its own, chosen at compile time (the slab loop is unrolled by S), and each step waits for
// its own slab's copies only (vmcnt) before a plain barrier: a barrier with the workgroup
// fence would wait for every copy in flight.  Copies past the last slab reload it into stages
// that no later step reads, so every step waits for the same count.  Both 16-wide k steps'
// operands of a slab are read before its first MFMA.  Taken when K is a multiple of 32 and
// the operands (rows of A included) are 16-byte aligned.
__device__ __forceinline__ int dma_swz(int r) { return ((r >> 1) & 2) | (((r >> 1) ^ (r >> 3)) & 1); }

template <int BM, int BN, int WGM, int WGN, int WPE, int S>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(WPE)))
void enc_gemm_dma_kernel(EncGemmArgs G) {
    constexpr int NW = WGM * WGN, TI = BM / WGM / 32, TJ = BN / WGN / 32;
    constexpr int PA = BM / 16 / NW, PW = BN / 16 / NW;     // 1 KB row blocks a wave copies
    static_assert(PA * 16 * NW == BM && PW * 16 * NW == BN && PA >= 1 && PW >= 1, "copy layout");
    static_assert(S >= 2 && S <= 4, "stages");
    typedef __attribute__((address_space(3))) void lds_void;
    __shared__ __align__(16) uint8_t sA0[BM * 64], sW0[BN * 64], sA1[BM * 64], sW1[BN * 64];
    __shared__ __align__(16) uint8_t sA2[S > 2 ? BM * 64 : 16], sW2[S > 2 ? BN * 64 : 16];
    __shared__ __align__(16) uint8_t sA3[S > 3 ? BM * 64 : 16], sW3[S > 3 ? BN * 64 : 16];
    auto stA = [&](auto st) -> uint8_t * {
        if constexpr (decltype(st)::value == 0) return sA0;
        else if constexpr (decltype(st)::value == 1) return sA1;
        else if constexpr (decltype(st)::value == 2) return sA2;
        else return sA3;
    };
    auto stW = [&](auto st) -> uint8_t * {
        if constexpr (decltype(st)::value == 0) return sW0;
        else if constexpr (decltype(st)::value == 1) return sW1;
        else if constexpr (decltype(st)::value == 2) return sW2;
        else return sW3;
    };
    const int tid = threadIdx.x, ln = __lane_id(), j = ln & 31, h = ln >> 5, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int N = G.N0 + G.N1;
    // tile order as in enc_gemm_tiled_kernel
    const int mT = (G.M + BM - 1) / BM, nTl = (N + BN - 1) / BN, total = mT * nTl;
    const int b = blockIdx.x, x = b % 8, per = total / 8, rem = total % 8;
    const int t = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + b / 8;
    const int grp = t / (kTGroupM * nTl), fm = grp * kTGroupM, gs = min(kTGroupM, mT - fm);
    const int within = t - grp * kTGroupM * nTl;
    const int m0 = (fm + within % gs) * BM, n0 = (within / gs) * BN;
    // wave w copies row blocks w P .. w P + P - 1 (16 rows each) of each tile; lane l carries
    // row 16 block + l / 4 and LDS piece l % 4, i.e. the row's piece (l % 4) ^ dma_swz(row)
    const uint16_t *srcA[PA], *srcW[PW];
#pragma unroll
    for (int i = 0; i < PA; ++i) {
        const int r = 16 * (PA * wave + i) + (ln >> 2);
        srcA[i] = G.A + (int64_t)min(m0 + r, G.M - 1) * G.lda + 8 * ((ln & 3) ^ dma_swz(r));
    }
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int r = 16 * (PW * wave + i) + (ln >> 2);
        const int n = min(n0 + r, N - 1);
        srcW[i] = (n < G.N0 ? G.W0 + (int64_t)n * G.K : G.W1 + (int64_t)(n - G.N0) * G.K) +
                  8 * ((ln & 3) ^ dma_swz(r));
    }
    const int nk = G.K / 32;
    auto issue = [&](auto st, int slab) {
        const int k0 = 32 * min(slab, nk - 1);
#pragma unroll
        for (int i = 0; i < PA; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(srcA[i] + k0),
                                             (lds_void *)(stA(st) + 1024 * (PA * wave + i)), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < PW; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(srcW[i] + k0),
                                             (lds_void *)(stW(st) + 1024 * (PW * wave + i)), 16, 0, 0);
    };
    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int jj = 0; jj < TJ; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;
    auto compute = [&](auto st) {
        const uint8_t *a_s = stA(st), *w_s = stW(st);
        u32x4 a[2][TI], bw[2][TJ];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const int r = wm * (BM / WGM) + 32 * i + j;
                a[ks][i] = *(const u32x4 *)(a_s + 64 * r + 16 * ((2 * ks + h) ^ dma_swz(r)));
            }
#pragma unroll
            for (int jj = 0; jj < TJ; ++jj) {
                const int r = wn * (BN / WGN) + 32 * jj + j;
                bw[ks][jj] = *(const u32x4 *)(w_s + 64 * r + 16 * ((2 * ks + h) ^ dma_swz(r)));
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int jj = 0; jj < TJ; ++jj) acc[i][jj] = mma(a[ks][i], bw[ks][jj], acc[i][jj]);
    };
    // s_waitcnt vmcnt(n), the other counters left alone (vmcnt in bits 3:0 and 15:14)
    constexpr int kWaitN = (PA + PW) * (S - 2);
    constexpr int kWaitImm = (kWaitN & 15) | ((kWaitN >> 4) << 14) | (7 << 4) | (15 << 8);
    auto step = [&](auto st, int slab) {
        __builtin_amdgcn_s_waitcnt(kWaitImm);              // this wave's copies of the slab
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();                      // every wave's; and the stage refilled
        __builtin_amdgcn_sched_barrier(0);                 // below was last read a step ago
        asm volatile("" ::: "memory");
        issue(std::integral_constant<int, (decltype(st)::value + S - 1) % S>(), slab + S - 1);
        compute(st);
    };
    issue(std::integral_constant<int, 0>(), 0);           // S - 1 slabs in flight
    if constexpr (S > 2) issue(std::integral_constant<int, 1>(), 1);
    if constexpr (S > 3) issue(std::integral_constant<int, 2>(), 2);
    int kt = 0;
    for (; kt + S <= nk; kt += S) {
        step(std::integral_constant<int, 0>(), kt);
        step(std::integral_constant<int, 1>(), kt + 1);
        if constexpr (S > 2) step(std::integral_constant<int, 2>(), kt + 2);
        if constexpr (S > 3) step(std::integral_constant<int, 3>(), kt + 3);
    }
    const int left = nk - kt;                              // the last nk % S slabs
    if (left > 0) step(std::integral_constant<int, 0>(), kt);
    if constexpr (S > 2) if (left > 1) step(std::integral_constant<int, 1>(), kt + 1);
    if constexpr (S > 3) if (left > 2) step(std::integral_constant<int, 2>(), kt + 2);
    __builtin_amdgcn_s_waitcnt(0);                         // no copy outlives the workgroup
    // accumulator v of lane j + 32 h: row 8 (v / 4) + 4 h + v % 4, column j of its MFMA tile
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int jj = 0; jj < TJ; ++jj) {
            const int col = n0 + wn * (BN / WGN) + 32 * jj + j;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * (BM / WGM) + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (row < G.M && col < N) G.C[(int64_t)row * N + col] = acc[i][jj][v];
            }
        }
}

}  // namespace

hipError_t launch_enc_gemm(const EncGemmArgs &g, hipStream_t s) {
    if (g.S == 1 && g.Z == 1 && g.M >= kTiledMinRows) {
        // the largest tile that still gives enough workgroups to fill the chip: 256 x 256
        // (eight waves of 64 x 128), 128 x 256 (four waves of 64 x 128: fewer LDS reads per
        // MFMA than 64 x 64), else 128 x 128
        const int n = g.N0 + g.N1;
        const int t256 = ((g.M + 255) / 256) * ((n + 255) / 256);
        const int wide = ((g.M + 127) / 128) * ((n + 255) / 256);
        const unsigned t128 = (unsigned)(((g.M + 127) / 128) * ((n + 127) / 128));
        // copies straight into LDS need whole 32-wide slabs and 16-byte aligned rows
        const bool dma = g.K % 32 == 0 && g.lda % 8 == 0 && (uintptr_t)g.A % 16 == 0 &&
                         (uintptr_t)g.W0 % 16 == 0 && (uintptr_t)g.W1 % 16 == 0;
        // The largest tiles that give kWideTiles workgroups: 256 x 256, then 128 x 256, then
        // 128 x 128 (two workgroups a CU).  When 128 x 128 tiles would spill past one round of
        // two a CU, 256 x 256 tiles are faster down to kBigTilesMin workgroups (half the CUs
        // idle).  The register-staged kernel takes the rest (K not a multiple of 32: the first
        // product when d_model is an odd multiple of 16).
        if (!dma)
            enc_gemm_tiled_kernel<128, 128, 2, 2, 2><<<dim3(t128), 256, 0, s>>>(g);
        else if (t256 >= kWideTiles ||
                 (wide < kWideTiles && (int)t128 > kWideTiles && t256 >= kBigTilesMin))
            enc_gemm_dma_kernel<256, 256, 4, 2, 2, 4><<<dim3((unsigned)t256), 512, 0, s>>>(g);
        else if (wide >= kWideTiles)
            enc_gemm_dma_kernel<128, 256, 2, 2, 2, 3><<<dim3((unsigned)wide), 256, 0, s>>>(g);
        else
            enc_gemm_dma_kernel<128, 128, 2, 2, 2, 4><<<dim3(t128), 256, 0, s>>>(g);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((g.N0 + g.N1) / 32), (unsigned)((g.M + 31) / 32), (unsigned)g.Z);
    switch (g.S) {
        case 1: enc_gemm_kernel<1><<<grid, 64, 0, s>>>(g); break;
        case 2: enc_gemm_kernel<2><<<grid, 128, 0, s>>>(g); break;
        case 4: enc_gemm_kernel<4><<<grid, 256, 0, s>>>(g); break;
        case 8: enc_gemm_kernel<8><<<grid, 512, 0, s>>>(g); break;
        case 16: enc_gemm_kernel<16><<<grid, 1024, 0, s>>>(g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_enc_norm(const EncNormArgs &a, hipStream_t s) {
    enc_norm_kernel<<<dim3((unsigned)a.M), kNormNT, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_enc_rope_had(const EncRopeArgs &a, hipStream_t s) {
    if (a.M >= 256) {
        const int64_t items = (int64_t)a.M * (a.n_heads / kRopeHeadsPerWave);
        enc_rope_had_kernel<kRopeHeadsPerWave><<<dim3((unsigned)((items + 3) / 4)), 256, 0, s>>>(a);
    } else {
        const int64_t items = (int64_t)a.M * a.n_heads;
        enc_rope_had_kernel<1><<<dim3((unsigned)((items + 3) / 4)), 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace fm
