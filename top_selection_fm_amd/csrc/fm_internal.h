// fm_internal.h -- kernel argument blocks and launch entry points shared by the HIP sources of
// libfm.so.  Host code validates every argument before it fills one of these blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fm.h"

namespace fm {

constexpr int kPage = FM_PAGE_SIZE;  // compressed entries per page
constexpr int kDim = FM_HEAD_DIM;    // head dimension
constexpr int kHeads = FM_N_HEADS;   // heads of one query row
constexpr int kRowFp8 = kDim + 4;    // 132-byte compressed-key row
constexpr int kRowBf16 = kDim * 2;
constexpr int kRowF32 = kDim * 4;

// key / query element formats the kernels are instantiated for
enum KeyFmt { KEY_F32 = 0, KEY_BF16 = 1, KEY_FP8 = 3 };
enum QFmt { Q_F32 = 0, Q_BF16 = 1, Q_FP8 = 2 };

// One query layer as the kernels see it.
struct QArgs {
    const void *q;          // [T, n_heads, 128]
    const float *q_scale;   // [T] (fp8 q)
    const void *w;          // [T, n_heads]
    int w_bf16;             // 1: w is bf16, 0: float32
    int n_heads;            // 64, or 128 (fp8 keys with bf16 q; fp32 keys)
    int T;
    const int32_t *row_req; // [T] or null
    int b_is_zero;          // row_req null and B == 1: every row is request 0
    const int32_t *q_pos;   // [T] or null
    int ratio;
    const int32_t *row_pool; // [T] or null: key layer of row t (null: layer 0)
};

struct KvArgs {
    const uint8_t *pool[FM_MAX_POOLS];
    int n_pools;
    const int32_t *bt;
    int64_t bt_ld;
    const int32_t *seq_lens;
    int64_t n_phys;
    int B;
};

// Scoring of query rows over pages, writing one float per entry.
//   res_pages == null: slot j of row t is logical page j; out column = 64 j + e.
//   res_pages != null: slot j is resident_pages[b, j] (j < n_res[b]); out column = 64 j + e.
struct ScoreArgs {
    QArgs q;
    KvArgs kv;
    const int32_t *res_pages;
    const int32_t *n_res;
    int64_t res_ld;
    float *out;
    int64_t out_ld;      // floats per output row
    int64_t n_slots;     // page slots per row covered by the grid
    int ppw;             // page slots per wave
};

// Tiled scoring of many query rows of one request (prefill), fp8 queries and fp8 keys.
struct PrefillArgs {
    QArgs q;
    KvArgs kv;           // B == 1: every row reads request 0's block table
    float *out;
    int64_t out_ld;      // floats per output row (columns 0 .. out_ld - 1 are written)
    int64_t n_pages;     // ceil(out_ld / 64)
    int64_t chunk_pages; // pages per workgroup chunk
    int n_chunks;
    int n_rowblocks;     // ceil(T / 8)
};

struct MaskArgs {
    QArgs q[FM_MAX_LAYERS];
    KvArgs kv;
    int n_layers;
    int mean_mode;
    float cut;           // MAX: logit cut ln(p/(1-p)); MEAN: probability p
    int32_t n_sink, n_recent;
    uint8_t *mask;
    int64_t mask_ld;
    float *union_score;  // nullable
    int64_t n_pages;     // ceil(mask_ld / 64)
    int ppw;             // pages per wave (set by the launcher)
    int32_t *dens_out;   // nullable: resident entries of every page, [B, dens_ld] (fp8 kernel)
    int64_t dens_ld;
    int shared_keys;     // every layer's pool is the same array (fp8, 64 heads): read it once
};

struct CompactArgs {
    const uint8_t *mask;
    int64_t mask_ld;
    const int32_t *dens_in;  // nullable: page densities [B, dens_ld] instead of the mask bytes
    int64_t dens_ld;
    int64_t n_pages;
    int32_t *page_count;
    int32_t *page_list;  // nullable
    int64_t page_list_ld;
    int32_t *page_density;  // nullable
};

struct TopkArgs {
    const float *logits;
    int64_t ld;
    int T;
    const int32_t *n_valid;    // [T] or null
    const uint8_t *mask;       // nullable
    int64_t mask_ld;
    const int32_t *row_req;    // request of row t (mask row and resident list), or null
    int b_is_zero;
    const int32_t *res_pages;  // two-level index map (nullable)
    const int32_t *n_res;
    int64_t res_ld;
    int res_cells;             // with res_pages: rank and emit reserve cells (row positions)
    int B;                     // requests (bounds row_req in two-level mode)
    int k;
    int32_t *out_idx;
    float *out_val;            // nullable
};

struct DensestArgs {
    const int32_t *density;    // [B, ld]
    int64_t ld;
    int64_t n_pages;
    int kmax;
    int32_t *out_pages;        // [B, kmax]
    int32_t *out_count;        // [B] or null
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Fused scoring + top-k.  Scoring grid (n_chunks, T): workgroup (c, t) scores page slots
// [c W ppw, (c + 1) W ppw) of row t into LDS (W waves, ppw slots each) and keeps at most cap
// candidates (a superset of the chunk's top-k) in the workspace; then one workgroup per row
// selects the row's top-k from its chunks' candidates.
constexpr int kFuseMaxChunks = 16;         // chunks of one row, at most
constexpr int kFuseMaxCand = 8192;         // chunks x cap, at most (the merge buffer in LDS)
struct FuseArgs {
    int k;
    int n_chunks;
    int cap;                     // candidates a chunk may keep: k <= cap, n_chunks cap <= 8192
    int ppw_pad;                 // slots a wave's LDS rows hold (ppw rounded up to the ring)
    const uint8_t *mask;         // Mode A: [rows of requests, mask_ld] by logical entry, or null
    int64_t mask_ld;
    int cells;                   // two-level: rank and emit reserve cells (list positions)
    int bit_words;               // entries below 32 bit_words (<= 8192 words, a multiple of 64)
                                 // are ordered through a bitmap; 0: by counting
    int32_t *cnt;                // [T, n_chunks]: candidates each chunk kept
    float4 *cstat;               // [T, n_chunks]: (bound of the kept values, chunk maximum,
                                 //  bound of the chunk's ceil(k / n_chunks) largest, -)
    float *cval;                 // [T, n_chunks, cap]
    int32_t *cidx;               // [T, n_chunks, cap]
    int32_t *out_idx;            // [T, k]
    float *out_val;              // [T, k] or null
};

// Top-k workspace: stage-1 survivors of every (row, kTopkChunk-entry chunk), kTopkCap each.
#ifndef FM_F8_WPE
#define FM_F8_WPE 3       // fp8-key scoring with bf16 queries: waves per SIMD it is sized for
#endif
#ifndef FM_TOPK_CHUNK
#define FM_TOPK_CHUNK 8192
#endif
constexpr int kTopkChunk = FM_TOPK_CHUNK;
constexpr int kTopkCap = 1024;
constexpr int kTopkMaxChunks = 256;   // staged path for rows of up to 2M entries
struct TopkWs {
    float *val;      // [T, n_chunks, kTopkCap]
    int32_t *idx;    // [T, n_chunks, kTopkCap]
    int32_t *cnt;    // [T, n_chunks]; > kTopkCap: overflow or no cut
    float4 *cut;     // [T]: the row's cut (bins lo, 1 / bin width, flat, cut bin as int bits)
    int n_chunks;
};
// Query encoder (encoder.hip): split-K products, RMSNorm + head weights, RoPE + Hadamard.
constexpr int kEncMaxPairs = FM_HEAD_DIM / 2;   // rotated pairs of a head, at most
struct EncGemmArgs {        // C[m, n] = sum over k of A[m, k] * W[n, k]
    const uint16_t *A;      // bf16 [M, lda]
    int64_t lda;
    int M;
    const uint16_t *W0;     // bf16 [N0, K]: columns 0 .. N0 - 1
    int N0;
    const uint16_t *W1;     // bf16 [N1, K]: columns N0 .. N0 + N1 - 1 (N1 may be 0)
    int N1;
    int K;
    int ksplit;             // K per wave, a multiple of 16
    int S;                  // waves per workgroup: 1, 2, 4, 8 or 16
    int Z;                  // workgroups per output tile (partial sums)
    float *C;               // [Z, M, N0 + N1]
};
struct EncNormArgs {
    const float *C;         // [Z, M, rank + n_heads]: partials of hidden . [wq_a ; w_proj]^T
    int Z, M, rank, n_heads;
    const uint16_t *g;      // bf16 [rank] RMSNorm weight
    float eps, w_scale;
    uint16_t *r;            // bf16 [M, rank]
    float *w;               // [M, n_heads]
};
struct EncRopeArgs {
    const float *C;         // [Z, M, n_heads * 128]: partials of r . wq_b^T
    int Z, M, n_heads, rope_dim;
    const int32_t *pos;     // [M]
    double inv_freq[kEncMaxPairs];
    uint16_t *q;            // bf16 [M, n_heads, 128]
};
hipError_t launch_enc_gemm(const EncGemmArgs &g, hipStream_t s);
hipError_t launch_enc_norm(const EncNormArgs &a, hipStream_t s);
hipError_t launch_enc_rope_had(const EncRopeArgs &a, hipStream_t s);

// Golden labels (labels.hip).
constexpr int kLabelMaxLd = 65536;      // entries of one token's row, at most
struct LabelArgs {
    const float *scores;      // [T, n_layers, ld]
    int64_t ld;
    int T, n_layers;
    const int32_t *n_valid;   // [T] or null
    float p;
    int min_votes, tau;
    int words;                // ceil(ld / 32)
    uint32_t *mbits;          // workspace [T, n_layers, words]: nucleus membership
    uint32_t *gbits;          // workspace [T, words]: golden sets
    uint32_t *pbits, *sbits;  // workspace [T, words]: prefix / suffix ORs within tau-blocks
    uint32_t *ybits;          // workspace [T - tau + 1, words]: label sets of the windows
    int32_t *counts;          // workspace [T - tau + 1, chunks]: labels, then first positions
    int chunks;               // 256-word chunks of a row
    int32_t *label_ptr;       // [T - tau + 2]
    int32_t *label_idx;       // [cap]
    float *label_score;       // [cap] or null
    int64_t cap;
};
size_t labels_ws_bytes(int T, int n_layers, int64_t ld, int tau);
void labels_ws_carve(LabelArgs &a, void *ws);
hipError_t launch_labels(const LabelArgs &a, hipStream_t s);

size_t topk_ws_bytes(int T, int64_t n);   // bytes for T rows of up to n entries (0: not used)
TopkWs topk_ws_carve(void *ws, int T, int64_t n);

hipError_t launch_score(const ScoreArgs &a, int key_fmt, int q_fmt, hipStream_t s);
// Fused scoring + top-k (ScoreArgs.out: the logits too, or null).  fuse_shape: W waves a
// workgroup (0: no fused kernel for the format) and the page count a wave's slots are padded to.
struct FuseShape {
    int waves, round, max_ppw;    // waves a workgroup, ring (page slots a multiple of), slots a wave
};
FuseShape fuse_shape(int key_fmt, int q_fmt, int n_heads);
hipError_t launch_score_topk(const ScoreArgs &a, const FuseArgs &f, int key_fmt, int q_fmt,
                             hipStream_t s);
void prefill_plan(PrefillArgs &a, int T, int64_t n_pages);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);
hipError_t launch_score_f32(const ScoreArgs &a, hipStream_t s);
hipError_t launch_mask(const MaskArgs &a, int key_fmt, int B, hipStream_t s);
hipError_t launch_compact(const CompactArgs &a, int B, hipStream_t s);
hipError_t launch_densest(const DensestArgs &a, int B, hipStream_t s);
hipError_t launch_topk(const TopkArgs &a, const TopkWs *ws, hipStream_t s);

}  // namespace fm
