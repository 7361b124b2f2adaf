/*
 * fm.h -- C ABI of libfm.so: compressed-key indexer scoring and selection on MI355X (gfx950).
 *
 * The indexer scores every compressed KV entry s of a request for a query row t as
 *
 *     L[t,s] = sum_h w[t,h] * ReLU( q[t,h,:] . k[s,:] )          (64 heads, head_dim 128)
 *
 * (FlashMemory-DeepSeek-V4 paper summary, section 3, the Memory-Indexer score I = sigmoid(L);
 * README "Retriever architecture"; DeepSeek-V4 CSA page, section 3, formula CSA-1 for the
 * native lightning indexer, which has the same form).  On top of the logits the library
 * provides the two decisions the pages build on them:
 *   - a Level-1 resident mask: sigmoid(L) >= p per query encoder, OR-ed over up to three
 *     encoders (paper summary, section 3, the threshold set and the R_t equation), compacted
 *     into 64-entry resident pages (README, page-granular recall);
 *   - a Level-2 top-k (k = 512 in DeepSeek-V4) per query row, optionally restricted to a
 *     resident mask or to a list of resident pages (paper summary, section 3, the C^CoreComp
 *     set; README "Two-level recall": non-resident logits are -inf before the native top-512,
 *     and decode scores only the resident set).
 *
 * Conventions for every entry point:
 *   - Descriptors are host structs; every pointer inside them and every buffer argument is a
 *     DEVICE pointer unless stated otherwise.  The caller owns all memory.  The library never
 *     allocates, frees, or keeps a pointer after the call returns.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs
 *     asynchronously; nothing synchronises the host.  Buffers must stay alive until the
 *     stream reaches the work.  Calls are stateless and thread-safe; a workspace needs no
 *     clearing, but work of two calls that may run at the same time on the GPU (different
 *     streams) must not share one.
 *   - Errors are detected on the host before anything is enqueued; on error nothing is
 *     launched and fm_last_error() (per thread) describes the problem.  No exception crosses
 *     the ABI.
 *   - Device-side preconditions that are NOT checked on the host: seq_lens[b] <=
 *     kv->max_seq_len; per-entry and per-token scales finite and > 0; q, w, keys free of NaN;
 *     resident page ids distinct.  Block-table and resident-list entries are bounds-checked
 *     on the device: an out-of-range physical page (e.g. -1) is never dereferenced and its
 *     entries score NaN, which no selection picks.
 */
#ifndef FM_H
#define FM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FM_VERSION 100          /* 1.0.0 */
#define FM_MAX_LAYERS 4          /* encoders of one fm_resident_mask call */
#define FM_MAX_POOLS 32          /* key layers of one fm_kv_desc */
#define FM_PAGE_SIZE 64         /* compressed entries per page */
#define FM_HEAD_DIM 128
#define FM_N_HEADS 64           /* indexer heads of every (q, key) dtype pair */
#define FM_N_HEADS_WIDE 128     /* the retriever's heads (FlashMemory README, "Hyperparameters") */
#define FM_MAX_K 1024

typedef enum {
    FM_OK = 0,
    FM_ERR_INVALID_ARG = 1,     /* null / negative / inconsistent argument */
    FM_ERR_UNSUPPORTED = 2,     /* valid but not implemented (dtype combination, n_heads...) */
    FM_ERR_WORKSPACE = 3,       /* workspace missing or smaller than fm_workspace_bytes() */
    FM_ERR_LAUNCH = 4           /* the HIP runtime refused a launch */
} fm_status;

typedef enum {
    FM_F32 = 0,                 /* float32 */
    FM_BF16 = 1,                /* bfloat16 bit patterns (uint16) */
    FM_FP8_E4M3 = 2,            /* OCP E4M3FN codes (uint8); a separate float32 scale applies */
    FM_FP8_E4M3_SCALED132 = 3   /* 132-byte compressed key: 128 E4M3FN codes + float32 scale */
} fm_dtype;

typedef enum { FM_UNION_MAX = 0, FM_UNION_MEAN = 1 } fm_union_mode;

typedef enum {
    FM_OP_INDEX_LOGITS = 0,
    FM_OP_TOPK = 1,
    FM_OP_RESIDENT_MASK = 2,
    FM_OP_SCORE_RESIDENT = 3,
    FM_OP_INDEX_TOPK = 4
} fm_op;

/*
 * Paged compressed-key pool(s).  Entry s of request b lives in logical page s / 64 at slot
 * s % 64; its physical page is block_table[b * bt_ld + s / 64].  Pool layer l is an array
 * [n_phys_pages][64][row] where row is 512 B (FM_F32), 256 B (FM_BF16) or 132 B
 * (FM_FP8_E4M3_SCALED132: bytes 0..127 E4M3FN codes, bytes 128..131 little-endian float32
 * scale; key = code * scale -- README "compressed_k format").  All layers share the block
 * table (each encoder scores its own keys at the same entry positions).  Pools 0 .. n_pools-1
 * must be non-NULL and 16-byte aligned (1 <= n_pools <= FM_MAX_POOLS).  Requires
 * bt_ld >= ceil(max_seq_len / 64).
 */
typedef struct {
    const void *pool[FM_MAX_POOLS];
    int n_pools;
    fm_dtype key_dtype;         /* FM_F32, FM_BF16 or FM_FP8_E4M3_SCALED132 */
    int page_size;              /* must be 64 */
    int head_dim;               /* must be 128 */
    const int32_t *block_table; /* [B, bt_ld] */
    int64_t bt_ld;
    const int32_t *seq_lens;    /* [B] valid entries per request */
    int B;
    int64_t max_seq_len;        /* host-side upper bound of every seq_lens[b] */
    int64_t n_phys_pages;
} fm_kv_desc;

/*
 * Query rows of one encoder / layer.  q is [T, n_heads, head_dim] row-major; w is
 * [T, n_heads] and already includes any weight scale (the library applies none).
 * row_req maps a row to its request (NULL: row t is request t when T == B, or request 0
 * when B == 1).  row_pool maps a row to the key layer it scores (NULL: every row scores
 * pool[0]), so one call can score the rows of many layers, each over its own pool, e.g. the
 * 21 compressed-attention layers of Mode A (paper summary, section 6; README "Two-level
 * recall": Level 2 runs in every c4 layer).  A row whose row_req or row_pool value is out of
 * range ([0, B), [0, n_pools)) has no visible entries.  row_pool is honoured by
 * fm_index_logits, fm_index_topk and the fm_score_resident calls; fm_resident_mask requires
 * it NULL (encoder l always scores pool[l]).
 * With q_pos, row t may only use entries s < floor(q_pos[t] / compress_ratio)
 * (DeepSeek-V4 CSA page, section 10: a token position maps to compressed block
 * floor(pos / ratio)); without it, every s < seq_len is visible.
 * Supported (q_dtype, key_dtype): (F32, F32), (BF16, BF16), (BF16, SCALED132),
 * (FP8_E4M3 with q_scale[T], SCALED132).  w_dtype: F32 or BF16.
 * n_heads: 64 for every pair; 128 (the retriever's head count, as fm_encode_queries produces
 * it) for (BF16, SCALED132) and (F32, F32); anything else is FM_ERR_UNSUPPORTED.  The score
 * is the same sum over all n_heads heads.  All layers of one fm_resident_mask call have the
 * same n_heads.
 */
typedef struct {
    const void *q;
    fm_dtype q_dtype;
    const float *q_scale;       /* [T], FP8_E4M3 q only; q = code * q_scale[t] */
    const void *w;
    fm_dtype w_dtype;
    int T;
    int n_heads;                /* 64, or 128 (see above) */
    const int32_t *row_req;     /* [T] or NULL */
    const int32_t *q_pos;       /* [T] or NULL */
    int compress_ratio;         /* > 0; used only with q_pos (4 for CSA) */
    const int32_t *row_pool;    /* [T] or NULL: key layer of row t */
} fm_query_desc;

/*
 * Index logits.  For every row t and 0 <= s < ld:
 *   logits[t * ld + s] = L[t,s] (float32) if s < n_vis(t), else -inf,
 * where n_vis(t) = seq_len[b] (cut to floor(q_pos / ratio) with positions).  Entries of an
 * unmapped page score NaN.  Row t scores key layer row_pool[t] (layer 0 without row_pool).
 * Accuracy: bf16 / fp8 inputs are decoded exactly and products accumulate in float32.  With
 * FP8_E4M3 q over SCALED132 keys, one request, T >= 16 and no row_pool (prefill), each
 * ReLU(q_h . k) term is rounded to f16 on a per-row power-of-two scale set by the row's
 * largest query code: the term's error is at most 2^-11 relative, or 2^(E-15) code-product
 * units absolute with E the largest E4M3 exponent field among the row's codes (one unit for
 * codes that fill the E4M3 range, 2^-10 units for codes below 1, as with q_scale = 1).  Key
 * codes are assumed to use the E4M3 range (scale = absmax / 448, as the compressed_k
 * quantiser produces them).
 */
fm_status fm_index_logits(const fm_query_desc *q, const fm_kv_desc *kv, float *logits,
                          int64_t ld, void *stream);

/*
 * Scoring and top-k in one call: fm_index_logits followed by fm_topk512 over every row's
 * visible entries (and, with a mask, its resident ones), with the same result as those two
 * calls (paper summary, section 3: the native top-k inside the resident set C^CoreComp;
 * README "Two-level recall": non-resident logits are -inf before the native top-512; CSA
 * page, section 3: index_topk = 512, all entries kept when fewer exist).
 *   Candidates of row t (request b = row_req[t], or t, or 0 when B == 1): the entries
 *   s < n_vis(t) whose logit is finite and, when mask is given, mask[b * mask_ld + s] != 0.
 *   out_idx[t * k + i]: the k of largest logit, ties to the lower s, ascending, padded -1;
 *   out_val (nullable): their logits, padded -inf.  logits (nullable): also receives the
 *   logits exactly as fm_index_logits writes them (columns s < logits_ld).
 * Shapes whose rows split into at most 16 chunks run fused: a workgroup scores each chunk of a
 * row into LDS and keeps a superset of the chunk's top-k in the workspace, then one workgroup
 * per row selects from those; no logit reaches memory unless asked for.  Other shapes score
 * into the workspace and select with the top-k kernels.  Both give the same result.
 * Requirements: 1 <= k <= FM_MAX_K; 1 <= max_seq_len <= 2^29; mask_ld >= 64 ceil(max_seq_len
 * / 64) and >= logits_ld (mask rows are requests, as for fm_resident_mask's output);
 * ws 256-byte aligned, ws_bytes >= fm_workspace_bytes(FM_OP_INDEX_TOPK, T, n) with
 * n = max(64 ceil(max_seq_len / 64), logits_ld rounded up to 64), its contents irrelevant.
 * Calls sharing a workspace must not overlap in time.
 */
fm_status fm_index_topk(const fm_query_desc *q, const fm_kv_desc *kv, const uint8_t *mask,
                        int64_t mask_ld, int k, int32_t *out_idx, float *out_val, float *logits,
                        int64_t logits_ld, void *ws, size_t ws_bytes, void *stream);

/*
 * Level-1 resident mask over n_layers encoders (1..FM_MAX_LAYERS), one query row per request
 * per encoder (q_layers[l].T == kv->B, row b = request b), encoder l scoring pool[l].
 *   FM_UNION_MAX : u[b,s] = max_l L_l[b,s]; resident iff u >= ln(p / (1 - p)), i.e.
 *                  max_l sigmoid(L_l) >= p (the OR of the per-encoder decisions);
 *   FM_UNION_MEAN: u[b,s] = mean_l sigmoid(L_l[b,s]); resident iff u >= p.
 * Entries s < n_sink or s >= seq_len[b] - n_recent are forced resident (README: threshold +
 * recent + sink).  mask[b * mask_ld + s] is 1/0 (torch.bool compatible) for s < mask_ld, 0
 * for s >= seq_len[b].  Pages are the 64-entry blocks of [0, mask_ld):
 *   page_count[b]   number of pages with >= 1 resident entry;
 *   page_list       (nullable) [B, page_list_ld]: those pages ascending, then -1;
 *   page_density    (nullable) [B, ceil(mask_ld / 64)]: resident entries per page;
 *   union_score     (nullable) [B, mask_ld] float32: u (-inf for s >= seq_len).
 * 0 < threshold < 1.  No workspace.
 */
fm_status fm_resident_mask(const fm_query_desc *q_layers, int n_layers, const fm_kv_desc *kv,
                           fm_union_mode mode, float threshold, int32_t n_sink,
                           int32_t n_recent, uint8_t *mask, int64_t mask_ld,
                           int32_t *page_count, int32_t *page_list, int64_t page_list_ld,
                           int32_t *page_density, float *union_score, void *stream);

/*
 * Top-k per row of a logit matrix logits[T, ld].  Candidates of row t are the entries
 * s < n_valid[t] (n_valid NULL: s < ld) whose logit is finite (not -inf, not NaN) and, when
 * mask is given, with mask[row_req[t] * mask_ld + s] != 0 (row_req NULL: mask row t).
 * Precondition (not checked on the device): every row_req[t] >= 0 indexes a row of the mask
 * buffer; the library does not know the mask's row count, so a larger value reads past it.
 * A negative row_req[t] gives row t no candidates.
 * Selects the k candidates of largest logit, ties broken by lower s (-0.0 == +0.0); with
 * fewer than k candidates, all of them.  out_idx[t * k + i] lists the selected s in
 * ascending order, padded with -1; out_val (nullable) holds their logits, padded with -inf.
 * 1 <= k <= FM_MAX_K.  For ld <= 65,536 one workgroup per row selects in a single pass over
 * the row and no workspace is used (fm_workspace_bytes(FM_OP_TOPK, T, ld) is 0).  For longer
 * rows the workspace is optional: with ws 256-byte aligned and ws_bytes >=
 * fm_workspace_bytes(FM_OP_TOPK, T, ld), each row's cut is taken from a sample by one
 * workgroup per row, the rows are filtered by one workgroup per 8,192-entry chunk, then
 * selected by one workgroup per row; otherwise one workgroup per row does everything.  Every
 * path gives the same result.
 */
fm_status fm_topk512(const float *logits, int64_t ld, int T, const int32_t *n_valid,
                     const uint8_t *mask, int64_t mask_ld, const int32_t *row_req, int k,
                     int32_t *out_idx, float *out_val, void *ws, size_t ws_bytes,
                     void *stream);

/*
 * Two-level scoring: for every row t (request b), score only the entries of the listed
 * resident logical pages resident_pages[b * res_ld + j], j < n_resident[b] (distinct ids,
 * any order), that are valid and visible, then select the top-k exactly as fm_topk512 over
 * those candidates (ties by lower logical index).  Indices are logical entry positions
 * 64 * page + slot, ascending, -1 padded.  Pages outside the list are never dereferenced.
 * Needs ws 256-byte aligned with ws_bytes >= fm_workspace_bytes(FM_OP_SCORE_RESIDENT, T,
 * res_ld * 64), its contents irrelevant.  Shapes that fit run fused as fm_index_topk does (the
 * chunks' candidates in the workspace); others score the listed pages into the workspace,
 * then select.
 */
fm_status fm_score_resident(const fm_query_desc *q, const fm_kv_desc *kv,
                            const int32_t *resident_pages, const int32_t *n_resident,
                            int64_t res_ld, int k, int32_t *out_idx, float *out_val,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Two-level scoring with the fused remap (README, "Key optimizations" table, the fused-remap
 * row: the top-512 columns map directly to reserve cells).  Recalled pages fill a reserve in
 * list order, so entry `offset` of the j-th listed page sits in reserve cell 64 * j + offset.
 * Same inputs, workspace and candidates as fm_score_resident; the selection ranks candidates by
 * logit, ties by lower cell, and out_cells[t * k + i] lists the selected cells in ascending
 * order, padded with -1 (out_val as in fm_score_resident).  With an ascending resident list (as
 * fm_densest_pages and fm_resident_mask produce) cells and logical entries are in the same
 * order, so the selection is fm_score_resident's, each entry given as its cell.
 */
fm_status fm_score_resident_cells(const fm_query_desc *q, const fm_kv_desc *kv,
                                  const int32_t *resident_pages, const int32_t *n_resident,
                                  int64_t res_ld, int k, int32_t *out_cells, float *out_val,
                                  void *ws, size_t ws_bytes, void *stream);

/*
 * fm_score_resident for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same arguments and results
 * as fm_score_resident (same kernels), but the workspace is the library's own static device
 * array of FM_STATIC_SCRATCH_BYTES (64 MiB) per GPU, held from the first call on that GPU
 * until the process ends; nothing is allocated or freed by the call.  The stream must belong
 * to the current device.  Calls whose fm_workspace_bytes(FM_OP_SCORE_RESIDENT, q->T,
 * res_ld * 64) exceeds FM_STATIC_SCRATCH_BYTES return FM_ERR_WORKSPACE before any launch
 * (e.g. 30 rows x 384 pages need 2.9 MB; 630 rows x 384 pages 62 MB).  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on different streams, or
 * from different threads without ordering) race and give undefined results.
 */
#define FM_STATIC_SCRATCH_BYTES (64ull << 20)

fm_status fm_score_resident_noalloc(const fm_query_desc *q, const fm_kv_desc *kv,
                                    const int32_t *resident_pages, const int32_t *n_resident,
                                    int64_t res_ld, int k, int32_t *out_idx, float *out_val,
                                    void *stream);

/*
 * The KMAX densest pages of each request (README, reference-performance notes: KMAX is the
 * number of densest pages recalled per request, about 10% of the history).  density is an
 * int32 [B, density_ld] matrix, e.g. the page_density of fm_resident_mask.  For request b,
 * the pages p < n_pages with density[b * density_ld + p] > 0 are ranked by density, ties by
 * lower page id; out_pages[b * kmax + i] lists the first min(kmax, count) in ascending page
 * id, padded with -1, and out_count[b] (nullable) holds min(kmax, count).  The result is a
 * resident list for fm_score_resident (res_ld = kmax, n_resident = out_count).
 * 1 <= kmax <= FM_MAX_K, n_pages <= density_ld.  Device precondition: densities <= 2^24 (a
 * page's density is at most 64).  No workspace.
 */
fm_status fm_densest_pages(const int32_t *density, int64_t density_ld, int B, int64_t n_pages,
                           int kmax, int32_t *out_pages, int32_t *out_count, void *stream);

/* Workspace bytes an operation needs for T rows of up to max_candidates entries each. */
size_t fm_workspace_bytes(fm_op op, int T, int64_t max_candidates);

/*
 * The retriever's query encoder, one CSA layer (FlashMemory-DeepSeek-V4 repository page,
 * section "Retriever architecture" and its "Hyperparameters" table).  For each row t:
 *   a = hidden[t] . wq_a^T                       (q_rank values)
 *   r = a / sqrt(mean(a^2) + rms_eps) * q_norm   (RMSNorm)
 *   x = r . wq_b^T, as [n_heads, head_dim]
 *   the last rope_dim dims of every head rotated by YaRN RoPE at position pos[t]: consecutive
 *     pairs (2i, 2i+1) turn by pos[t] * theta_i, theta_i = rope_base^(-2i/rope_dim) blended
 *     towards theta_i / rope_factor between the correction dims of beta_fast and beta_slow
 *     over rope_orig_len (YaRN's per-dimension interpolation; no temperature factor)
 *   q[t] = x . H / sqrt(head_dim), H Sylvester's Hadamard matrix (per head)
 *   w[t] = (hidden[t] . w_proj^T) * head_dim^-0.5 * n_heads^-0.5
 * Weights are Linear weights ([out, in] row-major bf16; wq_a, wq_b and w_proj 16-byte
 * aligned), all device pointers.  The products
 * accumulate in float32, r is rounded to bf16 (the operand of the second product), q is
 * rounded to bf16 at the end; w is float32.  q and w are the fm_query_desc inputs of the
 * scoring calls (q_dtype FM_BF16, w_dtype FM_F32) when n_heads is 64.
 */
typedef struct fm_encoder_desc {
    const void *wq_a;          /* bf16 [q_rank, d_model] */
    const void *q_norm;        /* bf16 [q_rank] */
    const void *wq_b;          /* bf16 [n_heads * head_dim, q_rank] */
    const void *w_proj;        /* bf16 [n_heads, d_model] */
    int d_model;               /* multiple of 16 (4096 on the page) */
    int q_rank;                /* multiple of 32, q_rank + n_heads <= 4096 (2048) */
    int n_heads;               /* multiple of 32 (128 on the page; 64 feeds the scoring calls) */
    int head_dim;              /* must be 128 */
    int rope_dim;              /* even, 0 .. head_dim (64) */
    float rms_eps;             /* >= 0 (1e-6) */
    float rope_base;           /* > 1 (160000) */
    float rope_factor;         /* >= 1 (16) */
    int rope_orig_len;         /* > 0 (65536) */
    float beta_fast;           /* > beta_slow (32) */
    float beta_slow;           /* > 0 (1) */
} fm_encoder_desc;

/* Workspace bytes fm_encode_queries needs for T rows (the two products' float32 results and r). */
size_t fm_encode_workspace_bytes(const fm_encoder_desc *e, int T);

/*
 * Encode T rows: hidden bf16 [T, d_model] (16-byte aligned), pos int32 [T] (>= 0), q bf16
 * [T, n_heads, head_dim] (4-byte aligned), w float32 [T, n_heads]; ws 256-byte aligned with
 * ws_bytes >= fm_encode_workspace_bytes(e, T), its contents irrelevant.  T = 0 is a no-op.
 * Errors: FM_ERR_INVALID_ARG (null pointer, bad size or alignment), FM_ERR_UNSUPPORTED
 * (head_dim != 128, shapes off the multiples above), FM_ERR_WORKSPACE; nothing is launched on
 * error.
 */
fm_status fm_encode_queries(const fm_encoder_desc *e, const void *hidden, int T,
                            const int32_t *pos, void *q, float *w, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * Golden labels for training the retriever from the future native selector's scores
 * (FlashMemory-DeepSeek-V4 paper summary, section 4, label construction; README "Data": CSR
 * labels).  scores: float32 [T, n_layers, ld], 4-byte aligned: the selector score of future
 * token i, CSA layer l and compressed entry s.  The candidates of token i are the entries
 * s < n_valid[i] (n_valid NULL: ld) whose score is not -inf or NaN; scores are finite or -inf.
 *   P[i,l,s] = softmax over the candidates;
 *   M[i,l]   = the candidates sorted by score (descending; equal scores by lower s) up to the
 *              last whose cumulative P is at most p (inclusive; a token whose largest P
 *              exceeds p has an empty M);
 *   V[i,s]   = the number of layers l with s in M[i,l];  A[i] = {s : V[i,s] >= min_votes};
 *   Y[t]     = union of A[i] for i = t .. t + tau - 1, for the windows t = 0 .. T - tau.
 * Output, CSR: label_ptr int32 [T - tau + 2] (always written in full); window t's labels are
 * label_idx[label_ptr[t] .. label_ptr[t + 1]) in ascending s, and label_score (nullable) holds
 * for each the fraction of the window's tau tokens whose A holds it (the page defines no
 * score).  Positions at or past cap are not written: a caller sizes the arrays from
 * label_ptr[T - tau + 1] (a first call with cap 0 may count only).
 * The membership decisions use float32 exponentials exp(x - max) rounded to 2^-44 fixed point,
 * with exact integer sums: a cumulative mass ratio is within 3e-6 of exact in the worst case
 * (each mass carries about (|x - max| + 1) 2^-23 relative error, the heavy ones the least,
 * plus 2^-45 of the largest per entry), so decisions agree with exact arithmetic except where
 * a cumulative mass lies that close to p.
 * Limits: 1 <= ld <= 65,536, 1 <= n_layers <= 64, 1 <= tau <= T, (T - tau + 1) * ld < 2^31,
 * 1 <= min_votes, 0 < p <= 1.  ws 256-byte aligned, ws_bytes >=
 * fm_golden_workspace_bytes(T, n_layers, ld, tau), its contents irrelevant.
 * Errors: FM_ERR_INVALID_ARG, FM_ERR_UNSUPPORTED (ld or n_layers past the limits),
 * FM_ERR_WORKSPACE; nothing is launched on error.
 */
size_t fm_golden_workspace_bytes(int T, int n_layers, int64_t ld, int tau);
fm_status fm_golden_labels(const float *scores, int64_t ld, int T, int n_layers,
                           const int32_t *n_valid, float p, int min_votes, int tau,
                           int32_t *label_ptr, int32_t *label_idx, float *label_score,
                           int64_t cap, void *ws, size_t ws_bytes, void *stream);

/* Static description of a status code. */
const char *fm_status_string(fm_status s);

/* Message of the last failed call on this thread ("" if none). */
const char *fm_last_error(void);

/* FM_VERSION of the library. */
int fm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FM_H */
