/*
 * fm_oracle.c -- plain, slow fp64 CPU oracle for compressed-key indexer scoring and
 * selection.  TEST INFRASTRUCTURE: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header or table with the HIP
 * library and must never serve a product result.
 *
 * What it computes, and where each step is defined:
 *
 *  - Key dequantisation (FlashMemory-DeepSeek-V4 README, "compressed_k format" table and the
 *    retriever dataflow under "Retriever architecture"): a compressed key is 128 E4M3 codes
 *    followed by a float32 scale; the key is code value times scale.  E4M3 here is the OCP
 *    FP8 E4M3FN encoding (bias 7, no infinities, S.1111.111 is NaN).  bf16 keys are the upper
 *    16 bits of a float32.
 *  - Index logit (paper summary, section 3 "Memory Indexer scoring function", the I_{t,s}
 *    equation; README "Retriever architecture", the score line; DeepSeek-V4 CSA page, section 3,
 *    formula CSA-1, which has the same form):
 *        L[t,s] = sum_h w[t,h] * max(0, sum_d q[t,h,d] * k[s,d]),
 *    evaluated here in fp64, d ascending inside, h ascending outside.  I = sigmoid(L).
 *  - Causal visibility (DeepSeek-V4 CSA page, section 10: a position maps to compressed block
 *    floor(pos / ratio)): row t may use entries s < floor(pos_t / ratio), and s < seq_len.
 *  - Threshold and three-encoder union (paper summary, section 3, the threshold set and the
 *    R_t equation): resident iff max_l sigmoid(L_l) >= p.  Since sigmoid is increasing this
 *    is max_l L_l >= ln(p / (1 - p)), which is 0 for p = 0.5.  The README's "mean" ensemble
 *    averages the sigmoids instead.  Optional sink / recent entries are forced resident
 *    (README, "Two-level recall": threshold + recent + sink).
 *  - Pages of 64 entries; a page is resident when any of its entries is.
 *  - Top-k (paper summary, section 3, the C^CoreComp set; README: non-resident logits are set
 *    to -inf before the native top-512; CSA page, section 8: with fewer than 512 entries all
 *    are taken): candidates are the entries with a finite logit that are valid, visible and
 *    resident; they are ordered by logit descending, ties by lower entry index, the first
 *    min(k, |C|) are kept, emitted in ascending entry order and padded with -1.
 *  - Two-level scoring (README, "Two-level recall" and the env table row for
 *    SGLANG_PATHP_SCORE_RESIDENT): the same top-k over the entries of the listed resident
 *    pages only.
 *  - Densest pages (README, reference-performance notes: KMAX is the number of densest pages
 *    recalled per request): the KMAX pages with the most resident entries, ties by lower page
 *    id, among the pages with at least one; listed in ascending page id.
 *  - Reserve cells (README env table, the fused-remap row: the top-512 columns map directly to
 *    reserve cells): recalled pages fill a reserve in list order, so entry `offset` of the
 *    j-th listed page sits in cell 64 j + offset; the fused top-k ranks and lists cells.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { O_F32 = 0, O_BF16 = 1, O_FP8 = 2, O_FP8X132 = 3 };
enum { O_UNION_MAX = 0, O_UNION_MEAN = 1 };
#define O_MAX_LAYERS 8

typedef struct {
    const void *pool[O_MAX_LAYERS]; /* per layer: [n_phys_pages, page_size, row] */
    int n_pools;
    int key_dtype;                  /* O_F32, O_BF16, O_FP8X132 */
    int page_size;
    int head_dim;
    const int32_t *block_table;     /* [B, bt_ld]; negative = unmapped */
    int64_t bt_ld;
    const int32_t *seq_lens;        /* [B] */
    int B;
    int64_t n_phys_pages;
} fmo_kv;

typedef struct {
    const void *q;                  /* [T, n_heads, head_dim] */
    int q_dtype;                    /* O_F32, O_BF16, O_FP8 */
    const float *q_scale;           /* [T] for O_FP8 */
    const void *w;                  /* [T, n_heads] */
    int w_dtype;                    /* O_F32, O_BF16 */
    int T;
    int n_heads;
    const int32_t *row_req;         /* [T] or NULL (row t -> request t, or 0 when B == 1) */
    const int32_t *q_pos;           /* [T] or NULL (no causal limit) */
    int compress_ratio;
} fmo_q;

/* ------------------------------------------------------------------ element decoding */
double fmo_decode_e4m3(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

double fmo_decode_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double row_scale(const uint8_t *row, int head_dim)
{
    float f;
    memcpy(&f, row + head_dim, 4);      /* little-endian host, as the format states */
    return (double)f;
}

/* key k[s, 0..D) of request b in layer `layer`; returns 0 when the entry is not mapped */
static int load_key(const fmo_kv *kv, int layer, int b, int64_t s, double *k)
{
    int D = kv->head_dim;
    int64_t page = s / kv->page_size, off = s % kv->page_size;
    if (s < 0 || page >= kv->bt_ld) return 0;
    int32_t phys = kv->block_table[(int64_t)b * kv->bt_ld + page];
    if (phys < 0 || phys >= kv->n_phys_pages) return 0;
    int64_t row = (int64_t)phys * kv->page_size + off;
    const void *pool = kv->pool[layer];
    if (kv->key_dtype == O_F32) {
        const float *p = (const float *)pool + row * D;
        for (int d = 0; d < D; ++d) k[d] = (double)p[d];
    } else if (kv->key_dtype == O_BF16) {
        const uint16_t *p = (const uint16_t *)pool + row * D;
        for (int d = 0; d < D; ++d) k[d] = fmo_decode_bf16(p[d]);
    } else {
        const uint8_t *p = (const uint8_t *)pool + row * (int64_t)(D + 4);
        double sc = row_scale(p, D);
        for (int d = 0; d < D; ++d) k[d] = fmo_decode_e4m3(p[d]) * sc;
    }
    return 1;
}

static void load_query(const fmo_q *q, int t, int D, double *qv, double *wv)
{
    int H = q->n_heads;
    int64_t base = (int64_t)t * H * D;
    for (int i = 0; i < H * D; ++i) {
        if (q->q_dtype == O_F32) qv[i] = ((const float *)q->q)[base + i];
        else if (q->q_dtype == O_BF16) qv[i] = fmo_decode_bf16(((const uint16_t *)q->q)[base + i]);
        else qv[i] = fmo_decode_e4m3(((const uint8_t *)q->q)[base + i]) * (double)q->q_scale[t];
    }
    for (int h = 0; h < H; ++h) {
        if (q->w_dtype == O_F32) wv[h] = ((const float *)q->w)[(int64_t)t * H + h];
        else wv[h] = fmo_decode_bf16(((const uint16_t *)q->w)[(int64_t)t * H + h]);
    }
}

int fmo_row_request(const fmo_q *q, const fmo_kv *kv, int t)
{
    if (q->row_req) return q->row_req[t];
    return kv->B == 1 ? 0 : t;
}

/* number of entries row t may use: seq_len, cut to floor(pos / ratio) when positions exist */
int64_t fmo_n_visible(const fmo_q *q, const fmo_kv *kv, int t)
{
    int b = fmo_row_request(q, kv, t);
    int64_t n = kv->seq_lens[b];
    if (q->q_pos) {
        int64_t c = (int64_t)q->q_pos[t] / q->compress_ratio;
        if (c < n) n = c;
    }
    return n < 0 ? 0 : n;
}

/* the definition: sum over heads of w * relu(q . k), fp64 */
static double logit_one(const double *qv, const double *wv, const double *k, int H, int D)
{
    double L = 0.0;
    for (int h = 0; h < H; ++h) {
        double x = 0.0;
        for (int d = 0; d < D; ++d) x += qv[(int64_t)h * D + d] * k[d];
        L += wv[h] * (x > 0.0 ? x : 0.0);
    }
    return L;
}

/*
 * Logits of rows rows[0..n_rows) over entries [s_begin, s_end) of layer `layer`:
 * out[i * ld + (s - s_begin)] = L[rows[i], s] for visible s, -inf otherwise (also for entries
 * whose page is not mapped).
 */
void fmo_logits(const fmo_q *q, const fmo_kv *kv, int layer, const int32_t *rows, int n_rows,
                int64_t s_begin, int64_t s_end, double *out, int64_t ld)
{
    int H = q->n_heads, D = kv->head_dim;
    int64_t span = s_end - s_begin;
#pragma omp parallel
    {
        double *qv = (double *)malloc(sizeof(double) * H * D);
        double *wv = (double *)malloc(sizeof(double) * H);
        double *k = (double *)malloc(sizeof(double) * D);
        int last = -1;
#pragma omp for schedule(static)
        for (int64_t job = 0; job < (int64_t)n_rows * span; ++job) {
            int i = (int)(job / span);
            int64_t s = s_begin + job % span;
            int t = rows ? rows[i] : i;
            if (t != last) { load_query(q, t, D, qv, wv); last = t; }
            int b = fmo_row_request(q, kv, t);
            double L = -INFINITY;
            if (s < fmo_n_visible(q, kv, t) && load_key(kv, layer, b, s, k))
                L = logit_one(qv, wv, k, H, D);
            out[(int64_t)i * ld + (s - s_begin)] = L;
        }
        free(qv); free(wv); free(k);
    }
}

/* the same logit at listed points: out[i] = L[rows[i], ents[i]] (-inf if not visible) */
void fmo_logits_at(const fmo_q *q, const fmo_kv *kv, int layer, const int32_t *rows,
                   const int64_t *ents, int64_t n, double *out)
{
    int H = q->n_heads, D = kv->head_dim;
#pragma omp parallel
    {
        double *qv = (double *)malloc(sizeof(double) * H * D);
        double *wv = (double *)malloc(sizeof(double) * H);
        double *k = (double *)malloc(sizeof(double) * D);
        int last = -1;
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            int t = rows[i];
            if (t != last) { load_query(q, t, D, qv, wv); last = t; }
            int b = fmo_row_request(q, kv, t);
            double L = -INFINITY;
            if (ents[i] >= 0 && ents[i] < fmo_n_visible(q, kv, t) &&
                load_key(kv, layer, b, ents[i], k))
                L = logit_one(qv, wv, k, H, D);
            out[i] = L;
        }
        free(qv); free(wv); free(k);
    }
}

/* ------------------------------------------------------------------ top-k */
typedef struct { double v; int64_t s; } cand_t;

static int by_score(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->v > y->v) return -1;          /* larger logit first; -0.0 == +0.0 here */
    if (x->v < y->v) return 1;
    return (x->s < y->s) ? -1 : (x->s > y->s);   /* ties: lower entry index first */
}

static int by_index(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    return (x->s < y->s) ? -1 : (x->s > y->s);
}

/*
 * Top-k of one row.  vals[i] is the logit of entry index[i] (index == NULL: entry i).
 * keep[i] (nullable) must be nonzero for a candidate; -inf and NaN logits never are.
 * Writes min(k, |C|) entries in ascending entry order to out_idx/out_val, pads -1 / -inf,
 * and returns the number selected.
 */
int fmo_topk(const double *vals, const int64_t *index, const uint8_t *keep, int64_t n, int k,
             int32_t *out_idx, double *out_val)
{
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (n > 0 ? n : 1));
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        double v = vals[i];
        if (keep && !keep[i]) continue;
        if (isnan(v) || v == -INFINITY) continue;
        c[m].v = v;
        c[m].s = index ? index[i] : i;
        ++m;
    }
    qsort(c, m, sizeof(cand_t), by_score);
    int64_t take = m < k ? m : k;
    qsort(c, take, sizeof(cand_t), by_index);
    for (int i = 0; i < k; ++i) {
        out_idx[i] = i < take ? (int32_t)c[i].s : -1;
        if (out_val) out_val[i] = i < take ? c[i].v : -INFINITY;
    }
    free(c);
    return (int)take;
}

/* top-k of many rows of a dense logit matrix, rows in parallel */
void fmo_topk_rows(const double *logits, int64_t ld, int T, const int64_t *n_valid,
                   const uint8_t *mask, int64_t mask_ld, const int32_t *row_mask_req, int k,
                   int32_t *out_idx, double *out_val, int32_t *out_count)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        int64_t n = n_valid ? n_valid[t] : ld;
        if (n > ld) n = ld;
        const uint8_t *keep = NULL;
        if (mask) keep = mask + (int64_t)(row_mask_req ? row_mask_req[t] : t) * mask_ld;
        int got = fmo_topk(logits + (int64_t)t * ld, NULL, keep, n, k, out_idx + (int64_t)t * k,
                           out_val ? out_val + (int64_t)t * k : NULL);
        if (out_count) out_count[t] = got;
    }
}

/* ------------------------------------------------------------------ Level-1 resident mask */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/*
 * One query row per request per layer (qs[l].T == B, row b belongs to request b).
 * union_score[b, s]: MAX -> max_l L_l; MEAN -> mean_l sigmoid(L_l); -inf outside seq_len.
 * mask[b, s] = union decision OR sink/recent forcing, 0 for s >= seq_len.  Pages cover
 * [0, mask_ld); page_density = resident entries per page; page_list ascending, -1 padded.
 */
void fmo_resident_mask(const fmo_q *qs, int n_layers, const fmo_kv *kv, int mode,
                       double threshold, int n_sink, int n_recent, uint8_t *mask,
                       int64_t mask_ld, double *union_score, int32_t *page_count,
                       int32_t *page_list, int64_t page_list_ld, int32_t *page_density)
{
    int B = kv->B, D = kv->head_dim, P = kv->page_size;
    double cut = (mode == O_UNION_MAX) ? log(threshold / (1.0 - threshold)) : threshold;
    if (mode == O_UNION_MAX && threshold == 0.5) cut = 0.0;
    for (int b = 0; b < B; ++b) {
        int64_t n = kv->seq_lens[b];
        double *scratch = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
        for (int64_t s = 0; s < n; ++s) scratch[s] = (mode == O_UNION_MAX) ? -INFINITY : 0.0;
        for (int l = 0; l < n_layers; ++l) {
            double *L = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
            int32_t row = b;
            fmo_logits(&qs[l], kv, l, &row, 1, 0, n, L, n);
            for (int64_t s = 0; s < n; ++s) {
                if (mode == O_UNION_MAX) { if (L[s] > scratch[s]) scratch[s] = L[s]; }
                else scratch[s] += sigmoid(L[s]) / n_layers;
            }
            free(L);
        }
        for (int64_t s = 0; s < mask_ld; ++s) {
            uint8_t m = 0;
            double u = -INFINITY;
            if (s < n) {
                u = scratch[s];
                m = (u >= cut) || (s < n_sink) || (s >= n - n_recent);
            }
            mask[(int64_t)b * mask_ld + s] = m;
            if (union_score) union_score[(int64_t)b * mask_ld + s] = u;
        }
        free(scratch);
        int64_t n_pages = (mask_ld + P - 1) / P;
        int32_t cnt = 0;
        for (int64_t p = 0; p < n_pages; ++p) {
            int32_t dens = 0;
            for (int64_t s = p * P; s < (p + 1) * P && s < mask_ld; ++s)
                dens += mask[(int64_t)b * mask_ld + s] != 0;
            if (page_density) page_density[(int64_t)b * n_pages + p] = dens;
            if (dens) {
                if (page_list && cnt < page_list_ld) page_list[(int64_t)b * page_list_ld + cnt] = (int32_t)p;
                ++cnt;
            }
        }
        if (page_list)
            for (int64_t i = cnt; i < page_list_ld; ++i) page_list[(int64_t)b * page_list_ld + i] = -1;
        if (page_count) page_count[b] = cnt;
    }
    (void)D;
}

/* ------------------------------------------------------------------ two-level scoring */
/*
 * For every row t (request b): candidates are the entries of the listed resident logical
 * pages resident_pages[b, 0..n_resident[b]) that are valid and visible; top-k as fmo_topk.
 */
void fmo_score_resident_ex(const fmo_q *q, const fmo_kv *kv, const int32_t *resident_pages,
                           const int32_t *n_resident, int64_t res_ld, int k, int cells,
                           int32_t *out_idx, double *out_val, int32_t *out_count)
{
    int H = q->n_heads, D = kv->head_dim, P = kv->page_size;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < q->T; ++t) {
        int b = fmo_row_request(q, kv, t);
        int64_t nv = fmo_n_visible(q, kv, t);
        int nr = n_resident[b];
        int64_t n = (int64_t)nr * P;
        double *vals = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
        int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
        double *qv = (double *)malloc(sizeof(double) * H * D);
        double *wv = (double *)malloc(sizeof(double) * H);
        double *kk = (double *)malloc(sizeof(double) * D);
        load_query(q, t, D, qv, wv);
        for (int j = 0; j < nr; ++j) {
            int64_t page = resident_pages[(int64_t)b * res_ld + j];
            for (int e = 0; e < P; ++e) {
                int64_t s = page * P + e;
                double L = -INFINITY;
                if (s < nv && load_key(kv, 0, b, s, kk)) L = logit_one(qv, wv, kk, H, D);
                vals[(int64_t)j * P + e] = L;
                idx[(int64_t)j * P + e] = cells ? (int64_t)j * P + e : s;   /* cell or entry */
            }
        }
        int got = fmo_topk(vals, idx, NULL, n, k, out_idx + (int64_t)t * k,
                           out_val ? out_val + (int64_t)t * k : NULL);
        if (out_count) out_count[t] = got;
        free(vals); free(idx); free(qv); free(wv); free(kk);
    }
}

void fmo_score_resident(const fmo_q *q, const fmo_kv *kv, const int32_t *resident_pages,
                        const int32_t *n_resident, int64_t res_ld, int k, int32_t *out_idx,
                        double *out_val, int32_t *out_count)
{
    fmo_score_resident_ex(q, kv, resident_pages, n_resident, res_ld, k, 0, out_idx, out_val,
                          out_count);
}

/* ------------------------------------------------------------------ densest pages */
/*
 * For every request b: the pages p < n_pages with density[b * density_ld + p] > 0 ranked by
 * density descending, ties by lower page id; the first min(kmax, count) in ascending page
 * id, padded with -1 (out_pages[b * kmax + i]); out_count[b] = how many.
 */
void fmo_densest_pages(const int32_t *density, int64_t density_ld, int B, int64_t n_pages,
                       int kmax, int32_t *out_pages, int32_t *out_count)
{
    for (int b = 0; b < B; ++b) {
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (n_pages > 0 ? n_pages : 1));
        int64_t m = 0;
        for (int64_t p = 0; p < n_pages; ++p) {
            const int32_t d = density[(int64_t)b * density_ld + p];
            if (d <= 0) continue;
            c[m].v = (double)d;
            c[m].s = p;
            ++m;
        }
        qsort(c, m, sizeof(cand_t), by_score);
        const int64_t take = m < kmax ? m : kmax;
        qsort(c, take, sizeof(cand_t), by_index);
        for (int i = 0; i < kmax; ++i) out_pages[(int64_t)b * kmax + i] = i < take ? (int32_t)c[i].s : -1;
        if (out_count) out_count[b] = (int32_t)take;
        free(c);
    }
}

int fmo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void fmo_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
