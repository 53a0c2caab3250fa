/*
 * CPU oracle for pooled block-sparse bidirectional attention (Step-dLLM style).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plainly written reference
 * that the GPU library is checked against.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or constant with the GPU library.
 *
 * Sources (cited by page title and place):
 *  [SD]  "Step-dLLM: Adaptive Step-aware Sparse Attention for Efficient
 *        Diffusion LLM Inference" (arXiv 2611.01320), abstract: a block-sparse
 *        mask refreshed at anchor steps and reused within each interval, a
 *        head-adaptive global budget, bidirectional attention.
 *  [SP]  "SparseD: Sparse Attention for Diffusion Language Models"
 *        (arXiv 2509.24014), abstract: full attention in early steps, then one
 *        precomputed sparse pattern reused for all later steps.
 *  [BA]  "Block Approximate Sparse Attention (BA-Att)" abstract: blocks are
 *        scored in a block-wise pre-downsampled space.
 *  [PC]  "PulseCol" abstract: periodically refreshed column-sparse attention
 *        (the column-sparse variant below).
 *
 * The pages do not say how blocks are scored; the reading taken here is:
 * mean-pool Q and K over each block of B tokens, score pooled pairs with
 * Qb.Kb^T / sqrt(d), softmax each (head, query-block) row over key blocks,
 * and keep the K = ceil((1-s) * H * nb^2) largest normalised scores over
 * all heads together (one global budget), ties going to the lowest flat
 * index (h*nb + i)*nb + j.
 *
 * Precision: the mask path (pool, score, softmax, select) is fp32, the
 * precision in which the GPU takes the same integer decision; inputs are
 * fp32 arrays holding bf16-rounded values.  Attention outputs are computed
 * in fp64 (nothing is decided there, so the reference is as exact as the
 * inputs allow).
 *
 * Layout: Q, O are [H, L, d]; K, V are [Hkv, L, d]; row-major, batch 1.
 * Query head h reads key/value head h / (H / Hkv).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- pool --- */
/* Block mean of B consecutive tokens ([BA] pre-downsampling; mean, not sum).
 * x: [heads, L, d] -> xb: [heads, L/B, d].  Sum in fp32 in ascending token
 * order, then scale by 1/B (a power of two here, so the scale is exact). */
void oracle_pool(const float *x, int heads, int L, int d, int B, float *xb)
{
    int nb = L / B;
    float inv_b = 1.0f / (float)B;
    for (int h = 0; h < heads; ++h)
        for (int i = 0; i < nb; ++i)
            for (int c = 0; c < d; ++c) {
                float sum = 0.0f;
                for (int t = i * B; t < (i + 1) * B; ++t)
                    sum = sum + x[((int64_t)h * L + t) * d + c];
                xb[((int64_t)h * nb + i) * d + c] = sum * inv_b;
            }
}

/* ------------------------------------------------------ score + softmax --- */
/* S[h,i,j] = (Qb[h,i,:] . Kb[g(h),j,:]) * (1/sqrt(d)), then a softmax over j
 * for each (h, i): the pooled scores, normalised per row, that the global
 * budget ranks.  Dot product in fp32, ascending c; softmax max-subtracted, sum in
 * ascending j. */
void oracle_scores(const float *qb, const float *kb, int H, int Hkv, int nb,
                   int d, float *P)
{
    int G = H / Hkv;
    float sigma = (float)(1.0 / sqrt((double)d));
    float *srow = (float *)malloc(sizeof(float) * (size_t)nb);
    for (int h = 0; h < H; ++h) {
        int g = h / G;
        for (int i = 0; i < nb; ++i) {
            const float *a = qb + ((int64_t)h * nb + i) * d;
            float m = -INFINITY;
            for (int j = 0; j < nb; ++j) {
                const float *b = kb + ((int64_t)g * nb + j) * d;
                float dot = 0.0f;
                for (int c = 0; c < d; ++c) {
                    float prod = a[c] * b[c];
                    dot = dot + prod;
                }
                srow[j] = dot * sigma;
                if (srow[j] > m)
                    m = srow[j];
            }
            float *prow = P + ((int64_t)h * nb + i) * nb;
            float sum = 0.0f;
            for (int j = 0; j < nb; ++j) {
                prow[j] = expf(srow[j] - m);
                sum = sum + prow[j];
            }
            for (int j = 0; j < nb; ++j)
                prow[j] = prow[j] / sum;
        }
    }
    free(srow);
}

/* ------------------------------------------------------------ keep count --- */
/* K = ceil((1 - s) * N) with N = H * nb^2 (the head-adaptive global budget of
 * [SD] counts all query heads together), s taken as the decimal number the
 * caller wrote: the decimal with the fewest significant digits that reads
 * back as the same double (the nearest one of that length).  With
 * s = m / 10^E the budget is the ceiling of the fraction (10^E - m) * N / 10^E,
 * exact in 128-bit integers for N < 2^31. */
int64_t oracle_keep_count(int64_t n, double s)
{
    if (s == 0.0)
        return n;
    if (s == 1.0)
        return 0;
    long long m = 0;
    int E = 0;
    for (int p = 1; p <= 17; ++p) {
        /* the nearest decimal with p significant digits, as digits * 10^-E */
        char b[64];
        snprintf(b, sizeof b, "%.*e", p - 1, s);
        if (strtod(b, NULL) != s)
            continue;
        char *c = b;
        for (; *c != 'e'; ++c)
            if (*c != '.')
                m = 10 * m + (*c - '0');
        E = (p - 1) - (int)strtol(c + 1, NULL, 10);
        break;
    }
    if (E > 27)     /* s < 1e-10, so 0 < s * N < 1 and (1 - s) * N is in (N-1, N) */
        return n;
    unsigned __int128 ten_e = 1;
    for (int i = 0; i < E; ++i)
        ten_e *= 10;
    unsigned __int128 num = (ten_e - (unsigned __int128)m) * (unsigned __int128)n;
    return (int64_t)((num + ten_e - 1) / ten_e);
}

/* ---------------------------------------------------------------- select --- */
/* Keep the K largest of all n normalised scores under the total order
 * (value descending, flat index ascending): a full sort, the brute force
 * definition of a global top-K with lowest-index ties. */
static const float *g_sort_vals;

static int by_value_desc_index_asc(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    float va = g_sort_vals[a], vb = g_sort_vals[b];
    if (va > vb) return -1;
    if (va < vb) return 1;
    return (a < b) ? -1 : (a > b);
}

void oracle_select(const float *P, int64_t n, int64_t K, uint8_t *keep)
{
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t f = 0; f < n; ++f)
        order[f] = f;
    g_sort_vals = P;
    qsort(order, (size_t)n, sizeof(int64_t), by_value_desc_index_asc);
    memset(keep, 0, (size_t)n);
    for (int64_t r = 0; r < K && r < n; ++r)
        keep[order[r]] = 1;
    free(order);
}

/* Value of the K-th kept score (the cut) under the same order; 0 if K == 0. */
float oracle_cut_value(const float *P, int64_t n, int64_t K)
{
    if (K <= 0 || n <= 0)
        return 0.0f;
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    for (int64_t f = 0; f < n; ++f)
        order[f] = f;
    g_sort_vals = P;
    qsort(order, (size_t)n, sizeof(int64_t), by_value_desc_index_asc);
    float v = P[order[(K < n ? K : n) - 1]];
    free(order);
    return v;
}

/* Uniform per-head budget, the baseline that the Step-dLLM abstract sets
 * against its head-adaptive one (every head gets the same share): head h
 * keeps the k_h = ceil((1-s) * nb^2) largest of its own nb^2 scores under the
 * same order (value descending, index ascending), i.e. the global select run
 * on each head's slice on its own. */
void oracle_select_per_head(const float *P, int H, int nb, int64_t k_h, uint8_t *keep)
{
    int64_t per = (int64_t)nb * nb;
    for (int h = 0; h < H; ++h)
        oracle_select(P + h * per, per, k_h, keep + h * per);
}

/* ------------------------------------------------------------------ lists --- */
/* Per (head, query-block) row, the kept key blocks in ascending order. */
void oracle_csr(const uint8_t *keep, int rows, int nb, int32_t *row_ptr,
                int32_t *col_idx)
{
    int32_t nnz = 0;
    for (int r = 0; r < rows; ++r) {
        row_ptr[r] = nnz;
        for (int j = 0; j < nb; ++j)
            if (keep[(int64_t)r * nb + j])
                col_idx[nnz++] = j;
    }
    row_ptr[rows] = nnz;
}

/* Full anchor-step mask build: pool, score, softmax, global select, lists.
 * qb_out / kb_out / p_out receive the intermediates (caller-sized). */
int64_t oracle_build_mask(const float *q, const float *k, int H, int Hkv, int L,
                          int d, int B, double s, float *qb_out, float *kb_out,
                          float *p_out, int32_t *row_ptr, int32_t *col_idx)
{
    int nb = L / B;
    int64_t n = (int64_t)H * nb * nb;
    oracle_pool(q, H, L, d, B, qb_out);
    oracle_pool(k, Hkv, L, d, B, kb_out);
    oracle_scores(qb_out, kb_out, H, Hkv, nb, d, p_out);
    int64_t K = oracle_keep_count(n, s);
    uint8_t *keep = (uint8_t *)malloc((size_t)n);
    oracle_select(p_out, n, K, keep);
    oracle_csr(keep, H * nb, nb, row_ptr, col_idx);
    free(keep);
    return K;
}

/* The mask build with the uniform per-head budget; returns K = H * k_h. */
int64_t oracle_build_mask_per_head(const float *q, const float *k, int H, int Hkv,
                                   int L, int d, int B, double s, float *qb_out,
                                   float *kb_out, float *p_out, int32_t *row_ptr,
                                   int32_t *col_idx)
{
    int nb = L / B;
    int64_t n = (int64_t)H * nb * nb;
    oracle_pool(q, H, L, d, B, qb_out);
    oracle_pool(k, Hkv, L, d, B, kb_out);
    oracle_scores(qb_out, kb_out, H, Hkv, nb, d, p_out);
    int64_t k_h = oracle_keep_count((int64_t)nb * nb, s);
    int64_t K = k_h * H;
    uint8_t *keep = (uint8_t *)malloc((size_t)n);
    oracle_select_per_head(p_out, H, nb, k_h, keep);
    oracle_csr(keep, H * nb, nb, row_ptr, col_idx);
    free(keep);
    return K;
}

/* ------------------------------------------------------------------- plan --- */
/* Work order for the attention launch on a GPU made of 8 dies (XCDs) that take
 * workgroups round robin, so that all rows of a head share one die's L2 and
 * each die's rows start longest first:
 *  - a head weighs w = (B/32)*kept + 4*nonempty: its kept blocks in 32-key
 *    steps plus four steps for each row with a kept block, the fixed start-up
 *    and write-out of a row (B is a multiple of 32);
 *  - heads are taken in order of weight (descending, ties by head id) and
 *    each goes to the die with the least weight so far among those that
 *    hold fewer than cap_h = min(H, ceil(H/8) + 2) heads (ties: lowest die);
 *    the slack over ceil(H/8) lets the greedy balance skewed heads;
 *  - die x's list is first the rows of its heads that keep a block (heads in
 *    that order, each head's rows by list length descending, ties by row id),
 *    then the rows that keep none (heads in the same order, rows ascending):
 *    empty rows only write zeros, so they go where the launch runs down;
 *  - list x fills work[x*cap .. x*cap + cap), cap = cap_h*nb, and unused
 *    positions hold -1.
 * Returns the number of rows with at least one kept block. */
static const int32_t *g_row_ptr;
static const int64_t *g_head_weight;

static int by_len_desc_row_asc(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    int32_t la = g_row_ptr[a + 1] - g_row_ptr[a];
    int32_t lb = g_row_ptr[b + 1] - g_row_ptr[b];
    if (la > lb) return -1;
    if (la < lb) return 1;
    return (a < b) ? -1 : (a > b);
}

static int by_weight_desc_head_asc(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    if (g_head_weight[a] > g_head_weight[b]) return -1;
    if (g_head_weight[a] < g_head_weight[b]) return 1;
    return (a < b) ? -1 : (a > b);
}

enum { ORACLE_DIES = 8 };

int32_t oracle_plan(const int32_t *row_ptr, int H, int nb, int B, int32_t *work)
{
    int cap_heads = (H + ORACLE_DIES - 1) / ORACLE_DIES + 2;
    if (cap_heads > H)
        cap_heads = H;
    int64_t cap = (int64_t)cap_heads * nb;
    int64_t *weight = (int64_t *)malloc(sizeof(int64_t) * (size_t)H);
    int32_t *heads = (int32_t *)malloc(sizeof(int32_t) * (size_t)H);
    int32_t *die_heads = (int32_t *)malloc(sizeof(int32_t) * (size_t)(ORACLE_DIES * cap_heads));
    int64_t load[ORACLE_DIES] = {0};
    int count[ORACLE_DIES] = {0};
    int32_t n_nonempty = 0;
    for (int h = 0; h < H; ++h) {
        int64_t kept = row_ptr[(h + 1) * nb] - row_ptr[h * nb];
        int64_t rows = 0;
        for (int i = 0; i < nb; ++i)
            rows += row_ptr[h * nb + i + 1] > row_ptr[h * nb + i];
        weight[h] = (B / 32) * kept + 4 * rows;
        n_nonempty += (int32_t)rows;
        heads[h] = h;
    }
    g_head_weight = weight;
    qsort(heads, (size_t)H, sizeof(int32_t), by_weight_desc_head_asc);
    for (int a = 0; a < H; ++a) {
        int best = -1;
        for (int x = 0; x < ORACLE_DIES; ++x)
            if (count[x] < cap_heads && (best < 0 || load[x] < load[best]))
                best = x;
        die_heads[best * cap_heads + count[best]++] = heads[a];
        load[best] += weight[heads[a]];
    }
    for (int64_t p = 0; p < ORACLE_DIES * cap; ++p)
        work[p] = -1;
    g_row_ptr = row_ptr;
    int32_t *tmp = (int32_t *)malloc(sizeof(int32_t) * (size_t)nb);
    for (int x = 0; x < ORACLE_DIES; ++x) {
        int32_t *out = work + x * cap;
        int64_t pos = 0;
        for (int c = 0; c < count[x]; ++c) {
            int h = die_heads[x * cap_heads + c];
            for (int i = 0; i < nb; ++i)
                tmp[i] = h * nb + i;
            qsort(tmp, (size_t)nb, sizeof(int32_t), by_len_desc_row_asc);
            for (int i = 0; i < nb; ++i)
                if (row_ptr[tmp[i] + 1] > row_ptr[tmp[i]])
                    out[pos++] = tmp[i];
        }
        for (int c = 0; c < count[x]; ++c) {
            int h = die_heads[x * cap_heads + c];
            for (int i = 0; i < nb; ++i)
                if (row_ptr[h * nb + i + 1] <= row_ptr[h * nb + i])
                    out[pos++] = h * nb + i;
        }
    }
    free(tmp);
    free(weight);
    free(heads);
    free(die_heads);
    return n_nonempty;
}

/* -------------------------------------------------------------- attention --- */
/* Bidirectional softmax attention of one query token over an explicit list of
 * key tokens (ascending), fp64:  o = sum_u softmax_u(q . k_u / sqrt(d)) v_u.
 * An empty list gives o = 0 (a row that kept no block attends to nothing). */
static void attend_token(const float *qt, const float *kh, const float *vh,
                         int d, const int32_t *toks, int ntok, double *z,
                         double *o)
{
    double scale = 1.0 / sqrt((double)d);
    for (int c = 0; c < d; ++c)
        o[c] = 0.0;
    if (ntok == 0)
        return;
    double m = -INFINITY;
    for (int a = 0; a < ntok; ++a) {
        const float *ku = kh + (int64_t)toks[a] * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += (double)qt[c] * (double)ku[c];
        z[a] = dot * scale;
        if (z[a] > m)
            m = z[a];
    }
    double l = 0.0;
    for (int a = 0; a < ntok; ++a) {
        z[a] = exp(z[a] - m);
        l += z[a];
    }
    for (int a = 0; a < ntok; ++a) {
        const float *vu = vh + (int64_t)toks[a] * d;
        double p = z[a] / l;
        for (int c = 0; c < d; ++c)
            o[c] += p * (double)vu[c];
    }
}

/* Block-sparse attention for the listed rows r = h*nb + i (all rows when
 * rows == NULL).  Each query token of block i in head h attends to every
 * token of the kept key blocks col_idx[row_ptr[r] .. row_ptr[r+1]) of key
 * head h / (H/Hkv).  Output o: [H, L, d] fp64; only listed rows are written. */
void oracle_sparse_attn(const float *q, const float *k, const float *v, int H,
                        int Hkv, int L, int d, int B, const int32_t *row_ptr,
                        const int32_t *col_idx, const int32_t *rows, int n_rows,
                        double *o)
{
    int nb = L / B, G = H / Hkv;
    int total = rows ? n_rows : H * nb;
    int32_t *toks = (int32_t *)malloc(sizeof(int32_t) * (size_t)L);
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    for (int x = 0; x < total; ++x) {
        int r = rows ? rows[x] : x;
        int h = r / nb, i = r % nb, g = h / G;
        int ntok = 0;
        for (int e = row_ptr[r]; e < row_ptr[r + 1]; ++e)
            for (int t = 0; t < B; ++t)
                toks[ntok++] = col_idx[e] * B + t;
        const float *kh = k + (int64_t)g * L * d;
        const float *vh = v + (int64_t)g * L * d;
        for (int t = i * B; t < (i + 1) * B; ++t)
            attend_token(q + ((int64_t)h * L + t) * d, kh, vh, d, toks, ntok, z,
                         o + ((int64_t)h * L + t) * d);
    }
    free(toks);
    free(z);
}

/* Dense bidirectional attention (every block kept) for the listed rows. */
void oracle_dense_attn(const float *q, const float *k, const float *v, int H,
                       int Hkv, int L, int d, int B, const int32_t *rows,
                       int n_rows, double *o)
{
    int nb = L / B, G = H / Hkv;
    int total = rows ? n_rows : H * nb;
    int32_t *toks = (int32_t *)malloc(sizeof(int32_t) * (size_t)L);
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    for (int u = 0; u < L; ++u)
        toks[u] = u;
    for (int x = 0; x < total; ++x) {
        int r = rows ? rows[x] : x;
        int h = r / nb, i = r % nb, g = h / G;
        const float *kh = k + (int64_t)g * L * d;
        const float *vh = v + (int64_t)g * L * d;
        for (int t = i * B; t < (i + 1) * B; ++t)
            attend_token(q + ((int64_t)h * L + t) * d, kh, vh, d, toks, L, z,
                         o + ((int64_t)h * L + t) * d);
    }
    free(toks);
    free(z);
}

/* ------------------------------------------------------------ mask quality --- */
/* True block attention mass, fp64: A[h,i,j] is the mean over the B query
 * tokens t of block i of the full bidirectional softmax probability that t
 * puts on the B key tokens of block j (head h, key head g(h)).  This is the
 * block-level map of the exact attention that a pooled mask approximates
 * (the post-downsampling comparison of the BA-Att abstract).  Each row of A
 * sums to 1.  rows: optional list of rows r = h*nb + i to compute (others are
 * left untouched); A is [H, nb, nb]. */
void oracle_block_mass(const float *q, const float *k, int H, int Hkv, int L,
                       int d, int B, const int32_t *rows, int n_rows, double *A)
{
    int nb = L / B, G = H / Hkv;
    int total = rows ? n_rows : H * nb;
    double scale = 1.0 / sqrt((double)d);
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    for (int x = 0; x < total; ++x) {
        int r = rows ? rows[x] : x;
        int h = r / nb, i = r % nb, g = h / G;
        const float *kh = k + (int64_t)g * L * d;
        double *arow = A + (int64_t)r * nb;
        for (int j = 0; j < nb; ++j)
            arow[j] = 0.0;
        for (int t = i * B; t < (i + 1) * B; ++t) {
            const float *qt = q + ((int64_t)h * L + t) * d;
            double m = -INFINITY;
            for (int u = 0; u < L; ++u) {
                const float *ku = kh + (int64_t)u * d;
                double dot = 0.0;
                for (int c = 0; c < d; ++c)
                    dot += (double)qt[c] * (double)ku[c];
                z[u] = dot * scale;
                if (z[u] > m)
                    m = z[u];
            }
            double l = 0.0;
            for (int u = 0; u < L; ++u) {
                z[u] = exp(z[u] - m);
                l += z[u];
            }
            for (int u = 0; u < L; ++u)
                arow[u / B] += z[u] / l / B;
        }
    }
    free(z);
}

/* Recall of a mask: per row, the block mass A[h,i,j] summed over the row's
 * kept blocks j (1 when the kept blocks hold all of the row's attention). */
void oracle_mask_recall(const double *A, int rows, int nb, const int32_t *row_ptr,
                        const int32_t *col_idx, double *recall)
{
    for (int r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e)
            acc += A[(int64_t)r * nb + col_idx[e]];
        recall[r] = acc;
    }
}

/* --------------------------------------------------------- column-sparse --- */
/* [PC] "PulseCol" abstract: column-sparse attention (individual key columns
 * instead of blocks), its pattern found at an early denoising step, reused,
 * and refreshed at a few intermediate steps.  The pages do not say how the
 * columns are scored or counted; the reading taken mirrors the block path:
 *  - each query block's pooled query (block mean, as in oracle_pool) is
 *    rounded to bf16, the matrix-core input type, and scored against every
 *    key token u with q.k_u / sqrt(d), softmaxed over all L keys;
 *  - the column mass c[h,u] is the mean of those probabilities over the nb
 *    pooled queries of head h (an estimate of the share of the head's
 *    attention that lands on key u); each head's masses sum to 1;
 *  - head h keeps its k_c = ceil((1-s) * L) largest columns (value
 *    descending, index ascending), the same count for every head;
 *  - every query token of head h attends to exactly the kept key tokens. */

/* Round to the nearest bf16, ties to even (finite inputs). */
static float bf16_round(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    memcpy(&x, &u, sizeof u);
    return x;
}

void oracle_bf16_round(const float *x, int64_t n, float *y)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = bf16_round(x[i]);
}

/* c: [H, L] fp64 column masses. */
void oracle_col_scores(const float *q, const float *k, int H, int Hkv, int L,
                       int d, int B, double *c)
{
    int nb = L / B, G = H / Hkv;
    double scale = 1.0 / sqrt((double)d);
    float *qb = (float *)malloc(sizeof(float) * (size_t)H * nb * d);
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    oracle_pool(q, H, L, d, B, qb);
    for (int64_t x = 0; x < (int64_t)H * nb * d; ++x)
        qb[x] = bf16_round(qb[x]);
    for (int h = 0; h < H; ++h) {
        int g = h / G;
        const float *kh = k + (int64_t)g * L * d;
        double *ch = c + (int64_t)h * L;
        for (int u = 0; u < L; ++u)
            ch[u] = 0.0;
        for (int i = 0; i < nb; ++i) {
            const float *a = qb + ((int64_t)h * nb + i) * d;
            double m = -INFINITY;
            for (int u = 0; u < L; ++u) {
                const float *ku = kh + (int64_t)u * d;
                double dot = 0.0;
                for (int e = 0; e < d; ++e)
                    dot += (double)a[e] * (double)ku[e];
                z[u] = dot * scale;
                if (z[u] > m)
                    m = z[u];
            }
            double l = 0.0;
            for (int u = 0; u < L; ++u) {
                z[u] = exp(z[u] - m);
                l += z[u];
            }
            for (int u = 0; u < L; ++u)
                ch[u] += z[u] / l / nb;
        }
    }
    free(qb);
    free(z);
}

/* Per head, the k_c largest of the head's L column masses (fp32, the
 * precision the GPU decides in) under (value descending, index ascending),
 * listed in ascending column order: cols [H, k_c]. */
void oracle_col_select(const float *c, int H, int L, int64_t k_c, int32_t *cols)
{
    uint8_t *keep = (uint8_t *)malloc((size_t)L);
    for (int h = 0; h < H; ++h) {
        oracle_select(c + (int64_t)h * L, L, k_c, keep);
        int64_t n = 0;
        for (int u = 0; u < L; ++u)
            if (keep[u])
                cols[(int64_t)h * k_c + n++] = u;
    }
    free(keep);
}

/* The whole column mask: masses in fp64, rounded to fp32 (c_out, [H, L]),
 * then the per-head select.  Returns k_c. */
int64_t oracle_build_col_mask(const float *q, const float *k, int H, int Hkv,
                              int L, int d, int B, double s, float *c_out,
                              int32_t *cols)
{
    int64_t k_c = oracle_keep_count(L, s);
    double *c = (double *)malloc(sizeof(double) * (size_t)H * L);
    oracle_col_scores(q, k, H, Hkv, L, d, B, c);
    for (int64_t x = 0; x < (int64_t)H * L; ++x)
        c_out[x] = (float)c[x];
    oracle_col_select(c_out, H, L, k_c, cols);
    free(c);
    return k_c;
}

/* Column-sparse attention for the listed rows r = h*nb + i (all when rows ==
 * NULL): each query token of block i in head h attends to the key tokens
 * cols[h*k_c .. h*k_c + k_c) of key head h / (H/Hkv).  o: [H, L, d] fp64. */
void oracle_col_attn(const float *q, const float *k, const float *v, int H,
                     int Hkv, int L, int d, int B, const int32_t *cols,
                     int64_t k_c, const int32_t *rows, int n_rows, double *o)
{
    int nb = L / B, G = H / Hkv;
    int total = rows ? n_rows : H * nb;
    double *z = (double *)malloc(sizeof(double) * (size_t)(k_c > 0 ? k_c : 1));
    for (int x = 0; x < total; ++x) {
        int r = rows ? rows[x] : x;
        int h = r / nb, i = r % nb, g = h / G;
        const float *kh = k + (int64_t)g * L * d;
        const float *vh = v + (int64_t)g * L * d;
        for (int t = i * B; t < (i + 1) * B; ++t)
            attend_token(q + ((int64_t)h * L + t) * d, kh, vh, d,
                         cols + (int64_t)h * k_c, (int)k_c, z,
                         o + ((int64_t)h * L + t) * d);
    }
    free(z);
}

/* Recall of a column mask (mask quality, as oracle_mask_recall for blocks):
 * for row r = h*nb + i, the mean over the B query tokens t of block i of the
 * full bidirectional softmax probability that t puts on the kept key tokens
 * cols[h*k_c .. h*k_c + k_c) (all L keys in the normaliser), fp64.  1 when the
 * kept columns hold all of the rows' attention. */
void oracle_col_recall(const float *q, const float *k, int H, int Hkv, int L,
                       int d, int B, const int32_t *cols, int64_t k_c,
                       const int32_t *rows, int n_rows, double *recall)
{
    int nb = L / B, G = H / Hkv;
    int total = rows ? n_rows : H * nb;
    double scale = 1.0 / sqrt((double)d);
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    for (int x = 0; x < total; ++x) {
        int r = rows ? rows[x] : x;
        int h = r / nb, i = r % nb, g = h / G;
        const float *kh = k + (int64_t)g * L * d;
        const int32_t *ch = cols + (int64_t)h * k_c;
        double acc = 0.0;
        for (int t = i * B; t < (i + 1) * B; ++t) {
            const float *qt = q + ((int64_t)h * L + t) * d;
            double m = -INFINITY;
            for (int u = 0; u < L; ++u) {
                const float *ku = kh + (int64_t)u * d;
                double dot = 0.0;
                for (int e = 0; e < d; ++e)
                    dot += (double)qt[e] * (double)ku[e];
                z[u] = dot * scale;
                if (z[u] > m)
                    m = z[u];
            }
            double l = 0.0;
            for (int u = 0; u < L; ++u)
                l += exp(z[u] - m);
            double kept = 0.0;
            for (int64_t a = 0; a < k_c; ++a)
                kept += exp(z[ch[a]] - m);
            acc += kept / l;
        }
        recall[r] = acc / B;
    }
    free(z);
}

/* ----------------------------------------------------------------- driver --- */
/* What a denoising step runs ([SD] anchors + reuse; [SP] dense warm-up then
 * one mask reused): 0 = dense attention, 1 = anchor (rebuild the mask from
 * this step's Q/K, then sparse attention), 2 = sparse attention on the stored
 * mask.  refresh_every == 0 means the mask is built once, at the first
 * sparse step, and never refreshed. */
int oracle_step_kind(int step, int dense_steps, int refresh_every)
{
    if (step < dense_steps)
        return 0;
    int since = step - dense_steps;
    if (since == 0)
        return 1;
    if (refresh_every > 0 && since % refresh_every == 0)
        return 1;
    return 2;
}
