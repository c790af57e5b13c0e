/* oracle.c - FP64 CPU oracle for multi-row verify attention over a paged
 * FP8-E4M3 KV cache.  TEST INFRASTRUCTURE ONLY (see oracle.h): the product
 * library never calls it, and it shares no code with the HIP path.
 *
 * What it computes, and where the pages say so:
 *  - E4M3 bytes are decoded to exact values and attention runs on the
 *    dequantised cache.  The null-block fix commit of [NB] uses as its
 *    kernel-independent ground truth a decode of the E4M3 K/V to floating
 *    point followed by attention over the selected tokens only; the Test
 *    Plan of [QSA] compares the kernel with a reference on the dequantised
 *    cache; and "Rebuilt operator results" of [DN] quotes an FP64 companion
 *    reference.  This oracle is that reference, in FP64.
 *  - Row i sees the first len_i tokens ("live per-query lengths, including
 *    zero padding", [DN] first section).  A zero-length row outputs 0.
 *  - k_scale multiplies the logits and v_scale the output: [QSA] folds the
 *    K scale into the softmax scale on the host and treats the V scale as
 *    the kernel's output scale (review thread on host-side KV scales, and
 *    the commit moving k_scale out of the loop).  In exact arithmetic this is
 *    the same as dequantising K and V first.
 *  - Split partials: FP32 unnormalised partition numerators with a separate
 *    max and sum and a final combination ([DN] first section).  Here they are
 *    FP64 and use base 2 (logits times log2(e)), the base of the LSE that the
 *    DCP merge of [NB] exchanges.
 *  - The cache write quantises each FP16 K/V element x as E4M3(x / scale),
 *    the quotient formed in FP32 and rounded to the nearest code (ties to
 *    even, saturation at 448): [QSA] writes the uint8 cache with the layer's
 *    per-tensor scales through the unchanged write path.
 *
 * Plain loops, no blocking, no reordering: a reader can check each function
 * against the definition above.  The ORC_MUTANT switch plants one known
 * mistake at a time; it exists only so the tests can show that the pins
 * catch each of them, and is never set in the normal build.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORC_MUTANT
#define ORC_MUTANT 0
#endif

#define LOG2E 1.4426950408889634073599246810019

/* ------------------------------------------------------------------ */
/* Number formats                                                       */
/* ------------------------------------------------------------------ */

/* E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
 * is subnormal (m * 2^-9); no infinities; S.1111.111 is NaN; max 448. */
static double e4m3_value(unsigned code)
{
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double mag;
    if (e == 15u && m == 7u)
        return NAN;
    if (e == 0u)
        mag = ldexp((double)m, ORC_MUTANT == 10 ? -10 : -9);
    else
        mag = ldexp(8.0 + (double)m, (int)e - (ORC_MUTANT == 11 ? 11 : 10));
    return s ? -mag : mag;
}

void orc_e4m3_table(double tab[256])
{
    for (unsigned c = 0; c < 256u; ++c)
        tab[c] = e4m3_value(c);
}

/* Brute force: the code whose value is nearest to |x| among the 127
 * non-negative finite codes; on a tie the even code (mantissa LSB 0) wins. */
uint8_t orc_e4m3_encode(double x)
{
    unsigned sign, best = 0;
    double a, bd = INFINITY;
    if (isnan(x))
        return 0x7F;
    sign = signbit(x) ? 0x80u : 0u;
    a = fabs(x);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7Eu);
    for (unsigned c = 0; c <= 0x7Eu; ++c) {
        double d = fabs(e4m3_value(c) - a);
        int tie_wins = (ORC_MUTANT == 12) ? (c & 1u) == 1u : (c & 1u) == 0u;
        if (d < bd || (d == bd && tie_wins)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)(sign | best);
}

void orc_e4m3_encode_array(const double *x, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(x[i]);
}

/* Cache write: token t of k/v ([num_tokens][num_kv_heads][head_dim] FP16 bits)
 * goes to slot slot_mapping[t] (page = slot / page_size, row = slot % page_size;
 * negative = skip), element (g, d) to byte page*page_stride + row*token_stride
 * + g*head_stride + d of each plane, as E4M3(fp32(x) / fp32(scale)).  Returns
 * -1 if a slot lies past num_pages * page_size. */
int orc_cache_write(const uint16_t *k, const uint16_t *v, int64_t num_tokens,
                    int32_t num_kv_heads, int32_t head_dim, const int64_t *slot_mapping,
                    uint8_t *k_pool, uint8_t *v_pool, int64_t page_stride, int64_t token_stride,
                    int64_t head_stride, int32_t num_pages, int32_t page_size, float k_scale,
                    float v_scale)
{
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0)
            continue;
        if (slot >= (int64_t)num_pages * page_size)
            return -1;
        int64_t page = slot / page_size, row = slot % page_size;
        for (int32_t g = 0; g < num_kv_heads; ++g) {
            for (int32_t d = 0; d < head_dim; ++d) {
                int64_t src = (t * num_kv_heads + g) * head_dim + d;
                int64_t dst = page * page_stride + row * token_stride + g * head_stride + d;
                float xk = (float)orc_fp16_value(k[src]) / k_scale;
                float xv = (float)orc_fp16_value(v[src]) / v_scale;
                k_pool[dst] = orc_e4m3_encode((double)xk);
                v_pool[dst] = orc_e4m3_encode((double)xv);
            }
        }
    }
    return 0;
}

/* binary16: 5 exponent bits (bias 15), 10 mantissa bits. */
double orc_fp16_value(uint16_t h)
{
    unsigned s = (h >> 15) & 1u, e = (h >> 10) & 31u, m = h & 1023u;
    double mag;
    if (e == 31u)
        mag = m ? NAN : INFINITY;
    else if (e == 0u)
        mag = ldexp((double)m, -24);
    else
        mag = ldexp(1024.0 + (double)m, (int)e - 25);
    return s ? -mag : mag;
}

/* bfloat16: 8 exponent bits (bias 127), 7 mantissa bits. */
double orc_bf16_value(uint16_t h)
{
    unsigned s = (h >> 15) & 1u, e = (h >> 7) & 255u, m = h & 127u;
    double mag;
    if (e == 255u)
        mag = m ? NAN : INFINITY;
    else if (e == 0u)
        mag = ldexp((double)m, -133);
    else
        mag = ldexp(128.0 + (double)m, (int)e - 134);
    return s ? -mag : mag;
}

/* ------------------------------------------------------------------ */
/* One output row: the token list, then softmax attention over it       */
/* ------------------------------------------------------------------ */

typedef struct {
    const uint8_t *k_pool, *v_pool;
    int64_t page_stride, token_stride, head_stride;
    int32_t num_pages, page_size, head_dim;
} pool_t;

/* Byte offset of token u of physical page p, KV head g. */
static int64_t kv_offset(const pool_t *pl, int64_t p, int64_t u, int64_t g)
{
    return p * pl->page_stride + u * pl->token_stride + g * pl->head_stride;
}

/* Attention of one query row over a list of n tokens given by byte offsets.
 * qv[d] are the query values.  Writes the FP64 output row (times v_scale). */
static void attend_row(const pool_t *pl, const double *tab, const double *qv,
                       const int64_t *off, int64_t n, double logit_scale, double v_scale,
                       double *s, double *out)
{
    int D = pl->head_dim;
    double m = -INFINITY, den = 0.0;
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (n == 0)
        return;
    for (int64_t t = 0; t < n; ++t) {
        const uint8_t *kp = pl->k_pool + off[t];
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qv[d] * tab[kp[d]];
        s[t] = logit_scale * dot;
        if (s[t] > m)
            m = s[t];
    }
    for (int64_t t = 0; t < n; ++t) {
        const uint8_t *vp = pl->v_pool + off[t];
        double w = (ORC_MUTANT == 4) ? exp(m - s[t]) : exp(s[t] - m);
        den += w;
        for (int d = 0; d < D; ++d)
            out[d] += w * tab[vp[d]];
    }
    for (int d = 0; d < D; ++d)
        out[d] = (ORC_MUTANT == 6 ? 1.0 : v_scale) * out[d] / den;
}

/* Split partials of one row over a list of n tokens, split by list index. */
static void split_row(const pool_t *pl, const double *tab, const double *qv,
                      const int64_t *off, const int64_t *pos, int64_t n,
                      double logit_scale, int S, int64_t T, int num_rows, int row,
                      double *y, double *ws_acc, double *ws_max, double *ws_sum)
{
    int D = pl->head_dim;
    for (int64_t t = 0; t < n; ++t) {
        const uint8_t *kp = pl->k_pool + off[t];
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qv[d] * tab[kp[d]];
        y[t] = logit_scale * dot * LOG2E;
    }
    for (int sp = 0; sp < S; ++sp) {
        int64_t lo = (int64_t)sp * T + (ORC_MUTANT == 8 ? 1 : 0), hi = lo + T;
        double m = -INFINITY, l = 0.0;
        double *acc = ws_acc + ((int64_t)sp * num_rows + row) * D;
        for (int d = 0; d < D; ++d)
            acc[d] = 0.0;
        for (int64_t t = 0; t < n; ++t)
            if (pos[t] >= lo && pos[t] < hi && y[t] > m)
                m = y[t];
        for (int64_t t = 0; t < n; ++t) {
            if (pos[t] >= lo && pos[t] < hi) {
                const uint8_t *vp = pl->v_pool + off[t];
                double w = exp2(y[t] - m);
                l += w;
                for (int d = 0; d < D; ++d)
                    acc[d] += w * tab[vp[d]];
            }
        }
        ws_max[(int64_t)sp * num_rows + row] = m;
        ws_sum[(int64_t)sp * num_rows + row] = l;
    }
}

/* ------------------------------------------------------------------ */
/* Problem descriptions and the per-row token lists                      */
/* ------------------------------------------------------------------ */

typedef struct {
    int sparse;                 /* 0: dense one request, 1: QSA batch over selected
                                   blocks, 2: QSA batch over selected token ids */
    const uint16_t *q;
    pool_t pool;
    const int32_t *block_table;
    int32_t num_entries;        /* dense: table length; QSA: max_blocks */
    const int32_t *sel;
    int32_t topk;
    const int32_t *row_lens;
    int32_t max_tokens;         /* dense clamp bound */
    int32_t batch, q_rows, num_heads, num_kv_heads;
    double sm_scale, k_scale, v_scale;
    /* split mode */
    int split;
    int32_t num_splits, tokens_per_split;
    double *out, *ws_acc, *ws_max, *ws_sum;
    /* threading */
    int32_t nthreads, tid;
    int status;
} problem_t;

static double q_value(const problem_t *pb, int b, int i, int h, int d)
{
    int D = pb->pool.head_dim;
    int64_t idx;
    if (ORC_MUTANT == 5)
        idx = (((int64_t)b * pb->num_heads + h) * pb->q_rows + i) * D + d;
    else
        idx = (((int64_t)b * pb->q_rows + i) * pb->num_heads + h) * D + d;
    return pb->sparse ? orc_bf16_value(pb->q[idx]) : orc_fp16_value(pb->q[idx]);
}

static int kv_head_of(const problem_t *pb, int h)
{
    int G = pb->num_heads / pb->num_kv_heads;
    return (ORC_MUTANT == 1) ? h % pb->num_kv_heads : h / G;
}

/* Token list of row (b, i) of KV head g: byte offsets and list positions.
 * Returns the count, or -1 on an out-of-range page id or selection. */
static int64_t token_list(const problem_t *pb, int b, int i, int g, int64_t *off, int64_t *pos)
{
    const pool_t *pl = &pb->pool;
    int64_t n = 0, L;
    if (!pb->sparse) {
        L = pb->row_lens[i];
        if (L < 0)
            L = 0;
        if (L > pb->max_tokens)
            L = pb->max_tokens;
        if (ORC_MUTANT == 3 && L < pb->max_tokens)
            L += 1;
        for (int64_t t = 0; t < L; ++t) {
            int64_t lp = t / pl->page_size, u = t % pl->page_size, phys;
            if (lp >= pb->num_entries)
                return -1;
            phys = (ORC_MUTANT == 7) ? lp : pb->block_table[lp];
            if (phys < 0 || phys >= pl->num_pages)
                return -1;
            off[n] = kv_offset(pl, phys, u, g);
            pos[n] = t;
            ++n;
        }
    } else if (pb->sparse == 2) {
        /* list entry j is a logical token id (-1: empty); the row sees it when
         * id < its length; the entry's block is located through the table */
        int64_t cap = (int64_t)pb->num_entries * pl->page_size;
        L = pb->row_lens[(int64_t)b * pb->q_rows + i];
        if (L < 0)
            L = 0;
        if (L > cap)
            L = cap;
        for (int j = 0; j < pb->topk; ++j) {
            int64_t t = pb->sel[((int64_t)b * pb->num_kv_heads + g) * pb->topk + j];
            int64_t lp, u, phys;
            if (t < 0 || (ORC_MUTANT == 15 ? t > L : t >= L))
                continue;
            lp = t / pl->page_size;
            u = t % pl->page_size;
            phys = pb->block_table[(ORC_MUTANT == 16 ? 0 : (int64_t)b * pb->num_entries) + lp];
            if (phys < 0 || phys >= pl->num_pages)
                return -1;
            off[n] = kv_offset(pl, phys, u, g);
            pos[n] = j;
            ++n;
        }
    } else {
        int64_t cap = (int64_t)pb->num_entries * pl->page_size;
        L = pb->row_lens[(int64_t)b * pb->q_rows + i];
        if (L < 0)
            L = 0;
        if (L > cap)
            L = cap;
        for (int j = 0; j < pb->topk; ++j) {
            int32_t blk = pb->sel[((int64_t)b * pb->num_kv_heads + g) * pb->topk + j];
            int64_t phys;
            if (ORC_MUTANT == 13 && blk >= 0)
                blk = j;
            if (blk < 0)
                continue;
            if (blk >= pb->num_entries)
                return -1;
            phys = pb->block_table[(int64_t)b * pb->num_entries + blk];
            if (phys < 0 || phys >= pl->num_pages)
                return -1;
            for (int64_t u = 0; u < pl->page_size; ++u) {
                int64_t t = (ORC_MUTANT == 14) ? (int64_t)j * pl->page_size + u
                                               : (int64_t)blk * pl->page_size + u;
                if (t < L) {
                    off[n] = kv_offset(pl, phys, u, g);
                    pos[n] = (int64_t)j * pl->page_size + u;
                    ++n;
                }
            }
        }
    }
    return n;
}

static void *worker(void *arg)
{
    problem_t *pb = (problem_t *)arg;
    const pool_t *pl = &pb->pool;
    int D = pl->head_dim, H = pb->num_heads;
    int64_t cap = pb->sparse == 2 ? (int64_t)pb->topk
                  : pb->sparse ? (int64_t)pb->topk * pl->page_size : pb->max_tokens;
    int num_rows = pb->batch * pb->q_rows * H;
    double tab[256], *qv, *s;
    int64_t *off, *pos;
    double logit_scale = pb->sm_scale * (ORC_MUTANT == 2 ? 1.0 : pb->k_scale);

    orc_e4m3_table(tab);
    qv = (double *)malloc(sizeof(double) * (size_t)D);
    s = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
    pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
    if (!qv || !s || !off || !pos) {
        pb->status = -2;
        goto done;
    }
    for (int row = pb->tid; row < num_rows; row += pb->nthreads) {
        int h = row % H, i = (row / H) % pb->q_rows, b = row / (H * pb->q_rows);
        int g = kv_head_of(pb, h);
        int64_t n = token_list(pb, b, i, g, off, pos);
        if (n < 0) {
            pb->status = -1;
            goto done;
        }
        for (int d = 0; d < D; ++d)
            qv[d] = q_value(pb, b, i, h, d);
        if (!pb->split)
            attend_row(pl, tab, qv, off, n, logit_scale, pb->v_scale, s,
                       pb->out + (int64_t)row * D);
        else
            split_row(pl, tab, qv, off, pos, n, logit_scale, pb->num_splits,
                      pb->tokens_per_split, num_rows, row, s, pb->ws_acc, pb->ws_max,
                      pb->ws_sum);
    }
done:
    free(qv);
    free(s);
    free(off);
    free(pos);
    return NULL;
}

static int run(const problem_t *tmpl)
{
    int nt = tmpl->nthreads < 1 ? 1 : tmpl->nthreads;
    problem_t *jobs;
    pthread_t *th;
    int status = 0;
    if (tmpl->num_kv_heads <= 0 || tmpl->num_heads % tmpl->num_kv_heads != 0 ||
        tmpl->pool.page_size <= 0 || tmpl->pool.head_dim <= 0)
        return -1;
    if (tmpl->split && (tmpl->num_splits <= 0 || tmpl->tokens_per_split <= 0))
        return -1;
    jobs = (problem_t *)calloc((size_t)nt, sizeof(problem_t));
    th = (pthread_t *)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -2;
    }
    for (int t = 0; t < nt; ++t) {
        jobs[t] = *tmpl;
        jobs[t].nthreads = nt;
        jobs[t].tid = t;
        jobs[t].status = 0;
    }
    for (int t = 1; t < nt; ++t)
        if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0)
            jobs[t].status = -3;
    worker(&jobs[0]);
    for (int t = 1; t < nt; ++t)
        if (jobs[t].status != -3)
            pthread_join(th[t], NULL);
    for (int t = 0; t < nt; ++t)
        if (jobs[t].status < status)
            status = jobs[t].status;
    free(jobs);
    free(th);
    return status;
}

static problem_t base_problem(int sparse, const uint16_t *q, const uint8_t *k_pool,
                              const uint8_t *v_pool, int64_t page_stride,
                              int64_t token_stride, int64_t head_stride, int32_t num_pages,
                              int32_t page_size, int32_t head_dim)
{
    problem_t pb;
    memset(&pb, 0, sizeof pb);
    pb.sparse = sparse;
    pb.q = q;
    pb.pool.k_pool = k_pool;
    pb.pool.v_pool = v_pool;
    pb.pool.page_stride = page_stride;
    pb.pool.token_stride = token_stride;
    pb.pool.head_stride = head_stride;
    pb.pool.num_pages = num_pages;
    pb.pool.page_size = page_size;
    pb.pool.head_dim = head_dim;
    pb.batch = 1;
    return pb;
}

int orc_verify_dense(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                     int64_t page_stride, int64_t token_stride, int64_t head_stride,
                     int32_t num_pages, int32_t page_size,
                     const int32_t *block_table, int32_t num_entries,
                     const int32_t *row_lens, int32_t max_tokens,
                     int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                     int32_t head_dim, double sm_scale, double k_scale, double v_scale,
                     int32_t nthreads, double *out)
{
    problem_t pb = base_problem(0, q, k_pool, v_pool, page_stride, token_stride, head_stride,
                                num_pages, page_size, head_dim);
    pb.block_table = block_table;
    pb.num_entries = num_entries;
    pb.row_lens = row_lens;
    pb.max_tokens = max_tokens;
    pb.q_rows = q_rows;
    pb.num_heads = num_heads;
    pb.num_kv_heads = num_kv_heads;
    pb.sm_scale = sm_scale;
    pb.k_scale = k_scale;
    pb.v_scale = v_scale;
    pb.nthreads = nthreads;
    pb.out = out;
    return run(&pb);
}

int orc_verify_dense_split(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                           int64_t page_stride, int64_t token_stride, int64_t head_stride,
                           int32_t num_pages, int32_t page_size,
                           const int32_t *block_table, int32_t num_entries,
                           const int32_t *row_lens, int32_t max_tokens,
                           int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, double sm_scale, double k_scale,
                           int32_t num_splits, int32_t tokens_per_split, int32_t nthreads,
                           double *ws_acc, double *ws_max, double *ws_sum)
{
    problem_t pb = base_problem(0, q, k_pool, v_pool, page_stride, token_stride, head_stride,
                                num_pages, page_size, head_dim);
    pb.block_table = block_table;
    pb.num_entries = num_entries;
    pb.row_lens = row_lens;
    pb.max_tokens = max_tokens;
    pb.q_rows = q_rows;
    pb.num_heads = num_heads;
    pb.num_kv_heads = num_kv_heads;
    pb.sm_scale = sm_scale;
    pb.k_scale = k_scale;
    pb.split = 1;
    pb.num_splits = num_splits;
    pb.tokens_per_split = tokens_per_split;
    pb.nthreads = nthreads;
    pb.ws_acc = ws_acc;
    pb.ws_max = ws_max;
    pb.ws_sum = ws_sum;
    return run(&pb);
}

int orc_qsa_verify(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                   int64_t page_stride, int64_t token_stride, int64_t head_stride,
                   int32_t num_pages, int32_t page_size,
                   const int32_t *block_table, int32_t max_blocks,
                   const int32_t *sel, int32_t topk, const int32_t *row_lens,
                   int32_t batch, int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                   int32_t head_dim, double sm_scale, double k_scale, double v_scale,
                   int32_t nthreads, double *out)
{
    problem_t pb = base_problem(1, q, k_pool, v_pool, page_stride, token_stride, head_stride,
                                num_pages, page_size, head_dim);
    pb.block_table = block_table;
    pb.num_entries = max_blocks;
    pb.sel = sel;
    pb.topk = topk;
    pb.row_lens = row_lens;
    pb.batch = batch;
    pb.q_rows = q_rows;
    pb.num_heads = num_heads;
    pb.num_kv_heads = num_kv_heads;
    pb.sm_scale = sm_scale;
    pb.k_scale = k_scale;
    pb.v_scale = v_scale;
    pb.nthreads = nthreads;
    pb.out = out;
    return run(&pb);
}

int orc_qsa_split(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                  int64_t page_stride, int64_t token_stride, int64_t head_stride,
                  int32_t num_pages, int32_t page_size,
                  const int32_t *block_table, int32_t max_blocks,
                  const int32_t *sel, int32_t topk, const int32_t *row_lens,
                  int32_t batch, int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                  int32_t head_dim, double sm_scale, double k_scale,
                  int32_t num_splits, int32_t tokens_per_split, int32_t nthreads,
                  double *ws_acc, double *ws_max, double *ws_sum)
{
    problem_t pb = base_problem(1, q, k_pool, v_pool, page_stride, token_stride, head_stride,
                                num_pages, page_size, head_dim);
    pb.block_table = block_table;
    pb.num_entries = max_blocks;
    pb.sel = sel;
    pb.topk = topk;
    pb.row_lens = row_lens;
    pb.batch = batch;
    pb.q_rows = q_rows;
    pb.num_heads = num_heads;
    pb.num_kv_heads = num_kv_heads;
    pb.sm_scale = sm_scale;
    pb.k_scale = k_scale;
    pb.split = 1;
    pb.num_splits = num_splits;
    pb.tokens_per_split = tokens_per_split;
    pb.nthreads = nthreads;
    pb.ws_acc = ws_acc;
    pb.ws_max = ws_max;
    pb.ws_sum = ws_sum;
    return run(&pb);
}

int orc_qsa_tokens_verify(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                          int64_t page_stride, int64_t token_stride, int64_t head_stride,
                          int32_t num_pages, int32_t page_size,
                          const int32_t *block_table, int32_t max_blocks,
                          const int32_t *sel_tokens, int32_t num_sel, const int32_t *row_lens,
                          int32_t batch, int32_t q_rows, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, double sm_scale,
                          double k_scale, double v_scale, int32_t nthreads, double *out)
{
    problem_t pb = base_problem(2, q, k_pool, v_pool, page_stride, token_stride, head_stride,
                                num_pages, page_size, head_dim);
    pb.block_table = block_table;
    pb.num_entries = max_blocks;
    pb.sel = sel_tokens;
    pb.topk = num_sel;
    pb.row_lens = row_lens;
    pb.batch = batch;
    pb.q_rows = q_rows;
    pb.num_heads = num_heads;
    pb.num_kv_heads = num_kv_heads;
    pb.sm_scale = sm_scale;
    pb.k_scale = k_scale;
    pb.v_scale = v_scale;
    pb.nthreads = nthreads;
    pb.out = out;
    return run(&pb);
}

int orc_qsa_tokens_split(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                         int64_t page_stride, int64_t token_stride, int64_t head_stride,
                         int32_t num_pages, int32_t page_size,
                         const int32_t *block_table, int32_t max_blocks,
                         const int32_t *sel_tokens, int32_t num_sel, const int32_t *row_lens,
                         int32_t batch, int32_t q_rows, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, double sm_scale,
                         double k_scale, int32_t num_splits, int32_t tokens_per_split,
                         int32_t nthreads, double *ws_acc, double *ws_max, double *ws_sum)
{
    problem_t pb = base_problem(2, q, k_pool, v_pool, page_stride, token_stride, head_stride,
                                num_pages, page_size, head_dim);
    pb.block_table = block_table;
    pb.num_entries = max_blocks;
    pb.sel = sel_tokens;
    pb.topk = num_sel;
    pb.row_lens = row_lens;
    pb.batch = batch;
    pb.q_rows = q_rows;
    pb.num_heads = num_heads;
    pb.num_kv_heads = num_kv_heads;
    pb.sm_scale = sm_scale;
    pb.k_scale = k_scale;
    pb.split = 1;
    pb.num_splits = num_splits;
    pb.tokens_per_split = tokens_per_split;
    pb.nthreads = nthreads;
    pb.ws_acc = ws_acc;
    pb.ws_max = ws_max;
    pb.ws_sum = ws_sum;
    return run(&pb);
}

/* ------------------------------------------------------------------ */
/* Combination of split partials                                        */
/* ------------------------------------------------------------------ */

static int combine_any(const double *acc64, const float *acc32, const double *mx64,
                       const float *mx32, const double *sm64, const float *sm32, int S,
                       int R, int D, double v_scale, double *out, double *lse)
{
    if (S <= 0 || R < 0 || D <= 0)
        return -1;
    for (int r = 0; r < R; ++r) {
        double M = -INFINITY, den = 0.0;
        for (int s = 0; s < S; ++s) {
            int64_t k = (int64_t)s * R + r;
            double l = sm64 ? sm64[k] : (double)(ORC_MUTANT == 17 ? mx32[k] : sm32[k]);
            double m = mx64 ? mx64[k] : (double)mx32[k];
            if (l != 0.0 && m > M)
                M = m;
        }
        for (int d = 0; d < D; ++d)
            out[(int64_t)r * D + d] = 0.0;
        for (int s = 0; s < S; ++s) {
            int64_t k = (int64_t)s * R + r;
            double l = sm64 ? sm64[k] : (double)(ORC_MUTANT == 17 ? mx32[k] : sm32[k]);
            double m = mx64 ? mx64[k] : (double)mx32[k];
            double w;
            if (l == 0.0)              /* empty split; a NaN sum is not empty */
                continue;
            w = (ORC_MUTANT == 9) ? 1.0 : exp2(m - M);
            den += w * l;
            for (int d = 0; d < D; ++d) {
                int64_t a = k * D + d;
                int64_t a32 = (ORC_MUTANT == 18) ? (int64_t)r * D + d : a;
                out[(int64_t)r * D + d] += w * (acc64 ? acc64[a] : (double)acc32[a32]);
            }
        }
        for (int d = 0; d < D; ++d)
            out[(int64_t)r * D + d] = den != 0.0 ? v_scale * out[(int64_t)r * D + d] / den : 0.0;
        /* base-2 log of the row's whole sum: log2 sum_t 2^(y_t) = M + log2(den) */
        if (lse)
            lse[r] = den != 0.0 ? M + log2(den) : -INFINITY;
    }
    return 0;
}

int orc_combine(const double *ws_acc, const double *ws_max, const double *ws_sum,
                int32_t num_splits, int32_t num_rows, int32_t head_dim, double v_scale,
                double *out)
{
    return combine_any(ws_acc, NULL, ws_max, NULL, ws_sum, NULL, num_splits, num_rows,
                       head_dim, v_scale, out, NULL);
}

int orc_combine_f32(const float *ws_acc, const float *ws_max, const float *ws_sum,
                    int32_t num_splits, int32_t num_rows, int32_t head_dim, double v_scale,
                    double *out)
{
    return combine_any(NULL, ws_acc, NULL, ws_max, NULL, ws_sum, num_splits, num_rows,
                       head_dim, v_scale, out, NULL);
}

int orc_combine_lse(const double *ws_acc, const double *ws_max, const double *ws_sum,
                    int32_t num_splits, int32_t num_rows, int32_t head_dim, double v_scale,
                    double *out, double *lse)
{
    return combine_any(ws_acc, NULL, ws_max, NULL, ws_sum, NULL, num_splits, num_rows,
                       head_dim, v_scale, out, lse);
}

int orc_combine_lse_f32(const float *ws_acc, const float *ws_max, const float *ws_sum,
                        int32_t num_splits, int32_t num_rows, int32_t head_dim, double v_scale,
                        double *out, double *lse)
{
    return combine_any(NULL, ws_acc, NULL, ws_max, NULL, ws_sum, num_splits, num_rows,
                       head_dim, v_scale, out, lse);
}
