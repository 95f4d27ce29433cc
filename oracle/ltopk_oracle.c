/*
 * CPU oracle for CSA indexer top-k index selection.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no source, header, table or helper with the HIP library.
 *
 * What it computes (the plain definition, written out):
 *
 *   The CSA layer of DeepSeek-V4 keeps one compressed KV position per 4 tokens
 *   and lets each query attend only to the positions its indexer ranks highest
 *   ("SGLang DeepSeek V4 speaker page", aicon.infoq.cn, abstract and outline
 *   item 一.1). An index-source layer scores the query against the row's valid
 *   compressed positions and keeps at most 512 of them ("SGLang 与 Miles 为
 *   DeepSeek-V4.1 提供首日支持", xhh.club, Q&A on cross-layer sharing).
 *
 *   For one row s[0..n_max) with valid length len (clamped to [0, n_max]) and
 *   an optional candidate set C, the valid set is V = {i : 0 <= i < len} (and
 *   i in C when candidates are given). The selection order on V is
 *
 *       i before j  <=>  s_i ranks above s_j, or s_i ties s_j and i < j,
 *
 *   where the ranking is the real-number order with -0.0 equal to +0.0, +inf
 *   highest, -inf the lowest non-NaN value, and every NaN below -inf (NaNs tie
 *   with each other). The pages do not fix the tie rule; lower index first is
 *   the reading taken, so that the result is a pure function of the scores
 *   (the V4.1 page's commentary notes that the indexer top-k is recomputed
 *   during training rather than replayed, which needs exactly that).
 *
 *   The result is the first m = min(k, |V|) elements of V in that order; the
 *   remaining k - m output slots hold -1 ("up to 512": a row with fewer valid
 *   positions returns all of them). Output slots [0, m) are written in
 *   selection order here; callers compare as sets.
 *
 * Algorithm: collect (s_i, i) for i in V in increasing i, sort with a
 * comparator that is a strict total order (so any correct sort gives the same
 * sequence), copy the first m indices. O(|V| log |V|) per row.
 *
 * Block variant (the layer that publishes shared candidates, V4.1 page, Q&A on
 * cross-layer sharing: up to 2048 blocks of eight positions): block b covers
 * positions [b*bs, b*bs + bs); the blocks with at least one valid position are
 * b < ceil(len / bs); a block's score is the score of its first valid position
 * in the selection order (its maximum, NaN lowest). The single-row definition
 * is then applied to the block scores with block ids as indices. How a block
 * is scored is not stated on the pages; the maximum is the reading taken.
 *
 * Candidate variant (later index-source layers restrict their top-512 to the
 * published candidates, same page and answer): C = {b*bs + j : b a listed
 * block id >= 0, 0 <= j < bs}, treated as a set; output indices are global
 * positions.
 *
 * Build without -ffast-math: it would let the compiler assume no NaN and set
 * flush-to-zero/denormals-are-zero on x86, which changes comparisons.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    float s;
    int32_t i;
} lto_item;

/* 1 if a comes before b in the selection order. */
static int lto_before(const lto_item *a, const lto_item *b)
{
    int a_nan = isnan(a->s);
    int b_nan = isnan(b->s);
    if (a_nan != b_nan)
        return b_nan; /* every non-NaN ranks above every NaN */
    if (!a_nan && a->s != b->s)
        return a->s > b->s; /* real-number order; -0.0 == +0.0 here */
    return a->i < b->i; /* equal scores: lower index first */
}

static int lto_cmp(const void *pa, const void *pb)
{
    const lto_item *a = (const lto_item *)pa;
    const lto_item *b = (const lto_item *)pb;
    if (lto_before(a, b))
        return -1;
    if (lto_before(b, a))
        return 1;
    return 0;
}

static int64_t lto_clamp_len(int64_t len, int64_t n_max)
{
    if (len < 0)
        return 0;
    if (len > n_max)
        return n_max;
    return len;
}

/* Sort the items, write the first min(k, n) indices, pad with -1. */
static void lto_take(lto_item *items, int64_t n, int32_t k, int32_t *out)
{
    qsort(items, (size_t)n, sizeof(lto_item), lto_cmp);
    int64_t m = n < k ? n : k;
    for (int64_t r = 0; r < m; ++r)
        out[r] = items[r].i;
    for (int64_t r = m; r < k; ++r)
        out[r] = -1;
}

/*
 * One row. cand == NULL: no candidate restriction. Otherwise cand holds
 * n_cand block ids (negative ids are empty slots) of bs positions each.
 * out has k slots. Returns 0, or -1 on bad arguments / allocation failure.
 */
int lt_oracle_topk(const float *row, int64_t n_max, int64_t len, int32_t k,
                   const int32_t *cand, int32_t n_cand, int32_t bs,
                   int32_t *out)
{
    if (!row || !out || k < 1 || n_max < 0)
        return -1;
    if (cand && (bs < 1 || n_cand < 0))
        return -1;
    len = lto_clamp_len(len, n_max);

    unsigned char *member = NULL;
    if (cand) {
        member = (unsigned char *)calloc((size_t)(len > 0 ? len : 1), 1);
        if (!member)
            return -1;
        for (int32_t c = 0; c < n_cand; ++c) {
            int64_t b = cand[c];
            if (b < 0)
                continue;
            for (int64_t j = 0; j < bs; ++j) {
                int64_t pos = b * (int64_t)bs + j;
                if (pos < len)
                    member[pos] = 1;
            }
        }
    }

    lto_item *items = (lto_item *)malloc(sizeof(lto_item) * (size_t)(len > 0 ? len : 1));
    if (!items) {
        free(member);
        return -1;
    }
    int64_t n = 0;
    for (int64_t i = 0; i < len; ++i) {
        if (member && !member[i])
            continue;
        items[n].s = row[i];
        items[n].i = (int32_t)i;
        ++n;
    }
    lto_take(items, n, k, out);
    free(items);
    free(member);
    return 0;
}

/*
 * Block stage of one row: top-kb blocks of bs positions, each scored by the
 * first valid position of the block in the selection order.
 * out has kb slots and receives block ids. Returns 0 or -1.
 */
int lt_oracle_blocks(const float *row, int64_t n_max, int64_t len, int32_t bs,
                     int32_t kb, int32_t *out)
{
    if (!row || !out || bs < 1 || kb < 1 || n_max < 0)
        return -1;
    len = lto_clamp_len(len, n_max);
    int64_t nb = (len + bs - 1) / bs;
    lto_item *items = (lto_item *)malloc(sizeof(lto_item) * (size_t)(nb > 0 ? nb : 1));
    if (!items)
        return -1;
    for (int64_t b = 0; b < nb; ++b) {
        int64_t lo = b * (int64_t)bs;
        int64_t hi = lo + bs < len ? lo + bs : len;
        lto_item best = {row[lo], (int32_t)lo};
        for (int64_t i = lo + 1; i < hi; ++i) {
            lto_item cur = {row[i], (int32_t)i};
            if (lto_before(&cur, &best))
                best = cur;
        }
        items[b].s = best.s;
        items[b].i = (int32_t)b;
    }
    lto_take(items, nb, kb, out);
    free(items);
    return 0;
}

/* ---- batches: rows split into contiguous ranges over host threads ---- */

typedef struct {
    const float *scores;
    int64_t row_stride;
    const int32_t *lengths;
    int64_t n_max;
    int32_t k;
    const int32_t *cand;
    int32_t n_cand;
    int32_t bs;
    int32_t *out;
    int32_t row_lo, row_hi;
    int blocks_mode;
    int status;
} lto_job;

static void *lto_worker(void *arg)
{
    lto_job *j = (lto_job *)arg;
    j->status = 0;
    for (int32_t r = j->row_lo; r < j->row_hi; ++r) {
        const float *row = j->scores + (int64_t)r * j->row_stride;
        int32_t *o = j->out + (int64_t)r * j->k;
        int rc;
        if (j->blocks_mode)
            rc = lt_oracle_blocks(row, j->n_max, j->lengths[r], j->bs, j->k, o);
        else
            rc = lt_oracle_topk(row, j->n_max, j->lengths[r], j->k,
                                j->cand ? j->cand + (int64_t)r * j->n_cand : NULL,
                                j->n_cand, j->bs, o);
        if (rc)
            j->status = rc;
    }
    return NULL;
}

static int lto_run_batch(lto_job proto, int32_t B, int nthreads)
{
    if (B < 0 || !proto.scores || !proto.lengths || !proto.out)
        return -1;
    if (B == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > B)
        nthreads = B;
    lto_job *jobs = (lto_job *)calloc((size_t)nthreads, sizeof(lto_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -1;
    }
    int status = 0;
    int32_t per = B / nthreads, extra = B % nthreads, lo = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].row_lo = lo;
        lo += per + (t < extra ? 1 : 0);
        jobs[t].row_hi = lo;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, lto_worker, &jobs[t]) != 0) {
            /* run the rest of the work on this thread */
            for (int u = t; u < nthreads; ++u)
                lto_worker(&jobs[u]);
            break;
        }
        started = t;
    }
    lto_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tids[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status)
            status = jobs[t].status;
    free(jobs);
    free(tids);
    return status;
}

/* out: [B, k]; cand (optional): [B, n_cand]. Returns 0 or -1. */
int lt_oracle_topk_batch(const float *scores, int64_t row_stride,
                         const int32_t *lengths, int32_t B, int64_t n_max,
                         int32_t k, const int32_t *cand, int32_t n_cand,
                         int32_t bs, int32_t *out, int nthreads)
{
    if (row_stride < n_max || k < 1)
        return -1;
    lto_job p;
    memset(&p, 0, sizeof(p));
    p.scores = scores;
    p.row_stride = row_stride;
    p.lengths = lengths;
    p.n_max = n_max;
    p.k = k;
    p.cand = cand;
    p.n_cand = n_cand;
    p.bs = bs;
    p.out = out;
    return lto_run_batch(p, B, nthreads);
}

/* out: [B, kb] block ids. Returns 0 or -1. */
int lt_oracle_blocks_batch(const float *scores, int64_t row_stride,
                           const int32_t *lengths, int32_t B, int64_t n_max,
                           int32_t bs, int32_t kb, int32_t *out, int nthreads)
{
    if (row_stride < n_max || kb < 1 || bs < 1)
        return -1;
    lto_job p;
    memset(&p, 0, sizeof(p));
    p.scores = scores;
    p.row_stride = row_stride;
    p.lengths = lengths;
    p.n_max = n_max;
    p.k = kb;
    p.bs = bs;
    p.out = out;
    p.blocks_mode = 1;
    return lto_run_batch(p, B, nthreads);
}
