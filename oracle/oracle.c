/*
 * oracle.c -- plain fp64 CPU oracle for block/page-sparse decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no code, header, table or helper with
 * the HIP path.
 *
 * What it computes, step by step, in the order the pages describe it:
 *
 *   1. page summaries  -- Quest-style per-channel min and max of the keys of a
 *      page (hybrid sparse attention page: full-attention layers attend a
 *      256-token prefix, a recent window and the pages that Quest scores
 *      highest); MoBA-style block key taken as the mean of the block's keys
 *      (course module 14, section 14.3; the page's gate key is a trained
 *      parameter, which we replace by the mean because no weights exist);
 *      semantic-block centroid = unit-norm mean of unit-norm keys (semantic
 *      blocks page: keys are normalised and grouped by spherical k-means into
 *      blocks, and a query is compared with the block centres); compressed
 *      key of the block of two pages starting at the page, the mean of its
 *      keys (self-indexing attention page, "Compressed keys": blocks of l
 *      keys with stride d, stride/block about 0.5; the trained MLP that
 *      compresses a block is replaced by the mean because no weights exist).
 *   2. regions -- attention sink [0, S), sliding window of the last W
 *      positions [L-W, L), middle [S, L-W) (course module 14, section 14.2,
 *      StreamingLLM; self-indexing attention page, "Sliding window").
 *   3. scores -- per q-head, the exact maximum of q.x over the page's
 *      per-channel bounding box, sum_c max(q_c*mx_c, q_c*mn_c); or q.mean; or
 *      q.centroid; or, for compressed keys, the larger of q.c over the two
 *      blocks that cover the page (starting at the page before and at the
 *      page itself; the page's softmax over blocks is monotone, so it is
 *      skipped).  One selection per KV head: the group score is the maximum
 *      over the G query heads that share the KV head (GQA, attention-mechanisms
 *      article, "MQA/GQA"; MSA picks blocks per GQA group, same article,
 *      "Learned top-k sparse attention").
 *   4. top-k -- keep the k = min(floor(budget/P), #candidates) candidates with
 *      the largest group score, ties to the lower page index.
 *   5. token set -- sink, window and the middle-region part of every selected
 *      page, as a set, restricted to positions <= the query's position.
 *   6. exact softmax attention over the set, scale 1/sqrt(hd) (course module
 *      14, exercise 14.1: logits q.k/sqrt(d), max-subtracted softmax).
 *
 * All arithmetic is IEEE double.  Stored inputs (fp32 or bf16 bit patterns)
 * are converted to double exactly.  Every sum runs in plain index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_QUEST = 0, ORC_MEAN = 1, ORC_CENTROID = 2, ORC_COMPRESSED = 3 };

/* A paged KV cache: K and V are each [num_phys][Hkv][P][hd] in `dtype`. */
typedef struct {
    int B, Hq, Hkv, hd, P, max_pages, num_phys, dtype;
    const void* k;
    const void* v;
    const int32_t* block_table; /* [B][max_pages] logical page -> physical page */
    const int32_t* seq_lens;    /* [B] tokens in the cache, current token included */
} orc_cache;

/* ---- exact element conversion ------------------------------------------ */

static double elem(const void* base, int dtype, size_t idx)
{
    if (dtype == ORC_F32) return (double)((const float*)base)[idx];
    /* bf16: the upper 16 bits of an IEEE single */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* flat index of element c of token `t` of sequence b, KV head kvh */
static size_t kv_index(const orc_cache* c, int b, int kvh, int t, int ch)
{
    int page = t / c->P;
    int off = t % c->P;
    int phys = c->block_table[(size_t)b * c->max_pages + page];
    return (((size_t)phys * c->Hkv + kvh) * c->P + off) * c->hd + ch;
}

int orc_summary_size(int mode, int hd) { return mode == ORC_QUEST ? 2 * hd : hd; }

/* ---- step 1: summary of one logical page -------------------------------- */

/* Writes the summary of logical page `page` of (b, kvh) over its valid tokens
 * [page*P, min((page+1)*P, L)).  Quest: out[0..hd) = min, out[hd..2hd) = max.
 * Mean: out[c] = mean of k_c.  Centroid: u = sum of k/|k| (zero keys skipped),
 * out = u/|u| (all zeros when u = 0).  Compressed: the mean of the valid keys
 * of the two pages starting at `page`, [page*P, min((page+2)*P, L)).
 * Returns the number of tokens summarised. */
int orc_page_summary(const orc_cache* c, int mode, int b, int kvh, int page, double* out)
{
    int L = c->seq_lens[b];
    int t0 = page * c->P;
    int span = mode == ORC_COMPRESSED ? 2 * c->P : c->P;
    int t1 = t0 + span < L ? t0 + span : L;
    int n = t1 - t0;
    int hd = c->hd;
    if (n <= 0) return 0;
    if (mode == ORC_QUEST) {
        for (int ch = 0; ch < hd; ++ch) {
            double mn = INFINITY, mx = -INFINITY;
            for (int t = t0; t < t1; ++t) {
                double x = elem(c->k, c->dtype, kv_index(c, b, kvh, t, ch));
                if (x < mn) mn = x;
                if (x > mx) mx = x;
            }
            out[ch] = mn;
            out[hd + ch] = mx;
        }
    } else if (mode == ORC_MEAN || mode == ORC_COMPRESSED) {
        for (int ch = 0; ch < hd; ++ch) {
            double s = 0.0;
            for (int t = t0; t < t1; ++t) s += elem(c->k, c->dtype, kv_index(c, b, kvh, t, ch));
            out[ch] = s / n;
        }
    } else {
        for (int ch = 0; ch < hd; ++ch) out[ch] = 0.0;
        for (int t = t0; t < t1; ++t) {
            double nn = 0.0;
            for (int ch = 0; ch < hd; ++ch) {
                double x = elem(c->k, c->dtype, kv_index(c, b, kvh, t, ch));
                nn += x * x;
            }
            if (nn == 0.0) continue;
            double inv = 1.0 / sqrt(nn);
            for (int ch = 0; ch < hd; ++ch)
                out[ch] += elem(c->k, c->dtype, kv_index(c, b, kvh, t, ch)) * inv;
        }
        double un = 0.0;
        for (int ch = 0; ch < hd; ++ch) un += out[ch] * out[ch];
        if (un > 0.0) {
            double inv = 1.0 / sqrt(un);
            for (int ch = 0; ch < hd; ++ch) out[ch] *= inv;
        }
    }
    return n;
}

/* ---- step 3: the score of one page for one query head -------------------- */

double orc_page_score(int mode, const double* summ, const double* q, int hd)
{
    double s = 0.0;
    if (mode == ORC_QUEST) {
        for (int ch = 0; ch < hd; ++ch) {
            double a = q[ch] * summ[ch];      /* q_c * min_c */
            double b = q[ch] * summ[hd + ch]; /* q_c * max_c */
            s += a > b ? a : b;
        }
    } else {
        for (int ch = 0; ch < hd; ++ch) s += q[ch] * summ[ch];
    }
    return s;
}

/* ---- step 2: candidate test ---------------------------------------------- */

/* A page is a candidate when at least one of its valid tokens lies in the
 * middle region [S, L-W). */
static int is_candidate(int page, int P, int L, int S, int W)
{
    long lo = (long)page * P;
    long hi = lo + P < L ? lo + P : L;
    long mlo = S;
    long mhi = (long)L - W;
    long a = lo > mlo ? lo : mlo;
    long z = hi < mhi ? hi : mhi;
    return a < z;
}

/* ---- step 4: top-k ------------------------------------------------------- */

typedef struct {
    double s;
    int p;
} scored_page;

static int by_score_then_page(const void* x, const void* y)
{
    const scored_page* a = (const scored_page*)x;
    const scored_page* b = (const scored_page*)y;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return a->p < b->p ? -1 : (a->p > b->p);
}

static int ascending_int(const void* x, const void* y)
{
    int a = *(const int32_t*)x, b = *(const int32_t*)y;
    return a < b ? -1 : (a > b);
}

/* Orders the candidates (cand[p] != 0) by (score desc, page asc), keeps the
 * first min(k, #candidates) and writes them to sel in ascending page order.
 * Returns the number kept. */
int orc_topk(const double* score, const unsigned char* cand, int n_pages, int k, int32_t* sel)
{
    scored_page* v = (scored_page*)malloc(sizeof(scored_page) * (size_t)(n_pages > 0 ? n_pages : 1));
    int n = 0;
    for (int p = 0; p < n_pages; ++p)
        if (cand[p]) {
            v[n].s = score[p];
            v[n].p = p;
            ++n;
        }
    qsort(v, (size_t)n, sizeof(scored_page), by_score_then_page);
    int m = k < n ? k : n;
    if (m < 0) m = 0;
    for (int i = 0; i < m; ++i) sel[i] = v[i].p;
    qsort(sel, (size_t)m, sizeof(int32_t), ascending_int);
    free(v);
    return m;
}

/* ---- steps 5 and 6: token set and exact attention ------------------------ */

/* Marks the token set of a query at position `pos` in a cache of L tokens:
 * sink [0,S), window [L-W,L), and for each selected page its tokens inside
 * the middle region [S, L-W); everything restricted to t <= pos. */
static void mark_token_set(unsigned char* mark, int L, int P, int S, int W, int pos,
                           const int32_t* sel, int nsel)
{
    memset(mark, 0, (size_t)L);
    for (int t = 0; t < L; ++t)
        if (t < S || t >= L - W) mark[t] = 1;
    for (int i = 0; i < nsel; ++i) {
        long t0 = (long)sel[i] * P;
        for (long t = t0; t < t0 + P && t < L; ++t)
            if (t >= S && t < (long)L - W) mark[t] = 1;
    }
    for (int t = pos + 1; t < L; ++t) mark[t] = 0;
}

/* Softmax attention of one query head over the marked tokens of (b, kvh).
 * out[hd] = sum_t e^{z_t - m} v_t / l, *lse = m + ln l, z_t = scale * q.k_t.
 * Returns the number of tokens attended. */
static int attend_marked(const orc_cache* c, int b, int kvh, const double* q, const unsigned char* mark,
                         int L, double scale, double* z, double* out, double* lse)
{
    int hd = c->hd;
    double m = -INFINITY;
    int n = 0;
    for (int t = 0; t < L; ++t) {
        if (!mark[t]) continue;
        double d = 0.0;
        for (int ch = 0; ch < hd; ++ch) d += q[ch] * elem(c->k, c->dtype, kv_index(c, b, kvh, t, ch));
        z[t] = scale * d;
        if (z[t] > m) m = z[t];
        ++n;
    }
    double l = 0.0;
    for (int ch = 0; ch < hd; ++ch) out[ch] = 0.0;
    for (int t = 0; t < L; ++t) {
        if (!mark[t]) continue;
        double w = exp(z[t] - m);
        l += w;
        for (int ch = 0; ch < hd; ++ch) out[ch] += w * elem(c->v, c->dtype, kv_index(c, b, kvh, t, ch));
    }
    for (int ch = 0; ch < hd; ++ch) out[ch] /= l;
    *lse = m + log(l);
    return n;
}

/* ---- log-sum-exp merge of partial results -------------------------------- */

/* Merges n partial softmax states (o_s normalised by l_s, running max m_s)
 * into the attention over the union of their token sets: with m* = max m_s,
 * l = sum e^{m_s-m*} l_s and o = sum e^{m_s-m*} l_s o_s / l.  A part with
 * l_s = 0 (no tokens) contributes nothing.  Writes out[hd] and *lse. */
void orc_merge(int n, int hd, const double* o, const double* m, const double* l, double* out, double* lse)
{
    double mx = -INFINITY;
    for (int s = 0; s < n; ++s)
        if (l[s] > 0.0 && m[s] > mx) mx = m[s];
    double tot = 0.0;
    for (int ch = 0; ch < hd; ++ch) out[ch] = 0.0;
    for (int s = 0; s < n; ++s) {
        if (!(l[s] > 0.0)) continue;
        double w = exp(m[s] - mx) * l[s];
        tot += w;
        for (int ch = 0; ch < hd; ++ch) out[ch] += w * o[(size_t)s * hd + ch];
    }
    for (int ch = 0; ch < hd; ++ch) out[ch] /= tot;
    *lse = mx + log(tot);
}

/* ---- the whole step ----------------------------------------------------- */

/*
 * Runs steps 1-6 for every (b, kv head, query row).
 *
 *   q        [B][Hq][Q][hd] in the cache dtype; row i of sequence b sits at
 *            position L_b - Q + i.
 *   budget   token budget; k = floor(budget / P).
 *   sel_in   optional [B][Hkv][Q][kmax_in] logical pages (with cnt_in
 *            [B][Hkv][Q]); when given, steps 1-4 are skipped and this set is
 *            attended (parity on another implementation's selection).
 *   sel_out  [B][Hkv][Q][kmax] ascending, padded with -1; cnt_out [B][Hkv][Q]
 *   scores_out   optional [B][Hkv][Q][max_pages]; NaN for non-candidates
 *   hscores_out  optional [B][Hq][Q][max_pages] per-head scores; NaN likewise
 *   out      [B][Hq][Q][hd], lse [B][Hq][Q]
 *   ntok_out optional [B][Hq][Q] tokens attended
 * Returns 0, or -1 on an argument it cannot use.
 */
int orc_run(const orc_cache* c, int mode, const void* q, int Q, int S, int W, int budget, double scale,
            const int32_t* sel_in, const int32_t* cnt_in, int kmax_in, int32_t* sel_out, int32_t* cnt_out,
            double* scores_out, double* hscores_out, double* out, double* lse, int32_t* ntok_out, int nthreads)
{
    if (c->Hkv <= 0 || c->Hq % c->Hkv != 0 || W < 1 || S < 0 || budget < 0 || Q < 1) return -1;
    int G = c->Hq / c->Hkv;
    int hd = c->hd;
    int P = c->P;
    int kmax = budget / P;
    int msz = orc_summary_size(mode, hd);
    int jobs = c->B * c->Hkv;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int j = 0; j < jobs; ++j) {
        int b = j / c->Hkv, kvh = j % c->Hkv;
        int L = c->seq_lens[b];
        if (L < Q || L > c->max_pages * P) {
            err = 1;
            continue;
        }
        double* summ = (double*)calloc((size_t)c->max_pages * msz, sizeof(double));
        double* gscore = (double*)malloc(sizeof(double) * (size_t)c->max_pages);
        unsigned char* cand = (unsigned char*)calloc((size_t)c->max_pages, 1);
        int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(c->max_pages + 1));
        double* qh = (double*)malloc(sizeof(double) * (size_t)hd);
        unsigned char* mark = (unsigned char*)malloc((size_t)L + 1);
        double* z = (double*)malloc(sizeof(double) * ((size_t)L + 1));
        int n_pages = (L + P - 1) / P;
        if (!sel_in)
            for (int p = 0; p < n_pages; ++p) orc_page_summary(c, mode, b, kvh, p, summ + (size_t)p * msz);
        for (int i = 0; i < Q; ++i) {
            int pos = L - Q + i;
            int nsel;
            size_t row = ((size_t)b * c->Hkv + kvh) * Q + i;
            if (sel_in) {
                nsel = cnt_in[row];
                if (nsel < 0 || nsel > kmax_in || nsel > c->max_pages) {
                    err = 1;
                    nsel = 0;
                }
                memcpy(sel, sel_in + row * kmax_in, sizeof(int32_t) * (size_t)nsel);
            } else {
                for (int p = 0; p < c->max_pages; ++p) {
                    cand[p] = p < n_pages && is_candidate(p, P, L, S, W);
                    gscore[p] = NAN;
                }
                for (int g = 0; g < G; ++g) {
                    int h = kvh * G + g;
                    size_t qrow = (((size_t)b * c->Hq + h) * Q + i) * hd;
                    for (int ch = 0; ch < hd; ++ch) qh[ch] = elem(q, c->dtype, qrow + ch);
                    for (int p = 0; p < c->max_pages; ++p) {
                        double u = cand[p] ? orc_page_score(mode, summ + (size_t)p * msz, qh, hd) : NAN;
                        if (cand[p] && mode == ORC_COMPRESSED && p > 0) {
                            /* the block starting at the page before also covers this page */
                            double v = orc_page_score(mode, summ + (size_t)(p - 1) * msz, qh, hd);
                            if (v > u) u = v;
                        }
                        if (hscores_out) hscores_out[(((size_t)b * c->Hq + h) * Q + i) * c->max_pages + p] = u;
                        if (cand[p] && (g == 0 || u > gscore[p])) gscore[p] = u;
                    }
                }
                nsel = orc_topk(gscore, cand, c->max_pages, kmax, sel);
                if (scores_out) memcpy(scores_out + row * c->max_pages, gscore, sizeof(double) * (size_t)c->max_pages);
            }
            if (sel_out) {
                for (int s = 0; s < kmax; ++s) sel_out[row * kmax + s] = s < nsel ? sel[s] : -1;
            }
            if (cnt_out) cnt_out[row] = nsel;
            mark_token_set(mark, L, P, S, W, pos, sel, nsel);
            for (int g = 0; g < G; ++g) {
                int h = kvh * G + g;
                size_t hrow = ((size_t)b * c->Hq + h) * Q + i;
                for (int ch = 0; ch < hd; ++ch) qh[ch] = elem(q, c->dtype, hrow * hd + ch);
                int nt = attend_marked(c, b, kvh, qh, mark, L, scale, z, out + hrow * hd, lse + hrow);
                if (ntok_out) ntok_out[hrow] = nt;
            }
        }
        free(summ);
        free(gscore);
        free(cand);
        free(sel);
        free(qh);
        free(mark);
        free(z);
    }
    return err ? -1 : 0;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
