/*
 * oracle.c -- plain CPU fp64 reference of selector-driven top-k sparse attention.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP library, and the HIP library never calls it.
 *
 * It writes the definitions out directly, in double precision, from the exact
 * fp32 / bf16 input values, with no blocking, fusion or reordering:
 *
 *   compress  K~_j = mean of the keys of block j (g consecutive tokens, one KV
 *             head): the parameter-free mean pooling of keys that InfLLM-V2
 *             uses (SparDA summary, Method).  L2SUM: each key divided by its
 *             L2 norm, then the keys summed (LSA deep-read, §2.2).  The pooling
 *             window of block j is its own tokens [jg, e_j] reaching `overlap`
 *             tokens further back (clipped at token 0): kernel g + overlap,
 *             stride g, the overlapping compressed keys of InfLLM-V2 (SparDA
 *             summary, Method); overlap 0 gives disjoint blocks.  A last
 *             partial block pools the tokens it has.  A zero key contributes
 *             zero to L2SUM.
 *
 *   select    one score per candidate block and GQA group (SparDA summary,
 *             Method: one selector head per GQA group).  Mode SUM: the group's
 *             query heads summed, dotted with K~_j, over sqrt(d) (LSA
 *             deep-read, §2.4: the heads summed into one index query).  Mode
 *             SOFTMAX: for every head h, the softmax over the row's candidates
 *             of q_h.K~_j / tau, summed over the group's heads (the SparDA
 *             training target, SparDA summary, Method).  Mode MAX: the largest
 *             over the group's heads of q_h.K~_j / sqrt(d) (N-LSA scores a
 *             bucket by its best head, LSA deep-read, §2.5).  Mode ATTN: the
 *             attention mass a dense verify pass puts on the block, summed over
 *             the row's queries i and the group's heads h: the sum over the
 *             block's tokens t of exp(q_ih.k_t / sqrt(d) - lse_ih), lse_ih the
 *             log-sum-exp of query i, head h over every key up to its position
 *             (S3R review: the verifier's attention weights refresh the subset
 *             the next drafts read).  With several queries in a row, q_h sums
 *             head h over them (modes SUM, SOFTMAX, MAX).  Candidates are the blocks
 *             that lie wholly at or before the selection position p_sel and
 *             hold at least one token outside the init/window set F(p_sel).
 *             The k best by (score descending, block index ascending) are kept
 *             and written in ascending block order.  With shared selection
 *             (S3R review, sparse drafting: one selection reused by k drafts)
 *             a sequence has one row at p_sel = first query position - 1, and
 *             its score query sums every query of the sequence as well.
 *
 *   attend    softmax over the attended set only, o = sum_t softmax(l)_t v_t
 *             with l_t = scale * q.k_t (PulseCol, §3.1 Eq. (1) and Eq. (2)
 *             with M(S) = 0 on the set and -inf elsewhere; S3R review, sparse
 *             drafting formula).  The set is the union of the init tokens, the
 *             local window [p_sel - w + 1, p] and the tokens of the selected
 *             blocks, cut at the query position p (SparDA summary, Method:
 *             init tokens, sliding window and top-k blocks merged into one
 *             sparse attention).
 *
 * Element types: 0 = fp32, 1 = bf16 given as raw 16-bit patterns.
 * Layouts: Q [sum M_b, Hq, d]; K, V [sum N_b, Hkv, d]; K~ [Hkv, batch, nb_max, d];
 * selection tables [Hkv, rows, kcap].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1
#define OR_MEAN 0
#define OR_L2SUM 1
#define OR_SEL_SUM 0
#define OR_SEL_SOFTMAX 1
#define OR_SEL_MAX 2
#define OR_SEL_ATTN 3

static double elem(const void *base, int dtype, int64_t i)
{
    if (dtype == OR_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void or_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* First query position of sequence b: q_pos0[b], else right-aligned N_b - M_b. */
static int64_t first_query_pos(int b, const int32_t *cu_q, const int32_t *cu_k, const int32_t *q_pos0)
{
    if (q_pos0)
        return q_pos0[b];
    return (int64_t)(cu_k[b + 1] - cu_k[b]) - (int64_t)(cu_q[b + 1] - cu_q[b]);
}

static int seq_of_query(int64_t i, int batch, const int32_t *cu_q)
{
    int b = 0;
    while (b + 1 < batch && i >= cu_q[b + 1])
        b++;
    return b;
}

/* ---------------------------------------------------------------- compress */

int or_compress(int batch, int h_kv, int d, const int32_t *cu_k, int g, int pool, int overlap, int dtype,
                const void *k, int64_t nb_max, double *k_cmp)
{
    if (g < 1 || d < 1 || overlap < 0)
        return 1;
    int64_t n_items = (int64_t)h_kv * batch * nb_max;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t it = 0; it < n_items; it++) {
        int64_t j = it % nb_max;
        int b = (int)((it / nb_max) % batch);
        int c = (int)(it / (nb_max * batch));
        int64_t n_b = cu_k[b + 1] - cu_k[b];
        int64_t t0 = j * g - overlap, t1 = (j + 1) * (int64_t)g;
        double *out = k_cmp + it * d;
        if (t0 < 0)
            t0 = 0;
        if (t1 > n_b)
            t1 = n_b;
        for (int e = 0; e < d; e++)
            out[e] = 0.0;
        if (j * g >= n_b)
            continue;
        for (int64_t t = t0; t < t1; t++) {
            int64_t row = ((cu_k[b] + t) * h_kv + c) * (int64_t)d;
            double scale = 1.0;
            if (pool == OR_L2SUM) {
                double ss = 0.0;
                for (int e = 0; e < d; e++) {
                    double x = elem(k, dtype, row + e);
                    ss += x * x;
                }
                scale = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
            }
            for (int e = 0; e < d; e++)
                out[e] += elem(k, dtype, row + e) * scale;
        }
        if (pool == OR_MEAN)
            for (int e = 0; e < d; e++)
                out[e] /= (double)(t1 - t0);
    }
    return 0;
}

/* ------------------------------------------------------------------ select */

typedef struct {
    double s;
    int32_t j;
} cand;

/* Higher score first; equal scores: lower block index first. */
static int cand_order(const void *a, const void *b)
{
    const cand *x = (const cand *)a, *y = (const cand *)b;
    if (x->s > y->s)
        return -1;
    if (x->s < y->s)
        return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int int_order(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Token t (t <= p_sel) is in F(p_sel) = [0, min(n_init, p_sel + 1)) U [max(0, p_sel - w + 1), p_sel]. */
static int in_fixed_set(int64_t t, int64_t p_sel, int n_init, int window)
{
    if (t < 0 || t > p_sel)
        return 0;
    return t < n_init || t >= p_sel - window + 1;
}

int or_select(int batch, int h_q, int h_kv, int d, const int32_t *cu_q, const int32_t *cu_k,
              const int32_t *q_pos0, int g, int topk, const int32_t *topk_per_seq, int n_init,
              int window, int shared, int mode, double tau, int dtype, const void *q_sel, const double *k_cmp,
              int64_t nb_max, const void *k, int64_t n_req, const int64_t *req_row,
              const int32_t *req_kvh, int kcap, int32_t *out_idx, int32_t *out_n, double *out_sk,
              double *out_sk1, double *out_floor, int32_t *out_ncand, double *out_scores,
              int64_t score_stride)
{
    int G = h_q / h_kv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n_req; r++) {
        int64_t row = req_row[r];
        int c = req_kvh[r];
        int b;
        int64_t qa, qb, p_sel;
        if (shared) {
            b = (int)row;
            qa = cu_q[b];
            qb = cu_q[b + 1];
            p_sel = first_query_pos(b, cu_q, cu_k, q_pos0) - 1;
        } else {
            b = seq_of_query(row, batch, cu_q);
            qa = row;
            qb = row + 1;
            p_sel = first_query_pos(b, cu_q, cu_k, q_pos0) + (row - cu_q[b]);
        }
        int64_t n_b = cu_k[b + 1] - cu_k[b];
        int64_t nb_b = (n_b + g - 1) / g;

        /* per-head queries q_h (summed over the row's queries) and their sum */
        double *qh = (double *)calloc((size_t)G * d, sizeof(double));
        double *qs = (double *)calloc((size_t)d, sizeof(double));
        for (int64_t i = qa; i < qb; i++)
            for (int hh = 0; hh < G; hh++)
                for (int e = 0; e < d; e++)
                    qh[hh * d + e] += elem(q_sel, dtype, (i * h_q + c * G + hh) * (int64_t)d + e);
        for (int hh = 0; hh < G; hh++)
            for (int e = 0; e < d; e++)
                qs[e] += qh[hh * d + e];
        double qnorm = 0.0, qhmax = 0.0;
        for (int e = 0; e < d; e++)
            qnorm += qs[e] * qs[e];
        qnorm = sqrt(qnorm);
        for (int hh = 0; hh < G; hh++) {
            double n2 = 0.0;
            for (int e = 0; e < d; e++)
                n2 += qh[hh * d + e] * qh[hh * d + e];
            if (sqrt(n2) > qhmax)
                qhmax = sqrt(n2);
        }

        cand *cs = (cand *)malloc(sizeof(cand) * (size_t)(nb_b > 0 ? nb_b : 1));
        /* SOFTMAX: every head's logit of every candidate, [candidate][head] */
        double *lg = mode == OR_SEL_SOFTMAX ? (double *)malloc(sizeof(double) * (size_t)G *
                                                               (size_t)(nb_b > 0 ? nb_b : 1)) : NULL;
        int64_t nc = 0;
        double kmax = 0.0;
        for (int64_t j = 0; j < nb_b; j++) {
            int64_t t0 = j * g, t1 = (j + 1) * (int64_t)g - 1;
            if (t1 > n_b - 1)
                t1 = n_b - 1;
            if (t1 > p_sel)
                continue; /* not wholly visible */
            int outside_f = 0;
            for (int64_t t = t0; t <= t1; t++)
                if (!in_fixed_set(t, p_sel, n_init, window))
                    outside_f = 1;
            if (!outside_f)
                continue; /* wholly inside init/window */
            double dot = 0.0, kn = 0.0, best = -INFINITY;
            double *kv = (double *)malloc(sizeof(double) * (size_t)d);
            for (int e = 0; e < d; e++) {
                if (g == 1)
                    kv[e] = elem(k, dtype, ((cu_k[b] + j) * h_kv + c) * (int64_t)d + e);
                else if (mode == OR_SEL_ATTN)
                    kv[e] = 0.0;                    /* scored from the raw keys below */
                else
                    kv[e] = k_cmp[(((int64_t)c * batch + b) * nb_max + j) * d + e];
                dot += qs[e] * kv[e];
                kn += kv[e] * kv[e];
            }
            for (int hh = 0; hh < G && (mode == OR_SEL_SOFTMAX || mode == OR_SEL_MAX); hh++) {
                double dh = 0.0;
                for (int e = 0; e < d; e++)
                    dh += qh[hh * d + e] * kv[e];
                if (mode == OR_SEL_SOFTMAX)
                    lg[nc * G + hh] = dh / tau;
                else if (dh > best)
                    best = dh;
            }
            free(kv);
            if (sqrt(kn) > kmax)
                kmax = sqrt(kn);
            cs[nc].s = mode == OR_SEL_MAX ? best / sqrt((double)d) : dot / sqrt((double)d);
            cs[nc].j = (int32_t)j;
            nc++;
        }
        if (mode == OR_SEL_ATTN) {
            /* every (query, head) of the row: its dense causal log-sum-exp, then the
               attention mass it puts on each candidate block's tokens */
            for (int64_t x = 0; x < nc; x++)
                cs[x].s = 0.0;
            double q0b = (double)first_query_pos(b, cu_q, cu_k, q_pos0);
            for (int64_t i = qa; i < qb; i++) {
                int64_t p_i = (int64_t)q0b + (i - cu_q[b]);
                if (p_i > n_b - 1)
                    p_i = n_b - 1;
                for (int hh = 0; hh < G; hh++) {
                    int64_t qoff = (i * h_q + c * G + hh) * (int64_t)d;
                    double *lgt = (double *)malloc(sizeof(double) * (size_t)(p_i + 1 > 0 ? p_i + 1 : 1));
                    double m = -INFINITY, z = 0.0;
                    for (int64_t t = 0; t <= p_i; t++) {
                        int64_t koff = ((cu_k[b] + t) * h_kv + c) * (int64_t)d;
                        double dot = 0.0;
                        for (int e = 0; e < d; e++)
                            dot += elem(q_sel, dtype, qoff + e) * elem(k, dtype, koff + e);
                        lgt[t] = dot / sqrt((double)d);
                        if (lgt[t] > m)
                            m = lgt[t];
                    }
                    for (int64_t t = 0; t <= p_i; t++)
                        z += exp(lgt[t] - m);
                    double lse_ih = m + log(z);
                    for (int64_t x = 0; x < nc; x++) {
                        int64_t t0 = (int64_t)cs[x].j * g, t1 = t0 + g - 1;
                        if (t1 > p_i)
                            t1 = p_i;
                        for (int64_t t = t0; t <= t1; t++)
                            cs[x].s += exp(lgt[t] - lse_ih);
                    }
                    free(lgt);
                }
            }
        }
        if (mode == OR_SEL_SOFTMAX) {
            /* S_j = sum over heads of exp(l_hj - m_h) / Z_h over the row's candidates */
            for (int64_t x = 0; x < nc; x++)
                cs[x].s = 0.0;
            for (int hh = 0; hh < G; hh++) {
                double m = -INFINITY, z = 0.0;
                for (int64_t x = 0; x < nc; x++)
                    if (lg[x * G + hh] > m)
                        m = lg[x * G + hh];
                for (int64_t x = 0; x < nc; x++)
                    z += exp(lg[x * G + hh] - m);
                for (int64_t x = 0; x < nc; x++)
                    cs[x].s += exp(lg[x * G + hh] - m) / z;
            }
        }
        if (out_scores)
            for (int64_t x = 0; x < nc; x++)
                if (cs[x].j < score_stride)
                    out_scores[r * score_stride + cs[x].j] = cs[x].s;
        qsort(cs, (size_t)nc, sizeof(cand), cand_order);
        int64_t kr = topk_per_seq ? topk_per_seq[b] : topk;
        int64_t ns = kr < nc ? kr : nc;
        if (ns > kcap) {
            bad |= 1;
            ns = kcap;
        }
        int32_t *dst = out_idx + r * (int64_t)kcap;
        for (int64_t s = 0; s < ns; s++)
            dst[s] = cs[s].j;
        qsort(dst, (size_t)ns, sizeof(int32_t), int_order);
        for (int64_t s = ns; s < kcap; s++)
            dst[s] = -1;
        out_n[r] = (int32_t)ns;
        if (out_ncand)
            out_ncand[r] = (int32_t)nc;
        if (out_sk)
            out_sk[r] = ns >= 1 ? cs[ns - 1].s : NAN;
        if (out_sk1)
            out_sk1[r] = nc > ns ? cs[ns].s : NAN;
        if (out_floor) {
            /* the size of fp32 rounding in a score: dot products of these norms, and for
               SOFTMAX the logit error carried into the largest selected probability sum */
            if (mode == OR_SEL_SUM)
                out_floor[r] = 1e-6 * qnorm * kmax / sqrt((double)d);
            else if (mode == OR_SEL_MAX)
                out_floor[r] = 1e-6 * qhmax * kmax / sqrt((double)d);
            else if (mode == OR_SEL_SOFTMAX)
                out_floor[r] = 4e-6 * qhmax * kmax / tau * (ns >= 1 ? cs[0].s : 0.0);
            else
                out_floor[r] = 1e-5 * (ns >= 1 ? cs[0].s : 0.0);
        }
        free(lg);
        free(cs);
        free(qs);
        free(qh);
    }
    return bad;
}

/* ------------------------------------------------------------------ attend */

int or_attend(int batch, int h_q, int h_kv, int d, const int32_t *cu_q, const int32_t *cu_k,
              const int32_t *q_pos0, int g, int n_init, int window, int shared, double scale,
              int dtype, const void *q, const void *k, const void *v, const int32_t *idx,
              const int32_t *n_idx, int64_t idx_rows, int kcap, int64_t n_req,
              const int64_t *req_q, const int32_t *req_h, double *out, double *lse,
              int64_t *out_count, uint8_t *out_mask, int64_t mask_stride)
{
    int G = h_q / h_kv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_req; r++) {
        int64_t i = req_q[r];
        int h = req_h[r], c = h / G;
        int b = seq_of_query(i, batch, cu_q);
        int64_t q0 = first_query_pos(b, cu_q, cu_k, q_pos0);
        int64_t p = q0 + (i - cu_q[b]);
        int64_t p_sel = shared ? q0 - 1 : p;
        int64_t row = shared ? b : i;
        int64_t n_b = cu_k[b + 1] - cu_k[b];
        int64_t nb_b = (n_b + g - 1) / g;

        uint8_t *sel = (uint8_t *)calloc((size_t)(nb_b > 0 ? nb_b : 1), 1);
        const int32_t *lst = idx + ((int64_t)c * idx_rows + row) * kcap;
        int32_t nl = n_idx[(int64_t)c * idx_rows + row];
        for (int32_t s = 0; s < nl && s < kcap; s++)
            if (lst[s] >= 0 && lst[s] < nb_b)
                sel[lst[s]] = 1;

        /* attended set A: t <= p and (init or window or selected block) */
        int64_t limit = p < n_b - 1 ? p : n_b - 1;
        uint8_t *in_a = (uint8_t *)calloc((size_t)(limit + 1 > 0 ? limit + 1 : 1), 1);
        int64_t count = 0;
        for (int64_t t = 0; t <= limit; t++) {
            int member = t < n_init || t >= p_sel - window + 1 || sel[t / g];
            in_a[t] = (uint8_t)member;
            count += member;
        }

        const int64_t qoff = (i * h_q + h) * (int64_t)d;
        double *logit = (double *)malloc(sizeof(double) * (size_t)(limit + 1 > 0 ? limit + 1 : 1));
        double m = -INFINITY;
        for (int64_t t = 0; t <= limit; t++) {
            if (!in_a[t])
                continue;
            int64_t koff = ((cu_k[b] + t) * h_kv + c) * (int64_t)d;
            double dot = 0.0;
            for (int e = 0; e < d; e++)
                dot += elem(q, dtype, qoff + e) * elem(k, dtype, koff + e);
            logit[t] = scale * dot;
            if (logit[t] > m)
                m = logit[t];
        }
        double den = 0.0;
        double *o = out + r * (int64_t)d;
        for (int e = 0; e < d; e++)
            o[e] = 0.0;
        for (int64_t t = 0; t <= limit; t++) {
            if (!in_a[t])
                continue;
            double wgt = exp(logit[t] - m);
            int64_t voff = ((cu_k[b] + t) * h_kv + c) * (int64_t)d;
            den += wgt;
            for (int e = 0; e < d; e++)
                o[e] += wgt * elem(v, dtype, voff + e);
        }
        for (int e = 0; e < d; e++)
            o[e] = count ? o[e] / den : 0.0;
        if (lse)
            lse[r] = count ? m + log(den) : -INFINITY;
        if (out_count)
            out_count[r] = count;
        if (out_mask) {
            uint8_t *mk = out_mask + r * mask_stride;
            memset(mk, 0, (size_t)mask_stride);
            for (int64_t t = 0; t <= limit && t < mask_stride; t++)
                mk[t] = in_a[t];
        }
        free(logit);
        free(in_a);
        free(sel);
    }
    return 0;
}

/* ------------------------------------------------------------- LSA buckets */

/*
 * bucket_build: the LSA flat index (LSA deep-read, §2.2).  The pooled keys of every
 * complete cluster block (C consecutive tokens = C/g pooled groups of one sequence
 * and KV head) start as one bucket each; every round, each bucket finds its
 * cheapest partner under Ward's criterion among the buckets it may join (merged
 * size <= cap groups), and the pairs that are each other's cheapest merge together
 * (if that would leave fewer than NB buckets, only the cheapest pairs do, enough to
 * reach NB); rounds repeat until NB buckets remain or no pair may merge.  Ward's
 * criterion for buckets A, B with member sums S and sizes n is the growth of the
 * within-bucket sum of squares when they merge,
 * n_A n_B / (n_A + n_B) |S_A/n_A - S_B/n_B|^2, computed as written in fp64 from
 * the fp64 pooled keys (member sums in fp64 too).  Ties: the lower bucket (a
 * bucket is named by its smallest member).  A bucket's centroid
 * is the normalised sum of its members.  Output per block: members grouped by
 * bucket (buckets in name order, members ascending), NB + 1 offsets, NB centroids
 * (fp64), and the smallest relative margin of any decision taken (second best vs
 * best partner; first excluded vs last merged pair), so tests can tell a
 * near-tied block from a wrong one.
 */
static double ward_cost(const double *sa, int na, const double *sb, int nb, int d)
{
    double dist2 = 0.0;                      /* |mean_A - mean_B|^2 */
    for (int e = 0; e < d; e++) {
        const double diff = sa[e] / na - sb[e] / nb;
        dist2 += diff * diff;
    }
    return (double)na * nb / (na + nb) * dist2;
}

int or_bucket_build(int batch, int h_kv, int d, const int32_t *cu_k, int g, int C, int NB, int cap_tok,
                    const double *k_cmp, int64_t nb_max, int64_t ncb_max, int32_t *member, int32_t *offset,
                    double *centroid, double *margin)
{
    const int M = C / g, capg = cap_tok / g;
    /* capg * NB >= 2M: merging can always continue while more than NB buckets remain
       (a stuck partition has every bucket above capg / 2, hence fewer than 2M / capg) */
    if (C % g || cap_tok % g || NB < 1 || NB > M || capg < 1 || (int64_t)capg * NB < 2 * (int64_t)M)
        return 1;
    int64_t n_items = (int64_t)h_kv * batch * ncb_max;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t it = 0; it < n_items; it++) {
        int64_t cb = it % ncb_max;
        int b = (int)((it / ncb_max) % batch);
        int c = (int)(it / (ncb_max * batch));
        int64_t n_b = cu_k[b + 1] - cu_k[b];
        int32_t *mem = member + it * M;
        int32_t *off = offset + it * (NB + 1);
        double *cen = centroid + it * (int64_t)NB * d;
        margin[it] = INFINITY;
        if ((cb + 1) * C > n_b) {                      /* incomplete: no buckets */
            for (int x = 0; x < M; x++)
                mem[x] = -1;
            for (int x = 0; x <= NB; x++)
                off[x] = 0;
            continue;
        }
        double *S = (double *)malloc(sizeof(double) * (size_t)M * d);
        int *size = (int *)malloc(sizeof(int) * M), *alive = (int *)malloc(sizeof(int) * M);
        int *root = (int *)malloc(sizeof(int) * M), *nn = (int *)malloc(sizeof(int) * M);
        double *nnc = (double *)malloc(sizeof(double) * M);
        for (int x = 0; x < M; x++) {
            const double *src = k_cmp + (((int64_t)c * batch + b) * nb_max + cb * M + x) * d;
            for (int e = 0; e < d; e++)
                S[x * d + e] = src[e];
            size[x] = 1;
            alive[x] = 1;
            root[x] = x;
        }
        int count = M;
        double mg = INFINITY;
        while (count > NB) {
            int any = 0;
            for (int a = 0; a < M; a++) {
                nn[a] = -1;
                if (!alive[a])
                    continue;
                double best = INFINITY, second = INFINITY;
                for (int o = 0; o < M; o++) {
                    if (o == a || !alive[o] || size[a] + size[o] > capg)
                        continue;
                    double w = ward_cost(S + a * d, size[a], S + o * d, size[o], d);
                    if (w < best) {
                        second = best;
                        best = w;
                        nn[a] = o;
                    } else if (w < second) {
                        second = w;
                    }
                }
                nnc[a] = best;
                if (nn[a] >= 0) {
                    any = 1;
                    if (second < INFINITY) {
                        double r = best > 0.0 ? (second - best) / best : (second > 0.0 ? INFINITY : 0.0);
                        if (r < mg)
                            mg = r;
                    }
                }
            }
            if (!any)
                break;
            /* mutual pairs (a < o), cheapest first, ties by a */
            int np = 0;
            int *pa = (int *)malloc(sizeof(int) * M);
            for (int a = 0; a < M; a++)
                if (alive[a] && nn[a] > a && nn[nn[a]] == a)
                    pa[np++] = a;
            for (int x = 1; x < np; x++)               /* insertion sort by (cost, a) */
                for (int y = x; y > 0 && (nnc[pa[y]] < nnc[pa[y - 1]] ||
                                          (nnc[pa[y]] == nnc[pa[y - 1]] && pa[y] < pa[y - 1])); y--) {
                    int t = pa[y];
                    pa[y] = pa[y - 1];
                    pa[y - 1] = t;
                }
            int take = np < count - NB ? np : count - NB;
            if (take < np && take > 0) {
                double lo = nnc[pa[take - 1]], hi = nnc[pa[take]];
                double r = lo > 0.0 ? (hi - lo) / lo : (hi > 0.0 ? INFINITY : 0.0);
                if (r < mg)
                    mg = r;
            }
            for (int x = 0; x < take; x++) {
                int a = pa[x], o = nn[a];
                for (int e = 0; e < d; e++)
                    S[a * d + e] += S[o * d + e];
                size[a] += size[o];
                alive[o] = 0;
                for (int y = 0; y < M; y++)
                    if (root[y] == o)
                        root[y] = a;
                count--;
            }
            free(pa);
            if (take == 0)
                break;
        }
        /* buckets in name order (a bucket is named by its smallest member = its root) */
        int nbk = 0, pos = 0;
        for (int a = 0; a < M && nbk < NB; a++) {
            if (!alive[a])
                continue;
            off[nbk] = pos;
            double nrm = 0.0;
            for (int e = 0; e < d; e++)
                nrm += (double)S[a * d + e] * S[a * d + e];
            nrm = sqrt(nrm);
            for (int e = 0; e < d; e++)
                cen[(int64_t)nbk * d + e] = nrm > 0.0 ? S[a * d + e] / nrm : 0.0;
            for (int y = 0; y < M; y++)
                if (root[y] == a)
                    mem[pos++] = y;
            nbk++;
        }
        for (; nbk <= NB; nbk++)
            off[nbk] = pos;
        margin[it] = mg;
        free(S);
        free(size);
        free(alive);
        free(root);
        free(nn);
        free(nnc);
    }
    return 0;
}

/*
 * bucket_select: flat retrieval (LSA deep-read, §2.3).  The row's selector query
 * (the group's heads summed, over the row's queries) scores every bucket of the
 * complete cluster blocks that end at or before p_sel, s = qs . centroid / sqrt(d);
 * the kb best (score descending, bucket index ascending) are expanded to their
 * member groups, keeping those that meet the non-fixed region [n_init, p_sel - w + 1)
 * (the sink and window are attended anyway: a group wholly inside them is left out,
 * as for block candidates), written in ascending group order (width kcap, -1
 * padded).  The near-tie data (sk, sk1, floor) refer to the bucket scores.
 */
int or_bucket_select(int batch, int h_q, int h_kv, int d, const int32_t *cu_q, const int32_t *cu_k,
                     const int32_t *q_pos0, int g, int n_init, int window, int C, int NB, int kb, int shared,
                     int dtype, const void *q_sel,
                     const int32_t *member, const int32_t *offset, const double *centroid, int64_t ncb_max,
                     int64_t n_req, const int64_t *req_row, const int32_t *req_kvh, int kcap, int32_t *out_idx,
                     int32_t *out_n, double *out_sk, double *out_sk1, double *out_floor, int32_t *out_nbk)
{
    const int G = h_q / h_kv, M = C / g;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n_req; r++) {
        int64_t row = req_row[r];
        int c = req_kvh[r];
        int b;
        int64_t qa, qb, p_sel;
        if (shared) {
            b = (int)row;
            qa = cu_q[b];
            qb = cu_q[b + 1];
            p_sel = first_query_pos(b, cu_q, cu_k, q_pos0);
            p_sel -= 1;                                /* the boundary before the row's queries */
        } else {
            b = seq_of_query(row, batch, cu_q);
            qa = row;
            qb = row + 1;
            p_sel = first_query_pos(b, cu_q, cu_k, q_pos0) + (row - cu_q[b]);
        }
        int64_t n_b = cu_k[b + 1] - cu_k[b];
        int64_t ncb = (p_sel + 1) / C;                 /* complete blocks wholly at or before p_sel */
        if (ncb > n_b / C)
            ncb = n_b / C;
        if (ncb > ncb_max)
            ncb = ncb_max;
        double *qs = (double *)calloc((size_t)d, sizeof(double));
        for (int64_t i = qa; i < qb; i++)
            for (int h = c * G; h < (c + 1) * G; h++)
                for (int e = 0; e < d; e++)
                    qs[e] += elem(q_sel, dtype, (i * h_q + h) * (int64_t)d + e);
        double qnorm = 0.0;
        for (int e = 0; e < d; e++)
            qnorm += qs[e] * qs[e];
        qnorm = sqrt(qnorm);
        int64_t nc = ncb * NB;
        cand *cs = (cand *)malloc(sizeof(cand) * (size_t)(nc > 0 ? nc : 1));
        for (int64_t j = 0; j < nc; j++) {
            const double *cv = centroid + ((((int64_t)c * batch + b) * ncb_max + j / NB) * NB + j % NB) * d;
            double dot = 0.0;
            for (int e = 0; e < d; e++)
                dot += qs[e] * cv[e];
            cs[j].s = dot / sqrt((double)d);
            cs[j].j = (int32_t)j;
        }
        qsort(cs, (size_t)nc, sizeof(cand), cand_order);
        int64_t ns = kb < nc ? kb : nc;
        int32_t *dst = out_idx + r * (int64_t)kcap;
        int64_t n_out = 0;
        for (int64_t s = 0; s < ns; s++) {
            int64_t j = cs[s].j, blk = j / NB, lb = j % NB;
            const int64_t base = (((int64_t)c * batch + b) * ncb_max + blk);
            const int32_t *mem = member + base * M;
            const int32_t *off = offset + base * (NB + 1);
            for (int x = off[lb]; x < off[lb + 1]; x++) {
                const int64_t grp = blk * M + mem[x];
                if (!(grp * g < p_sel - window + 1 && (grp + 1) * g > n_init))
                    continue;                          /* wholly inside the sink or the window */
                if (n_out >= kcap) {
                    bad |= 1;
                    break;
                }
                dst[n_out++] = (int32_t)grp;
            }
        }
        qsort(dst, (size_t)n_out, sizeof(int32_t), int_order);
        for (int64_t s = n_out; s < kcap; s++)
            dst[s] = -1;
        out_n[r] = (int32_t)n_out;
        if (out_nbk)
            out_nbk[r] = (int32_t)ns;
        if (out_sk)
            out_sk[r] = ns >= 1 ? cs[ns - 1].s : NAN;
        if (out_sk1)
            out_sk1[r] = nc > ns ? cs[ns].s : NAN;
        if (out_floor)
            out_floor[r] = 1e-6 * qnorm / sqrt((double)d);     /* centroids have unit norm */
        free(cs);
        free(qs);
    }
    return bad;
}
