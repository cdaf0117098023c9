/*
 * lsh_oracle.c -- plain double-precision CPU oracle for the forward pass of
 * Reformer's LSH attention.
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library. The GPU library
 * never calls it and shares no code, header or table with it.
 *
 * Every step follows the method as the source pages state it, in their order,
 * with no blocking, fusion or reordering of the arithmetic. All arithmetic is
 * in IEEE double; inputs arrive already widened to double (bf16 and fp32
 * values widen exactly). Parallelism (OpenMP) is only over independent units
 * (token, segment, head) and never changes any unit's arithmetic.
 *
 * Sources, cited by page and section:
 *   [GLOSSARY]  ultralytics.com glossary entry "Reformer", section
 *               "Atenção LSH": angular LSH -- multiply by a random matrix R,
 *               bucket = index of the largest entry of [xR, -xR]; sort tokens
 *               by bucket, cut the sorted sequence into equal blocks, each
 *               token attends within its own block and the one before it;
 *               several hash rounds in parallel. Its worked example uses
 *               R of shape [rounds, dim, n_buckets/2] and torch's argmax
 *               over the concatenation [proj, -proj].
 *   [WALKTHRU]  twgreatdaily.com walkthrough of the ICLR 2020 paper, section
 *               "1 LSH Attention": attention restricted to a set P_i through a
 *               mask over a larger set, shared Q = K, sort by bucket and then
 *               by position inside the bucket, chunks of m consecutive sorted
 *               items where a chunk looks back exactly one chunk, and
 *               multi-round hashing whose attended set is the union over the
 *               rounds' sets.
 *   [SCHOLAR]   ai-scholar.tech summary, section "Transformerの問題点とは":
 *               scaled dot-product attention with the 1/sqrt(d_k) factor;
 *               section "・LSH Attention": Q = K, bucket, sort, equal chunks,
 *               attend own chunk and the preceding one; section
 *               "Reformerを用いた結果": model width d_model 1024 with 8 heads.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes):
 *   - keys are the queries themselves, not normalised;
 *   - a query may not attend to itself unless nothing else is valid: its own
 *     score is lowered by ORACLE_SELF_PENALTY;
 *   - causal masking compares original positions (key position <= query
 *     position);
 *   - chunk 0 has no look-back and windows never wrap or cross rounds;
 *   - rounds are combined with weights exp(lse_r - logsumexp_r lse_r), with
 *     no de-duplication of keys seen in several rounds;
 *   - ties in the argmax go to the first (lowest) index, as torch's argmax.
 * Variant (key_norm = 1): the key side of a score uses the unit vector
 * x_j / |x_j| ([WALKTHRU] "1 LSH Attention": its stripped formula is where
 * the method normalises keys); queries stay as they are and the hash is
 * unchanged (it is invariant to positive scaling). A zero vector keeps a zero
 * key.
 * Variant (per_head_r = 1): R is [H, n_hashes, d, n_buckets/2] and head h
 * hashes with R[h] in every batch.
 * Ablation Q1 (separate queries and keys): [WALKTHRU] "1 LSH Attention"
 * describes the bucket-sorted attention matrix before Q = K -- queries and
 * keys each hashed and sorted by bucket, so a bucket's query and key counts
 * need not match and a bucket may hold queries but no keys. Reading: round r
 * hashes queries and keys with the same R_r; queries and keys are sorted
 * separately by (bucket, position); query chunk c sees the keys of key
 * chunks c-1 and c; a key counts when its bucket equals the query's (and,
 * causal, its position is not later); no self penalty (it exists only
 * because a shared vector would attend to itself); a window with no such key
 * gives that round lse = -inf and a zero output, so the round takes no
 * weight, and a query with no key in any round outputs zero.
 * F1, the chunked feed-forward ([WALKTHRU] "3 分塊"; [SCHOLAR] "Reformerを
 * 用いた結果" for d_model 1024 and d_ff 4096): reading -- the Transformer's
 * position-wise feed-forward relu(x W1^T + b1) W2^T + b2, rows processed a
 * chunk at a time.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define ORACLE_SELF_PENALTY 1.0e5

/* Number of threads the oracle's parallel loops use (for reporting). */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* O1. Angular LSH ([GLOSSARY] "Atenção LSH"; [WALKTHRU] "1 LSH Attention"   */
/* for the different hash function per round).                              */
/*                                                                           */
/*   x        [n, d]             token vectors (one (batch, head) slice or    */
/*                               any list of tokens)                          */
/*   R        [n_hashes, d, n_buckets/2]   one random matrix per round        */
/*   buckets  [n_hashes, n]      out: first index of the max of [xR, -xR]     */
/*   margin   [n_hashes, n]      out (may be NULL): max minus the largest     */
/*                               entry at any other index (0 on exact ties)   */
/* ------------------------------------------------------------------------ */
int oracle_hash(const double *x, int64_t n, int d, const double *R,
                int n_hashes, int n_buckets, int32_t *buckets, double *margin)
{
    if (n_buckets < 2 || (n_buckets % 2) != 0 || d < 1 || n_hashes < 1 || n < 0)
        return -1;
    const int half = n_buckets / 2;
    int failed = 0;
#pragma omp parallel
    {
        double *c = (double *)malloc(sizeof(double) * (size_t)n_buckets);
        if (!c) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static) collapse(2)
        for (int r = 0; r < n_hashes; ++r) {
            for (int64_t i = 0; i < n; ++i) {
                if (!c) continue;
                const double *xi = x + i * d;
                /* projection p = x R_r, then the concatenation [p, -p] */
                for (int b = 0; b < half; ++b) {
                    double p = 0.0;
                    for (int k = 0; k < d; ++k)
                        p += xi[k] * R[((int64_t)r * d + k) * half + b];
                    c[b] = p;
                    c[b + half] = -p;
                }
                /* first index attaining the maximum */
                int best = 0;
                for (int b = 1; b < n_buckets; ++b)
                    if (c[b] > c[best]) best = b;
                buckets[(int64_t)r * n + i] = best;
                if (margin) {
                    double second = -INFINITY;
                    for (int b = 0; b < n_buckets; ++b)
                        if (b != best && c[b] > second) second = c[b];
                    margin[(int64_t)r * n + i] = c[best] - second;
                }
            }
        }
        free(c);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* O2. Sort of one round's positions by (bucket, position)                   */
/* ([WALKTHRU] "1 LSH Attention": two-level sort, bucket first, then the     */
/* position inside the bucket; [SCHOLAR] "・LSH Attention").                */
/*                                                                           */
/*   bucket [L]   bucket of each position                                    */
/*   perm   [L]   out: perm[s] = position held by sorted slot s              */
/*   inv    [L]   out: inv[i]  = sorted slot of position i                   */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t bucket;
    int32_t pos;
} oracle_key;

static int oracle_key_cmp(const void *pa, const void *pb)
{
    const oracle_key *a = (const oracle_key *)pa, *b = (const oracle_key *)pb;
    if (a->bucket != b->bucket) return a->bucket < b->bucket ? -1 : 1;
    if (a->pos != b->pos) return a->pos < b->pos ? -1 : 1;
    return 0;
}

int oracle_sort(const int32_t *bucket, int64_t L, int32_t *perm, int32_t *inv)
{
    if (L < 0) return -1;
    if (L == 0) return 0;
    oracle_key *k = (oracle_key *)malloc(sizeof(oracle_key) * (size_t)L);
    if (!k) return -2;
    for (int64_t i = 0; i < L; ++i) {
        k[i].bucket = bucket[i];
        k[i].pos = (int32_t)i;
    }
    /* (bucket, position) pairs are all distinct, so the order is total */
    qsort(k, (size_t)L, sizeof(oracle_key), oracle_key_cmp);
    for (int64_t s = 0; s < L; ++s) {
        perm[s] = k[s].pos;
        inv[k[s].pos] = (int32_t)s;
    }
    free(k);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O3 + O4. Chunked attention of one (batch, head, round) segment.           */
/* Windows: [WALKTHRU] "1 LSH Attention" (chunks of m sorted items, each     */
/* looking back one chunk); [GLOSSARY] "Atenção LSH" (own block and the      */
/* previous block). Scores and restriction: [SCHOLAR] (1/sqrt(d_k) scaling),  */
/* [WALKTHRU] (only keys in the query's bucket take part; the rest are       */
/* masked out of a larger candidate set; keys are the queries, Q = K).       */
/*                                                                           */
/*   x, v    [L, d]  by original position                                    */
/*   bucket  [L]     this round's bucket of each position                    */
/*   perm    [L]     this round's sorted order (from O2)                     */
/*   slots   list of query slots to compute (NULL: all L)                    */
/*   o       [L, d]  out, by sorted slot: softmax-weighted sum of v           */
/*   lse     [L]     out, by sorted slot: natural-log partition function     */
/* ------------------------------------------------------------------------ */
/* 1 / |x| (0 for the zero vector): the key scale of the key_norm variant */
static double inv_norm(const double *x, int d)
{
    double s = 0.0;
    for (int k = 0; k < d; ++k) s += x[k] * x[k];
    return s > 0.0 ? 1.0 / sqrt(s) : 0.0;
}

int oracle_attend(const double *x, const double *v, int64_t L, int d,
                  const int32_t *bucket, const int32_t *perm, int m, int causal,
                  const int64_t *slots, int64_t n_slots, double *o, double *lse,
                  int key_norm)
{
    if (L < 0 || d < 1 || m < 1 || (L % m) != 0) return -1;
    const int64_t n_q = slots ? n_slots : L;
    const double scale = 1.0 / sqrt((double)d);
    int failed = 0;
#pragma omp parallel
    {
        double *score = (double *)malloc(sizeof(double) * 2 * (size_t)m);
        int *valid = (int *)malloc(sizeof(int) * 2 * (size_t)m);
        if (!score || !valid) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 64)
        for (int64_t q = 0; q < n_q; ++q) {
            if (!score || !valid) continue;
            const int64_t s = slots ? slots[q] : q;
            const int64_t i = perm[s];
            const int64_t c = s / m;
            const int64_t t0 = (c > 0) ? (c - 1) * m : 0; /* no look-back for chunk 0 */
            const int64_t t1 = (c + 1) * m;                /* end of the query's own chunk */
            const double *xi = x + i * d;
            double mx = -INFINITY;
            for (int64_t t = t0; t < t1; ++t) {
                const int64_t j = perm[t];
                int ok = (bucket[j] == bucket[i]) && (!causal || j <= i);
                valid[t - t0] = ok;
                if (!ok) continue;
                const double *xj = x + j * d;
                double dot = 0.0;
                for (int k = 0; k < d; ++k) dot += xi[k] * xj[k];
                double sc = dot * scale;
                if (key_norm) sc *= inv_norm(xj, d);
                if (j == i) sc -= ORACLE_SELF_PENALTY;
                score[t - t0] = sc;
                if (sc > mx) mx = sc;
            }
            /* self is always valid, so the set is never empty */
            double sum = 0.0;
            for (int64_t t = t0; t < t1; ++t)
                if (valid[t - t0]) sum += exp(score[t - t0] - mx);
            const double l = mx + log(sum);
            lse[s] = l;
            double *os = o + s * d;
            for (int k = 0; k < d; ++k) os[k] = 0.0;
            for (int64_t t = t0; t < t1; ++t) {
                if (!valid[t - t0]) continue;
                const double w = exp(score[t - t0] - l);
                const double *vj = v + (int64_t)perm[t] * d;
                for (int k = 0; k < d; ++k) os[k] += w * vj[k];
            }
        }
        free(score);
        free(valid);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* O5. Un-sort and combine the rounds of one (batch, head)                   */
/* ([WALKTHRU] "1 LSH Attention": the attended set is the union of the       */
/* rounds' sets; each round's partial result is weighted by its share of     */
/* the total partition function, i.e. by exp(lse_r - logsumexp over r)).     */
/*                                                                           */
/*   o    [n_hashes, L, d]  per-round outputs by sorted slot                 */
/*   lse  [n_hashes, L]     per-round log partition functions by sorted slot */
/*   inv  [n_hashes, L]     per-round slot of each position                  */
/*   toks list of positions to compute (NULL: all L)                         */
/*   out  [L, d]            out, by original position                        */
/* A round whose lse is -inf (no key, separate queries and keys only) takes  */
/* weight 0; with no round left the output row is zero.                      */
/* ------------------------------------------------------------------------ */
int oracle_combine(const double *o, const double *lse, const int32_t *inv,
                   int n_hashes, int64_t L, int d, const int64_t *toks,
                   int64_t n_toks, double *out)
{
    if (n_hashes < 1 || L < 0 || d < 1) return -1;
    const int64_t n_t = toks ? n_toks : L;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < n_t; ++q) {
        const int64_t i = toks ? toks[q] : q;
        double mx = -INFINITY;
        for (int r = 0; r < n_hashes; ++r) {
            const double l = lse[(int64_t)r * L + inv[(int64_t)r * L + i]];
            if (l > mx) mx = l;
        }
        double *oi = out + i * d;
        if (mx == -INFINITY) {
            /* no round has a key (only with separate queries and keys): an
               empty softmax, read as a zero output */
            for (int k = 0; k < d; ++k) oi[k] = 0.0;
            continue;
        }
        double sum = 0.0;
        for (int r = 0; r < n_hashes; ++r)
            sum += exp(lse[(int64_t)r * L + inv[(int64_t)r * L + i]] - mx);
        const double z = mx + log(sum);
        for (int k = 0; k < d; ++k) oi[k] = 0.0;
        for (int r = 0; r < n_hashes; ++r) {
            const int64_t s = inv[(int64_t)r * L + i];
            const double w = exp(lse[(int64_t)r * L + s] - z);
            const double *os = o + ((int64_t)r * L + s) * d;
            for (int k = 0; k < d; ++k) oi[k] += w * os[k];
        }
    }
    return 0;
}

/* Rotations used by (batch, head) bh: the shared R, or head (bh mod H)'s own */
/* block of n_hashes rounds when each head has its rotations.               */
static const double *head_rotations(const double *R, int64_t bh, int H, int n_hashes, int d,
                                    int n_buckets, int per_head_r)
{
    if (!per_head_r) return R;
    const int64_t per_head = (int64_t)n_hashes * d * (n_buckets / 2);
    return R + (bh % H) * per_head;
}

/* ------------------------------------------------------------------------ */
/* Whole forward over [B, H]: O1 -> O2 -> O3/O4 -> O5 for every (b, h).      */
/*                                                                           */
/*   qk, v  [B, H, L, d]                                                     */
/*   R      [n_hashes, d, n_buckets/2] shared by every batch and head, or,   */
/*          with per_head_r, [H, n_hashes, d, n_buckets/2]: head h hashes     */
/*          with its own rotations R[h] in every batch                       */
/*   out    [B, H, L, d]                                                     */
/*   optional outputs (each may be NULL):                                    */
/*     buckets, perm, inv [B, H, n_hashes, L]; margin, lse [B, H, n_hashes, L]*/
/*     o_sorted           [B, H, n_hashes, L, d]                             */
/* ------------------------------------------------------------------------ */
int oracle_forward(const double *qk, const double *v, const double *R,
                   int B, int H, int64_t L, int d, int n_buckets, int n_hashes,
                   int chunk_len, int causal, double *out, int32_t *buckets_out,
                   double *margin_out, int32_t *perm_out, int32_t *inv_out,
                   double *o_sorted_out, double *lse_out, int key_norm, int per_head_r)
{
    if (B < 0 || H < 0 || L < 0 || d < 1 || n_hashes < 1 || chunk_len < 1 ||
        n_buckets < 2 || (n_buckets % 2) != 0 || (L % chunk_len) != 0)
        return -1;
    const int64_t seg = (int64_t)n_hashes * L;
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        const double *x = qk + bh * L * d;
        const double *vv = v + bh * L * d;
        int32_t *bk = (int32_t *)malloc(sizeof(int32_t) * (size_t)(seg ? seg : 1));
        int32_t *pm = (int32_t *)malloc(sizeof(int32_t) * (size_t)(seg ? seg : 1));
        int32_t *iv = (int32_t *)malloc(sizeof(int32_t) * (size_t)(seg ? seg : 1));
        double *mg = (double *)malloc(sizeof(double) * (size_t)(seg ? seg : 1));
        double *ls = (double *)malloc(sizeof(double) * (size_t)(seg ? seg : 1));
        double *os = (double *)malloc(sizeof(double) * (size_t)(seg ? seg * d : 1));
        int rc = (bk && pm && iv && mg && ls && os) ? 0 : -2;
        const double *Rh = head_rotations(R, bh, H, n_hashes, d, n_buckets, per_head_r);
        if (!rc) rc = oracle_hash(x, L, d, Rh, n_hashes, n_buckets, bk, mg);
        for (int r = 0; !rc && r < n_hashes; ++r)
            rc = oracle_sort(bk + r * L, L, pm + r * L, iv + r * L);
        for (int r = 0; !rc && r < n_hashes; ++r)
            rc = oracle_attend(x, vv, L, d, bk + r * L, pm + r * L, chunk_len,
                               causal, NULL, 0, os + r * L * d, ls + r * L, key_norm);
        if (!rc)
            rc = oracle_combine(os, ls, iv, n_hashes, L, d, NULL, 0, out + bh * L * d);
        if (!rc) {
            if (buckets_out) memcpy(buckets_out + bh * seg, bk, sizeof(int32_t) * (size_t)seg);
            if (margin_out) memcpy(margin_out + bh * seg, mg, sizeof(double) * (size_t)seg);
            if (perm_out) memcpy(perm_out + bh * seg, pm, sizeof(int32_t) * (size_t)seg);
            if (inv_out) memcpy(inv_out + bh * seg, iv, sizeof(int32_t) * (size_t)seg);
            if (lse_out) memcpy(lse_out + bh * seg, ls, sizeof(double) * (size_t)seg);
            if (o_sorted_out)
                memcpy(o_sorted_out + bh * seg * d, os, sizeof(double) * (size_t)(seg * d));
        }
        free(bk);
        free(pm);
        free(iv);
        free(mg);
        free(ls);
        free(os);
        if (rc) return rc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Q1 (ablation). Chunked attention of one segment with separate queries     */
/* and keys ([WALKTHRU] "1 LSH Attention": the bucket-sorted matrix before   */
/* Q = K, where a bucket may hold queries but no keys).                      */
/*                                                                           */
/*   q, k, v      [L, d] by original position                                */
/*   bucket_q/_k  [L]    this round's bucket of each query / key position    */
/*   perm_q/_k    [L]    the queries' / keys' sorted order (from O2)          */
/*   slots        query slots to compute (NULL: all L)                       */
/*   o   [L, d]   out, by query slot; lse [L] out, by query slot (-inf and a */
/*                zero row when no key of the window counts)                 */
/* ------------------------------------------------------------------------ */
int oracle_attend_qk(const double *q, const double *k, const double *v, int64_t L, int d,
                     const int32_t *bucket_q, const int32_t *bucket_k,
                     const int32_t *perm_q, const int32_t *perm_k, int m, int causal,
                     const int64_t *slots, int64_t n_slots, double *o, double *lse)
{
    if (L < 0 || d < 1 || m < 1 || (L % m) != 0) return -1;
    const int64_t n_q = slots ? n_slots : L;
    const double scale = 1.0 / sqrt((double)d);
    int failed = 0;
#pragma omp parallel
    {
        double *score = (double *)malloc(sizeof(double) * 2 * (size_t)m);
        int *valid = (int *)malloc(sizeof(int) * 2 * (size_t)m);
        if (!score || !valid) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 64)
        for (int64_t qi = 0; qi < n_q; ++qi) {
            if (!score || !valid) continue;
            const int64_t s = slots ? slots[qi] : qi;
            const int64_t i = perm_q[s];
            const int64_t c = s / m;
            /* the same chunk and the previous one, in the keys' sorted order */
            const int64_t t0 = (c > 0) ? (c - 1) * m : 0;
            const int64_t t1 = (c + 1) * m;
            const double *qv = q + i * d;
            double mx = -INFINITY;
            int any = 0;
            for (int64_t t = t0; t < t1; ++t) {
                const int64_t j = perm_k[t];
                const int ok = (bucket_k[j] == bucket_q[i]) && (!causal || j <= i);
                valid[t - t0] = ok;
                if (!ok) continue;
                const double *kv = k + j * d;
                double dot = 0.0;
                for (int e = 0; e < d; ++e) dot += qv[e] * kv[e];
                const double sc = dot * scale;
                score[t - t0] = sc;
                if (!any || sc > mx) mx = sc;
                any = 1;
            }
            double *os = o + s * d;
            for (int e = 0; e < d; ++e) os[e] = 0.0;
            if (!any) {
                lse[s] = -INFINITY;
                continue;
            }
            double sum = 0.0;
            for (int64_t t = t0; t < t1; ++t)
                if (valid[t - t0]) sum += exp(score[t - t0] - mx);
            const double l = mx + log(sum);
            lse[s] = l;
            for (int64_t t = t0; t < t1; ++t) {
                if (!valid[t - t0]) continue;
                const double w = exp(score[t - t0] - l);
                const double *vj = v + (int64_t)perm_k[t] * d;
                for (int e = 0; e < d; ++e) os[e] += w * vj[e];
            }
        }
        free(score);
        free(valid);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Q1 forward over [B, H]: O1 on the queries and on the keys (the same R),    */
/* O2 on each, chunked attention with separate queries and keys, O5 through  */
/* the queries' inverse order.                                               */
/*                                                                           */
/*   q, k, v  [B, H, L, d];  R as in oracle_forward;  out [B, H, L, d]        */
/*   optional outputs (each may be NULL), [B, H, n_hashes, L]: buckets_q,    */
/*   buckets_k, margin_q, margin_k, perm_q, perm_k, inv_q, lse (by query      */
/*   slot); o_sorted [B, H, n_hashes, L, d] by query slot                    */
/* ------------------------------------------------------------------------ */
int oracle_forward_qk(const double *q, const double *k, const double *v, const double *R,
                      int B, int H, int64_t L, int d, int n_buckets, int n_hashes,
                      int chunk_len, int causal, double *out, int32_t *bq_out,
                      int32_t *bk_out, double *mq_out, double *mk_out, int32_t *pq_out,
                      int32_t *pk_out, int32_t *iq_out, double *o_sorted_out,
                      double *lse_out, int per_head_r)
{
    if (B < 0 || H < 0 || L < 0 || d < 1 || n_hashes < 1 || chunk_len < 1 ||
        n_buckets < 2 || (n_buckets % 2) != 0 || (L % chunk_len) != 0)
        return -1;
    const int64_t seg = (int64_t)n_hashes * L;
    const size_t n1 = (size_t)(seg ? seg : 1);
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        const double *qq = q + bh * L * d;
        const double *kk = k + bh * L * d;
        const double *vv = v + bh * L * d;
        int32_t *bq = (int32_t *)malloc(sizeof(int32_t) * n1);
        int32_t *bk = (int32_t *)malloc(sizeof(int32_t) * n1);
        double *mq = (double *)malloc(sizeof(double) * n1);
        double *mk = (double *)malloc(sizeof(double) * n1);
        int32_t *pq = (int32_t *)malloc(sizeof(int32_t) * n1);
        int32_t *iq = (int32_t *)malloc(sizeof(int32_t) * n1);
        int32_t *pk = (int32_t *)malloc(sizeof(int32_t) * n1);
        int32_t *ik = (int32_t *)malloc(sizeof(int32_t) * n1);
        double *ls = (double *)malloc(sizeof(double) * n1);
        double *os = (double *)malloc(sizeof(double) * (size_t)(seg ? seg * d : 1));
        int rc = (bq && bk && mq && mk && pq && iq && pk && ik && ls && os) ? 0 : -2;
        const double *Rh = head_rotations(R, bh, H, n_hashes, d, n_buckets, per_head_r);
        if (!rc) rc = oracle_hash(qq, L, d, Rh, n_hashes, n_buckets, bq, mq);
        if (!rc) rc = oracle_hash(kk, L, d, Rh, n_hashes, n_buckets, bk, mk);
        for (int r = 0; !rc && r < n_hashes; ++r) {
            rc = oracle_sort(bq + r * L, L, pq + r * L, iq + r * L);
            if (!rc) rc = oracle_sort(bk + r * L, L, pk + r * L, ik + r * L);
        }
        for (int r = 0; !rc && r < n_hashes; ++r)
            rc = oracle_attend_qk(qq, kk, vv, L, d, bq + r * L, bk + r * L, pq + r * L,
                                  pk + r * L, chunk_len, causal, NULL, 0, os + r * L * d,
                                  ls + r * L);
        if (!rc) rc = oracle_combine(os, ls, iq, n_hashes, L, d, NULL, 0, out + bh * L * d);
        if (!rc) {
            const size_t ni = sizeof(int32_t) * (size_t)seg, nd = sizeof(double) * (size_t)seg;
            if (bq_out) memcpy(bq_out + bh * seg, bq, ni);
            if (bk_out) memcpy(bk_out + bh * seg, bk, ni);
            if (mq_out) memcpy(mq_out + bh * seg, mq, nd);
            if (mk_out) memcpy(mk_out + bh * seg, mk, nd);
            if (pq_out) memcpy(pq_out + bh * seg, pq, ni);
            if (pk_out) memcpy(pk_out + bh * seg, pk, ni);
            if (iq_out) memcpy(iq_out + bh * seg, iq, ni);
            if (lse_out) memcpy(lse_out + bh * seg, ls, nd);
            if (o_sorted_out) memcpy(o_sorted_out + bh * seg * d, os, nd * (size_t)d);
        }
        free(bq); free(bk); free(mq); free(mk); free(pq); free(iq); free(pk); free(ik);
        free(ls); free(os);
        if (rc) return rc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* G1 -- backward of the whole forward for one (batch, head) and beyond.    */
/* The hash and the sort are piecewise constant, so only the attention       */
/* carries a gradient. By O4/O5 the output of position i is one softmax over */
/* every (round, key) hit: out_i = sum_{r,j} P_i(r,j) v_j with               */
/* P_i(r,j) = exp(s_ij - Z_i), s_ij the masked, penalised score of key j in  */
/* round r's window of i, and Z_i = log sum_r exp(lse_r(i)). For a loss with */
/* gradient g_i = dL/dout_i this gives, with D_i = g_i . out_i:              */
/*   dv_j     += P_i(r,j) g_i                                                */
/*   dS_i(r,j) = P_i(r,j) (g_i . v_j - D_i)                                  */
/*   dq_i     += dS_i(r,j) x_j / sqrt(d)     (x_i as the query)              */
/*   dk_j     += dS_i(r,j) x_i / sqrt(d)     (x_j as the key)                */
/* and, queries and keys being the same vectors, dqk = dq + dk. The penalty  */
/* on the self score is a constant and has no derivative of its own.         */
/*                                                                           */
/*   qk, v, dout  [B, H, L, d]                                               */
/*   R            [n_hashes, d, n_buckets/2], or [H, n_hashes, d, nb/2] with */
/*                per_head_r (as in oracle_forward)                          */
/*   dqk, dv      [B, H, L, d]  out                                          */
/* ------------------------------------------------------------------------ */
int oracle_backward(const double *qk, const double *v, const double *R, const double *dout,
                    int B, int H, int64_t L, int d, int n_buckets, int n_hashes,
                    int chunk_len, int causal, double *dqk, double *dv, int key_norm,
                    int per_head_r)
{
    if (B < 0 || H < 0 || L < 0 || d < 1 || n_hashes < 1 || chunk_len < 1 ||
        n_buckets < 2 || (n_buckets % 2) != 0 || (L % chunk_len) != 0)
        return -1;
    const int64_t seg = (int64_t)n_hashes * L;
    const int64_t m = chunk_len;
    const double scale = 1.0 / sqrt((double)d);
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        const double *x = qk + bh * L * d;
        const double *vv = v + bh * L * d;
        const double *g = dout + bh * L * d;
        double *gx = dqk + bh * L * d;
        double *gv = dv + bh * L * d;
        const size_t n1 = (size_t)(seg ? seg : 1), nl = (size_t)(L ? L : 1);
        int32_t *bk = (int32_t *)malloc(sizeof(int32_t) * n1);
        int32_t *pm = (int32_t *)malloc(sizeof(int32_t) * n1);
        int32_t *iv = (int32_t *)malloc(sizeof(int32_t) * n1);
        double *mg = (double *)malloc(sizeof(double) * n1);
        double *ls = (double *)malloc(sizeof(double) * n1);
        double *os = (double *)malloc(sizeof(double) * n1 * (size_t)d);
        double *out = (double *)malloc(sizeof(double) * nl * (size_t)d);
        double *z = (double *)malloc(sizeof(double) * nl);
        double *dd = (double *)malloc(sizeof(double) * nl);
        int rc = (bk && pm && iv && mg && ls && os && out && z && dd) ? 0 : -2;
        /* the forward's own steps */
        const double *Rh = head_rotations(R, bh, H, n_hashes, d, n_buckets, per_head_r);
        if (!rc) rc = oracle_hash(x, L, d, Rh, n_hashes, n_buckets, bk, mg);
        for (int r = 0; !rc && r < n_hashes; ++r)
            rc = oracle_sort(bk + r * L, L, pm + r * L, iv + r * L);
        for (int r = 0; !rc && r < n_hashes; ++r)
            rc = oracle_attend(x, vv, L, d, bk + r * L, pm + r * L, chunk_len, causal, NULL, 0,
                               os + r * L * d, ls + r * L, key_norm);
        if (!rc) rc = oracle_combine(os, ls, iv, n_hashes, L, d, NULL, 0, out);
        if (!rc) {
            /* Z_i (log of the total partition function) and D_i */
            for (int64_t i = 0; i < L; ++i) {
                double mx = -INFINITY;
                for (int r = 0; r < n_hashes; ++r) {
                    const double l = ls[(int64_t)r * L + iv[(int64_t)r * L + i]];
                    if (l > mx) mx = l;
                }
                double sum = 0.0;
                for (int r = 0; r < n_hashes; ++r)
                    sum += exp(ls[(int64_t)r * L + iv[(int64_t)r * L + i]] - mx);
                z[i] = mx + log(sum);
                double dot = 0.0;
                for (int k = 0; k < d; ++k) dot += g[i * d + k] * out[i * d + k];
                dd[i] = dot;
            }
            for (int64_t e = 0; e < L * d; ++e) {
                gx[e] = 0.0;
                gv[e] = 0.0;
            }
            /* every (round, query slot, window key): serial, so the sums into
               the keys' gradients need no care */
            for (int r = 0; r < n_hashes; ++r) {
                const int32_t *bucket = bk + (int64_t)r * L;
                const int32_t *perm = pm + (int64_t)r * L;
                for (int64_t s = 0; s < L; ++s) {
                    const int64_t i = perm[s];
                    const int64_t c = s / m;
                    const int64_t t0 = (c > 0) ? (c - 1) * m : 0;
                    const int64_t t1 = (c + 1) * m;
                    const double *xi = x + i * d, *gi = g + i * d;
                    for (int64_t t = t0; t < t1; ++t) {
                        const int64_t j = perm[t];
                        if (!((bucket[j] == bucket[i]) && (!causal || j <= i))) continue;
                        const double *xj = x + j * d, *vj = vv + j * d;
                        double dot = 0.0, gdv = 0.0;
                        for (int k = 0; k < d; ++k) {
                            dot += xi[k] * xj[k];
                            gdv += gi[k] * vj[k];
                        }
                        /* key_norm: s = x_i . x_j rn / sqrt(d), rn = 1 / |x_j|; its
                           derivative in x_j is rn (x_i - (x_i . x_j) rn^2 x_j) / sqrt(d) */
                        const double rn = key_norm ? inv_norm(xj, d) : 1.0;
                        double sc = dot * scale * rn;
                        if (j == i) sc -= ORACLE_SELF_PENALTY;
                        const double p = exp(sc - z[i]);
                        const double ds = p * (gdv - dd[i]);
                        for (int k = 0; k < d; ++k) {
                            gv[j * d + k] += p * gi[k];
                            gx[i * d + k] += ds * scale * rn * xj[k];
                            if (key_norm)
                                gx[j * d + k] += ds * scale * rn * (xi[k] - dot * rn * rn * xj[k]);
                            else
                                gx[j * d + k] += ds * scale * xi[k];
                        }
                    }
                }
            }
        }
        free(bk);
        free(pm);
        free(iv);
        free(mg);
        free(ls);
        free(os);
        free(out);
        free(z);
        free(dd);
        if (rc) return rc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* G1 at chosen positions of one (batch, head): the rows dqk[p] and dv[p]   */
/* of G1 for each position p in toks, by the same sums restricted to the    */
/* terms that land in those rows. A position's rows receive terms only from */
/* query slots in its own chunk (as query and as key) and in the next chunk */
/* (queries that look back at it), in every round; those queries' Z_i and   */
/* D_i need their forward at every round's slot. So the forward runs at     */
/* exactly those slots and tokens, and the (round, slot, key) loop visits   */
/* the same terms in the same order as G1 does, skipping the ones that land */
/* in rows outside toks: each chosen row comes out as G1 computes it. Meant */
/* for sequences where G1 over every position is too slow.                  */
/*                                                                           */
/*   x, v, dout  [L, d]  one (batch, head) by original position             */
/*   R           [n_hashes, d, n_buckets/2]  this head's rotations          */
/*   toks        n_toks distinct positions                                  */
/*   dqk, dv     [n_toks, d]  out, row q for position toks[q]                */
/* ------------------------------------------------------------------------ */
int oracle_backward_rows(const double *x, const double *v, const double *R,
                         const double *dout, int64_t L, int d, int n_buckets, int n_hashes,
                         int chunk_len, int causal, int key_norm, const int64_t *toks,
                         int64_t n_toks, double *dqk, double *dv)
{
    if (L < 1 || d < 1 || n_hashes < 1 || chunk_len < 1 || n_buckets < 2 ||
        (n_buckets % 2) != 0 || (L % chunk_len) != 0 || n_toks < 0)
        return -1;
    const int64_t seg = (int64_t)n_hashes * L;
    const int64_t m = chunk_len, n_chunks = L / chunk_len;
    const double scale = 1.0 / sqrt((double)d);
    int32_t *bk = (int32_t *)malloc(sizeof(int32_t) * (size_t)seg);
    int32_t *pm = (int32_t *)malloc(sizeof(int32_t) * (size_t)seg);
    int32_t *iv = (int32_t *)malloc(sizeof(int32_t) * (size_t)seg);
    double *mg = (double *)malloc(sizeof(double) * (size_t)seg);
    double *ls = (double *)malloc(sizeof(double) * (size_t)seg);
    double *os = (double *)malloc(sizeof(double) * (size_t)seg * (size_t)d);
    double *out = (double *)malloc(sizeof(double) * (size_t)L * (size_t)d);
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    double *dd = (double *)malloc(sizeof(double) * (size_t)L);
    int64_t *row = (int64_t *)malloc(sizeof(int64_t) * (size_t)L);     /* position -> q, or -1 */
    char *qchunk = (char *)calloc((size_t)(n_hashes * n_chunks), 1);  /* query chunks visited */
    char *need = (char *)calloc((size_t)seg, 1);                      /* slots to attend */
    char *qtok = (char *)calloc((size_t)L, 1);                        /* queries visited */
    int64_t *list = (int64_t *)malloc(sizeof(int64_t) * (size_t)(seg > L ? seg : L));
    int rc = (bk && pm && iv && mg && ls && os && out && z && dd && row && qchunk && need &&
              qtok && list) ? 0 : -2;
    if (!rc) rc = oracle_hash(x, L, d, R, n_hashes, n_buckets, bk, mg);
    for (int r = 0; !rc && r < n_hashes; ++r)
        rc = oracle_sort(bk + r * L, L, pm + r * L, iv + r * L);
    for (int64_t p = 0; !rc && p < L; ++p) row[p] = -1;
    for (int64_t q = 0; !rc && q < n_toks; ++q) {
        const int64_t p = toks[q];
        if (p < 0 || p >= L || row[p] >= 0) rc = -1;   /* out of range or repeated */
        else row[p] = q;
    }
    if (!rc) {
        /* query chunks whose terms reach a chosen row: its own and the next */
        for (int64_t q = 0; q < n_toks; ++q)
            for (int r = 0; r < n_hashes; ++r) {
                const int64_t c = iv[(int64_t)r * L + toks[q]] / m;
                qchunk[r * n_chunks + c] = 1;
                if (c + 1 < n_chunks) qchunk[r * n_chunks + c + 1] = 1;
            }
        /* their queries, and each of those queries' slots in every round */
        for (int r = 0; r < n_hashes; ++r)
            for (int64_t s = 0; s < L; ++s)
                if (qchunk[r * n_chunks + s / m]) qtok[pm[(int64_t)r * L + s]] = 1;
        for (int64_t i = 0; i < L; ++i)
            if (qtok[i])
                for (int r = 0; r < n_hashes; ++r) need[(int64_t)r * L + iv[(int64_t)r * L + i]] = 1;
        for (int r = 0; !rc && r < n_hashes; ++r) {
            int64_t n = 0;
            for (int64_t s = 0; s < L; ++s)
                if (need[(int64_t)r * L + s]) list[n++] = s;
            rc = oracle_attend(x, v, L, d, bk + r * L, pm + r * L, chunk_len, causal, list, n,
                               os + r * L * d, ls + r * L, key_norm);
        }
        int64_t n_q = 0;
        for (int64_t i = 0; i < L; ++i)
            if (qtok[i]) list[n_q++] = i;
        if (!rc) rc = oracle_combine(os, ls, iv, n_hashes, L, d, list, n_q, out);
    }
    if (!rc) {
        /* Z_i and D_i as G1 forms them, for the visited queries */
        for (int64_t i = 0; i < L; ++i) {
            if (!qtok[i]) continue;
            double mx = -INFINITY;
            for (int r = 0; r < n_hashes; ++r) {
                const double l = ls[(int64_t)r * L + iv[(int64_t)r * L + i]];
                if (l > mx) mx = l;
            }
            double sum = 0.0;
            for (int r = 0; r < n_hashes; ++r)
                sum += exp(ls[(int64_t)r * L + iv[(int64_t)r * L + i]] - mx);
            z[i] = mx + log(sum);
            double dot = 0.0;
            for (int k = 0; k < d; ++k) dot += dout[i * d + k] * out[i * d + k];
            dd[i] = dot;
        }
        for (int64_t e = 0; e < n_toks * d; ++e) {
            dqk[e] = 0.0;
            dv[e] = 0.0;
        }
        for (int r = 0; r < n_hashes; ++r) {
            const int32_t *bucket = bk + (int64_t)r * L;
            const int32_t *perm = pm + (int64_t)r * L;
            for (int64_t s = 0; s < L; ++s) {
                const int64_t c = s / m;
                if (!qchunk[r * n_chunks + c]) continue;
                const int64_t i = perm[s];
                const int64_t t0 = (c > 0) ? (c - 1) * m : 0;
                const int64_t t1 = (c + 1) * m;
                const double *xi = x + i * d, *gi = dout + i * d;
                for (int64_t t = t0; t < t1; ++t) {
                    const int64_t j = perm[t];
                    if (row[i] < 0 && row[j] < 0) continue;
                    if (!((bucket[j] == bucket[i]) && (!causal || j <= i))) continue;
                    const double *xj = x + j * d, *vj = v + j * d;
                    double dot = 0.0, gdv = 0.0;
                    for (int k = 0; k < d; ++k) {
                        dot += xi[k] * xj[k];
                        gdv += gi[k] * vj[k];
                    }
                    const double rn = key_norm ? inv_norm(xj, d) : 1.0;
                    double sc = dot * scale * rn;
                    if (j == i) sc -= ORACLE_SELF_PENALTY;
                    const double p = exp(sc - z[i]);
                    const double ds = p * (gdv - dd[i]);
                    double *qi = row[i] >= 0 ? dqk + row[i] * d : NULL;
                    double *kj = row[j] >= 0 ? dqk + row[j] * d : NULL;
                    double *vo = row[j] >= 0 ? dv + row[j] * d : NULL;
                    for (int k = 0; k < d; ++k) {
                        if (vo) vo[k] += p * gi[k];
                        if (qi) qi[k] += ds * scale * rn * xj[k];
                        if (kj) {
                            if (key_norm)
                                kj[k] += ds * scale * rn * (xi[k] - dot * rn * rn * xj[k]);
                            else
                                kj[k] += ds * scale * xi[k];
                        }
                    }
                }
            }
        }
    }
    free(bk);
    free(pm);
    free(iv);
    free(mg);
    free(ls);
    free(os);
    free(out);
    free(z);
    free(dd);
    free(row);
    free(qchunk);
    free(need);
    free(qtok);
    free(list);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* P0 -- input projections ahead of the hash.                               */
/* [GLOSSARY] "Atenção LSH": queries and keys come from one shared          */
/* projection; [SCHOLAR] "Reformerを用いた結果": a model width of 1024       */
/* split over 8 heads. Reading: two bias-free linear maps of the token      */
/* vectors, one giving the shared query/key vectors and one the values,     */
/* each with H*d outputs, head h taking outputs h*d .. h*d + d - 1; the     */
/* weight of output n for input k is w[n * d_model + k].                    */
/*   x            [B, L, d_model]                                           */
/*   w_qk, w_v    [H * d, d_model]                                          */
/*   qk, v (out)  [B, H, L, d]                                              */
/*   qk[b,h,l,e] = sum_k x[b,l,k] * w_qk[h*d + e, k]   (likewise v with w_v) */
/* ------------------------------------------------------------------------ */
int oracle_project(const double *x, int B, int64_t L, int d_model,
                   const double *w_qk, const double *w_v, int H, int d,
                   double *qk, double *v)
{
    if (B < 0 || L < 0 || d_model < 1 || H < 1 || d < 1) return -1;
#ifdef _OPENMP
#pragma omp parallel for collapse(2) schedule(static)
#endif
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int64_t l = 0; l < L; ++l) {
                const double *xr = x + ((int64_t)b * L + l) * d_model;
                double *qo = qk + (((int64_t)b * H + h) * L + l) * d;
                double *vo = v + (((int64_t)b * H + h) * L + l) * d;
                for (int e = 0; e < d; ++e) {
                    const double *wq = w_qk + ((int64_t)h * d + e) * d_model;
                    const double *wv = w_v + ((int64_t)h * d + e) * d_model;
                    double sq = 0.0, sv = 0.0;
                    for (int k = 0; k < d_model; ++k) {
                        sq += xr[k] * wq[k];
                        sv += xr[k] * wv[k];
                    }
                    qo[e] = sq;
                    vo[e] = sv;
                }
            }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* F1 -- chunked feed-forward.                                              */
/* [WALKTHRU] "3 分塊": the feed-forward's inner width exceeds the model     */
/* width, and since positions are computed independently the sequence is    */
/* split into chunks processed one after another; [SCHOLAR] "Reformerを用い */
/* た結果": d_model 1024, d_ff 4096. Reading (the pages give no formula):   */
/* the Transformer's feed-forward, a ReLU between two linear maps with a    */
/* bias after each (NULL = zero), weights output-major (w[n * in + k]).     */
/*   x, out  [rows, d_model]   w1 [d_ff, d_model]   b1 [d_ff]               */
/*   w2 [d_model, d_ff]        b2 [d_model]                                 */
/* For each chunk of `chunk` rows: h = relu(x W1^T + b1) for the chunk,     */
/* then out = h W2^T + b2.                                                  */
/* ------------------------------------------------------------------------ */
int oracle_ffn(const double *x, int64_t rows, int d_model, const double *w1, const double *b1,
               const double *w2, const double *b2, int d_ff, int64_t chunk, double *out)
{
    if (rows < 0 || d_model < 1 || d_ff < 1 || chunk < 1) return -1;
    const int64_t cap = rows < chunk ? rows : chunk;
    double *h = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1) * (size_t)d_ff);
    if (!h) return -2;
    for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
        const int64_t n = (rows - r0) < chunk ? (rows - r0) : chunk;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
        for (int64_t i = 0; i < n; ++i) {
            const double *xr = x + (r0 + i) * d_model;
            for (int f = 0; f < d_ff; ++f) {
                const double *w = w1 + (int64_t)f * d_model;
                double s = 0.0;
                for (int k = 0; k < d_model; ++k) s += xr[k] * w[k];
                if (b1) s += b1[f];
                h[i * d_ff + f] = s > 0.0 ? s : 0.0;
            }
        }
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
        for (int64_t i = 0; i < n; ++i) {
            const double *hr = h + i * d_ff;
            for (int o = 0; o < d_model; ++o) {
                const double *w = w2 + (int64_t)o * d_ff;
                double s = 0.0;
                for (int f = 0; f < d_ff; ++f) s += hr[f] * w[f];
                if (b2) s += b2[o];
                out[(r0 + i) * d_model + o] = s;
            }
        }
    }
    free(h);
    return 0;
}
