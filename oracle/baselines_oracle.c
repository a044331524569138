/*
 * CPU oracle for the sparse-KV baselines the diagonal method is compared with.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library.  It shares no code with the
 * GPU library (nor with dsa_oracle.c) and never calls it.
 *
 * Source: "Understanding and Exploiting Diagonal Attention Sparsity in
 * Autoregressive Image Generation" (arxiv 2609.19702), Section 2.3 "KV cache
 * sparsity techniques" (position-based: SlidingWindow keeps the most recent
 * KV, StreamingLLM adds the first few tokens as attention sinks; score-based:
 * H2O keeps heavy hitters by accumulated attention score, TOVA drops the
 * lowest-scoring key at each step) and Section 5.1 "Sparse KV baselines"
 * (StreamingLLM keeps the first 4 decode tokens as sinks because the prompt KV
 * is kept whole; the sparsity ratio counts decode KV left out of attention).
 *
 * Readings taken where the pages leave a step open (the same budget
 * accounting as Algorithm 1: prompt always attended, N_att decode entries
 * attended per step once the decode is long enough, the current token
 * included):
 *   - SlidingWindow: decode positions max(0, t - N_att + 1) .. t;
 *   - StreamingLLM: decode positions 0 .. 3 (those that exist) plus the
 *     N_att - 4 most recent positions; the sinks count inside N_att;
 *   - TOVA, per lane: a cache of at most N_att decode entries.  Step t puts
 *     token t in the cache and attends prompt + cache; if the cache then holds
 *     N_att entries, the entry with the lowest score of this step's query
 *     leaves it (the current token is a candidate).  The softmax is monotone
 *     in the raw logit q . k, so the lowest score is the lowest logit; ties
 *     go to the lowest position;
 *   - H2O, per lane: the same cache, of which the N_recent most recent
 *     positions are protected (the caller picks N_recent; the split the
 *     benchmarks use is N_att - floor(N_att / 2) recent, floor(N_att / 2)
 *     heavy hitters).  Every entry's accumulated score is the sum of its
 *     softmax probability (normalised over prompt + cache) over the steps it
 *     has been attended, its own step included.  If the cache holds N_att
 *     entries after step t, the unprotected entry (position <= t - N_recent)
 *     with the lowest accumulated score leaves it; ties go to the lowest
 *     position.
 * All arithmetic is fp64 on the exact inputs, widened by the caller.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* q . k over d doubles, in index order */
static double dot(int d, const double* q, const double* k) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += q[i] * k[i];
    return s;
}

/*
 * Softmax attention of query q over n rows: s[j] = q . k_j (raw), p[j] the
 * normalised probability with scale 1 / sqrt(d) (two passes: max, then exp and
 * sum), out = sum_j p[j] v_j.
 */
static void softmax_attend(int d, const double* q, int n, const double** rk, const double** rv, double* s,
                           double* p, double* out) {
    const double scale = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        s[j] = dot(d, q, rk[j]);
        if (s[j] > m) m = s[j];
    }
    double sum = 0.0;
    for (int j = 0; j < n; ++j) {
        p[j] = exp((s[j] - m) * scale);
        sum += p[j];
    }
    for (int i = 0; i < d; ++i) out[i] = 0.0;
    for (int j = 0; j < n; ++j) {
        p[j] /= sum;
        for (int i = 0; i < d; ++i) out[i] += p[j] * rv[j][i];
    }
}

typedef struct {
    const double** rk;
    const double** rv;
    double* s;
    double* p;
} rows_t;

static int rows_alloc(rows_t* r, int n) {
    r->rk = (const double**)malloc(sizeof(double*) * (size_t)n);
    r->rv = (const double**)malloc(sizeof(double*) * (size_t)n);
    r->s = (double*)malloc(sizeof(double) * (size_t)n);
    r->p = (double*)malloc(sizeof(double) * (size_t)n);
    return r->rk && r->rv && r->s && r->p ? 0 : -3;
}

static void rows_free(rows_t* r) {
    free(r->rk);
    free(r->rv);
    free(r->s);
    free(r->p);
}

/* rows 0 .. L_p-1: the prompt */
static int put_prompt(rows_t* r, int L_p, int d, const double* Kp, const double* Vp) {
    for (int j = 0; j < L_p; ++j) {
        r->rk[j] = Kp + (size_t)j * d;
        r->rv[j] = Vp + (size_t)j * d;
    }
    return L_p;
}

/*
 * SlidingWindow (S = 0) and StreamingLLM (S = 4), from their definitions.
 *   Q, K, V : [T][d]; Kp, Vp : [L_p][d]
 *   out [T][d]; n_dec [T] decode positions attended; att_mask (nullable) [T][T]
 * Returns 0, -1 on invalid parameters, -3 on allocation failure.
 */
int oracle_window_lane(int L_p, int N_att, int S, int d, int T, const double* Q, const double* Kp,
                       const double* Vp, const double* K, const double* V, double* out, int32_t* n_dec,
                       uint8_t* att_mask) {
    if (L_p < 0 || d < 1 || T < 0 || N_att < 1 || (S != 0 && S != 4) || (S == 4 && N_att <= S)) return -1;
    rows_t r;
    if (rows_alloc(&r, L_p + N_att + 1)) {
        rows_free(&r);
        return -3;
    }
    for (int t = 0; t < T; ++t) {
        int n = put_prompt(&r, L_p, d, Kp, Vp);
        if (att_mask) memset(att_mask + (size_t)t * T, 0, (size_t)T);
        int lo = t - (N_att - S) + 1; /* oldest recent position */
        if (lo < S) lo = S;
        for (int p = 0; p <= t; ++p) {
            if (!(p < S || p >= lo)) continue;
            r.rk[n] = K + (size_t)p * d;
            r.rv[n] = V + (size_t)p * d;
            ++n;
            if (att_mask) att_mask[(size_t)t * T + p] = 1;
        }
        n_dec[t] = n - L_p;
        softmax_attend(d, Q + (size_t)t * d, n, r.rk, r.rv, r.s, r.p, out + (size_t)t * d);
    }
    rows_free(&r);
    return 0;
}

/*
 * TOVA (policy 0) and H2O (policy 1) over a cache of N_att decode entries.
 *   N_recent : H2O's protected recent positions, 1 <= N_recent <= N_att - 1 (ignored by TOVA)
 *   follow   : optional [T]; at an eviction step the entry that leaves is
 *              follow[t] instead of the oracle's own choice (lockstep with
 *              another implementation); it must be a candidate, else -2.
 * Outputs: out [T][d]; choice [T] the oracle's own pick at step t (-1: no
 * eviction); n_dec [T]; gap (nullable) [T] at eviction steps with follow:
 * (key[follow] - key[choice]) / max(|key|), key = logit (TOVA) or accumulated
 * score (H2O), else 0; att_mask (nullable) [T][T]; score (nullable) [T][T]:
 * H2O's accumulated score of every cached position after step t (0 if not cached).
 * Returns 0, -1 on invalid parameters, -2 on a bad follow entry, -3 on allocation failure.
 */
int oracle_score_lane(int policy, int L_p, int N_att, int N_recent, int d, int T, const double* Q,
                      const double* Kp, const double* Vp, const double* K, const double* V,
                      const int32_t* follow, double* out, int32_t* choice, int32_t* n_dec, double* gap,
                      uint8_t* att_mask, double* score) {
    if (L_p < 0 || d < 1 || T < 0 || N_att < 1 || (policy != 0 && policy != 1)) return -1;
    if (policy == 1 && (N_recent < 1 || N_recent > N_att - 1)) return -1;
    rows_t r;
    int32_t* cache = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N_att + 1)); /* positions, ascending */
    double* acc = (double*)calloc((size_t)(T > 0 ? T : 1), sizeof(double));  /* H2O score by position */
    if (rows_alloc(&r, L_p + N_att + 1) || !cache || !acc) {
        rows_free(&r);
        free(cache);
        free(acc);
        return -3;
    }
    int rc = 0, nc = 0;
    for (int t = 0; t < T; ++t) {
        choice[t] = -1;
        if (gap) gap[t] = 0.0;
        cache[nc++] = t; /* token t enters the cache */
        int n = put_prompt(&r, L_p, d, Kp, Vp);
        for (int j = 0; j < nc; ++j, ++n) {
            r.rk[n] = K + (size_t)cache[j] * d;
            r.rv[n] = V + (size_t)cache[j] * d;
        }
        softmax_attend(d, Q + (size_t)t * d, n, r.rk, r.rv, r.s, r.p, out + (size_t)t * d);
        n_dec[t] = nc;
        if (att_mask) {
            memset(att_mask + (size_t)t * T, 0, (size_t)T);
            for (int j = 0; j < nc; ++j) att_mask[(size_t)t * T + cache[j]] = 1;
        }
        if (policy == 1)
            for (int j = 0; j < nc; ++j) acc[cache[j]] += r.p[L_p + j];

        if (nc == N_att) {
            /* the key each candidate is ranked by; candidates ascend in position,
             * so the first minimum is the lowest position among equals */
            int best = -1;
            double best_key = 0.0;
            for (int j = 0; j < nc; ++j) {
                if (policy == 1 && cache[j] > t - N_recent) continue;
                double key = policy == 0 ? r.s[L_p + j] : acc[cache[j]];
                if (best < 0 || key < best_key) {
                    best = j;
                    best_key = key;
                }
            }
            choice[t] = cache[best];
            int leave = best;
            if (follow) {
                int found = -1;
                for (int j = 0; j < nc; ++j)
                    if (cache[j] == follow[t] && !(policy == 1 && cache[j] > t - N_recent)) found = j;
                if (found < 0) {
                    rc = -2;
                    break;
                }
                if (gap) {
                    double a = policy == 0 ? r.s[L_p + found] : acc[cache[found]];
                    double mag = fabs(a) > fabs(best_key) ? fabs(a) : fabs(best_key);
                    gap[t] = mag > 0.0 ? (a - best_key) / mag : 0.0;
                }
                leave = found;
            }
            acc[cache[leave]] = 0.0;
            for (int j = leave; j + 1 < nc; ++j) cache[j] = cache[j + 1];
            --nc;
        }
        if (score) {
            double* row = score + (size_t)t * T;
            memset(row, 0, sizeof(double) * (size_t)T);
            for (int j = 0; j < nc; ++j) row[cache[j]] = acc[cache[j]];
        }
    }
    rows_free(&r);
    free(cache);
    free(acc);
    return rc;
}
