/*
 * CPU oracle for diagonal-aware sparse decode attention.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library.  It shares no code with the
 * GPU library and never calls it.
 *
 * Source: "Understanding and Exploiting Diagonal Attention Sparsity in
 * Autoregressive Image Generation" (arxiv 2609.19702), Section 4, Algorithm 1
 * ("Diagonal-Aware Sparse Attention"), its "Detailed explanation" (the worked
 * example with N_r = 7, N_att = 4) and Section 5.1 "Our methods" (the
 * Diagonal+Sink4 variant).  The method is a selection heuristic, not a faster
 * route to a closed form, so this file runs the algorithm step by step in the
 * pages' notation: absolute decode positions, an explicit skip_idx list that
 * is shifted by +1 each step, an explicit window, explicit eviction.  All
 * arithmetic is fp64; the inputs are the exact fp32 / bf16 values the GPU
 * receives, widened without loss by the caller.
 *
 * Readings taken where the pages leave a step open:
 *   - the window [max(0, t - N_r) .. t] includes the current token t (the
 *     t = 4 set {K0, K2, K3, K4} of the worked example contains K4);
 *   - in phase 3 the evicted entry t - N_r is in that window but holds no KV
 *     any more, so it is never attended (the attended count stays N_att);
 *   - eviction happens at step t before attention;
 *   - Attn is one softmax over the concatenation of prompt rows and the
 *     selected decode rows, scaled by 1 / sqrt(d), no other mask;
 *   - argmin_j softmax(...) is taken on the raw logits q . k (same order,
 *     no scaling that could merge values), ties go to the lowest position;
 *   - the candidates are the decode entries in idx at step t, the current
 *     token included, prompt and sink entries excluded;
 *   - Diagonal+Sink4 (S = 4): decode positions 0..3 are sinks, attended from
 *     the step they exist on, never in the window, never evicted, never
 *     skipped; the algorithm runs unchanged on positions >= S with
 *     N_r - S and N_att - S, so the window is [max(S, t - (N_r - S)) .. t]
 *     and phase 3 evicts t - (N_r - S).  The phase boundaries in t stay
 *     N_att - 1 and N_r, and the budgets N_r (memory) and N_att (attended
 *     decode entries) include the sinks.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Attn(q, rows): one two-pass softmax over the given rows.  rows_k[j] / rows_v[j]
 * point at d doubles each; s[j] receives the raw logit q . k_j. */
static void attend(int d, const double* q, int n, const double** rows_k, const double** rows_v, double* s,
                   double* out) {
    double scale = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += q[i] * rows_k[j][i];
        s[j] = acc;
        if (acc * scale > m) m = acc * scale;
    }
    double denom = 0.0;
    for (int i = 0; i < d; ++i) out[i] = 0.0;
    for (int j = 0; j < n; ++j) {
        double w = exp(s[j] * scale - m);
        denom += w;
        for (int i = 0; i < d; ++i) out[i] += w * rows_v[j][i];
    }
    for (int i = 0; i < d; ++i) out[i] /= denom;
}

/*
 * One lane, decode steps t = 0 .. T-1.
 *   Q, K, V     : [T][d] query / key / value of decode token t (K, V indexed by position)
 *   Kp, Vp      : [L_p][d] prompt keys / values
 *   follow      : optional [T]; at a selection step the position appended to
 *                 skip_idx is follow[t] instead of the oracle's own argmin
 *                 (lockstep with another implementation).  It must be a
 *                 candidate, else the call fails with -2.
 * Outputs (each [T], or [T][d] / [T][T]; the optional ones may be NULL):
 *   out         : attention output of step t
 *   choice      : the oracle's own argmin position at step t, -1 when no selection
 *   evicted     : position evicted at step t, -1 when none
 *   n_dec       : number of decode positions attended at step t (sinks included)
 *   gap         : optional; at selection steps with follow, (s[follow] - s[choice]) / max(|s|), else 0
 *   att_mask    : optional; att_mask[t*T + p] = 1 iff decode position p is attended at step t
 *   skip_mask   : optional; skip_mask[t*T + p] = 1 iff p is in skip_idx when step t attends
 * Returns 0, -1 on invalid parameters, -2 on a follow entry that is not a candidate,
 * -3 on allocation failure.
 */
int oracle_dsa_lane(int L_p, int N_r, int N_att, int S, int d, int T, const double* Q, const double* Kp,
                    const double* Vp, const double* K, const double* V, const int32_t* follow, double* out,
                    int32_t* choice, int32_t* evicted, int32_t* n_dec, double* gap, uint8_t* att_mask,
                    uint8_t* skip_mask) {
    if (L_p < 0 || d < 1 || T < 0 || N_att < 1 || N_r < N_att || (S != 0 && S != 4) || (S == 4 && N_att <= S))
        return -1;
    int rc = 0;
    int32_t* skip_idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N_r + 1));
    uint8_t* present = (uint8_t*)calloc((size_t)(T > 0 ? T : 1), 1);   /* decode KV held in the cache */
    uint8_t* in_skip = (uint8_t*)calloc((size_t)(T > 0 ? T : 1), 1);
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T + 1));
    int nrows_max = L_p + S + T + 1;
    const double** rk = (const double**)malloc(sizeof(double*) * (size_t)nrows_max);
    const double** rv = (const double**)malloc(sizeof(double*) * (size_t)nrows_max);
    double* s = (double*)malloc(sizeof(double) * (size_t)nrows_max);
    if (!skip_idx || !present || !in_skip || !idx || !rk || !rv || !s) {
        rc = -3;
        goto done;
    }
    int nskip = 0;
    int Nr_w = N_r - S; /* window length over non-sink positions */

    for (int t = 0; t < T; ++t) {
        /* the new token's K, V enter the cache */
        present[t] = 1;
        choice[t] = -1;
        evicted[t] = -1;
        if (gap) gap[t] = 0.0;

        /* window <- [max(0, t - N_r), ..., t]  (non-sink positions) */
        int lo = t - Nr_w;
        if (lo < S) lo = S;
        int select = 0;

        if (t < N_att - 1) {
            /* Phase 1: full attention, idx <- window */
        } else if (t < N_r) {
            /* Phase 2: skip_idx <- [j + 1 for j in skip_idx]; idx <- window - skip_idx */
            for (int j = 0; j < nskip; ++j) skip_idx[j] += 1;
            if (nskip < N_r - N_att) select = 1;
        } else {
            /* Phase 3: K[t - N_r], V[t - N_r] <- empty; shift skip_idx by +1 */
            int e = t - Nr_w;
            present[e] = 0;
            evicted[t] = e;
            for (int j = 0; j < nskip; ++j) skip_idx[j] += 1;
        }

        /* idx <- window - skip_idx (only entries that still hold KV) */
        memset(in_skip, 0, (size_t)T);
        for (int j = 0; j < nskip; ++j)
            if (skip_idx[j] >= 0 && skip_idx[j] < T) in_skip[skip_idx[j]] = 1;
        int nidx = 0;
        for (int p = lo; p <= t; ++p)
            if (!in_skip[p] && present[p]) idx[nidx++] = p;

        /* rows: prompt KV, sink KV that exists by now, then K[idx] */
        int n = 0;
        for (int j = 0; j < L_p; ++j, ++n) {
            rk[n] = Kp + (size_t)j * d;
            rv[n] = Vp + (size_t)j * d;
        }
        int nsink = 0;
        for (int p = 0; p < S && p <= t; ++p, ++n, ++nsink) {
            rk[n] = K + (size_t)p * d;
            rv[n] = V + (size_t)p * d;
        }
        int first_idx_row = n;
        for (int j = 0; j < nidx; ++j, ++n) {
            rk[n] = K + (size_t)idx[j] * d;
            rv[n] = V + (size_t)idx[j] * d;
        }
        attend(d, Q + (size_t)t * d, n, rk, rv, s, out + (size_t)t * d);
        n_dec[t] = nsink + nidx;

        if (att_mask) {
            uint8_t* row = att_mask + (size_t)t * T;
            memset(row, 0, (size_t)T);
            for (int p = 0; p < nsink; ++p) row[p] = 1;
            for (int j = 0; j < nidx; ++j) row[idx[j]] = 1;
        }
        if (skip_mask) {
            uint8_t* row = skip_mask + (size_t)t * T;
            memset(row, 0, (size_t)T);
            for (int j = 0; j < nskip; ++j) row[skip_idx[j]] = 1;
        }

        if (select) {
            /* w <- softmax(Q_t K[idx]^T); j* <- argmin_j w[j]: the lowest raw logit,
             * first (lowest position) among equals since idx ascends */
            int best = 0;
            for (int j = 1; j < nidx; ++j)
                if (s[first_idx_row + j] < s[first_idx_row + best]) best = j;
            int jstar = idx[best];
            choice[t] = jstar;
            int app = jstar;
            if (follow) {
                int f = follow[t], found = -1;
                for (int j = 0; j < nidx; ++j)
                    if (idx[j] == f) found = j;
                if (found < 0) {
                    rc = -2;
                    goto done;
                }
                if (gap) {
                    double a = s[first_idx_row + found], b = s[first_idx_row + best];
                    double mag = fabs(a) > fabs(b) ? fabs(a) : fabs(b);
                    gap[t] = mag > 0.0 ? (a - b) / mag : 0.0;
                }
                app = f;
            }
            /* skip_idx.append(idx[j*]) */
            skip_idx[nskip++] = app;
        }
    }
done:
    free(skip_idx);
    free(present);
    free(in_skip);
    free(idx);
    free(rk);
    free(rv);
    free(s);
    return rc;
}

/*
 * Dense decode attention ("No sparsity", page 4 Sec. 2.3 (1)): step t attends
 * every prompt row and every decode position 0 .. t.  Arrays as above.
 */
int oracle_dense_lane(int L_p, int d, int T, const double* Q, const double* Kp, const double* Vp,
                      const double* K, const double* V, double* out) {
    if (L_p < 0 || d < 1 || T < 0) return -1;
    int nmax = L_p + T + 1;
    const double** rk = (const double**)malloc(sizeof(double*) * (size_t)nmax);
    const double** rv = (const double**)malloc(sizeof(double*) * (size_t)nmax);
    double* s = (double*)malloc(sizeof(double) * (size_t)nmax);
    if (!rk || !rv || !s) {
        free(rk);
        free(rv);
        free(s);
        return -3;
    }
    for (int t = 0; t < T; ++t) {
        int n = 0;
        for (int j = 0; j < L_p; ++j, ++n) {
            rk[n] = Kp + (size_t)j * d;
            rv[n] = Vp + (size_t)j * d;
        }
        for (int p = 0; p <= t; ++p, ++n) {
            rk[n] = K + (size_t)p * d;
            rv[n] = V + (size_t)p * d;
        }
        attend(d, Q + (size_t)t * d, n, rk, rv, s, out + (size_t)t * d);
    }
    free(rk);
    free(rv);
    free(s);
    return 0;
}
