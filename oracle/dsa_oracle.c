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
 * route to a closed form, so this file runs the algorithm step by step with
 * the pages' quantities: absolute decode positions, the skipped set as a list
 * of positions that each move +1 per step, an explicit window and an explicit
 * eviction.  All
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
 *   - the lowest-score entry is found on the raw logits q . k (softmax keeps
 *     their order; no scaling that could merge values), ties go to the
 *     lowest position;
 *   - the candidates are the decode entries attended at step t, the current
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
 * Lane state of the selection.  Decode positions are absolute (token t has
 * position t); `skip` holds the positions of the skipped set in the order
 * they were chosen, and moves along the attention diagonal by one position per
 * step; `held` says which decode positions the cache still holds.
 */
struct lane {
    int S;       /* sink count (0 or 4) */
    int Nr_w;    /* window length over non-sink positions, N_r - S */
    int room;    /* how many positions the skipped set may hold, N_r - N_att */
    int nskip;
    int32_t* skip;
    uint8_t* held;
};

/*
 * Which regime step t is in ([DAS] Section 4, Algorithm 1 and its "Detailed
 * explanation"): every decode entry attended until N_att - 1 steps have run;
 * then one entry joins the skipped set per step while the window grows; from
 * t = N_r on the window slides and its oldest entry leaves the cache.
 */
enum regime { ATTEND_ALL = 1, GROW_SKIPS = 2, SLIDE_WINDOW = 3 };

static enum regime regime_of(int t, int N_att, int N_r) {
    if (t < N_att - 1) return ATTEND_ALL;
    return t < N_r ? GROW_SKIPS : SLIDE_WINDOW;
}

/* The diagonal move: a position skipped for query t - 1 is skipped at its
 * successor for query t (Algorithm 1, phases 2 and 3). */
static void move_along_diagonal(struct lane* L) {
    for (int j = 0; j < L->nskip; ++j) L->skip[j] += 1;
}

/* Phase 3: the non-sink entry that falls out of the window loses its K/V.
 * Returns its position. */
static int drop_oldest(struct lane* L, int t) {
    int p = t - L->Nr_w;
    L->held[p] = 0;
    return p;
}

/*
 * Decode positions step t attends, ascending: the sinks that exist by now,
 * then every window position (non-sink, within the last Nr_w positions up to
 * t itself) whose K/V is still held and that is not in the skipped set.
 * `mark` is scratch of T bytes.  Returns the count; *nsink gets the sinks.
 */
static int attended_positions(const struct lane* L, int t, int T, uint8_t* mark, int32_t* pos, int* nsink) {
    int n = 0;
    for (int p = 0; p < L->S && p <= t; ++p) pos[n++] = p;
    *nsink = n;
    memset(mark, 0, (size_t)T);
    for (int j = 0; j < L->nskip; ++j)
        if (L->skip[j] >= 0 && L->skip[j] < T) mark[L->skip[j]] = 1;
    int first = t - L->Nr_w;
    if (first < L->S) first = L->S;
    for (int p = first; p <= t; ++p)
        if (L->held[p] && !mark[p]) pos[n++] = p;
    return n;
}

/*
 * One lane, decode steps t = 0 .. T-1.
 *   Q, K, V     : [T][d] query / key / value of decode token t (K, V indexed by position)
 *   Kp, Vp      : [L_p][d] prompt keys / values
 *   follow      : optional [T]; at a selection step the position added to the
 *                 skipped set is follow[t] instead of the oracle's own choice
 *                 (lockstep with another implementation).  It must be a
 *                 candidate, else the call fails with -2.
 * Outputs (each [T], or [T][d] / [T][T]; the optional ones may be NULL):
 *   out         : attention output of step t
 *   choice      : the oracle's own lowest-score position at step t, -1 when no selection
 *   evicted     : position evicted at step t, -1 when none
 *   n_dec       : number of decode positions attended at step t (sinks included)
 *   gap         : optional; at selection steps with follow, (s[follow] - s[choice]) / max(|s[follow]|, |s[choice]|)
 *                 on the raw logits, else 0
 *   att_mask    : optional; att_mask[t*T + p] = 1 iff decode position p is attended at step t
 *   skip_mask   : optional; skip_mask[t*T + p] = 1 iff p is in the skipped set when step t attends
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
    struct lane L;
    L.S = S;
    L.Nr_w = N_r - S;
    L.room = N_r - N_att;
    L.nskip = 0;
    L.skip = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N_r + 1));
    L.held = (uint8_t*)calloc((size_t)(T > 0 ? T : 1), 1);
    uint8_t* mark = (uint8_t*)calloc((size_t)(T > 0 ? T : 1), 1);
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T + 1));
    int nrows_max = L_p + S + T + 1;
    const double** rk = (const double**)malloc(sizeof(double*) * (size_t)nrows_max);
    const double** rv = (const double**)malloc(sizeof(double*) * (size_t)nrows_max);
    double* s = (double*)malloc(sizeof(double) * (size_t)nrows_max);
    if (!L.skip || !L.held || !mark || !pos || !rk || !rv || !s) {
        rc = -3;
        goto done;
    }

    for (int t = 0; t < T; ++t) {
        enum regime ph = regime_of(t, N_att, N_r);
        L.held[t] = 1; /* token t's K/V joins the cache */
        choice[t] = -1;
        evicted[t] = -1;
        if (gap) gap[t] = 0.0;

        if (ph != ATTEND_ALL) move_along_diagonal(&L);
        if (ph == SLIDE_WINDOW) evicted[t] = drop_oldest(&L, t);

        int nsink = 0;
        int npos = attended_positions(&L, t, T, mark, pos, &nsink);
        n_dec[t] = npos;

        /* the prompt rows, then the attended decode rows, in one softmax */
        int n = 0;
        for (int j = 0; j < L_p; ++j, ++n) {
            rk[n] = Kp + (size_t)j * d;
            rv[n] = Vp + (size_t)j * d;
        }
        for (int j = 0; j < npos; ++j, ++n) {
            rk[n] = K + (size_t)pos[j] * d;
            rv[n] = V + (size_t)pos[j] * d;
        }
        attend(d, Q + (size_t)t * d, n, rk, rv, s, out + (size_t)t * d);

        if (att_mask) {
            uint8_t* row = att_mask + (size_t)t * T;
            memset(row, 0, (size_t)T);
            for (int j = 0; j < npos; ++j) row[pos[j]] = 1;
        }
        if (skip_mask) {
            uint8_t* row = skip_mask + (size_t)t * T;
            memset(row, 0, (size_t)T);
            for (int j = 0; j < L.nskip; ++j) row[L.skip[j]] = 1;
        }

        /* Phase 2 while the skipped set has room: the attended window entry
         * with the lowest score joins it (it is still attended at this step).
         * Softmax preserves the order of the raw logits, so the lowest logit
         * is compared; scanning positions upward, the first (oldest) of equal
         * logits wins.  Sinks are no candidates. */
        if (ph == GROW_SKIPS && L.nskip < L.room) {
            const double* sw = s + L_p + nsink; /* logits of the window entries */
            const int32_t* pw = pos + nsink;
            int nw = npos - nsink;
            int best = 0;
            for (int j = 1; j < nw; ++j)
                if (sw[j] < sw[best]) best = j;
            choice[t] = pw[best];
            int joins = pw[best];
            if (follow) {
                int found = -1;
                for (int j = 0; j < nw; ++j)
                    if (pw[j] == follow[t]) found = j;
                if (found < 0) {
                    rc = -2;
                    goto done;
                }
                if (gap) {
                    double a = sw[found], b = sw[best];
                    double mag = fabs(a) > fabs(b) ? fabs(a) : fabs(b);
                    gap[t] = mag > 0.0 ? (a - b) / mag : 0.0;
                }
                joins = follow[t];
            }
            L.skip[L.nskip++] = joins;
        }
    }
done:
    free(L.skip);
    free(L.held);
    free(mark);
    free(pos);
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
