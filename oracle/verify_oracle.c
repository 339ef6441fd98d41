/* fp64 CPU oracle of the batched speculative-sampling verify step, in plain C.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a second, independent transcription of the rule
 * the numpy oracle (spec_verify_oracle.py) implements, for checks that need many
 * sequences: it runs without Python's interpreter lock, so a thread pool over sequences
 * scales over the host's cores.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load it.  It shares no code, header, table or
 * constant with the HIP library; the status bits are restated from the documented
 * contract.
 *
 * What it computes, per sequence, following the lesson page "Decodificação
 * Especulativa e EAGLE" (ai-engineering.academy; the same text as "Việc giải mã giả
 * định và Eagle"):
 *   - p_t = softmax(zt_t / T), q_t = softmax(zd_t / T), the same T on both sides (the
 *     temperature softmax of the "Desenvolva" listing);
 *   - left to right, draft token x_t is accepted while ln u_t < ln p_t(x_t) - ln q_t(x_t),
 *     the test r < p(x)/q(x) of "A Regra de Exatidão" in log space (q = 0 with p > 0
 *     accepts, p = 0 rejects; no underflow of p or q on their own);
 *   - at the first rejection t, one token from the positive part of the pointwise
 *     difference (p_t - q_t)+ over the whole vocabulary ("A Regra de Exatidão");
 *   - after K acceptances, a bonus token from p_K ("O Conceito", step 4);
 *   - at T = 0, accept while argmax(zt_t) == x_t, else emit that argmax; after K
 *     matches emit argmax(zt_K) ("Caso ganancioso").
 * The readings where the pages are silent are the numpy oracle's: lowest-index argmax;
 * categorical draw = smallest i with C_i > u S (C the left-to-right fp64 prefix sums, S
 * the last one), the last index with positive weight if rounding leaves none; uniform
 * u[K] drives the final draw; zero residual mass falls back to p_t with the NOTE bit.
 *
 * Arithmetic: logits widen exactly to double (bf16 is the top half of an fp32); every
 * exponential, sum, quotient and prefix is fp64 (libm exp), sums left to right.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
    ORC_ERR_TOKEN = 1,
    ORC_ERR_LOGIT = 2,
    ORC_ERR_TEMPERATURE = 4,
    ORC_ERR_UNIFORM = 8,
    ORC_NOTE_FALLBACK = 16,
    ORC_ERROR_MASK = 1 | 2 | 4 | 8 | 32 | 64,
};

enum { ORC_DTYPE_F32 = 0, ORC_DTYPE_BF16 = 1, ORC_DTYPE_F64 = 2 };
enum { ORC_DRAW_TEST = 0, ORC_DRAW_RESIDUAL = 1, ORC_DRAW_BONUS = 2 };

/* Element i of a logit row, widened exactly to double. */
static double logit_at(const void *row, int dtype, int64_t i) {
    if (dtype == ORC_DTYPE_BF16) {
        uint32_t w = (uint32_t)((const uint16_t *)row)[i] << 16;
        float f;
        memcpy(&f, &w, sizeof f);
        return (double)f;
    }
    if (dtype == ORC_DTYPE_F64) return ((const double *)row)[i];
    return (double)((const float *)row)[i];
}

static void decode_row(const void *row, int dtype, int V, double *out) {
    for (int i = 0; i < V; ++i) out[i] = logit_at(row, dtype, i);
}

static double row_max(const double *z, int V) {
    double m = -INFINITY;
    for (int i = 0; i < V; ++i)
        if (z[i] > m) m = z[i];
    return m;
}

/* T is NaN, negative, infinite, or positive below the smallest normal fp32. */
static int temperature_error(double T) {
    if (isnan(T) || T < 0.0 || isinf(T)) return 1;
    return T > 0.0 && T < 0x1p-126;
}

/* NaN anywhere, a maximum of -inf, or (sampled rows) a +inf logit; with a valid
 * temperature T > 0 also a maximum m with |m| * c2 >= 2^30, c2 = log2(e)/T rounded to
 * fp32 (the range of scaled logits the library supports, a contract of its own; the
 * product of two fp32 values is exact in double). */
static int row_error(const double *z, int V, int sampled, double T) {
    for (int i = 0; i < V; ++i)
        if (isnan(z[i])) return 1;
    const double m = row_max(z, V);
    if (m == -INFINITY) return 1;
    if (sampled && m == INFINITY) return 1;
    if (sampled && T > 0.0 && !temperature_error(T)) {
        const double c2 = (double)(float)(1.4426950408889634 / T);
        if (fabs(m) * c2 >= 0x1p30) return 1;
    }
    return 0;
}

/* Lowest index of the maximum. */
static int argmax_first(const double *z, int V) {
    int best = 0;
    for (int i = 1; i < V; ++i)
        if (z[i] > z[best]) best = i;
    return best;
}

/* sum_i exp((z_i - m) / T), m the row maximum, left to right. */
static double sum_exp(const double *z, int V, double m, double T) {
    double s = 0.0;
    for (int i = 0; i < V; ++i) s += exp((z[i] - m) / T);
    return s;
}

/* p = softmax(z / T) in fp64 (shifted by the maximum; the quotient is unchanged). */
static void softmax_t(const double *z, int V, double T, double *p) {
    const double m = row_max(z, V);
    double s = 0.0;
    for (int i = 0; i < V; ++i) {
        p[i] = exp((z[i] - m) / T);
        s += p[i];
    }
    for (int i = 0; i < V; ++i) p[i] /= s;
}

/* Smallest i with C_i > u S, C_i = w_0 + ... + w_i (left to right), S = C_{V-1}.
 * *margin = distance from u to the nearer edge of the chosen cell [C_{i-1}/S, C_i/S);
 * *fell = no index satisfied the predicate (then the last index with w > 0).  c is
 * scratch of V doubles. */
static int categorical_draw(const double *w, int V, double u, double *c, double *margin, int *fell) {
    double run = 0.0;
    for (int i = 0; i < V; ++i) {
        run += w[i];
        c[i] = run;
    }
    const double S = c[V - 1];
    const double target = u * S;
    int i = 0;
    while (i < V && !(c[i] > target)) ++i;
    *fell = 0;
    if (i >= V) {
        *fell = 1;
        i = V - 1;
        while (i > 0 && !(w[i] > 0.0)) --i;
    }
    const double lo = (i > 0 ? c[i - 1] : 0.0) / S;
    const double hi = c[i] / S;
    *margin = fmin(fabs(u - lo), fabs(hi - u));
    return i;
}

/* One sequence.
 *   zt: [K+1][V] target logits, zd: [K][V] draft logits (may be NULL when T == 0), both
 *   dtype (0: fp32, 1: bf16 bit patterns, 2: fp64); x: [K] draft tokens; u: [K+1]
 *   uniforms widened to double (may be NULL when T == 0); T: temperature.
 * Outputs: tokens [K+1] (-1 padded), *n (accepted drafts, -1 on a data error), p, q [K]
 * (p_t(x_t), q_t(x_t); NaN on greedy or failed sequences), the draws in the order the
 * uniforms are consumed (kind, position, margin; at most K+1), *ndraws.
 * Returns the status bits.  -1: out of memory. */
int oracle_verify_sequence(const void *zt, const void *zd, int dtype, int K, int V,
                           const int32_t *x, const double *u, double T, int32_t *tokens,
                           int32_t *n, double *p, double *q, int32_t *draw_kind,
                           int32_t *draw_t, double *draw_margin, int32_t *ndraws) {
    const size_t esize = dtype == ORC_DTYPE_BF16 ? 2 : dtype == ORC_DTYPE_F64 ? 8 : 4;
    const int greedy = T == 0.0;
    int status = 0;
    *ndraws = 0;
    *n = -1;
    for (int t = 0; t <= K; ++t) tokens[t] = -1;
    for (int t = 0; t < K; ++t) p[t] = q[t] = NAN;

    if (temperature_error(T)) status |= ORC_ERR_TEMPERATURE;
    for (int t = 0; t < K; ++t)
        if (x[t] < 0 || x[t] >= V) status |= ORC_ERR_TOKEN;
    if (!greedy)
        for (int t = 0; t <= K; ++t)
            if (isnan(u[t]) || u[t] < 0.0 || u[t] >= 1.0) status |= ORC_ERR_UNIFORM;

    double *z = malloc(sizeof(double) * (size_t)V);
    double *zb = malloc(sizeof(double) * (size_t)V);
    double *w = malloc(sizeof(double) * (size_t)V);
    double *c = malloc(sizeof(double) * (size_t)V);
    if (!z || !zb || !w || !c) {
        free(z); free(zb); free(w); free(c);
        return -1;
    }
    double *lp = NULL, *lq = NULL;
    const char *trow = (const char *)zt;
    const char *drow = (const char *)zd;
    const size_t rowb = esize * (size_t)V;

    /* every row the sequence reads must be valid */
    for (int t = 0; t <= K; ++t) {
        decode_row(trow + rowb * t, dtype, V, z);
        if (row_error(z, V, !greedy, T)) status |= ORC_ERR_LOGIT;
    }
    if (!greedy)
        for (int t = 0; t < K; ++t) {
            decode_row(drow + rowb * t, dtype, V, z);
            if (row_error(z, V, 1, T)) status |= ORC_ERR_LOGIT;
        }
    if (status & ORC_ERROR_MASK) goto done;

    if (greedy) {
        int t = 0;
        for (; t < K; ++t) {
            decode_row(trow + rowb * t, dtype, V, z);
            const int a = argmax_first(z, V);
            if (a != x[t]) {
                tokens[t] = a;
                break;
            }
            tokens[t] = x[t];
        }
        if (t == K) {
            decode_row(trow + rowb * K, dtype, V, z);
            tokens[K] = argmax_first(z, V);
        }
        *n = t;
        goto done;
    }

    /* ln p_t(x_t), ln q_t(x_t) at every drafted position: (z_x - m)/T - ln sum */
    lp = malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    lq = malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!lp || !lq) {
        free(lp); free(lq); free(z); free(zb); free(w); free(c);
        return -1;
    }
    for (int t = 0; t < K; ++t) {
        decode_row(trow + rowb * t, dtype, V, z);
        double m = row_max(z, V);
        lp[t] = (z[x[t]] - m) / T - log(sum_exp(z, V, m, T));
        decode_row(drow + rowb * t, dtype, V, z);
        m = row_max(z, V);
        lq[t] = (z[x[t]] - m) / T - log(sum_exp(z, V, m, T));
        p[t] = exp(lp[t]);
        q[t] = exp(lq[t]);
    }
    for (int t = 0; t < K; ++t) {
        const double ut = u[t];
        /* the test r < p/q in log space: ln u < ln p - ln q; p = 0 rejects, q = 0 with
           p > 0 accepts (then u does not matter: margin infinite) */
        int accept;
        double margin;
        if (lp[t] == -INFINITY || lq[t] == -INFINITY) {
            accept = lp[t] != -INFINITY;
            margin = INFINITY;
        } else {
            accept = (ut > 0.0 ? log(ut) : -INFINITY) < lp[t] - lq[t];
            margin = fabs(ut - exp(lp[t] - lq[t]));
        }
        draw_kind[*ndraws] = ORC_DRAW_TEST;
        draw_t[*ndraws] = t;
        draw_margin[*ndraws] = margin;
        ++*ndraws;
        if (accept) {
            tokens[t] = x[t];
            continue;
        }
        /* first rejection: the replacement from (p_t - q_t)+ */
        decode_row(trow + rowb * t, dtype, V, z);
        decode_row(drow + rowb * t, dtype, V, zb);
        softmax_t(z, V, T, c);  /* p_t into c, then q_t into zb */
        softmax_t(zb, V, T, w);
        double mass = 0.0;
        for (int i = 0; i < V; ++i) {
            const double d = c[i] - w[i];
            w[i] = d > 0.0 ? d : 0.0;
            mass += w[i];
        }
        if (!(mass > 0.0)) {
            status |= ORC_NOTE_FALLBACK;
            memcpy(w, c, sizeof(double) * (size_t)V);
        }
        int fell;
        tokens[t] = categorical_draw(w, V, u[K], c, &margin, &fell);
        if (fell) status |= ORC_NOTE_FALLBACK;
        draw_kind[*ndraws] = ORC_DRAW_RESIDUAL;
        draw_t[*ndraws] = t;
        draw_margin[*ndraws] = margin;
        ++*ndraws;
        *n = t;
        goto done;
    }
    /* all K accepted: the bonus token from p_K */
    {
        decode_row(trow + rowb * K, dtype, V, z);
        softmax_t(z, V, T, w);
        double margin;
        int fell;
        tokens[K] = categorical_draw(w, V, u[K], c, &margin, &fell);
        if (fell) status |= ORC_NOTE_FALLBACK;
        draw_kind[*ndraws] = ORC_DRAW_BONUS;
        draw_t[*ndraws] = K;
        draw_margin[*ndraws] = margin;
        ++*ndraws;
        *n = K;
    }

done:
    if (status & ORC_ERROR_MASK) {
        *n = -1;
        *ndraws = 0;
        for (int t = 0; t <= K; ++t) tokens[t] = -1;
        for (int t = 0; t < K; ++t) p[t] = q[t] = NAN;
    }
    free(lp);
    free(lq);
    free(z);
    free(zb);
    free(w);
    free(c);
    return status;
}

int oracle_abi_version(void) { return 1; }
