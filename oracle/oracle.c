/*
 * CPU oracle for the forward pass of one Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code with
 * the HIP path: no header, helper, table or constant generator is common to
 * the two. Both sides take their inputs from the seeded generators, which hold
 * none of the layer's arithmetic.
 *
 * What the layer computes, and where the pages state it:
 *   - router in fp32, whatever the activation dtype
 *       (moe-200m-qwen3-100b README, "Per-layer numerics", first item;
 *        "SigmoidRouter": logits = x W_r^T on fp32 copies of both operands);
 *   - sigmoid scores, selection on scores plus a per-expert bias that moves
 *     selection only; combine weights gathered from the unbiased scores and
 *     divided by their sum plus 1e-9
 *       ("SigmoidRouter"; SpecForge PR #930, "What this adds" and "Tests");
 *   - softmax over all experts, top-k weights renormalised, no scaling, no
 *     shared expert (SpecForge PR #930, "What this adds", the qwen3 preset);
 *   - top-k sorted by descending selection value ("SigmoidRouter": topk);
 *   - tokens per expert ("SigmoidRouter": one-hot sum over tokens);
 *   - SwiGLU experts with weights stacked [E, out, in], an optional shared
 *     expert that every token uses with weight 1, and a weighted sum of the
 *     expert outputs (README "Architecture diagram"; PR #930 "Why FSDP is
 *     enough here").
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the design notes of the repository):
 *   - the fp32 gate product is one fused-multiply-add chain per (token,
 *     expert), over features in ascending order, starting from +0;
 *   - with no bias the selection value is the logit itself (softmax and
 *     sigmoid are strictly increasing, so the chosen set and order are those
 *     of the scores, with no rounding of exp in the way);
 *   - the bias is added to the score (sigmoid, or softmax probability);
 *   - exp inside the router is the canonical fp32 function cexpf below;
 *   - ties are broken towards the lower expert index;
 *   - softmax weights are exp(l_j - M) / sum_i exp(l_i - M) over the k
 *     selected logits, M their maximum (equal to p_j / sum p_i in real
 *     arithmetic because the full normaliser cancels);
 *   - sums over slots and over experts run in ascending index order;
 *   - rows of one expert are ordered by ascending token index;
 *   - the expert MLPs and the combine run in fp64 on the exact values of the
 *     inputs (bf16 widens exactly), so the oracle's own rounding is far below
 *     any tolerance used against it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define DT_F32 0
#define DT_BF16 1
#define SCORE_SOFTMAX 0
#define SCORE_SIGMOID 1

/* ------------------------------------------------------------------------ */
/* element access                                                            */
/* ------------------------------------------------------------------------ */

static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Element i of a row-major array holding fp32 values or bf16 bit patterns. */
static float elem(const void *p, int dtype, size_t i)
{
    if (dtype == DT_BF16)
        return bf16_to_float(((const uint16_t *)p)[i]);
    return ((const float *)p)[i];
}

static float bits_to_float(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ------------------------------------------------------------------------ */
/* canonical fp32 exp                                                        */
/* ------------------------------------------------------------------------ */

/*
 * exp(a) in fp32 from IEEE +, -, *, / and fma only, so that any machine with
 * IEEE arithmetic gets the same bits.
 *   1. n = nearest integer to a / ln 2 (a * log2(e), rounded half to even).
 *   2. r = a - n ln 2 with ln 2 split into two fp32 constants (Cody and
 *      Waite, 1980): hi = ln 2 rounded to fp32, lo = (ln 2 - hi) rounded to
 *      fp32; each step is one fma. |r| <= about 0.347.
 *   3. exp(r) by its Taylor series to degree 7 in Horner form with fma; the
 *      dropped term is below r^8/8! < 6e-9 relative, under half an fp32 ulp.
 *   4. exp(a) = exp(r) * 2^n, the power of two built from its bit pattern;
 *      when 2^n itself is not a normal fp32 the scaling is split in two so
 *      that only the final multiply rounds (subnormal results included).
 * Overflow above 88.72283935546875 gives +inf, underflow below
 * -103.972084045410 gives +0 (exp there is under half the least subnormal).
 */
float oracle_cexpf(float a)
{
    const float LOG2E = 1.44269504088896340736f;
    const float LN2_HI = 0.693147182464599609375f;      /* fp32(ln 2) */
    const float LN2_LO = -1.9046542121259336e-09f;     /* fp32(ln 2 - LN2_HI) */
    const float C2 = 1.0f / 2.0f, C3 = 1.0f / 6.0f, C4 = 1.0f / 24.0f;
    const float C5 = 1.0f / 120.0f, C6 = 1.0f / 720.0f, C7 = 1.0f / 5040.0f;
    float n, r, p;
    int ni;

    if (a != a)
        return a;
    if (a > 88.72283935546875f)
        return INFINITY;
    if (a < -103.972084045410f)
        return 0.0f;

    n = rintf(a * LOG2E);
    r = fmaf(-n, LN2_HI, a);
    r = fmaf(-n, LN2_LO, r);

    p = C7;
    p = fmaf(p, r, C6);
    p = fmaf(p, r, C5);
    p = fmaf(p, r, C4);
    p = fmaf(p, r, C3);
    p = fmaf(p, r, C2);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);

    ni = (int)n;
    if (ni > 127)
        return (p * 2.0f) * bits_to_float((uint32_t)(ni - 1 + 127) << 23);
    if (ni < -126)
        return (p * bits_to_float((uint32_t)(ni + 64 + 127) << 23)) * bits_to_float((uint32_t)(-64 + 127) << 23);
    return p * bits_to_float((uint32_t)(ni + 127) << 23);
}

void oracle_cexpf_array(const float *a, float *out, int64_t n)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; i++)
        out[i] = oracle_cexpf(a[i]);
}

/* ------------------------------------------------------------------------ */
/* router                                                                    */
/* ------------------------------------------------------------------------ */

/*
 * logits[t, e] = sum_j x[t, j] * W_r[e, j] in fp32, as one fma chain over j
 * ascending from +0 ("SigmoidRouter": F.linear on fp32 copies).
 * Written with experts innermost so that the chains of one token run side by
 * side; each chain still sees its terms in ascending j.
 */
void oracle_logits(int dtype, const void *x, int64_t T, int d, const float *w_router, int E, float *logits)
{
    float *wt = (float *)malloc(sizeof(float) * (size_t)d * (size_t)E); /* W_r transposed: [d][E] */
    int64_t t;
    int j, e;
    for (e = 0; e < E; e++)
        for (j = 0; j < d; j++)
            wt[(size_t)j * E + e] = w_router[(size_t)e * d + j];
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; t++) {
        float *acc = logits + (size_t)t * E;
        int jj, ee;
        for (ee = 0; ee < E; ee++)
            acc[ee] = 0.0f;
        for (jj = 0; jj < d; jj++) {
            const float xv = elem(x, dtype, (size_t)t * d + jj);
            const float *wrow = wt + (size_t)jj * E;
            for (ee = 0; ee < E; ee++)
                acc[ee] = fmaf(xv, wrow[ee], acc[ee]);
        }
    }
    free(wt);
}

static float sigmoidf_canon(float l)
{
    return 1.0f / (1.0f + oracle_cexpf(-l));
}

/*
 * Routing of one token from its fp32 logits l[0..E-1]: selection values,
 * top-k, combine weights.
 */
static void route_token(const float *l, const float *bias, int bias_on_logits, const float *noise, int E, int k,
                        int score, int renorm, float *v, unsigned char *taken, int32_t *idx, float *w)
{
    int e, j;
    float m = 0.0f, z = 0.0f;

    /* Softmax normaliser over all experts: only needed for a softmax score
     * that is biased in score space or not renormalised. */
    if (score == SCORE_SOFTMAX && ((bias && !bias_on_logits) || !renorm)) {
        m = l[0];
        for (e = 1; e < E; e++)
            if (l[e] > m)
                m = l[e];
        z = 0.0f;
        for (e = 0; e < E; e++)
            z += oracle_cexpf(l[e] - m);
    }

    /* selection value; the bias enters the score (default) or the logit
     * (the README's SigmoidRouter code), exploration noise (training only)
     * is added last */
    for (e = 0; e < E; e++) {
        if (!bias)
            v[e] = l[e];
        else if (bias_on_logits)
            v[e] = l[e] + bias[e];
        else if (score == SCORE_SIGMOID)
            v[e] = sigmoidf_canon(l[e]) + bias[e];
        else
            v[e] = oracle_cexpf(l[e] - m) / z + bias[e];
        if (noise)
            v[e] = v[e] + noise[e];
    }

    /* top-k: k times, the largest remaining value; on a tie the lower index
     * is kept because only a strictly larger value replaces the candidate. */
    memset(taken, 0, (size_t)E);
    for (j = 0; j < k; j++) {
        int best = -1;
        for (e = 0; e < E; e++) {
            if (taken[e])
                continue;
            if (best < 0 || v[e] > v[best])
                best = e;
        }
        taken[best] = 1;
        idx[j] = best;
    }

    /* combine weights from the unbiased scores */
    if (score == SCORE_SOFTMAX) {
        if (renorm) {
            float mk = l[idx[0]], s = 0.0f;
            for (j = 1; j < k; j++)
                if (l[idx[j]] > mk)
                    mk = l[idx[j]];
            for (j = 0; j < k; j++) {
                w[j] = oracle_cexpf(l[idx[j]] - mk);
                s += w[j];
            }
            for (j = 0; j < k; j++)
                w[j] = w[j] / s;
        } else {
            for (j = 0; j < k; j++)
                w[j] = oracle_cexpf(l[idx[j]] - m) / z;
        }
    } else {
        float s = 0.0f;
        for (j = 0; j < k; j++) {
            w[j] = sigmoidf_canon(l[idx[j]]);
            s += w[j];
        }
        if (renorm)
            for (j = 0; j < k; j++)
                w[j] = w[j] / (s + 1e-9f);
    }
}

/*
 * Router for T tokens: idx [T, k] (slots in descending selection value),
 * w [T, k] fp32, counts [E] (tokens per expert). logits_out [T, E] is
 * optional. Returns 0, or -1 on bad arguments.
 */
int oracle_route_ex(int dtype, const void *x, int64_t T, int d, const float *w_router, const float *sel_bias,
                    int bias_on_logits, const float *noise, int E, int k, int score, int renorm, int32_t *idx,
                    float *w, int32_t *counts, float *logits_out)
{
    float *logits;
    int64_t t;
    int e;
    if (T < 0 || d < 1 || E < 1 || k < 1 || k > E)
        return -1;
    logits = logits_out ? logits_out : (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * (size_t)E);
    oracle_logits(dtype, x, T, d, w_router, E, logits);
#pragma omp parallel
    {
        float *v = (float *)malloc(sizeof(float) * (size_t)E);
        unsigned char *taken = (unsigned char *)malloc((size_t)E);
#pragma omp for schedule(static)
        for (t = 0; t < T; t++)
            route_token(logits + (size_t)t * E, sel_bias, bias_on_logits, noise ? noise + (size_t)t * E : NULL, E, k,
                        score, renorm, v, taken, idx + (size_t)t * k, w + (size_t)t * k);
        free(v);
        free(taken);
    }
    for (e = 0; e < E; e++)
        counts[e] = 0;
    for (t = 0; t < T * k; t++)
        counts[idx[t]]++;
    if (!logits_out)
        free(logits);
    return 0;
}

int oracle_route(int dtype, const void *x, int64_t T, int d, const float *w_router, const float *sel_bias,
                 int E, int k, int score, int renorm, int32_t *idx, float *w, int32_t *counts, float *logits_out)
{
    return oracle_route_ex(dtype, x, T, d, w_router, sel_bias, 0, NULL, E, k, score, renorm, idx, w, counts,
                           logits_out);
}

/*
 * Router losses and health metrics of one forward pass (README,
 * "SigmoidRouter": z-loss, aux loss, counts, coefficient of variation,
 * entropy of the mean score distribution; SpecForge PR #931, "What to
 * watch": max/mean load and the share of unused experts), in fp64 from the
 * fp32 logits and the chosen ids:
 *   out[0] z_loss         mean over tokens of logsumexp(logits)^2
 *   out[1] aux_loss       E * sum_i f_i P_i, f_i = counts_i / T,
 *                         P_i = mean over tokens of the score of expert i
 *   out[2] cv             std(counts, unbiased) / max(mean(counts), 1); 0 for E = 1
 *   out[3] entropy_bits   -sum p log2 p, p = max(P, 1e-9) normalised to sum 1
 *   out[4] load_max_ratio max(counts) / mean(counts)
 *   out[5] unused_frac    share of experts with no token
 * Scores are sigmoid(logit) or the softmax over all experts.
 */
void oracle_router_metrics(const float *logits, const int32_t *idx, int64_t T, int E, int k, int score, double *out)
{
    double *P = (double *)calloc((size_t)E, sizeof(double));
    double *cnt = (double *)calloc((size_t)E, sizeof(double));
    double z = 0.0, aux = 0.0, mean, var = 0.0, ent = 0.0, psum = 0.0, mx = 0.0;
    int64_t t;
    int e, unused = 0;
    for (t = 0; t < T; t++) {
        const float *l = logits + (size_t)t * E;
        double m = l[0], s = 0.0, lse;
        for (e = 1; e < E; e++)
            if (l[e] > m)
                m = l[e];
        for (e = 0; e < E; e++)
            s += exp((double)l[e] - m);
        lse = m + log(s);
        z += lse * lse;
        for (e = 0; e < E; e++)
            P[e] += score == SCORE_SIGMOID ? 1.0 / (1.0 + exp(-(double)l[e])) : exp((double)l[e] - m) / s;
    }
    for (t = 0; t < T * k; t++)
        cnt[idx[t]] += 1.0;
    mean = (double)(T * k) / E;
    for (e = 0; e < E; e++) {
        P[e] /= (double)T;
        aux += (cnt[e] / (double)T) * P[e];
        var += (cnt[e] - mean) * (cnt[e] - mean);
        if (cnt[e] > mx)
            mx = cnt[e];
        if (cnt[e] == 0.0)
            unused++;
        psum += P[e] > 1e-9 ? P[e] : 1e-9;
    }
    for (e = 0; e < E; e++) {
        double p = (P[e] > 1e-9 ? P[e] : 1e-9) / psum;
        ent -= p * log(p);
    }
    out[0] = T > 0 ? z / (double)T : 0.0;
    out[1] = (double)E * aux;
    out[2] = E > 1 ? sqrt(var / (double)(E - 1)) / (mean > 1.0 ? mean : 1.0) : 0.0;
    out[3] = ent / log(2.0);
    out[4] = mean > 0.0 ? mx / mean : 0.0;
    out[5] = (double)unused / E;
    free(P);
    free(cnt);
}

/*
 * Aux-loss-free balance controller, applied after a forward pass so that the
 * next forward selects with the new bias (README, "SigmoidRouter",
 * step_bias_update; SpecForge PR #930 "Tests": deferred balance update).
 * In fp32, in the order of that code:
 *   p_i = counts_i / max(sum counts, 1);  err = 1/E - p_i;
 *   err += 0.5 where p_i < 0.1 / E (starved expert);  bias += err * rate;
 *   bias = clamp(bias, -10, 10).
 * The constants 1/E and 0.1/E are formed in fp64 and rounded to fp32 once,
 * as a Python scalar meets an fp32 tensor; the sum of counts is exact
 * integer arithmetic.
 */
void oracle_bias_update(const int32_t *counts, int E, float rate, float *bias)
{
    int64_t sum = 0;
    float total, target = (float)(1.0 / E), starved = (float)(0.1 * (1.0 / E));
    int e;
    for (e = 0; e < E; e++)
        sum += counts[e];
    total = (float)sum;
    if (total < 1.0f)
        total = 1.0f;
    for (e = 0; e < E; e++) {
        float p = (float)counts[e] / total;
        float err = target - p;
        if (p < starved)
            err = err + 0.5f;
        bias[e] = bias[e] + err * rate;
        if (bias[e] < -10.0f)
            bias[e] = -10.0f;
        if (bias[e] > 10.0f)
            bias[e] = 10.0f;
    }
}

/*
 * Expert-contiguous order. offsets = exclusive scan of counts (E+1 entries);
 * row_of[t, j] = offsets[e] + number of tokens t' < t that chose e, with
 * e = idx[t, j]. Each token holds k distinct experts, so this is a stable
 * ordering of the (token, slot) pairs by expert.
 */
int oracle_dispatch(int64_t T, int E, int k, const int32_t *idx, int32_t *counts, int32_t *offsets, int32_t *row_of)
{
    int32_t *cursor = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int64_t t;
    int e, j;
    for (e = 0; e < E; e++)
        counts[e] = 0;
    for (t = 0; t < T * k; t++) {
        if (idx[t] < 0 || idx[t] >= E) {
            free(cursor);
            return -1;
        }
        counts[idx[t]]++;
    }
    offsets[0] = 0;
    for (e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + counts[e];
    for (t = 0; t < T; t++)
        for (j = 0; j < k; j++) {
            e = idx[t * k + j];
            row_of[t * k + j] = offsets[e] + cursor[e]++;
        }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* experts                                                                   */
/* ------------------------------------------------------------------------ */

static double silu(double z)
{
    return z / (1.0 + exp(-z));
}

#define PAIR_BLOCK 16

/*
 * SwiGLU expert outputs for a list of (row, expert) pairs, in fp64:
 *   out[p] = W_down[e] (silu(W_gate[e] a) * (W_up[e] a)),  a = x[row[p]],
 * with W_gate, W_up [E, d_ff, d] and W_down [E, d, d_ff]. The pairs are
 * visited expert by expert (the "sorted loop"), PAIR_BLOCK rows at a time so
 * that each weight row is read once per block.
 */
static int experts_impl(int dtype, int d, int d_ff, const void *x, int64_t n_pairs, const int64_t *pair_row,
                        const int32_t *pair_expert, int E, const void *w_gate, const void *w_up, const void *w_down,
                        double *out, int absolute)
{
    int64_t *order, *starts, n_blocks = 0, p;
    int64_t *count;
    int e;
    if (n_pairs <= 0)
        return 0;
    /* stable counting sort of the pairs by expert */
    count = (int64_t *)calloc((size_t)E + 1, sizeof(int64_t));
    order = (int64_t *)malloc(sizeof(int64_t) * (size_t)n_pairs);
    for (p = 0; p < n_pairs; p++) {
        if (pair_expert[p] < 0 || pair_expert[p] >= E) {
            free(count);
            free(order);
            return -1;
        }
        count[pair_expert[p] + 1]++;
    }
    for (e = 0; e < E; e++)
        count[e + 1] += count[e];
    {
        int64_t *cur = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
        memcpy(cur, count, sizeof(int64_t) * (size_t)E);
        for (p = 0; p < n_pairs; p++)
            order[cur[pair_expert[p]]++] = p;
        free(cur);
    }
    /* work items: blocks of up to PAIR_BLOCK pairs of one expert */
    starts = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_pairs + E + 1));
    for (e = 0; e < E; e++)
        for (p = count[e]; p < count[e + 1]; p += PAIR_BLOCK)
            starts[n_blocks++] = p;

#pragma omp parallel
    {
        double *xb = (double *)malloc(sizeof(double) * (size_t)d * PAIR_BLOCK);   /* [d][B] */
        double *hb = (double *)malloc(sizeof(double) * (size_t)d_ff * PAIR_BLOCK); /* [d_ff][B] */
        double *wr = (double *)malloc(sizeof(double) * (size_t)(d > d_ff ? d : d_ff));
        double *wr2 = (double *)malloc(sizeof(double) * (size_t)d);
        int64_t bi;
#pragma omp for schedule(dynamic, 1)
        for (bi = 0; bi < n_blocks; bi++) {
            int64_t s = starts[bi];
            int ex = pair_expert[order[s]];
            int64_t end = count[ex + 1];
            int nb = (int)((end - s) < PAIR_BLOCK ? (end - s) : PAIR_BLOCK);
            int b, i, f, c;
            const size_t wg_off = (size_t)ex * d_ff * d, wd_off = (size_t)ex * d * d_ff;
            for (b = 0; b < nb; b++) {
                int64_t row = pair_row[order[s + b]];
                for (i = 0; i < d; i++)
                    xb[(size_t)i * PAIR_BLOCK + b] = (double)elem(x, dtype, (size_t)row * d + i);
            }
            /* gate and up projections, SwiGLU */
            for (f = 0; f < d_ff; f++) {
                double g[PAIR_BLOCK], u[PAIR_BLOCK];
                for (b = 0; b < PAIR_BLOCK; b++)
                    g[b] = u[b] = 0.0;
                for (i = 0; i < d; i++) {
                    wr[i] = (double)elem(w_gate, dtype, wg_off + (size_t)f * d + i);
                    wr2[i] = (double)elem(w_up, dtype, wg_off + (size_t)f * d + i);
                }
                for (i = 0; i < d; i++) {
                    const double *xi = xb + (size_t)i * PAIR_BLOCK;
                    for (b = 0; b < PAIR_BLOCK; b++) {
                        g[b] += wr[i] * xi[b];
                        u[b] += wr2[i] * xi[b];
                    }
                }
                for (b = 0; b < PAIR_BLOCK; b++) {
                    double h = silu(g[b]) * u[b];
                    hb[(size_t)f * PAIR_BLOCK + b] = absolute ? fabs(h) : h;
                }
            }
            /* down projection */
            for (c = 0; c < d; c++) {
                double o[PAIR_BLOCK];
                for (b = 0; b < PAIR_BLOCK; b++)
                    o[b] = 0.0;
                for (f = 0; f < d_ff; f++) {
                    wr[f] = (double)elem(w_down, dtype, wd_off + (size_t)c * d_ff + f);
                    if (absolute)
                        wr[f] = fabs(wr[f]);
                }
                for (f = 0; f < d_ff; f++) {
                    const double *hf = hb + (size_t)f * PAIR_BLOCK;
                    for (b = 0; b < PAIR_BLOCK; b++)
                        o[b] += wr[f] * hf[b];
                }
                for (b = 0; b < nb; b++)
                    out[(size_t)order[s + b] * d + c] = o[b];
            }
        }
        free(xb);
        free(hb);
        free(wr);
        free(wr2);
    }
    free(starts);
    free(order);
    free(count);
    return 0;
}

int oracle_experts(int dtype, int d, int d_ff, const void *x, int64_t n_pairs, const int64_t *pair_row,
                   const int32_t *pair_expert, int E, const void *w_gate, const void *w_up, const void *w_down,
                   double *out)
{
    return experts_impl(dtype, d, d_ff, x, n_pairs, pair_row, pair_expert, E, w_gate, w_up, w_down, out, 0);
}

/*
 * Magnitude envelope of the same pairs: sum_f |W_down[e, c, f]| |h_f| with
 * h = silu(W_gate a) * (W_up a). A relative perturbation of at most u in
 * every h_f moves the expert output by at most u times this envelope; the
 * tests use it to bound the effect of storing h in a narrower type.
 */
int oracle_experts_abs(int dtype, int d, int d_ff, const void *x, int64_t n_pairs, const int64_t *pair_row,
                       const int32_t *pair_expert, int E, const void *w_gate, const void *w_up, const void *w_down,
                       double *out)
{
    return experts_impl(dtype, d, d_ff, x, n_pairs, pair_row, pair_expert, E, w_gate, w_up, w_down, out, 1);
}

/*
 * The layer's output for a subset of tokens, in fp64:
 *   y[t] = sum_{j<k} w[t, j] * E_{idx[t, j]}(x_t)  (+ S(x_t), weight 1)
 * summed over slots in order, the shared expert added last
 * (README "Architecture diagram": routed experts and the always-on shared
 * expert feed one weighted sum). tokens [n_tok] lists the token ids; y is
 * [n_tok, d]. The shared weights may be NULL.
 */
int oracle_combine(int dtype, int d, int d_ff, int d_ff_shared, const void *x, int64_t n_tok, const int64_t *tokens,
                   int k, const int32_t *idx, const float *w, int E, const void *w_gate, const void *w_up,
                   const void *w_down, const void *ws_gate, const void *ws_up, const void *ws_down, double *y)
{
    int64_t n_pairs = n_tok * k, p, i;
    int64_t *prow = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_pairs > 0 ? n_pairs : 1));
    int32_t *pexp = (int32_t *)calloc((size_t)(n_pairs > 0 ? n_pairs : 1), sizeof(int32_t));
    double *o = (double *)malloc(sizeof(double) * (size_t)(n_pairs > 0 ? n_pairs : 1) * (size_t)d);
    double *s = NULL;
    int rc, j, c;
    for (i = 0; i < n_tok; i++)
        for (j = 0; j < k; j++) {
            prow[i * k + j] = tokens[i];
            pexp[i * k + j] = idx[tokens[i] * k + j];
        }
    rc = oracle_experts(dtype, d, d_ff, x, n_pairs, prow, pexp, E, w_gate, w_up, w_down, o);
    if (rc == 0 && ws_gate) {
        int32_t *zero = (int32_t *)calloc((size_t)(n_tok > 0 ? n_tok : 1), sizeof(int32_t));
        s = (double *)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1) * (size_t)d);
        rc = oracle_experts(dtype, d, d_ff_shared, x, n_tok, tokens, zero, 1, ws_gate, ws_up, ws_down, s);
        free(zero);
    }
    if (rc == 0) {
        for (i = 0; i < n_tok; i++)
            for (c = 0; c < d; c++) {
                double acc = 0.0;
                for (j = 0; j < k; j++) {
                    p = i * k + j;
                    acc += (double)w[tokens[i] * k + j] * o[(size_t)p * d + c];
                }
                if (s)
                    acc += s[(size_t)i * d + c];
                y[(size_t)i * d + c] = acc;
            }
    }
    free(prow);
    free(pexp);
    free(o);
    free(s);
    return rc;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* backward                                                                  */
/* ------------------------------------------------------------------------ */

static double sigm(double z)
{
    return 1.0 / (1.0 + exp(-z));
}

/* One SwiGLU expert on one token in fp64, keeping what its backward needs:
 * g = W_gate a, u = W_up a, h = silu(g) u, out = W_down h. */
static void expert_forward(int dtype, int d, int d_ff, const double *a, const void *wg, const void *wu,
                           const void *wd, size_t off_gu, size_t off_d, double *g, double *u, double *h, double *out)
{
    int f, c;
    for (f = 0; f < d_ff; f++) {
        double sg = 0.0, su = 0.0;
        for (c = 0; c < d; c++) {
            sg += (double)elem(wg, dtype, off_gu + (size_t)f * d + c) * a[c];
            su += (double)elem(wu, dtype, off_gu + (size_t)f * d + c) * a[c];
        }
        g[f] = sg;
        u[f] = su;
        h[f] = silu(sg) * su;
    }
    if (out)
        for (c = 0; c < d; c++) {
            double s = 0.0;
            for (f = 0; f < d_ff; f++)
                s += (double)elem(wd, dtype, off_d + (size_t)c * d_ff + f) * h[f];
            out[c] = s;
        }
}

/* Backward of that expert given dout, the gradient of its output:
 * dh = W_down^T dout, dg = dh u silu'(g), du = dh silu(g), with
 * silu'(z) = s (1 + z (1 - s)), s = sigmoid(z). */
static void expert_backward(int dtype, int d, int d_ff, const void *wd, size_t off_d, const double *g,
                            const double *u, const double *dout, double *dg, double *du)
{
    int f, c;
    for (f = 0; f < d_ff; f++) {
        double dh = 0.0, s = sigm(g[f]);
        for (c = 0; c < d; c++)
            dh += (double)elem(wd, dtype, off_d + (size_t)c * d_ff + f) * dout[c];
        dg[f] = dh * u[f] * s * (1.0 + g[f] * (1.0 - s));
        du[f] = dh * g[f] * s;
    }
}

/* da += W_gate^T dg + W_up^T du */
static void expert_input_grad(int dtype, int d, int d_ff, const void *wg, const void *wu, size_t off_gu,
                              const double *dg, const double *du, double *da)
{
    int f, c;
    for (f = 0; f < d_ff; f++)
        for (c = 0; c < d; c++)
            da[c] += (double)elem(wg, dtype, off_gu + (size_t)f * d + c) * dg[f] +
                     (double)elem(wu, dtype, off_gu + (size_t)f * d + c) * du[f];
}

/*
 * Gradient of the router logits of one token (fp64, from the fp32 logits l
 * and the combine-weight gradients dtw of its k slots), for the weight rule
 * of the forward pass (README "SigmoidRouter": weights gathered from the
 * unbiased scores and renormalised; PR #930 "What this adds": softmax over
 * all experts, top-k renormalised), plus the z-loss and aux-loss terms of
 * "SigmoidRouter" scaled by their coefficients:
 *   z_loss = mean_t lse_t^2                -> 2 lse_t softmax(l_t) / T
 *   aux    = E sum_e f_e mean_t score_te,  f_e = counts_e / T (a constant)
 * The selection itself (top-k, bias, noise) is piecewise constant and passes
 * no gradient.
 */
static void router_token_grad(const float *l, int E, int k, const int32_t *idx, const double *dtw, int score,
                              int renorm, int64_t T, const double *f, double z_coef, double aux_coef, double *dl)
{
    int e, j;
    double m = l[0], z = 0.0, lse;
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    for (e = 1; e < E; e++)
        if (l[e] > m)
            m = l[e];
    for (e = 0; e < E; e++)
        z += exp((double)l[e] - m);
    lse = m + log(z);
    for (e = 0; e < E; e++) {
        p[e] = exp((double)l[e] - m) / z;
        dl[e] = 0.0;
    }
    if (score == SCORE_SOFTMAX && renorm) {
        double mk = l[idx[0]], zk = 0.0, dot = 0.0;
        for (j = 1; j < k; j++)
            if (l[idx[j]] > mk)
                mk = l[idx[j]];
        for (j = 0; j < k; j++)
            zk += exp((double)l[idx[j]] - mk);
        for (j = 0; j < k; j++)
            dot += exp((double)l[idx[j]] - mk) / zk * dtw[j];
        for (j = 0; j < k; j++)
            dl[idx[j]] += exp((double)l[idx[j]] - mk) / zk * (dtw[j] - dot);
    } else if (score == SCORE_SOFTMAX) {
        double dot = 0.0;
        for (j = 0; j < k; j++)
            dot += p[idx[j]] * dtw[j];
        for (e = 0; e < E; e++)
            dl[e] -= p[e] * dot;
        for (j = 0; j < k; j++)
            dl[idx[j]] += p[idx[j]] * dtw[j];
    } else if (renorm) {
        double S = 0.0, dot = 0.0, D;
        for (j = 0; j < k; j++)
            S += sigm(l[idx[j]]);
        D = S + 1e-9;
        for (j = 0; j < k; j++)
            dot += dtw[j] * sigm(l[idx[j]]);
        for (j = 0; j < k; j++) {
            double s = sigm(l[idx[j]]);
            dl[idx[j]] += (dtw[j] / D - dot / (D * D)) * s * (1.0 - s);
        }
    } else {
        for (j = 0; j < k; j++) {
            double s = sigm(l[idx[j]]);
            dl[idx[j]] += dtw[j] * s * (1.0 - s);
        }
    }
    if (z_coef != 0.0)
        for (e = 0; e < E; e++)
            dl[e] += z_coef * 2.0 * lse * p[e] / (double)T;
    if (aux_coef != 0.0) {
        double fp = 0.0;
        for (e = 0; e < E; e++)
            fp += f[e] * p[e];
        for (e = 0; e < E; e++) {
            if (score == SCORE_SIGMOID) {
                double s = sigm(l[e]);
                dl[e] += aux_coef * (double)E / (double)T * f[e] * s * (1.0 - s);
            } else {
                dl[e] += aux_coef * (double)E / (double)T * p[e] * (f[e] - fp);
            }
        }
    }
    free(p);
}

/*
 * Backward pass of the layer for a given routing (idx, w from the forward
 * pass) and output gradient dy [T, d] fp32, all in fp64 on the exact inputs:
 *   d_topk_w[t, j] = <dy_t, E_e(x_t)>,        e = idx[t, j]
 *   expert e, token t:  dout = w[t, j] dy_t;  dW_down[e] += dout h^T;
 *     dW_gate[e] += dg x_t^T;  dW_up[e] += du x_t^T;  dx_t += W_gate^T dg + W_up^T du
 *   shared expert: the same with dout = dy_t
 *   router: dlogits from d_topk_w (router_token_grad); dW_router = dlogits^T x;
 *     dx_t += W_router^T dlogits_t
 * The logits are the forward's fp32 ones (oracle_logits). Weight gradients
 * are summed over tokens in ascending order. The shared weights and their
 * gradients may be NULL (no shared expert). Returns nonzero for an expert id
 * out of range.
 */
int oracle_backward(int dtype, const void *x, int64_t T, int d, int E, int k, int d_ff, int d_ff_s,
                    const float *w_router, const void *w_gate, const void *w_up, const void *w_down,
                    const void *ws_gate, const void *ws_up, const void *ws_down, int score, int renorm,
                    const int32_t *idx, const float *w, const float *dy, double z_coef, double aux_coef, double *dx,
                    double *dw_router, double *dw_gate, double *dw_up, double *dw_down, double *dws_gate,
                    double *dws_up, double *dws_down, double *d_topk_w)
{
    float *lg;
    double *f, *dl;
    int64_t t, n = T * k;
    int e, bad = 0;
    for (t = 0; t < n; t++)
        if (idx[t] < 0 || idx[t] >= E)
            return 1;
    lg = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * (size_t)E);
    f = (double *)calloc((size_t)E, sizeof(double));
    dl = (double *)calloc((size_t)(T > 0 ? T : 1) * (size_t)E, sizeof(double));
    oracle_logits(dtype, x, T, d, w_router, E, lg);
    for (t = 0; t < n; t++)
        f[idx[t]] += 1.0 / (double)T;

    /* per token: combine-weight gradients, router logit gradients, dx */
#pragma omp parallel for schedule(dynamic, 4)
    for (t = 0; t < T; t++) {
        int c, j, ds = d_ff_s > 0 ? d_ff_s : 1;
        int mf = d_ff > ds ? d_ff : ds;
        double *a = (double *)malloc(sizeof(double) * (size_t)d);
        double *g = (double *)malloc(sizeof(double) * (size_t)mf);
        double *u = (double *)malloc(sizeof(double) * (size_t)mf);
        double *h = (double *)malloc(sizeof(double) * (size_t)mf);
        double *dg = (double *)malloc(sizeof(double) * (size_t)mf);
        double *du = (double *)malloc(sizeof(double) * (size_t)mf);
        double *out = (double *)malloc(sizeof(double) * (size_t)d);
        double *dout = (double *)malloc(sizeof(double) * (size_t)d);
        double *dtw = (double *)malloc(sizeof(double) * (size_t)k);
        double *da = dx + (size_t)t * d;
        for (c = 0; c < d; c++) {
            a[c] = (double)elem(x, dtype, (size_t)t * d + c);
            da[c] = 0.0;
        }
        for (j = 0; j < k; j++) {
            int ee = idx[t * k + j];
            size_t ogu = (size_t)ee * d_ff * d, od = (size_t)ee * d * d_ff;
            double s = 0.0;
            expert_forward(dtype, d, d_ff, a, w_gate, w_up, w_down, ogu, od, g, u, h, out);
            for (c = 0; c < d; c++) {
                s += (double)dy[(size_t)t * d + c] * out[c];
                dout[c] = (double)w[t * k + j] * (double)dy[(size_t)t * d + c];
            }
            dtw[j] = s;
            if (d_topk_w)
                d_topk_w[t * k + j] = s;
            expert_backward(dtype, d, d_ff, w_down, od, g, u, dout, dg, du);
            expert_input_grad(dtype, d, d_ff, w_gate, w_up, ogu, dg, du, da);
        }
        if (ws_gate) {
            for (c = 0; c < d; c++)
                dout[c] = (double)dy[(size_t)t * d + c];
            expert_forward(dtype, d, d_ff_s, a, ws_gate, ws_up, ws_down, 0, 0, g, u, h, NULL);
            expert_backward(dtype, d, d_ff_s, ws_down, 0, g, u, dout, dg, du);
            expert_input_grad(dtype, d, d_ff_s, ws_gate, ws_up, 0, dg, du, da);
        }
        router_token_grad(lg + (size_t)t * E, E, k, idx + t * k, dtw, score, renorm, T, f, z_coef, aux_coef,
                          dl + (size_t)t * E);
        for (j = 0; j < E; j++)
            for (c = 0; c < d; c++)
                da[c] += dl[(size_t)t * E + j] * (double)w_router[(size_t)j * d + c];
        free(a);
        free(g);
        free(u);
        free(h);
        free(dg);
        free(du);
        free(out);
        free(dout);
        free(dtw);
    }

    /* weight gradients, one expert (or the shared expert, index E) at a time */
#pragma omp parallel for schedule(dynamic, 1)
    for (e = 0; e <= E; e++) {
        int shared = e == E, ff = shared ? d_ff_s : d_ff, c, j, q;
        size_t ogu = shared ? 0 : (size_t)e * d_ff * d, od = shared ? 0 : (size_t)e * d * d_ff;
        const void *wg = shared ? ws_gate : w_gate, *wu = shared ? ws_up : w_up, *wd = shared ? ws_down : w_down;
        double *Gg = shared ? dws_gate : dw_gate + ogu, *Gu = shared ? dws_up : dw_up + ogu;
        double *Gd = shared ? dws_down : dw_down + od;
        double *a, *g, *u, *h, *dg, *du, *dout;
        int64_t tt;
        if (shared && !ws_gate)
            continue;
        a = (double *)malloc(sizeof(double) * (size_t)d);
        g = (double *)malloc(sizeof(double) * (size_t)ff);
        u = (double *)malloc(sizeof(double) * (size_t)ff);
        h = (double *)malloc(sizeof(double) * (size_t)ff);
        dg = (double *)malloc(sizeof(double) * (size_t)ff);
        du = (double *)malloc(sizeof(double) * (size_t)ff);
        dout = (double *)malloc(sizeof(double) * (size_t)d);
        memset(Gg, 0, sizeof(double) * (size_t)ff * d);
        memset(Gu, 0, sizeof(double) * (size_t)ff * d);
        memset(Gd, 0, sizeof(double) * (size_t)d * ff);
        for (tt = 0; tt < T; tt++) {
            for (j = 0; j < (shared ? 1 : k); j++) {
                double wt = 1.0;
                if (!shared) {
                    if (idx[tt * k + j] != e)
                        continue;
                    wt = (double)w[tt * k + j];
                }
                for (c = 0; c < d; c++) {
                    a[c] = (double)elem(x, dtype, (size_t)tt * d + c);
                    dout[c] = wt * (double)dy[(size_t)tt * d + c];
                }
                expert_forward(dtype, d, ff, a, wg, wu, wd, ogu, od, g, u, h, NULL);
                expert_backward(dtype, d, ff, wd, od, g, u, dout, dg, du);
                for (c = 0; c < d; c++)
                    for (q = 0; q < ff; q++)
                        Gd[(size_t)c * ff + q] += dout[c] * h[q];
                for (q = 0; q < ff; q++)
                    for (c = 0; c < d; c++) {
                        Gg[(size_t)q * d + c] += dg[q] * a[c];
                        Gu[(size_t)q * d + c] += du[q] * a[c];
                    }
            }
        }
        free(a);
        free(g);
        free(u);
        free(h);
        free(dg);
        free(du);
        free(dout);
    }

    /* router weight gradient: dW_router[e] = sum_t dlogits[t, e] x_t */
#pragma omp parallel for
    for (e = 0; e < E; e++) {
        int c;
        int64_t tt;
        for (c = 0; c < d; c++)
            dw_router[(size_t)e * d + c] = 0.0;
        for (tt = 0; tt < T; tt++) {
            double v = dl[(size_t)tt * E + e];
            if (v == 0.0)
                continue;
            for (c = 0; c < d; c++)
                dw_router[(size_t)e * d + c] += v * (double)elem(x, dtype, (size_t)tt * d + c);
        }
    }
    free(lg);
    free(f);
    free(dl);
    return bad;
}
