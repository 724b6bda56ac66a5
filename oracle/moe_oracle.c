/*
 * moe_oracle.c -- plain, slow, obviously correct CPU oracle for the sparse
 * Mixture-of-Experts feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; the two meet only in the seeded inputs they are both fed.
 *
 * What it computes, and where that is defined:
 *   - The operation order is the one stated in the Feed-forward panel
 *     ("Decoder microscope", Feed-forward: Mixture of Experts) of the
 *     Qwen3.8-Flash-Next anatomy page on frontier-model-atlas: router logits,
 *     then a softmax, then the top-10 routed experts, then a normalisation of
 *     the selected weights; one shared expert runs beside the routed path and
 *     is scaled by a sigmoid gate of its own.
 *   - Experts are gated MLPs (llm-architectures-explained "Qwen3.8-Flash-Next",
 *     table "Every architecture field", row ffns.moe.gated) whose activation
 *     is SiLU (llm-atlas "Qwen3.8-Flash-Next", table "Raw config fields",
 *     row hidden_act).
 *
 * Readings where the pages say nothing (each is listed in the design notes):
 *   - The router logit is accumulated in binary32 in one fixed order, the
 *     "canonical order" below, so that a GPU that follows the same order
 *     reaches the same bits and the integer top-k decision is taken on the
 *     same numbers on both sides.
 *   - Selection key: the logit (softmax is strictly increasing, so the set is
 *     the same as for probabilities); ties go to the lower expert index; the
 *     selected experts are listed by descending logit.
 *   - Normalisation: divide each selected probability by the sum of the
 *     selected probabilities (no epsilon).
 *   - Gated MLP: silu(gate . x) * (up . x), gate = first F rows of the packed
 *     gate/up matrix, up = the next F rows.
 *   - Shared gate: s = sigmoid(g . x) with a vector g of length d, no bias.
 *   - An optional fp32 router bias b[E] is added to the finished dot product.
 *   - Everything after the router logit is computed in binary64 with no
 *     intermediate rounding.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC
 * (no fast-math: the binary32 router logit must round exactly as written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Read element i of an array that holds either binary32 values or bfloat16
 * bit patterns.  Widening bfloat16 to binary32 is exact (append 16 zero
 * mantissa bits). */
static float load_elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORACLE_F32)
        return ((const float *)base)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Router logit l = sum_k x[k] * w[k] + bias in binary32, canonical order:
 *   64 partial sums acc[j], all starting at +0.0f;
 *   for each 512-wide chunk (ascending), for q = 0..7 (ascending), for each
 *   j: element kk = chunk + 8*j + q (if kk < d) is folded in with one fused
 *   multiply-add, acc[j] = fmaf(x[kk], w[kk], acc[j]);
 *   then a fixed halving tree: for s = 32, 16, 8, 4, 2, 1 and j < s,
 *   acc[j] = acc[j] + acc[j + s];
 *   finally l = acc[0] + bias.
 * The definition of the logit is the plain dot product; this fixes only the
 * rounding order. */
static float router_logit(const void *x, int64_t xoff, const void *w,
                          int64_t woff, int d, int dtype, float bias)
{
    float acc[64];
    for (int j = 0; j < 64; j++)
        acc[j] = 0.0f;
    for (int chunk = 0; chunk < d; chunk += 512)
        for (int q = 0; q < 8; q++)
            for (int j = 0; j < 64; j++) {
                int kk = chunk + 8 * j + q;
                if (kk < d)
                    acc[j] = fmaf(load_elem(x, dtype, xoff + kk),
                                  load_elem(w, dtype, woff + kk), acc[j]);
            }
    for (int s = 32; s >= 1; s >>= 1)
        for (int j = 0; j < s; j++)
            acc[j] = acc[j] + acc[j + s];
    return acc[0] + bias;
}

/* logits[t*E + e] for all tokens and experts. */
int oracle_router_logits(int64_t T, int d, int E, int dtype, const void *x,
                         const void *w_router, const float *bias,
                         float *logits)
{
    if (T < 0 || d < 1 || E < 1 || !x || !w_router || !logits)
        return 1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < T; t++)
        for (int e = 0; e < E; e++)
            logits[t * E + e] = router_logit(x, t * d, w_router, (int64_t)e * d,
                                             d, dtype, bias ? bias[e] : 0.0f);
    return 0;
}

typedef struct {
    float l;
    int e;
} candidate;

/* Descending logit, then ascending expert index.  The key is total over
 * distinct experts, so the sorted order is unique. */
static int candidate_cmp(const void *a, const void *b)
{
    const candidate *p = (const candidate *)a;
    const candidate *q = (const candidate *)b;
    if (p->l > q->l)
        return -1;
    if (p->l < q->l)
        return 1;
    return (p->e > q->e) - (p->e < q->e);
}

/* Selection, softmax and normalisation for one token from its E logits.
 * idx[k]: the first k entries of a full sort; w[k]: p_sel / sum(p_sel) with
 * p the softmax over all E logits, in binary64. */
static void select_and_weigh(const float *l, int E, int k, int32_t *idx,
                             double *w, candidate *scratch)
{
    for (int e = 0; e < E; e++) {
        scratch[e].l = l[e];
        scratch[e].e = e;
    }
    qsort(scratch, (size_t)E, sizeof(candidate), candidate_cmp);

    /* softmax over all E logits, binary64 */
    double m = (double)scratch[0].l;
    double z = 0.0;
    for (int e = 0; e < E; e++)
        z += exp((double)l[e] - m);
    double sel = 0.0;
    for (int j = 0; j < k; j++) {
        idx[j] = scratch[j].e;
        w[j] = exp((double)l[idx[j]] - m) / z;
        sel += w[j];
    }
    /* selected-weight normalisation */
    for (int j = 0; j < k; j++)
        w[j] = w[j] / sel;
}

int oracle_route(int64_t T, int d, int E, int k, int dtype, const void *x,
                 const void *w_router, const float *bias, int32_t *topk_idx,
                 double *topk_w, float *logits_out)
{
    if (T < 0 || d < 1 || E < 1 || k < 1 || k > E || !x || !w_router ||
        !topk_idx || !topk_w)
        return 1;
    int fail = 0;
#pragma omp parallel
    {
        float *l = (float *)malloc(sizeof(float) * (size_t)E);
        candidate *scratch = (candidate *)malloc(sizeof(candidate) * (size_t)E);
        /* every thread reaches the loop; one without scratch only flags */
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < T; t++) {
            if (!l || !scratch) {
#pragma omp atomic write
                fail = 1;
                continue;
            }
            for (int e = 0; e < E; e++)
                l[e] = router_logit(x, t * d, w_router, (int64_t)e * d, d,
                                    dtype, bias ? bias[e] : 0.0f);
            if (logits_out)
                memcpy(logits_out + t * E, l, sizeof(float) * (size_t)E);
            select_and_weigh(l, E, k, topk_idx + t * k, topk_w + t * k,
                             scratch);
        }
        free(l);
        free(scratch);
    }
    return fail ? 2 : 0;
}

/* Shared-expert gate s = sigmoid(g . x), binary64, no bias. */
static double shared_gate(const void *x, int64_t xoff, const void *g, int d,
                          int dtype)
{
    double z = 0.0;
    for (int kk = 0; kk < d; kk++)
        z += (double)load_elem(x, dtype, xoff + kk) *
             (double)load_elem(g, dtype, kk);
    return 1.0 / (1.0 + exp(-z));
}

/* One gated-MLP expert on one token, binary64:
 *   a = W_gate x, u = W_up x, h = silu(a) * u with silu(a) = a / (1 + e^-a),
 *   y = W_down h.
 * w_gu points at the packed [2F, d] gate/up block (gate rows first), w_dn at
 * the [d, F] down block. */
static void gated_mlp(const void *x, int64_t xoff, const void *w_gu,
                      int64_t gu_off, const void *w_dn, int64_t dn_off, int d,
                      int F, int dtype, double *h, double *y)
{
    for (int n = 0; n < F; n++) {
        double a = 0.0, u = 0.0;
        for (int kk = 0; kk < d; kk++) {
            double xv = (double)load_elem(x, dtype, xoff + kk);
            a += (double)load_elem(w_gu, dtype, gu_off + (int64_t)n * d + kk) * xv;
            u += (double)load_elem(w_gu, dtype, gu_off + (int64_t)(F + n) * d + kk) * xv;
        }
        h[n] = a / (1.0 + exp(-a)) * u;
    }
    for (int m = 0; m < d; m++) {
        double acc = 0.0;
        for (int n = 0; n < F; n++)
            acc += (double)load_elem(w_dn, dtype, dn_off + (int64_t)m * F + n) * h[n];
        y[m] = acc;
    }
}

/* Expert stage with routing given: out[t] = sum_j w[t,j] * y_{idx[t,j]}(x_t)
 * + s_t * y_shared(x_t).  With Fs == 0 the shared term is absent.  s_out
 * (nullable) receives the shared gate values. */
int oracle_experts(int64_t T, int d, int E, int k, int F, int Fs, int dtype,
                   const void *x, const void *w_gate_up, const void *w_down,
                   const void *w_sh_gate_up, const void *w_sh_down,
                   const void *sh_gate, const int32_t *topk_idx,
                   const double *topk_w, double *out, double *s_out)
{
    if (T < 0 || d < 1 || E < 1 || k < 1 || F < 1 || Fs < 0 || !x ||
        !w_gate_up || !w_down || !topk_idx || !topk_w || !out)
        return 1;
    if (Fs > 0 && (!w_sh_gate_up || !w_sh_down || !sh_gate))
        return 1;
    for (int64_t i = 0; i < T * k; i++)
        if (topk_idx[i] < 0 || topk_idx[i] >= E)
            return 1;
    int fmax = F > Fs ? F : Fs;
    int fail = 0;
#pragma omp parallel
    {
        double *h = (double *)malloc(sizeof(double) * (size_t)fmax);
        double *y = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; t++) {
            if (!h || !y) {
#pragma omp atomic write
                fail = 1;
                continue;
            }
            double *o = out + t * d;
            for (int m = 0; m < d; m++)
                o[m] = 0.0;
            for (int j = 0; j < k; j++) {
                int e = topk_idx[t * k + j];
                gated_mlp(x, t * d, w_gate_up, (int64_t)e * 2 * F * d, w_down,
                          (int64_t)e * d * F, d, F, dtype, h, y);
                for (int m = 0; m < d; m++)
                    o[m] += topk_w[t * k + j] * y[m];
            }
            if (Fs > 0) {
                double s = shared_gate(x, t * d, sh_gate, d, dtype);
                if (s_out)
                    s_out[t] = s;
                gated_mlp(x, t * d, w_sh_gate_up, 0, w_sh_down, 0, d, Fs, dtype,
                          h, y);
                for (int m = 0; m < d; m++)
                    o[m] += s * y[m];
            }
        }
        free(h);
        free(y);
    }
    return fail ? 2 : 0;
}

/* The whole layer: routing (oracle_route) then the expert stage. */
int oracle_forward(int64_t T, int d, int E, int k, int F, int Fs, int dtype,
                   const void *x, const void *w_router, const float *bias,
                   const void *w_gate_up, const void *w_down,
                   const void *w_sh_gate_up, const void *w_sh_down,
                   const void *sh_gate, double *out, int32_t *topk_idx,
                   double *topk_w, double *s_out)
{
    int rc = oracle_route(T, d, E, k, dtype, x, w_router, bias, topk_idx,
                          topk_w, NULL);
    if (rc)
        return rc;
    return oracle_experts(T, d, E, k, F, Fs, dtype, x, w_gate_up, w_down,
                          w_sh_gate_up, w_sh_down, sh_gate, topk_idx, topk_w,
                          out, s_out);
}

/* Number of threads the parallel loops above use. */
#ifdef _OPENMP
#include <omp.h>
#endif
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
