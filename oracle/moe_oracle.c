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
 *   - Low-bit expert weights: the model's published weights are packed
 *     low-bit tensors (llm-atlas "Qwen3.8-Flash-Next", "Modelled costs",
 *     published-weights row); the pages do not name the encoding.  The
 *     reading taken here is MXFP4 from the OCP Microscaling (MX)
 *     specification v1.0: each run of 32 consecutive elements of a weight row
 *     (along the reduction axis) shares one E8M0 scale byte X, worth
 *     2^(X - 127), and every element is an FP4 E2M1 code (sign bit 3,
 *     exponent bits 2..1 with bias 1, mantissa bit 0; exponent 0 encodes
 *     0 or 0.5).  Codes are stored two per byte, element 2i in bits 3..0 and
 *     element 2i+1 in bits 7..4.  The oracle decodes every element exactly
 *     and then runs the same binary64 gated MLPs.
 *   - Pre-FFN RMSNorm (oracle_rmsnorm): the norm is RMSNorm with eps 1e-6
 *     (llm-atlas "Qwen3.8-Flash-Next", "Key facts" Norm and "Raw config
 *     fields" rms_norm_eps); its placement is not disclosed and is read as
 *     the usual pre-norm: the layer's input is x = h / sqrt(mean(h^2) + eps)
 *     * gamma.  Because the normalised x feeds the integer top-k decision,
 *     it is evaluated in one fixed binary32 order (below) and rounded to the
 *     layer's dtype, so that both sides route on the same bits.
 *   - Backward pass (oracle_backward): the training variant of the layer.
 *     The pages give only the coefficient of the router's auxiliary loss,
 *     0.001 (llm-atlas "Qwen3.8-Flash-Next", "Raw config fields",
 *     router_aux_loss_coef), not its formula.  The reading taken is the
 *     usual load-balancing loss: coef * E * sum_e f_e * P_e, where f_e is
 *     the share of the T*k routed assignments that went to expert e (a count,
 *     so it carries no gradient) and P_e the mean over tokens of the router's
 *     softmax probability of e.  The selection itself is piecewise constant
 *     and is taken as given; gradients reach the router through the
 *     normalised weights of the selected experts and through P.
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
#define ORACLE_MXFP4 2

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

/* FP4 E2M1 element (OCP MX v1.0): sign bit 3, 2-bit exponent field e with
 * bias 1, 1-bit mantissa m.  e = 0 is the subnormal range, m * 2^(1-1) / 2;
 * otherwise 2^(e-1) * (1 + m/2).  The format has no infinity or NaN. */
static double e2m1_value(unsigned code)
{
    unsigned sign = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double v = e == 0 ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return sign ? -v : v;
}

/* E8M0 scale (OCP MX v1.0): 2^(X - 127); X = 255 is NaN. */
static double e8m0_value(unsigned x)
{
    return x == 255u ? NAN : ldexp(1.0, (int)x - 127);
}

/* An expert weight matrix of `cols` elements per row (the reduction axis):
 * binary32 or bfloat16 elements, or MXFP4 codes with one scale byte per 32
 * elements of a row (scales [rows, cols/32]). */
typedef struct {
    int fmt;
    const void *data;
    const uint8_t *scales;
    int64_t cols;
} wsrc;

/* Element (row, kk) of w, exactly, in binary64. */
static double load_w(const wsrc *w, int64_t row, int64_t kk)
{
    if (w->fmt != ORACLE_MXFP4)
        return (double)load_elem(w->data, w->fmt, row * w->cols + kk);
    int64_t i = row * w->cols + kk;
    unsigned byte = ((const uint8_t *)w->data)[i / 2];
    unsigned code = (i % 2) ? (byte >> 4) : (byte & 15u);
    unsigned x = w->scales[row * (w->cols / 32) + kk / 32];
    return e2m1_value(code) * e8m0_value(x);
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

/* binary32 -> bfloat16 bits, round to nearest, ties to even (finite input). */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Pre-FFN RMSNorm of each row of h [T, d] with weight gamma [d], in binary32:
 *   ss   = sum_k h_k^2, in the canonical order of the router logit (the same
 *          64 partials, fused multiply-adds and halving tree, no bias);
 *   mean = ss / d;  v = mean + eps;  r = 1 / sqrtf(v)   (each rounded once);
 *   x_k  = (h_k * r) * gamma_k                          (each product rounded),
 * then rounded to bfloat16 (nearest even) for bfloat16 layers.  x_out has
 * the layout and dtype of h. */
int oracle_rmsnorm(int64_t T, int d, int dtype, const void *h, const void *gamma,
                   float eps, void *x_out)
{
    if (T < 0 || d < 1 || !h || !gamma || !x_out || !(eps >= 0.0f))
        return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        float ss = router_logit(h, t * d, h, t * d, d, dtype, 0.0f);
        float mean = ss / (float)d;
        float v = mean + eps;
        float r = 1.0f / sqrtf(v);
        for (int kk = 0; kk < d; kk++) {
            float hr = load_elem(h, dtype, t * d + kk) * r;
            float xv = hr * load_elem(gamma, dtype, kk);
            if (dtype == ORACLE_BF16)
                ((uint16_t *)x_out)[t * d + kk] = f32_to_bf16(xv);
            else
                ((float *)x_out)[t * d + kk] = xv;
        }
    }
    return 0;
}

/* Residual update after the layer.  The layer's output joins the residual
 * stream, which the model carries as gated residual streams (anatomy page on
 * frontier-model-atlas, "Residual topology", Gated Residual).  The stream
 * gates are not defined on the pages and stay with the caller, so the update
 * is the plain sum (the gate-1, single-stream case):
 *   res[t, c] = resid[t, c] + out[t, c]      (binary64; resid is binary32)
 * res may alias out. */
int oracle_residual(int64_t T, int d, const float *resid, const double *out,
                    double *res)
{
    if (T < 0 || d < 1 || !resid || !out || !res)
        return 1;
    for (int64_t i = 0; i < T * d; i++)
        res[i] = (double)resid[i] + out[i];
    return 0;
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
 * The expert's gate/up block is rows gu_row .. gu_row + 2F - 1 of w_gu
 * (gate rows first, d elements each); its down block is rows
 * dn_row .. dn_row + d - 1 of w_dn (F elements each). */
static void gated_mlp(const void *x, int64_t xoff, int dtype, const wsrc *w_gu,
                      int64_t gu_row, const wsrc *w_dn, int64_t dn_row, int d,
                      int F, double *h, double *y)
{
    for (int n = 0; n < F; n++) {
        double a = 0.0, u = 0.0;
        for (int kk = 0; kk < d; kk++) {
            double xv = (double)load_elem(x, dtype, xoff + kk);
            a += load_w(w_gu, gu_row + n, kk) * xv;
            u += load_w(w_gu, gu_row + F + n, kk) * xv;
        }
        h[n] = a / (1.0 + exp(-a)) * u;
    }
    for (int m = 0; m < d; m++) {
        double acc = 0.0;
        for (int n = 0; n < F; n++)
            acc += load_w(w_dn, dn_row + m, n) * h[n];
        y[m] = acc;
    }
}

/* Expert stage with routing given: out[t] = sum_j w[t,j] * y_{idx[t,j]}(x_t)
 * + s_t * y_shared(x_t).  With Fs == 0 the shared term is absent.  s_out
 * (nullable) receives the shared gate values.  x and sh_gate are in dtype;
 * the four expert weight tensors are described by their wsrc. */
static int experts_impl(int64_t T, int d, int E, int k, int F, int Fs,
                        int dtype, const void *x, const wsrc *w_gu,
                        const wsrc *w_dn, const wsrc *w_sgu, const wsrc *w_sdn,
                        const void *sh_gate, const int32_t *topk_idx,
                        const double *topk_w, double *out, double *s_out)
{
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
                gated_mlp(x, t * d, dtype, w_gu, (int64_t)e * 2 * F, w_dn,
                          (int64_t)e * d, d, F, h, y);
                for (int m = 0; m < d; m++)
                    o[m] += topk_w[t * k + j] * y[m];
            }
            if (Fs > 0) {
                double s = shared_gate(x, t * d, sh_gate, d, dtype);
                if (s_out)
                    s_out[t] = s;
                gated_mlp(x, t * d, dtype, w_sgu, 0, w_sdn, 0, d, Fs, h, y);
                for (int m = 0; m < d; m++)
                    o[m] += s * y[m];
            }
        }
        free(h);
        free(y);
    }
    return fail ? 2 : 0;
}

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
    wsrc gu = {dtype, w_gate_up, NULL, d}, dn = {dtype, w_down, NULL, F};
    wsrc sgu = {dtype, w_sh_gate_up, NULL, d}, sdn = {dtype, w_sh_down, NULL, Fs};
    return experts_impl(T, d, E, k, F, Fs, dtype, x, &gu, &dn, &sgu, &sdn,
                        sh_gate, topk_idx, topk_w, out, s_out);
}

/* The expert stage with MXFP4 expert weights (routed and shared): codes
 * [E,2F,d/2], [E,d,F/2], [2Fs,d/2], [d,Fs/2]; scales [E,2F,d/32],
 * [E,d,F/32], [2Fs,d/32], [d,Fs/32].  x and sh_gate are bfloat16.  d, F and
 * Fs must be multiples of 32. */
int oracle_experts_mx4(int64_t T, int d, int E, int k, int F, int Fs,
                       const void *x, const uint8_t *gu_codes,
                       const uint8_t *gu_scales, const uint8_t *dn_codes,
                       const uint8_t *dn_scales, const uint8_t *sgu_codes,
                       const uint8_t *sgu_scales, const uint8_t *sdn_codes,
                       const uint8_t *sdn_scales, const void *sh_gate,
                       const int32_t *topk_idx, const double *topk_w,
                       double *out, double *s_out)
{
    if (T < 0 || d < 1 || E < 1 || k < 1 || F < 1 || Fs < 0 || !x ||
        !gu_codes || !gu_scales || !dn_codes || !dn_scales || !topk_idx ||
        !topk_w || !out || d % 32 || F % 32 || Fs % 32)
        return 1;
    if (Fs > 0 && (!sgu_codes || !sgu_scales || !sdn_codes || !sdn_scales ||
                   !sh_gate))
        return 1;
    wsrc gu = {ORACLE_MXFP4, gu_codes, gu_scales, d};
    wsrc dn = {ORACLE_MXFP4, dn_codes, dn_scales, F};
    wsrc sgu = {ORACLE_MXFP4, sgu_codes, sgu_scales, d};
    wsrc sdn = {ORACLE_MXFP4, sdn_codes, sdn_scales, Fs};
    return experts_impl(T, d, E, k, F, Fs, ORACLE_BF16, x, &gu, &dn, &sgu,
                        &sdn, sh_gate, topk_idx, topk_w, out, s_out);
}

/* Decoded value of every MXFP4 element of a [rows, cols] tensor, binary64
 * (for tests of the decoder itself). */
int oracle_mx4_decode(int64_t rows, int64_t cols, const uint8_t *codes,
                      const uint8_t *scales, double *out)
{
    if (rows < 0 || cols < 1 || cols % 32 || !codes || !scales || !out)
        return 1;
    wsrc w = {ORACLE_MXFP4, codes, scales, cols};
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            out[r * cols + c] = load_w(&w, r, c);
    return 0;
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

/* The whole layer with MXFP4 expert weights: routing on the bfloat16 router
 * (oracle_route), then oracle_experts_mx4. */
int oracle_forward_mx4(int64_t T, int d, int E, int k, int F, int Fs,
                       const void *x, const void *w_router, const float *bias,
                       const uint8_t *gu_codes, const uint8_t *gu_scales,
                       const uint8_t *dn_codes, const uint8_t *dn_scales,
                       const uint8_t *sgu_codes, const uint8_t *sgu_scales,
                       const uint8_t *sdn_codes, const uint8_t *sdn_scales,
                       const void *sh_gate, double *out, int32_t *topk_idx,
                       double *topk_w, double *s_out)
{
    int rc = oracle_route(T, d, E, k, ORACLE_BF16, x, w_router, bias, topk_idx,
                          topk_w, NULL);
    if (rc)
        return rc;
    return oracle_experts_mx4(T, d, E, k, F, Fs, x, gu_codes, gu_scales,
                              dn_codes, dn_scales, sgu_codes, sgu_scales,
                              sdn_codes, sdn_scales, sh_gate, topk_idx, topk_w,
                              out, s_out);
}

/* ---------------------------------------------------------------------------
 * Backward pass.
 *
 * The scalar being differentiated is
 *     Lambda = sum_t dout_t . out_t  +  L_aux,
 *     L_aux  = coef * E * sum_e f_e * P_e,   f_e = c_e / (T k),
 *     P_e    = (1/T) sum_t p_te,             p_t = softmax over all E of l_t,
 * with c_e the number of routed assignments (t, j) with idx[t,j] = e.  dout
 * is the gradient arriving at the layer's output.  The routing idx is an
 * input (the selection is piecewise constant); the selected weights are
 * w_tj = softmax over the k selected logits (the normalised probabilities of
 * the forward pass), given as topk_w.  Everything is binary64, including the
 * router logits l_te = x_t . W_r[e] + b_e used for p (the selection being
 * given, no bit-exact order is needed here).
 *
 * Per (token t, slot j) with expert e and weight w (chain rule through the
 * gated MLP, silu(a) = a sigma(a), silu'(a) = sigma(a) (1 + a (1 - sigma(a)))):
 *     a = W_g,e x_t,  u = W_u,e x_t,  h = silu(a) u,
 *     G   = W_dn,e^T dout_t                 (F values)
 *     dw  = G . h                           (dLambda / dw_tj)
 *     dh  = w G
 *     da  = dh u silu'(a),   du = dh silu(a)
 *     dx_t     += W_g,e^T da + W_u,e^T du
 *     dW_g,e   += da x_t^T,  dW_u,e += du x_t^T,  dW_dn,e += (w dout_t) h^T
 * The shared expert is the same with w = s_t = sigma(z_t), z_t = g . x_t, and
 * ds_t = G_sh . h_sh gives dz_t = ds_t s_t (1 - s_t), dg += dz_t x_t,
 * dx_t += dz_t g.
 * Router, per token (w = softmax of the selected logits, so its Jacobian is
 * diag(w) - w w^T on the selected entries and zero elsewhere):
 *     dl_te  = [e selected as slot j] w_j (dw_j - sum_j' w_j' dw_j')
 *            + coef (E/T) p_te (f_e - sum_e' f_e' p_te')
 *     dW_r[e] += dl_te x_t,   dx_t += sum_e dl_te W_r[e]
 *
 * parts selects what is computed (the rest of the outputs is left as is):
 *     1 dx of the tokens in tok_sel (all tokens when tok_sel is NULL)
 *     2 dW_gu, dW_dn of the experts e with exp_slot[e] >= 0, written to
 *       slot exp_slot[e] of dw_gu / dw_dn (exp_slot NULL: every expert, slot e)
 *     4 dW_sgu, dW_sdn and dsh_gate (shared expert and its gate)
 *     8 dW_router
 * aux_loss (nullable) receives L_aux.  Returns 0, 1 on bad arguments, 2 when
 * out of memory.
 * ------------------------------------------------------------------------- */

/* Per-pair backward quantities (see above); returns dw = G . h. */
static double pair_backward(const void *x, int64_t xoff, int dtype,
                            const wsrc *w_gu, int64_t gu_row, const wsrc *w_dn,
                            int64_t dn_row, int d, int F, const double *dout_t,
                            double w, double *h, double *da, double *du)
{
    double dw = 0.0;
    for (int n = 0; n < F; n++) {
        double a = 0.0, u = 0.0, g = 0.0;
        for (int kk = 0; kk < d; kk++) {
            double xv = (double)load_elem(x, dtype, xoff + kk);
            a += load_w(w_gu, gu_row + n, kk) * xv;
            u += load_w(w_gu, gu_row + F + n, kk) * xv;
        }
        for (int m = 0; m < d; m++)
            g += load_w(w_dn, dn_row + m, n) * dout_t[m];
        double sg = 1.0 / (1.0 + exp(-a));
        double silu = a * sg;
        double dsilu = sg * (1.0 + a * (1.0 - sg));
        h[n] = silu * u;
        dw += g * h[n];
        double dh = w * g;
        da[n] = dh * u * dsilu;
        du[n] = dh * silu;
    }
    return dw;
}

int oracle_backward(int64_t T, int d, int E, int k, int F, int Fs, int dtype,
                    const void *x, const void *w_router, const float *bias,
                    const void *w_gate_up, const void *w_down,
                    const void *w_sh_gate_up, const void *w_sh_down,
                    const void *sh_gate, const int32_t *topk_idx,
                    const double *topk_w, const double *dout, double coef,
                    int parts, const int32_t *tok_sel, int64_t n_tok_sel,
                    const int32_t *exp_slot, double *dx, double *dw_router,
                    double *dw_gu, double *dw_dn, double *dw_sgu,
                    double *dw_sdn, double *dsh_gate, double *aux_loss)
{
    if (T < 1 || d < 1 || E < 1 || k < 1 || k > E || F < 1 || Fs < 0 || !x ||
        !w_router || !w_gate_up || !w_down || !topk_idx || !topk_w || !dout)
        return 1;
    if (Fs > 0 && (!w_sh_gate_up || !w_sh_down || !sh_gate))
        return 1;
    if (((parts & 1) && !dx) || ((parts & 2) && (!dw_gu || !dw_dn)) ||
        ((parts & 4) && Fs > 0 && (!dw_sgu || !dw_sdn || !dsh_gate)) ||
        ((parts & 8) && !dw_router))
        return 1;
    for (int64_t i = 0; i < T * k; i++)
        if (topk_idx[i] < 0 || topk_idx[i] >= E)
            return 1;
    if (tok_sel)
        for (int64_t i = 0; i < n_tok_sel; i++)
            if (tok_sel[i] < 0 || tok_sel[i] >= T)
                return 1;
    const int64_t P = T * k;
    wsrc gu = {dtype, w_gate_up, NULL, d}, dn = {dtype, w_down, NULL, F};
    wsrc sgu = {dtype, w_sh_gate_up, NULL, d}, sdn = {dtype, w_sh_down, NULL, Fs};

    /* which tokens and pairs need their per-pair quantities */
    uint8_t *tok_need = (uint8_t *)calloc((size_t)T, 1);
    uint8_t *pair_need = (uint8_t *)calloc((size_t)P, 1);
    double *f = (double *)calloc((size_t)E, sizeof(double));
    double *h = (double *)malloc(sizeof(double) * (size_t)(P * F));
    double *da = (double *)malloc(sizeof(double) * (size_t)(P * F));
    double *du = (double *)malloc(sizeof(double) * (size_t)(P * F));
    double *dwp = (double *)calloc((size_t)P, sizeof(double));
    int sh = Fs > 0;
    double *hs = sh ? (double *)malloc(sizeof(double) * (size_t)(T * Fs)) : NULL;
    double *das = sh ? (double *)malloc(sizeof(double) * (size_t)(T * Fs)) : NULL;
    double *dus = sh ? (double *)malloc(sizeof(double) * (size_t)(T * Fs)) : NULL;
    double *sv = sh ? (double *)calloc((size_t)T, sizeof(double)) : NULL;
    double *dl = (double *)calloc((size_t)(T * (E + 1)), sizeof(double));
    double *pt = (double *)calloc((size_t)(T * E), sizeof(double));
    int fail = !tok_need || !pair_need || !f || !h || !da || !du || !dwp || !dl ||
               !pt || (sh && (!hs || !das || !dus || !sv));
    if (fail)
        goto done;

    if (parts & 8)
        memset(tok_need, 1, (size_t)T);
    if (parts & 1) {
        if (tok_sel)
            for (int64_t i = 0; i < n_tok_sel; i++)
                tok_need[tok_sel[i]] = 1;
        else
            memset(tok_need, 1, (size_t)T);
    }
    for (int64_t i = 0; i < P; i++) {
        int e = topk_idx[i];
        f[e] += 1.0; /* count first, divide once below */
        if (tok_need[i / k] || ((parts & 2) && (!exp_slot || exp_slot[e] >= 0)))
            pair_need[i] = 1;
    }
    for (int e = 0; e < E; e++)
        f[e] /= (double)P;

    /* phase 1: per-pair, per-token quantities */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < P; i++) {
        if (!pair_need[i])
            continue;
        int64_t t = i / k;
        int e = topk_idx[i];
        dwp[i] = pair_backward(x, t * d, dtype, &gu, (int64_t)e * 2 * F, &dn,
                               (int64_t)e * d, d, F, dout + t * d, topk_w[i],
                               h + i * F, da + i * F, du + i * F);
    }
    int shared_all = sh && (parts & 4);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; t++) {
        int need_sh = sh && (tok_need[t] || shared_all);
        double s = 0.0, dsv = 0.0;
        if (need_sh) {
            s = shared_gate(x, t * d, sh_gate, d, dtype);
            sv[t] = s;
            dsv = pair_backward(x, t * d, dtype, &sgu, 0, &sdn, 0, d, Fs, dout + t * d,
                                s, hs + t * Fs, das + t * Fs, dus + t * Fs);
            dl[t * (E + 1) + E] = dsv * s * (1.0 - s);
        }
        /* router: binary64 logits, softmax over all E */
        double *p = pt + t * E;
        double m = -INFINITY;
        for (int e = 0; e < E; e++) {
            double l = bias ? (double)bias[e] : 0.0;
            for (int kk = 0; kk < d; kk++)
                l += (double)load_elem(x, dtype, t * d + kk) *
                     (double)load_elem(w_router, dtype, (int64_t)e * d + kk);
            p[e] = l;
            if (l > m)
                m = l;
        }
        double z = 0.0;
        for (int e = 0; e < E; e++) {
            p[e] = exp(p[e] - m);
            z += p[e];
        }
        double fp = 0.0;
        for (int e = 0; e < E; e++) {
            p[e] /= z;
            fp += f[e] * p[e];
        }
        if (!tok_need[t])
            continue;
        double *dlt = dl + t * (E + 1);
        double c = coef * (double)E / (double)T;
        for (int e = 0; e < E; e++)
            dlt[e] = c * p[e] * (f[e] - fp);
        double wdw = 0.0;
        for (int j = 0; j < k; j++)
            wdw += topk_w[t * k + j] * dwp[t * k + j];
        for (int j = 0; j < k; j++)
            dlt[topk_idx[t * k + j]] += topk_w[t * k + j] * (dwp[t * k + j] - wdw);
    }

    /* phase 2: the outputs */
    if (parts & 1) {
        int64_t n = tok_sel ? n_tok_sel : T;
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t ii = 0; ii < n; ii++) {
            int64_t t = tok_sel ? tok_sel[ii] : ii;
            double *o = dx + t * d;
            const double *dlt = dl + t * (E + 1);
            for (int kk = 0; kk < d; kk++) {
                double acc = 0.0;
                for (int j = 0; j < k; j++) {
                    int64_t i = t * k + j;
                    int64_t row = (int64_t)topk_idx[i] * 2 * F;
                    for (int nn = 0; nn < F; nn++)
                        acc += load_w(&gu, row + nn, kk) * da[i * F + nn] +
                               load_w(&gu, row + F + nn, kk) * du[i * F + nn];
                }
                if (sh) {
                    for (int nn = 0; nn < Fs; nn++)
                        acc += load_w(&sgu, nn, kk) * das[t * Fs + nn] +
                               load_w(&sgu, Fs + nn, kk) * dus[t * Fs + nn];
                    acc += dlt[E] * (double)load_elem(sh_gate, dtype, kk);
                }
                for (int e = 0; e < E; e++)
                    acc += dlt[e] * (double)load_elem(w_router, dtype, (int64_t)e * d + kk);
                o[kk] = acc;
            }
        }
    }
    if (parts & 2) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int e = 0; e < E; e++) {
            if (exp_slot && exp_slot[e] < 0)
                continue;
            int64_t slot = exp_slot ? exp_slot[e] : e;
            double *g = dw_gu + slot * 2 * F * d;
            double *dd = dw_dn + slot * d * F;
            memset(g, 0, sizeof(double) * (size_t)(2 * F * d));
            memset(dd, 0, sizeof(double) * (size_t)(d * F));
            for (int64_t i = 0; i < P; i++) {
                if (topk_idx[i] != e)
                    continue;
                int64_t t = i / k;
                double w = topk_w[i];
                for (int nn = 0; nn < F; nn++)
                    for (int kk = 0; kk < d; kk++) {
                        double xv = (double)load_elem(x, dtype, t * d + kk);
                        g[(int64_t)nn * d + kk] += da[i * F + nn] * xv;
                        g[(int64_t)(F + nn) * d + kk] += du[i * F + nn] * xv;
                    }
                for (int mm = 0; mm < d; mm++)
                    for (int nn = 0; nn < F; nn++)
                        dd[(int64_t)mm * F + nn] += w * dout[t * d + mm] * h[i * F + nn];
            }
        }
    }
    if ((parts & 4) && sh) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int nn = 0; nn < Fs; nn++)
            for (int kk = 0; kk < d; kk++) {
                double ag = 0.0, au = 0.0;
                for (int64_t t = 0; t < T; t++) {
                    double xv = (double)load_elem(x, dtype, t * d + kk);
                    ag += das[t * Fs + nn] * xv;
                    au += dus[t * Fs + nn] * xv;
                }
                dw_sgu[(int64_t)nn * d + kk] = ag;
                dw_sgu[(int64_t)(Fs + nn) * d + kk] = au;
            }
#pragma omp parallel for schedule(dynamic, 1)
        for (int mm = 0; mm < d; mm++) {
            for (int nn = 0; nn < Fs; nn++) {
                double acc = 0.0;
                for (int64_t t = 0; t < T; t++)
                    acc += sv[t] * dout[t * d + mm] * hs[t * Fs + nn];
                dw_sdn[(int64_t)mm * Fs + nn] = acc;
            }
            double ag = 0.0;
            for (int64_t t = 0; t < T; t++)
                ag += dl[t * (E + 1) + E] * (double)load_elem(x, dtype, t * d + mm);
            dsh_gate[mm] = ag;
        }
    }
    if (parts & 8) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int e = 0; e < E; e++)
            for (int kk = 0; kk < d; kk++) {
                double acc = 0.0;
                for (int64_t t = 0; t < T; t++)
                    acc += dl[t * (E + 1) + e] * (double)load_elem(x, dtype, t * d + kk);
                dw_router[(int64_t)e * d + kk] = acc;
            }
    }
    if (aux_loss) {
        double acc = 0.0;
        for (int e = 0; e < E; e++) {
            double Pe = 0.0;
            for (int64_t t = 0; t < T; t++)
                Pe += pt[t * E + e];
            acc += f[e] * (Pe / (double)T);
        }
        *aux_loss = coef * (double)E * acc;
    }
done:
    free(tok_need);
    free(pair_need);
    free(f);
    free(h);
    free(da);
    free(du);
    free(dwp);
    free(hs);
    free(das);
    free(dus);
    free(sv);
    free(dl);
    free(pt);
    return fail ? 2 : 0;
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
