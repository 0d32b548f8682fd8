/*
 * moe_ffn_oracle.c -- plain CPU reference for one decode-step MoE
 * feed-forward layer with a gated shared expert.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library: it has its own decoders and
 * its own argument structs.
 *
 * Every stored value is decoded exactly (bf16, fp16, 4-bit blocks) and all
 * arithmetic is IEEE double precision, evaluated in the order of the
 * definition below, one token at a time, with no blocking or fusion.
 *
 * Layer structure (page "ggml-cuda: overlap the MoE shared expert on a
 * separate stream", section "What this changes" and its commit messages):
 * routed experts and one gated shared expert run on the same input and their
 * outputs meet in a final add, the node pair ffn_moe_out / ffn_shexp.  The
 * expert FFN is SwiGLU with separate gate and up matrices (page "ggml operator
 * extensions", section "sd.cpp integration": the SwiGLU fusion takes separate
 * gate/up inputs).  The pages print no formula for routing or for the shared
 * gate; the plain reading taken here is the usual one for this layer type:
 *
 *   for each token x0 (the layer's input):
 *     0. input norm  (optional) x[h] = (x0[h] * rho) * wn[h],
 *                    rho = 1 / sqrt(sum_h x0[h]^2 / H + eps); else x = x0.
 *                    The FFN-input RMSNorm is the fork point of both branches
 *                    (same page, commit messages), RMSNorm followed by a
 *                    multiply with a one-dimensional weight (page "ggml operator
 *                    extensions", section "sd.cpp integration").
 *     1. logits      l[e] = sum_h x[h] * Wr[e][h]                  e < E
 *     2. selection   experts ranked by (l descending, index ascending);
 *                    ids = the first k, in rank order (exact ties -> lower index)
 *     3. softmax     p[e] = exp(l[e] - m) / sum_e' exp(l[e'] - m), m = max_e l[e]
 *     4. renormalise w[j] = p[ids[j]] / sum_j' p[ids[j']]
 *     5. experts     y[j] = Wd[e] . a,  a[i] = silu(g[i]) * u[i],
 *                    g = Wg[e] . x, u = Wu[e] . x, silu(z) = z / (1 + exp(-z))
 *     6. routed      r = sum_j w[j] * y[j]   (j in rank order)
 *     7. shared      S = Ws_d . (silu(Ws_g . x) * (Ws_u . x)),
 *                    s = 1 / (1 + exp(-(wg . x)))
 *     8. output      out = r + s * S
 *     9. residual    (optional) out = x0 + (r + s * S), the block's residual add
 *                    after the join (same page and section: gate multiply, then
 *                    residual add)
 *
 * 4-bit block storage (the pages do not give one): a block is 32 consecutive
 * elements along a row's reduction dimension; element c of a row sits in byte
 * c/2 of the row's packed bytes, low nibble for even c and high nibble for odd
 * c, stored as u = q + 8; its value is fp16(scale[row][c/32]) * (u - 8).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_Q4 = 2 };

typedef struct {
    int kind;               /* ORC_F32 | ORC_BF16 | ORC_Q4                     */
    const void *data;       /* f32 / bf16 bits [rows][cols], or q4 [rows][cols/2] */
    const uint16_t *scale;  /* ORC_Q4: fp16 bits [rows][cols/32], else unused   */
    long rows, cols;
} orc_matrix;

typedef struct {
    int hidden, n_experts, top_k, inter, shared_inter;
    int x_kind;                 /* ORC_F32 | ORC_BF16: tokens [T][hidden]        */
    const void *x;
    const float *router;        /* [E][H]                                        */
    orc_matrix gate, up;        /* rows = E*I (expert e owns rows e*I .. e*I+I-1), cols = H */
    orc_matrix down;            /* rows = E*H, cols = I                          */
    orc_matrix sh_gate, sh_up;  /* rows = I_s, cols = H                          */
    orc_matrix sh_down;         /* rows = H, cols = I_s                          */
    const float *gate_vec;      /* [H]                                           */
    const float *norm_w;        /* [H] RMSNorm weight, or NULL: no input norm     */
    double norm_eps;            /* RMSNorm epsilon (with norm_w)                  */
    int residual;               /* 1: out = x0 + layer output                     */
} orc_layer;

/* ---- exact decoders ---------------------------------------------------- */

double orc_bf16_value(uint16_t bits)
{
    /* bf16 is the upper half of an IEEE binary32 */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double orc_f16_value(uint16_t bits)
{
    /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits */
    int sign = bits >> 15;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);  /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -v : v;
}

double orc_matrix_elem(const orc_matrix *m, long row, long col)
{
    switch (m->kind) {
    case ORC_F32:
        return (double)((const float *)m->data)[row * m->cols + col];
    case ORC_BF16:
        return orc_bf16_value(((const uint16_t *)m->data)[row * m->cols + col]);
    case ORC_Q4: {
        uint8_t byte = ((const uint8_t *)m->data)[row * (m->cols / 2) + col / 2];
        int u = (col % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
        double scale = orc_f16_value(m->scale[row * (m->cols / 32) + col / 32]);
        return scale * (double)(u - 8);
    }
    }
    return NAN;
}

static double token_elem(const orc_layer *L, long t, long h)
{
    if (L->x_kind == ORC_F32)
        return (double)((const float *)L->x)[t * L->hidden + h];
    return orc_bf16_value(((const uint16_t *)L->x)[t * L->hidden + h]);
}

/* ---- plain linear algebra ---------------------------------------------- */

/* y[r] = sum_c M[row0 + r][c] * v[c], r < n_rows */
static void matvec(const orc_matrix *m, long row0, long n_rows, const double *v, double *y,
                   int nthreads)
{
    long r;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (r = 0; r < n_rows; ++r) {
        double acc = 0.0;
        for (long c = 0; c < m->cols; ++c)
            acc += orc_matrix_elem(m, row0 + r, c) * v[c];
        y[r] = acc;
    }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* SwiGLU FFN: y = D . (silu(G . x) * (U . x)); G, U own rows g0 .. g0+n_inter-1,
 * D owns rows d0 .. d0+n_out-1 */
static void swiglu_ffn(const orc_matrix *G, const orc_matrix *U, const orc_matrix *D, long g0,
                       long d0, long n_inter, long n_out, const double *x, double *y, int nthreads)
{
    double *g = malloc(sizeof(double) * n_inter);
    double *u = malloc(sizeof(double) * n_inter);
    double *a = malloc(sizeof(double) * n_inter);
    matvec(G, g0, n_inter, x, g, nthreads);
    matvec(U, g0, n_inter, x, u, nthreads);
    for (long i = 0; i < n_inter; ++i)
        a[i] = silu(g[i]) * u[i];
    matvec(D, d0, n_out, a, y, nthreads);
    free(g);
    free(u);
    free(a);
}

/* ---- the layer ---------------------------------------------------------- */

/*
 * Runs the layer on tokens 0 .. n_tokens-1.  Outputs (each may be NULL except
 * out): out/routed/shared [T][H], ids [T][k] (rank order), weights [T][k],
 * logits [T][E], gate_s [T].  If forced_ids is not NULL it replaces step 2:
 * token t uses experts forced_ids[t*k .. t*k+k-1] (still renormalised over
 * them by steps 3-4).  Returns 0, or -1 on a bad argument.
 */
int orc_forward(const orc_layer *L, long n_tokens, int nthreads, const int32_t *forced_ids,
                double *out, double *routed, double *shared, int32_t *ids, double *weights,
                double *logits, double *gate_s)
{
    const long H = L->hidden, E = L->n_experts, K = L->top_k, I = L->inter;
    const long Is = L->shared_inter;
    if (H <= 0 || E <= 0 || K <= 0 || K > E || I <= 0 || Is <= 0 || n_tokens < 0 || !out)
        return -1;
    if (L->norm_w && !(L->norm_eps >= 0.0))
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (forced_ids)
        for (long i = 0; i < n_tokens * K; ++i)
            if (forced_ids[i] < 0 || forced_ids[i] >= E)
                return -1;

    double *x0 = malloc(sizeof(double) * H);
    double *x = malloc(sizeof(double) * H);
    double *l = malloc(sizeof(double) * E);
    double *p = malloc(sizeof(double) * E);
    int *taken = malloc(sizeof(int) * E);
    long *sel = malloc(sizeof(long) * K);
    double *wsel = malloc(sizeof(double) * K);
    double *y = malloc(sizeof(double) * H);
    double *r = malloc(sizeof(double) * H);
    double *S = malloc(sizeof(double) * H);

    for (long t = 0; t < n_tokens; ++t) {
        for (long h = 0; h < H; ++h)
            x0[h] = token_elem(L, t, h);

        /* 0. optional RMSNorm of the input */
        if (L->norm_w) {
            double ss = 0.0;
            for (long h = 0; h < H; ++h)
                ss += x0[h] * x0[h];
            double rho = 1.0 / sqrt(ss / (double)H + L->norm_eps);
            for (long h = 0; h < H; ++h)
                x[h] = (x0[h] * rho) * (double)L->norm_w[h];
        } else {
            memcpy(x, x0, sizeof(double) * H);
        }

        /* 1. router logits */
        for (long e = 0; e < E; ++e) {
            double acc = 0.0;
            for (long h = 0; h < H; ++h)
                acc += x[h] * (double)L->router[e * H + h];
            l[e] = acc;
        }

        /* 2. top-k by (logit desc, index asc): k passes of a strict-greater scan */
        if (forced_ids) {
            for (long j = 0; j < K; ++j)
                sel[j] = forced_ids[t * K + j];
        } else {
            for (long e = 0; e < E; ++e)
                taken[e] = 0;
            for (long j = 0; j < K; ++j) {
                long best = -1;
                for (long e = 0; e < E; ++e)
                    if (!taken[e] && (best < 0 || l[e] > l[best]))
                        best = e;
                taken[best] = 1;
                sel[j] = best;
            }
        }

        /* 3. softmax over all E experts */
        double m = l[0];
        for (long e = 1; e < E; ++e)
            if (l[e] > m)
                m = l[e];
        double z = 0.0;
        for (long e = 0; e < E; ++e)
            z += exp(l[e] - m);
        for (long e = 0; e < E; ++e)
            p[e] = exp(l[e] - m) / z;

        /* 4. renormalise over the selected experts */
        double psum = 0.0;
        for (long j = 0; j < K; ++j)
            psum += p[sel[j]];
        for (long j = 0; j < K; ++j)
            wsel[j] = p[sel[j]] / psum;

        /* 5-6. routed experts, weighted sum in rank order */
        for (long h = 0; h < H; ++h)
            r[h] = 0.0;
        for (long j = 0; j < K; ++j) {
            long e = sel[j];
            swiglu_ffn(&L->gate, &L->up, &L->down, e * I, e * H, I, H, x, y, nthreads);
            for (long h = 0; h < H; ++h)
                r[h] += wsel[j] * y[h];
        }

        /* 7. shared expert and its scalar gate */
        swiglu_ffn(&L->sh_gate, &L->sh_up, &L->sh_down, 0, 0, Is, H, x, S, nthreads);
        double gl = 0.0;
        for (long h = 0; h < H; ++h)
            gl += (double)L->gate_vec[h] * x[h];
        double s = sigmoid(gl);

        /* 8. join, 9. optional residual */
        for (long h = 0; h < H; ++h) {
            const double joined = r[h] + s * S[h];
            out[t * H + h] = L->residual ? x0[h] + joined : joined;
        }

        if (routed)
            memcpy(routed + t * H, r, sizeof(double) * H);
        if (shared)
            memcpy(shared + t * H, S, sizeof(double) * H);
        if (ids)
            for (long j = 0; j < K; ++j)
                ids[t * K + j] = (int32_t)sel[j];
        if (weights)
            memcpy(weights + t * K, wsel, sizeof(double) * K);
        if (logits)
            memcpy(logits + t * E, l, sizeof(double) * E);
        if (gate_s)
            gate_s[t] = s;
    }

    free(x0);
    free(x);
    free(l);
    free(p);
    free(taken);
    free(sel);
    free(wsel);
    free(y);
    free(r);
    free(S);
    return 0;
}

/* Decodes rows [row0, row0+n_rows) of a matrix to doubles (for tests). */
void orc_matrix_decode(const orc_matrix *m, long row0, long n_rows, double *dst)
{
    for (long r = 0; r < n_rows; ++r)
        for (long c = 0; c < m->cols; ++c)
            dst[r * m->cols + c] = orc_matrix_elem(m, row0 + r, c);
}
