/*
 * CPU oracle for the sparse mixture-of-experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library and includes none of its
 * files; it defines its own types.  Plain C99 loops, OpenMP over independent
 * tokens/experts only, double-precision arithmetic unless a step says
 * otherwise.
 *
 * What it computes (the pages describe the layer, not its arithmetic):
 *  - "single RTX 5090 runs a 125B model", section "MoE experts scheduled on
 *    demand": a light gating network (router) picks the top-K experts for
 *    each token and the remaining experts do not compute.
 *  - "How Strata works", section "three storage tiers": router and a shared
 *    expert are resident; the model has 24,576 experts, 10 used per token.
 *  - The layer's output is the top-k-weighted sum of SwiGLU expert outputs
 *    plus the ungated shared expert; experts are block-32 quantised
 *    (int4/int8 with one fp16 scale per 32 weights along each row).
 *
 * Readings taken where the pages are silent (each is applied below):
 *  - router logits z[t,e] = sum_i x[t,i] * Wr[e,i] (+ bias[e]), summed in
 *    double with i ascending; every product is exact in double.
 *  - selection is on logits: experts ordered by (z descending, e ascending),
 *    the first k kept in that order (ties go to the lower expert index).
 *  - gates are the softmax over the k selected logits (equal to the full
 *    softmax renormalised over the top k), computed in double, stored fp32.
 *  - expert FFN: y = Wd (silu(Wg x) * (Wu x)), silu(z) = z / (1 + exp(-z)),
 *    no biases, no norms.
 *  - int8 activation mode ("Q8"): per 32 consecutive features, s = amax/127
 *    (fp32 IEEE division), q = clamp(rint(x / s), -127, 127) with
 *    round-to-nearest-even, s = 0 and q = 0 for an all-zero block; applied to
 *    the hidden state x and to the SwiGLU intermediate h (h rounded to fp32
 *    first); block sums of int8 products are exact integers.
 *  - combine: out[t] = residual[t] + shared(x_t) + sum_j g[t,j] * y_{t,j},
 *    in double, j ascending, stored fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENOMEM 2

#define ORC_WFMT_I4B32 4
#define ORC_WFMT_I8B32 8
#define ORC_ACT_FLOAT 0
#define ORC_ACT_Q8 1

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* IEEE 754 binary16 -> double, from the format's definition. */
double orc_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);    /* (1024 + m) * 2^(e-25) */
    return sign ? -v : v;
}

/* ---- canonical expert blob ---------------------------------------------- */

typedef struct {
    size_t qg, qu, qd, sg, su, sd, total;
} orc_layout;

static int fmt_ok(int wfmt) { return wfmt == ORC_WFMT_I4B32 || wfmt == ORC_WFMT_I8B32; }

static orc_layout layout_of(int wfmt, int d, int f) {
    orc_layout L;
    size_t n = (size_t)d * (size_t)f;
    size_t qb = (wfmt == ORC_WFMT_I4B32) ? n / 2 : n;
    size_t sb = (n / 32) * 2;
    L.qg = 0;
    L.qu = qb;
    L.qd = 2 * qb;
    L.sg = 3 * qb;
    L.su = L.sg + sb;
    L.sd = L.su + sb;
    L.total = L.sd + sb;
    return L;
}

size_t orc_expert_bytes(int wfmt, int d, int f) {
    if (!fmt_ok(wfmt) || d <= 0 || f <= 0) return 0;
    return layout_of(wfmt, d, f).total;
}

/* Signed quant value of element idx of a row-major quant array. */
static int quant_at(const uint8_t* q, size_t idx, int wfmt) {
    if (wfmt == ORC_WFMT_I8B32) return (int)(int8_t)q[idx];
    uint8_t byte = q[idx >> 1];
    int u = (idx & 1) ? (byte >> 4) : (byte & 15); /* offset-binary nibble */
    return u - 8;
}

static uint16_t scale_bits_at(const uint8_t* s, size_t idx) {
    return (uint16_t)(s[2 * idx] | (s[2 * idx + 1] << 8));
}

/* w[r][c] = half(scale[r][c/32]) * q[r][c] for an R x K block-32 matrix. */
int orc_dequant_matrix(const uint8_t* q, const uint8_t* s, int R, int K, int wfmt, double* out) {
    if (!q || !s || !out || R <= 0 || K <= 0 || K % 32 || !fmt_ok(wfmt)) return ORC_EINVAL;
    int nb = K / 32;
    for (int r = 0; r < R; ++r)
        for (int c = 0; c < K; ++c) {
            double sc = orc_half_to_double(scale_bits_at(s, (size_t)r * nb + c / 32));
            out[(size_t)r * K + c] = sc * (double)quant_at(q, (size_t)r * K + c, wfmt);
        }
    return ORC_OK;
}

/* Dequantise the three matrices of one expert: Wg, Wu [f x d], Wd [d x f]. */
int orc_dequant_expert(const uint8_t* blob, int wfmt, int d, int f, double* wg, double* wu, double* wd) {
    if (!blob || !fmt_ok(wfmt) || d % 32 || f % 32) return ORC_EINVAL;
    orc_layout L = layout_of(wfmt, d, f);
    int rc = orc_dequant_matrix(blob + L.qg, blob + L.sg, f, d, wfmt, wg);
    if (!rc) rc = orc_dequant_matrix(blob + L.qu, blob + L.su, f, d, wfmt, wu);
    if (!rc) rc = orc_dequant_matrix(blob + L.qd, blob + L.sd, d, f, wfmt, wd);
    return rc;
}

/* ---- router ------------------------------------------------------------- */

/* One token: logits, top-k selection (z desc, e asc), renormalised softmax. */
static void route_token(const float* x, int d, const float* Wr, const float* bias, int E, int k,
                        double* z, unsigned char* taken, int32_t* ids, float* gates, double* p) {
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += (double)x[i] * (double)Wr[(size_t)e * d + i];
        if (bias) acc += (double)bias[e];
        z[e] = acc;
        taken[e] = 0;
    }
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || z[e] > z[best]) best = e; /* strict: equal logit keeps lower index */
        }
        taken[best] = 1;
        ids[j] = best;
    }
    double m = z[ids[0]], sum = 0.0;
    for (int j = 0; j < k; ++j) {
        p[j] = exp(z[ids[j]] - m);
        sum += p[j];
    }
    for (int j = 0; j < k; ++j) gates[j] = (float)(p[j] / sum);
}

int orc_route(const float* x, int T, int d, const float* Wr, const float* bias, int E, int k,
              int32_t* ids, float* gates, double* logits /* [T,E] or NULL */) {
    if (T < 0 || d <= 0 || E <= 0 || k < 1 || k > E) return ORC_EINVAL;
    if (T == 0) return ORC_OK;
    if (!x || !Wr || !ids || !gates) return ORC_EINVAL;
    int fail = 0;
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)E);
        double* p = (double*)malloc(sizeof(double) * (size_t)k);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
        int ok = z && p && taken;
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
        /* every thread reaches the work-sharing loop; one without scratch skips its share */
#pragma omp for schedule(dynamic, 4)
        for (int t = 0; t < T; ++t) {
            if (!ok) continue;
            route_token(x + (size_t)t * d, d, Wr, bias, E, k, z, taken, ids + (size_t)t * k,
                        gates + (size_t)t * k, p);
            if (logits) memcpy(logits + (size_t)t * E, z, sizeof(double) * (size_t)E);
        }
        free(z);
        free(p);
        free(taken);
    }
    return fail ? ORC_ENOMEM : ORC_OK;
}

/* ---- permutation -------------------------------------------------------- */

/* Stable counting sort of the T*k routing slots by expert id.
 * counts[e], offsets[e] = sum_{e'<e} counts[e'] (offsets[E] = T*k),
 * sorted_idx lists flat slots f = t*k + j in (ids[f], f) order,
 * dest[f] is the position of slot f in sorted_idx. */
int orc_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                int32_t* sorted_idx, int32_t* dest) {
    if (T < 0 || k < 1 || E <= 0 || !counts || !offsets) return ORC_EINVAL;
    long n = (long)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (long f = 0; f < n; ++f) {
        if (ids[f] < 0 || ids[f] >= E) return ORC_EINVAL;
        counts[ids[f]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) return ORC_ENOMEM;
    memcpy(cursor, offsets, sizeof(int32_t) * (size_t)E);
    for (long f = 0; f < n; ++f) {
        int32_t p = cursor[ids[f]]++;
        sorted_idx[p] = (int32_t)f;
        dest[f] = p;
    }
    free(cursor);
    return ORC_OK;
}

/* ---- pre-norm of a layer's input (layer stack) ---------------------------- */

/* out[t,i] = x[t,i] / sqrt(mean_i(x[t,i]^2) + eps), in double, stored fp32.
 * The pages do not describe the block around the MoE layer; a stack of layers
 * with a residual add needs the usual pre-norm to stay finite (reading taken:
 * RMSNorm without a learned gain). */
int orc_rmsnorm(const float* x, int T, int d, double eps, float* out) {
    if (T < 0 || d <= 0 || (T && (!x || !out))) return ORC_EINVAL;
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int i = 0; i < d; ++i) ss += (double)x[(size_t)t * d + i] * (double)x[(size_t)t * d + i];
        double r = 1.0 / sqrt(ss / (double)d + eps);
        for (int i = 0; i < d; ++i) out[(size_t)t * d + i] = (float)((double)x[(size_t)t * d + i] * r);
    }
    return ORC_OK;
}

/* ---- int8 activation quantisation -------------------------------------- */

static void quant8_row(const float* x, int K, int8_t* q, float* s) {
    for (int b = 0; b < K / 32; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(x[b * 32 + i]);
            if (a > amax) amax = a;
        }
        float sc = amax / 127.0f;
        s[b] = sc;
        for (int i = 0; i < 32; ++i) {
            int v = 0;
            if (sc != 0.0f) {
                float r = rintf(x[b * 32 + i] / sc);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                v = (int)r;
            }
            q[b * 32 + i] = (int8_t)v;
        }
    }
}

int orc_quant8(const float* x, int rows, int K, int8_t* q, float* s) {
    if (rows < 0 || K <= 0 || K % 32 || (rows && (!x || !q || !s))) return ORC_EINVAL;
    for (int r = 0; r < rows; ++r) quant8_row(x + (size_t)r * K, K, q + (size_t)r * K, s + (size_t)r * (K / 32));
    return ORC_OK;
}

/* ---- expert FFN --------------------------------------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Per-expert state: fp64 weights (float mode) or raw quants + scales (Q8 mode). */
typedef struct {
    int d, f, wfmt, act_mode;
    double *wg, *wu, *wd;          /* float mode */
    int8_t *qg, *qu, *qd;          /* q8 mode: signed quants, row-major */
    double *sg, *su, *sd;          /* q8 mode: block scales as doubles */
} orc_expert;

static void expert_free(orc_expert* X) {
    free(X->wg); free(X->wu); free(X->wd);
    free(X->qg); free(X->qu); free(X->qd);
    free(X->sg); free(X->su); free(X->sd);
    memset(X, 0, sizeof(*X));
}

static int unpack_quants(const uint8_t* q, const uint8_t* s, int R, int K, int wfmt, int8_t** qo, double** so) {
    size_t n = (size_t)R * K, nb = n / 32;
    *qo = (int8_t*)malloc(n);
    *so = (double*)malloc(sizeof(double) * nb);
    if (!*qo || !*so) return ORC_ENOMEM;
    for (size_t i = 0; i < n; ++i) (*qo)[i] = (int8_t)quant_at(q, i, wfmt);
    for (size_t i = 0; i < nb; ++i) (*so)[i] = orc_half_to_double(scale_bits_at(s, i));
    return ORC_OK;
}

static int expert_load(orc_expert* X, const uint8_t* blob, int wfmt, int d, int f, int act_mode) {
    memset(X, 0, sizeof(*X));
    X->d = d; X->f = f; X->wfmt = wfmt; X->act_mode = act_mode;
    if (act_mode == ORC_ACT_FLOAT) {
        size_t n = (size_t)d * f;
        X->wg = (double*)malloc(sizeof(double) * n);
        X->wu = (double*)malloc(sizeof(double) * n);
        X->wd = (double*)malloc(sizeof(double) * n);
        if (!X->wg || !X->wu || !X->wd) return ORC_ENOMEM;
        return orc_dequant_expert(blob, wfmt, d, f, X->wg, X->wu, X->wd);
    }
    orc_layout L = layout_of(wfmt, d, f);
    int rc = unpack_quants(blob + L.qg, blob + L.sg, f, d, wfmt, &X->qg, &X->sg);
    if (!rc) rc = unpack_quants(blob + L.qu, blob + L.su, f, d, wfmt, &X->qu, &X->su);
    if (!rc) rc = unpack_quants(blob + L.qd, blob + L.sd, d, f, wfmt, &X->qd, &X->sd);
    return rc;
}

/* sum_b s_act[b] * s_w[n,b] * (exact integer sum over block b of qa * qw[n,.]) */
static double q8_dot(const int8_t* qa, const float* sa, const int8_t* qw, const double* sw, int K) {
    double acc = 0.0;
    for (int b = 0; b < K / 32; ++b) {
        int32_t blk = 0;
        for (int i = 0; i < 32; ++i) blk += (int32_t)qa[b * 32 + i] * (int32_t)qw[b * 32 + i];
        acc += (double)sa[b] * sw[b] * (double)blk;
    }
    return acc;
}

/* One token through one expert; scratch must hold 3*f + 2*d doubles-worth. */
static void expert_apply(const orc_expert* X, const float* x, double* y, double* g_out, double* u_out,
                         double* g, double* u, float* hf, int8_t* xq, float* xs, int8_t* hq, float* hs) {
    int d = X->d, f = X->f;
    if (X->act_mode == ORC_ACT_FLOAT) {
        for (int n = 0; n < f; ++n) {
            double ag = 0.0, au = 0.0;
            for (int i = 0; i < d; ++i) {
                ag += X->wg[(size_t)n * d + i] * (double)x[i];
                au += X->wu[(size_t)n * d + i] * (double)x[i];
            }
            g[n] = ag;
            u[n] = au;
        }
        double* h = (double*)hf; /* float mode keeps h in double; hf holds f doubles */
        for (int n = 0; n < f; ++n) h[n] = silu(g[n]) * u[n];
        for (int o = 0; o < d; ++o) {
            double acc = 0.0;
            for (int n = 0; n < f; ++n) acc += X->wd[(size_t)o * f + n] * h[n];
            y[o] = acc;
        }
    } else {
        quant8_row(x, d, xq, xs);
        for (int n = 0; n < f; ++n) {
            g[n] = q8_dot(xq, xs, X->qg + (size_t)n * d, X->sg + (size_t)n * (d / 32), d);
            u[n] = q8_dot(xq, xs, X->qu + (size_t)n * d, X->su + (size_t)n * (d / 32), d);
        }
        for (int n = 0; n < f; ++n) hf[n] = (float)(silu(g[n]) * u[n]);
        quant8_row(hf, f, hq, hs);
        for (int o = 0; o < d; ++o)
            y[o] = q8_dot(hq, hs, X->qd + (size_t)o * f, X->sd + (size_t)o * (f / 32), f);
    }
    if (g_out) memcpy(g_out, g, sizeof(double) * (size_t)f);
    if (u_out) memcpy(u_out, u, sizeof(double) * (size_t)f);
}

typedef struct {
    double *g, *u;
    float* hf;       /* f doubles in float mode, f floats in q8 mode */
    int8_t *xq, *hq;
    float *xs, *hs;
} orc_scratch;

static int scratch_alloc(orc_scratch* S, int d, int f) {
    S->g = (double*)malloc(sizeof(double) * (size_t)f);
    S->u = (double*)malloc(sizeof(double) * (size_t)f);
    S->hf = (float*)malloc(sizeof(double) * (size_t)f);
    S->xq = (int8_t*)malloc((size_t)d);
    S->hq = (int8_t*)malloc((size_t)f);
    S->xs = (float*)malloc(sizeof(float) * (size_t)(d / 32));
    S->hs = (float*)malloc(sizeof(float) * (size_t)(f / 32));
    return (S->g && S->u && S->hf && S->xq && S->hq && S->xs && S->hs) ? ORC_OK : ORC_ENOMEM;
}

static void scratch_free(orc_scratch* S) {
    free(S->g); free(S->u); free(S->hf); free(S->xq); free(S->hq); free(S->xs); free(S->hs);
}

/* One expert applied to M rows X[M,d] -> Y[M,d] (double).  G/U (optional,
 * [M,f]) receive the gate and up projections before the activation. */
int orc_expert_ffn(const float* X, int M, int d, int f, const uint8_t* blob, int wfmt, int act_mode,
                   double* Y, double* G, double* U) {
    if (M < 0 || d <= 0 || f <= 0 || d % 32 || f % 32 || !fmt_ok(wfmt) || !blob ||
        (act_mode != ORC_ACT_FLOAT && act_mode != ORC_ACT_Q8))
        return ORC_EINVAL;
    if (M == 0) return ORC_OK;
    orc_expert W;
    int rc = expert_load(&W, blob, wfmt, d, f, act_mode);
    if (rc) { expert_free(&W); return rc; }
    int fail = 0;
#pragma omp parallel
    {
        orc_scratch S;
        int ok = scratch_alloc(&S, d, f) == ORC_OK;
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int m = 0; m < M; ++m) {
            if (!ok) continue;
            expert_apply(&W, X + (size_t)m * d, Y + (size_t)m * d, G ? G + (size_t)m * f : NULL,
                         U ? U + (size_t)m * f : NULL, S.g, S.u, S.hf, S.xq, S.xs, S.hq, S.hs);
        }
        scratch_free(&S);
    }
    expert_free(&W);
    return fail ? ORC_ENOMEM : ORC_OK;
}

/* ---- whole layer -------------------------------------------------------- */

/* route -> permute -> routed experts -> shared expert -> combine.
 * Routing outputs cover all T tokens.  FFN outputs are produced for the
 * tokens listed in tok (n_tok of them, out is [n_tok, d]); tok == NULL means
 * all tokens in order.  residual (optional) is [T, d]. */
int orc_moe_layer(const float* x, int T, int d, int f, int E, int k, const float* Wr, const float* bias,
                  const uint8_t* const* experts, const uint8_t* shared, int wfmt, int act_mode,
                  const float* residual, const int32_t* tok, int n_tok,
                  int32_t* ids, float* gates, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                  int32_t* dest, float* out) {
    if (T < 0 || d <= 0 || f <= 0 || d % 32 || f % 32 || E <= 0 || k < 1 || k > E || !fmt_ok(wfmt) ||
        (act_mode != ORC_ACT_FLOAT && act_mode != ORC_ACT_Q8) || !experts)
        return ORC_EINVAL;
    if (!tok) n_tok = T;
    if (n_tok < 0) return ORC_EINVAL;
    for (int i = 0; tok && i < n_tok; ++i)
        if (tok[i] < 0 || tok[i] >= T) return ORC_EINVAL;
    int rc = orc_route(x, T, d, Wr, bias, E, k, ids, gates, NULL);
    if (rc) return rc;
    rc = orc_permute(ids, T, k, E, counts, offsets, sorted_idx, dest);
    if (rc || T == 0 || n_tok == 0) return rc;

    /* position of each token in the output list (-1: not requested) */
    int32_t* where = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
    double* ysel = (double*)calloc((size_t)n_tok * k * d, sizeof(double));
    double* ysh = shared ? (double*)calloc((size_t)n_tok * d, sizeof(double)) : NULL;
    if (!where || !ysel || (shared && !ysh)) { free(where); free(ysel); free(ysh); return ORC_ENOMEM; }
    for (int t = 0; t < T; ++t) where[t] = tok ? -1 : t;
    for (int i = 0; tok && i < n_tok; ++i) where[tok[i]] = i;

    int fail = 0;
#pragma omp parallel
    {
        orc_scratch S;
        int ok = scratch_alloc(&S, d, f) == ORC_OK;
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int e = 0; e < E; ++e) {
            if (!ok || counts[e] == 0) continue;
            int any = 0;
            for (int p = offsets[e]; p < offsets[e + 1]; ++p) any |= where[sorted_idx[p] / k] >= 0;
            if (!any) continue;
            orc_expert W;
            if (expert_load(&W, experts[e], wfmt, d, f, act_mode)) {
#pragma omp atomic write
                fail = 1;
                expert_free(&W);
                continue;
            }
            for (int p = offsets[e]; p < offsets[e + 1]; ++p) {
                int slot = sorted_idx[p], t = slot / k, j = slot % k, w = where[t];
                if (w < 0) continue;
                expert_apply(&W, x + (size_t)t * d, ysel + ((size_t)w * k + j) * d, NULL, NULL, S.g, S.u, S.hf,
                             S.xq, S.xs, S.hq, S.hs);
            }
            expert_free(&W);
        }
        scratch_free(&S);
    }
    if (!fail && shared) {
        orc_expert W;
        if (expert_load(&W, shared, wfmt, d, f, act_mode)) {
            fail = 1;
        } else {
#pragma omp parallel
            {
                orc_scratch S;
                int ok = scratch_alloc(&S, d, f) == ORC_OK;
                if (!ok) {
#pragma omp atomic write
                    fail = 1;
                }
#pragma omp for schedule(dynamic, 1)
                for (int i = 0; i < n_tok; ++i) {
                    if (!ok) continue;
                    int t = tok ? tok[i] : i;
                    expert_apply(&W, x + (size_t)t * d, ysh + (size_t)i * d, NULL, NULL, S.g, S.u, S.hf,
                                 S.xq, S.xs, S.hq, S.hs);
                }
                scratch_free(&S);
            }
        }
        expert_free(&W);
    }
    if (!fail) {
        for (int i = 0; i < n_tok; ++i) {
            int t = tok ? tok[i] : i;
            for (int o = 0; o < d; ++o) {
                double acc = residual ? (double)residual[(size_t)t * d + o] : 0.0;
                if (ysh) acc += ysh[(size_t)i * d + o];
                for (int j = 0; j < k; ++j)
                    acc += (double)gates[(size_t)t * k + j] * ysel[((size_t)i * k + j) * d + o];
                out[(size_t)i * d + o] = (float)acc;
            }
        }
    }
    free(where);
    free(ysel);
    free(ysh);
    return fail ? ORC_ENOMEM : ORC_OK;
}
