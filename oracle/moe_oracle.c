/*
 * moe_oracle.c -- plain CPU oracle of the single-token quantized MoE decode layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg.  It shares no code with the HIP library.
 *
 * It computes the plain definition of the layer in double precision from
 * exactly decoded inputs, one output at a time, with no blocking, fusion or
 * reordering.  OpenMP only distributes independent output rows over threads;
 * every dot product is one serial double-precision loop in element order.
 *
 * The layer, as the pages describe it:
 *  - mlxcel PR #276, "two-kernel decode-MoE that beats gather_qmm",
 *    section "What changed", step 2: kernel A computes the gate and up
 *    projections of each selected expert followed by SwiGLU into act[K, Dff];
 *    kernel B computes the down projection times the expert's score into
 *    partial[K, Din]; the K partials are then summed.
 *  - same page, "Scope / flags" and "Next": 4- and 8-bit affine weights, and
 *    6-bit / mixed-bit unpacking for a 6-bit down projection.
 *  - Red Lite dev39, "fused expert tail (GPU-routed decode)", section "Change":
 *    routed = sum over the selected experts, in the pool's order, of
 *    weight[e] * out_e[i]; then x = resid + (routed + shared * scalar).
 * Routing (router logits, softmax over all experts, top-k, optional
 * renormalisation of the selected probabilities) is the GPU-routed step the
 * Red Lite page names; its exact form is the plain reading of that step.
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *  - weight w[r, j] = scale[r, j/64] * q[r, j] + bias[r, j/64], groups of 64
 *    along the contraction index j; codes packed LSB-first in little-endian
 *    uint32 words per row (6-bit codes may straddle two words);
 *  - top-k orders by logit, descending, ties to the lower expert index;
 *  - SwiGLU(g, u) = g * sigmoid(g) * u with sigmoid(z) = 1 / (1 + exp(-z));
 *  - an expert id outside [0, n_experts) contributes an all-zero row;
 *  - with no shared expert the shared term is zero; a missing gate means 1.
 *
 * dtype codes: 0 = float32, 1 = IEEE binary16, 2 = bfloat16.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* ------------------------------------------------------------- decoding -- */

/* Exact value of an IEEE binary16 bit pattern. */
static double half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)mant, -24);              /* subnormal: mant * 2^-24 */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(mant | 0x400), expo - 25); /* (1.mant) * 2^(e-15) */
    return sign ? -v : v;
}

/* Exact value of a bfloat16 bit pattern (the top half of a float32). */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Element i of an array of dtype dt, as a double. */
static double load_val(const void *p, int dt, size_t i)
{
    switch (dt) {
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_F16: return half_to_double(((const uint16_t *)p)[i]);
    default:      return bf16_to_double(((const uint16_t *)p)[i]);
    }
}

double oracle_decode_value(const void *p, int dt, int64_t i) { return load_val(p, dt, (size_t)i); }

/* Code j of a row: bits [bits*j, bits*j + bits) of the row's LSB-first bit stream. */
static uint32_t code_at(const uint32_t *row, int bits, int64_t j)
{
    uint64_t bit = (uint64_t)bits * (uint64_t)j;
    uint64_t w = bit / 32, sh = bit % 32;
    uint64_t v = row[w] >> sh;
    if (sh + (uint64_t)bits > 32)
        v |= (uint64_t)row[w + 1] << (32 - sh);
    return (uint32_t)(v & ((1u << bits) - 1u));
}

void oracle_unpack_row(const uint32_t *row, int bits, int64_t cols, uint32_t *codes)
{
    for (int64_t j = 0; j < cols; ++j)
        codes[j] = code_at(row, bits, j);
}

/* A quantized projection stack [n_experts, rows, cols]. */
typedef struct {
    const uint32_t *q;        /* [n_experts, rows, cols*bits/32] */
    const uint16_t *scales;   /* [n_experts, rows, cols/64] */
    const uint16_t *biases;   /* [n_experts, rows, cols/64] */
    int32_t n_experts, rows, cols, bits, sb_dtype;
} oracle_qmat;

/* Dequantised weight w[e, r, j] = scale * q + bias, exact in double. */
static double weight_at(const oracle_qmat *m, int64_t e, int64_t r, int64_t j)
{
    int64_t words = (int64_t)m->cols * m->bits / 32;
    int64_t groups = m->cols / 64;
    const uint32_t *row = m->q + (e * m->rows + r) * words;
    size_t gi = (size_t)((e * m->rows + r) * groups + j / 64);
    double s = load_val(m->scales, m->sb_dtype, gi);
    double b = load_val(m->biases, m->sb_dtype, gi);
    return s * (double)code_at(row, m->bits, j) + b;
}

/* Dot product of dequantised row r of expert e with a double vector v[cols]. */
static double qrow_dot(const oracle_qmat *m, int64_t e, int64_t r, const double *v)
{
    double acc = 0.0;
    for (int64_t j = 0; j < m->cols; ++j)
        acc += weight_at(m, e, r, j) * v[j];
    return acc;
}

void oracle_dequant_row(const oracle_qmat *m, int64_t e, int64_t r, double *w)
{
    for (int64_t j = 0; j < m->cols; ++j)
        w[j] = weight_at(m, e, r, j);
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------- route -- */
/*
 * Per token t: logits[e] = sum_j Wr[e, j] * x[t, j];
 * probs = softmax(logits) over all n_experts (max-subtracted);
 * ids = the top_k experts by logit, descending, ties to the lower index;
 * scores[k] = probs[ids[k]] / sum_k' probs[ids[k']] if renormalize else probs[ids[k]];
 * gate[t] = sigmoid(sum_j w_g[j] * x[t, j]) when w_g is given.
 * Returns 0, or -1 on invalid sizes.
 */
int oracle_route(const void *x, int x_dt, int n_tokens, int d_in,
                 const void *wr, int wr_dt, int n_experts, int top_k, int renormalize,
                 const void *wg, int wg_dt,
                 double *logits, double *probs, int32_t *ids, double *scores, double *gate)
{
    if (n_tokens < 1 || d_in < 1 || n_experts < 1 || top_k < 1 || top_k > n_experts)
        return -1;
    for (int t = 0; t < n_tokens; ++t) {
        double *l = logits + (size_t)t * n_experts;
        double *p = probs + (size_t)t * n_experts;
#pragma omp parallel for schedule(static)
        for (int e = 0; e < n_experts; ++e) {
            double acc = 0.0;
            for (int j = 0; j < d_in; ++j)
                acc += load_val(wr, wr_dt, (size_t)e * d_in + j) *
                       load_val(x, x_dt, (size_t)t * d_in + j);
            l[e] = acc;
        }
        double m = l[0];
        for (int e = 1; e < n_experts; ++e)
            if (l[e] > m) m = l[e];
        double z = 0.0;
        for (int e = 0; e < n_experts; ++e) {
            p[e] = exp(l[e] - m);
            z += p[e];
        }
        for (int e = 0; e < n_experts; ++e)
            p[e] /= z;

        /* selection of the top_k by (logit descending, index ascending) */
        int32_t *id = ids + (size_t)t * top_k;
        for (int k = 0; k < top_k; ++k) {
            int best = -1;
            for (int e = 0; e < n_experts; ++e) {
                int taken = 0;
                for (int kk = 0; kk < k; ++kk)
                    if (id[kk] == e) taken = 1;
                if (taken) continue;
                if (best < 0 || l[e] > l[best]) best = e;   /* strict: ties keep the lower index */
            }
            id[k] = best;
        }
        double *sc = scores + (size_t)t * top_k;
        double sel = 0.0;
        for (int k = 0; k < top_k; ++k)
            sel += p[id[k]];
        for (int k = 0; k < top_k; ++k)
            sc[k] = renormalize ? p[id[k]] / sel : p[id[k]];

        if (wg && gate) {
            double acc = 0.0;
            for (int j = 0; j < d_in; ++j)
                acc += load_val(wg, wg_dt, (size_t)j) * load_val(x, x_dt, (size_t)t * d_in + j);
            gate[t] = sigmoid(acc);
        }
    }
    return 0;
}

/* ----------------------------------------------------------- expert FFN -- */
/*
 * For every token t and slot k with e = ids[t, k] in [0, n_experts):
 *   g[r] = sum_j wg[e, r, j] x[t, j],  u[r] = sum_j wu[e, r, j] x[t, j]
 *   act[t, k, r] = g[r] * sigmoid(g[r]) * u[r]                    (kernel A)
 *   partial[t, k, i] = score[t, k] * sum_r wd[e, i, r] act[t, k, r]  (kernel B)
 * with score = 1 when scores is NULL.  Out-of-range ids give zero rows.
 * Returns 0, or -1 on inconsistent shapes.
 */
int oracle_expert_ffn(const void *x, int x_dt, int n_tokens, int d_in, int d_ff,
                      const oracle_qmat *gp, const oracle_qmat *up, const oracle_qmat *dp,
                      const int32_t *ids, const double *scores, int top_k,
                      double *act, double *partial)
{
    if (gp->rows != d_ff || up->rows != d_ff || dp->cols != d_ff ||
        gp->cols != d_in || up->cols != d_in || dp->rows != d_in ||
        gp->n_experts != up->n_experts || gp->n_experts != dp->n_experts)
        return -1;
    int n_pairs = n_tokens * top_k;
    double *xv = (double *)malloc(sizeof(double) * (size_t)d_in);
    if (!xv)
        return -1;
    for (int pidx = 0; pidx < n_pairs; ++pidx) {
        int t = pidx / top_k;
        int e = ids[pidx];
        double *a = act + (size_t)pidx * d_ff;
        double *o = partial + (size_t)pidx * d_in;
        if (e < 0 || e >= gp->n_experts) {
            for (int r = 0; r < d_ff; ++r) a[r] = 0.0;
            for (int i = 0; i < d_in; ++i) o[i] = 0.0;
            continue;
        }
        for (int j = 0; j < d_in; ++j)
            xv[j] = load_val(x, x_dt, (size_t)t * d_in + j);
#pragma omp parallel for schedule(static)
        for (int r = 0; r < d_ff; ++r) {
            double g = qrow_dot(gp, e, r, xv);
            double u = qrow_dot(up, e, r, xv);
            a[r] = g * sigmoid(g) * u;
        }
        double s = scores ? scores[pidx] : 1.0;
#pragma omp parallel for schedule(static)
        for (int i = 0; i < d_in; ++i)
            o[i] = s * qrow_dot(dp, e, i, a);
    }
    free(xv);
    return 0;
}

/* ----------------------------------------------------------------- tail -- */
/*
 * out[t, i] = resid[t, i] + ( routed[t, i] + shared[t, i] * gate[t] ), where
 * routed = (((partial[t,0,i] + partial[t,1,i]) + ...) + partial[t,K-1,i]) in
 * slot order, shared = sum over s in order of shared_partial[t, s, i]
 * (zero when n_shared == 0) and gate = 1 when absent.
 */
int oracle_tail(const double *partial, int n_tokens, int top_k, int d_in,
                const double *shared, int n_shared, const double *gate,
                const void *resid, int resid_dt, double *out)
{
    if (n_tokens < 1 || top_k < 1 || d_in < 1 || n_shared < 0)
        return -1;
    for (int t = 0; t < n_tokens; ++t) {
        double gv = gate ? gate[t] : 1.0;
        for (int i = 0; i < d_in; ++i) {
            double routed = 0.0;
            for (int k = 0; k < top_k; ++k)
                routed += partial[((size_t)t * top_k + k) * d_in + i];
            double sh = 0.0;
            for (int s = 0; s < n_shared; ++s)
                sh += shared[((size_t)t * n_shared + s) * d_in + i];
            out[(size_t)t * d_in + i] =
                load_val(resid, resid_dt, (size_t)t * d_in + i) + (routed + sh * gv);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- rmsnorm -- */
/*
 * The next layer's RMSNorm applied to the layer output (Red Lite dev39, "fused
 * expert tail (GPU-routed decode)", section "Measurements": the tail variant
 * that also computed the next layer's RMSNorm).  The standard definition, per
 * token t:
 *   ms             = (1 / d) * sum_i y[t, i]^2
 *   normed[t, i]   = y[t, i] / sqrt(ms + eps) * weight[i]
 * y is the layer output [n_tokens][d] (double), weight [d] of dtype w_dt,
 * eps >= 0.  Returns 0, or -1 on invalid sizes.
 */
int oracle_rmsnorm(const double *y, int n_tokens, int d, const void *weight, int w_dt, double eps,
                   double *normed)
{
    if (n_tokens < 1 || d < 1 || eps < 0.0)
        return -1;
    for (int t = 0; t < n_tokens; ++t) {
        const double *yt = y + (size_t)t * d;
        double ss = 0.0;
        for (int i = 0; i < d; ++i)
            ss += yt[i] * yt[i];
        double ms = ss / (double)d;
        double inv = 1.0 / sqrt(ms + eps);
        for (int i = 0; i < d; ++i)
            normed[(size_t)t * d + i] = yt[i] * inv * load_val(weight, w_dt, (size_t)i);
    }
    return 0;
}

/* ----------------------------------------------------- 16-bit output dtype -- */
/*
 * The layer output (and the RMSNorm output) stored in a 16-bit dtype, as an
 * engine that keeps its hidden state in bf16 would hold it (mlxcel PR #276,
 * "Validation": the fused path checked inside the engine's decode loop).  The
 * reading taken: the exact result rounded once to the nearest value of the
 * dtype, ties to the value whose last significand bit is 0 (IEEE 754
 * round-to-nearest-even), past the largest finite value to infinity.
 *
 * A binary floating-point format with p significand bits (the leading one
 * included) and exponents emin..emax holds, in each binade [2^e, 2^(e+1)),
 * the multiples of 2^(e - p + 1); below 2^emin (subnormals) the multiples of
 * 2^(emin - p + 1).  Rounding is therefore: take the spacing q of v's binade,
 * round v / q to an integer with ties to even (rint in the default rounding
 * mode; v / q and the product back are exact in double), and overflow past
 * the largest finite value (2 - 2^(1-p)) * 2^emax to infinity.
 *   bfloat16: p = 8,  emin = -126, emax = 127
 *   binary16: p = 11, emin = -14,  emax = 15
 * v is rounded in place, n values; dt 0 leaves v unchanged.  Returns 0, or -1
 * for an unknown dtype.
 */
int oracle_round_to_dtype(double *v, size_t n, int dt)
{
    int p, emin, emax;
    if (dt == 0)
        return 0;
    if (dt == 2) {
        p = 8; emin = -126; emax = 127;
    } else if (dt == 1) {
        p = 11; emin = -14; emax = 15;
    } else {
        return -1;
    }
    const double vmax = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    for (size_t i = 0; i < n; ++i) {
        const double x = v[i];
        if (x == 0.0 || !isfinite(x))
            continue;
        int e2;
        frexp(x, &e2);                  /* |x| in [2^(e2-1), 2^e2) */
        int e = e2 - 1;
        if (e < emin)
            e = emin;
        const double q = ldexp(1.0, e - p + 1);
        double r = rint(x / q) * q;
        if (fabs(r) > vmax)
            r = copysign(INFINITY, x);
        v[i] = r;
    }
    return 0;
}
