/*
 * moe_oracle.c -- plain CPU oracle for the routed MoE expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  It shares no code
 * with the HIP library.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared
 * (-ffp-contract=off: no multiply-add is fused unless written as fmaf).
 *
 * Arithmetic: every floating-point step is done in double and rounded once to
 * the storage type where the pages place a storage rounding; the combine is
 * the one step written in fp32, because the pages fix an order for it (see
 * orc_combine).  OpenMP splits only independent output rows; each output
 * element is computed by one thread in a fixed order.
 *
 * What pins each function (tests/test_oracle_*.py):
 *   orc_round_f16 / orc_round_bf16  numpy's correctly rounded f64->f16 cast;
 *                                   hand-derived ties and double-rounding cases
 *   orc_route                       numpy lexsort brute force; scipy softmax /
 *                                   expit closed forms; all-equal-logit cases
 *   orc_dispatch_index, orc_counts  numpy stable argsort and bincount
 *   orc_awq_coeff / dequant         golden words for the AWQ nibble order
 *                                   (tests/golden/awq_words.txt); worked
 *                                   rounding values; numpy f16 casts
 *   orc_awq_project                 numpy float64 matmul, exact-arithmetic cases
 *   orc_swiglu                      scipy expit, clamp bound, one-sided gate clamp
 *   orc_combine                     order-sensitive fp32 case, k*x identity
 *   orc_copy_vjp                    adjoint identity with the COPY dispatch
 *   orc_awq_input_backward          adjoint identity, numpy matmul
 *   orc_dispatch_backward           adjoint identity with the COPY dispatch,
 *                                   order-sensitive fp32 case
 *   orc_dispatch_weights_backward   finite differences of a float64 softmax,
 *                                   two-expert closed form, zero sum
 *   orc_combine_backward            adjoint identity and exact finite
 *                                   differences of the combine
 *   orc_swiglu_backward             finite differences of the closed form,
 *                                   values at 0 and beyond the clamp
 *   orc_awq_swiglu_input_backward   finite differences of the gate/up + SwiGLU
 *                                   forward (fp32 activations)
 *   orc_e2m1_value, orc_e8m0_value  OCP MX element/scale tables
 *   orc_mxfp4_*                     golden byte, numpy matmul; a non-zero
 *                                   bias distinct per (expert, row), exact
 *   orc_moe_forward                 per-token dense float64 evaluation in numpy,
 *                                   for AWQ cubes and for MXFP4 banks (dense
 *                                   banks from the golden tables, gate and up
 *                                   banks interleaved by the test, clamped and
 *                                   one-sided SwiGLU, non-zero biases)
 * Parity unpinned by the pages (conventions only, frozen by golden values):
 *   the AWQ nibble permutation, the nibble order inside an MXFP4 byte, the
 *   row interleave of the fused gate/up bank, and the clamped-SwiGLU form.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* storage types                                                        */
/* ------------------------------------------------------------------ */

double orc_f16_value(uint16_t bits)
{
    int sign = bits >> 15;
    int ex = (bits >> 10) & 0x1F;
    int man = bits & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);              /* subnormal: man * 2^-24 */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25); /* (1.man) * 2^(ex-15) */
    return sign ? -v : v;
}

double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round v to the nearest multiple of the format's quantum at v's binade
 * (ties to even), where the format keeps `sig` significant bits and its
 * smallest quantum (subnormal spacing) is 2^min_q_exp. */
static double round_to_format(double v, int sig, int min_q_exp, double max_finite)
{
    if (v == 0.0 || isnan(v) || isinf(v))
        return v;
    int ex;
    frexp(v, &ex);                    /* |v| = m * 2^ex, 0.5 <= |m| < 1 */
    int q_exp = ex - sig;             /* spacing of `sig`-bit numbers at v */
    if (q_exp < min_q_exp)
        q_exp = min_q_exp;
    double scaled = ldexp(v, -q_exp); /* exact: power-of-two scaling */
    double r = ldexp(nearbyint(scaled), q_exp); /* default mode: ties to even */
    if (fabs(r) > max_finite)
        return v > 0 ? INFINITY : -INFINITY;
    return r;
}

uint16_t orc_round_f16(double v)
{
    /* IEEE binary16: 11 significant bits, subnormal spacing 2^-24, max 65504 */
    double r = round_to_format(v, 11, -24, 65504.0);
    if (isnan(r))
        return 0x7E00;
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (isinf(a))
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);
    int e16 = ex - 1 + 15;            /* biased exponent of a = 1.f * 2^(ex-1) */
    if (e16 <= 0)                     /* subnormal: a = man * 2^-24 */
        return sign | (uint16_t)(a / ldexp(1.0, -24));
    uint16_t man = (uint16_t)(ldexp(a, -(ex - 1)) * 1024.0 - 1024.0);
    return sign | (uint16_t)(e16 << 10) | man;
}

uint16_t orc_round_bf16(double v)
{
    /* bfloat16: 8 significant bits, fp32's exponent range, subnormal spacing
     * 2^-133, max finite (2 - 2^-7) * 2^127 */
    double maxf = ldexp(255.0, 120);
    double r = round_to_format(v, 8, -133, maxf);
    if (isnan(r))
        return 0x7FC0;
    float f = (float)r;               /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

double orc_load(const void *buf, int dtype, size_t i)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float *)buf)[i];
    case ORC_F16: return orc_f16_value(((const uint16_t *)buf)[i]);
    default:      return orc_bf16_value(((const uint16_t *)buf)[i]);
    }
}

void orc_store(void *buf, int dtype, size_t i, double v)
{
    switch (dtype) {
    case ORC_F32: ((float *)buf)[i] = (float)v; break; /* C cast: ties to even */
    case ORC_F16: ((uint16_t *)buf)[i] = orc_round_f16(v); break;
    default:      ((uint16_t *)buf)[i] = orc_round_bf16(v); break;
    }
}

static double round_to(int dtype, double v)
{
    switch (dtype) {
    case ORC_F32: return (double)(float)v;
    case ORC_F16: return orc_f16_value(orc_round_f16(v));
    default:      return orc_bf16_value(orc_round_bf16(v));
    }
}

/* ------------------------------------------------------------------ */
/* router                                                               */
/* ------------------------------------------------------------------ */

/* ruda-tensor moe_exchange.rs, MoeDispatchOps::moe_dispatch and the
 * MoeDispatched fields: per token, a discrete selection of top_k expert IDs
 * (U32 [tokens,top_k]) and FP32 continuous weights [tokens,top_k].
 * Readings: the score is logit + bias (one fp32 add); the k largest scores are
 * taken, ties going to the lower expert ID, listed in that order; the weights
 * are the softmax over the k selected scores, computed in double and rounded
 * once to fp32. */
void orc_route(int T, int E, int k, const float *logits, const float *bias,
               uint32_t *selected, float *weights)
{
#pragma omp parallel
    {
        float *s = (float *)malloc(sizeof(float) * (size_t)E);
        char *taken = (char *)malloc((size_t)E);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            for (int e = 0; e < E; ++e) {
                float sc = logits[(size_t)t * E + e];
                if (bias)
                    sc = sc + bias[e];      /* one IEEE single-precision add */
                s[e] = sc;
                taken[e] = 0;
            }
            for (int j = 0; j < k; ++j) {
                int best = -1;
                for (int e = 0; e < E; ++e) {
                    if (taken[e])
                        continue;
                    /* greater score wins; equal scores: the lower ID (first seen) */
                    if (best < 0 || s[e] > s[best])
                        best = e;
                }
                taken[best] = 1;
                selected[(size_t)t * k + j] = (uint32_t)best;
            }
            double m = s[selected[(size_t)t * k]];
            double den = 0.0;
            for (int j = 0; j < k; ++j)
                den += exp((double)s[selected[(size_t)t * k + j]] - m);
            for (int j = 0; j < k; ++j) {
                double num = exp((double)s[selected[(size_t)t * k + j]] - m);
                weights[(size_t)t * k + j] = (float)(num / den);
            }
        }
        free(s);
        free(taken);
    }
}

/* ------------------------------------------------------------------ */
/* COPY dispatch                                                        */
/* ------------------------------------------------------------------ */

/* ruda-tensor moe_exchange.rs, MoeDispatched: `values` holds expert-sorted
 * copies of source rows, one per selected assignment, and `row_experts` the
 * sorted U32 global expert IDs aligned with them.  Reading: the sort is stable
 * in flattened (token, slot) order, so rows of one expert keep token order.
 * offsets[e] is the first sorted row of expert e (offsets[E] = T*k). */
void orc_dispatch_index(int T, int E, int k, const uint32_t *selected,
                        int32_t *offsets, int32_t *row_src, int32_t *slot_pos,
                        uint32_t *row_experts)
{
    int32_t *cursor = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
    for (int e = 0; e <= E; ++e)
        offsets[e] = 0;
    for (long a = 0; a < (long)T * k; ++a)
        offsets[selected[a] + 1] += 1;           /* histogram, shifted by one */
    for (int e = 0; e < E; ++e)
        offsets[e + 1] += offsets[e];            /* inclusive scan -> starts */
    for (int e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int t = 0; t < T; ++t)                   /* tokens in ascending order */
        for (int j = 0; j < k; ++j) {
            uint32_t e = selected[(size_t)t * k + j];
            int32_t p = cursor[e]++;
            slot_pos[(size_t)t * k + j] = p;
            row_src[p] = t;
            row_experts[p] = e;
        }
    free(cursor);
}

void orc_copy_rows(int A, size_t row_bytes, const void *x, const int32_t *row_src,
                   void *values)
{
    for (int p = 0; p < A; ++p)
        memcpy((char *)values + (size_t)p * row_bytes,
               (const char *)x + (size_t)row_src[p] * row_bytes, row_bytes);
}

/* ruda-tensor moe_exchange.rs, MoeDispatchOps::moe_dispatch_counts: row counts
 * per caller-declared contiguous range of global expert IDs, read from the
 * expert-prefix metadata only.  Reading: prefix holds R+1 non-decreasing
 * boundaries within [0, E]; range r is [prefix[r], prefix[r+1]). */
int orc_counts(int E, const int32_t *offsets, int R, const int64_t *prefix,
               int64_t *counts)
{
    if (R < 0)
        return -1;
    for (int r = 0; r <= R; ++r) {
        if (prefix[r] < 0 || prefix[r] > E)
            return -1;
        if (r > 0 && prefix[r] < prefix[r - 1])
            return -1;
    }
    for (int r = 0; r < R; ++r)
        counts[r] = (int64_t)offsets[prefix[r + 1]] - (int64_t)offsets[prefix[r]];
    return 0;
}

/* ------------------------------------------------------------------ */
/* AWQ packed coefficients                                              */
/* ------------------------------------------------------------------ */

/* Which logical column of its group of eight each nibble of a packed word
 * holds (nibble i = bits 4i..4i+3).  The pages name "the AWQ nibble order" for
 * the permuted eight-code I32 words (packed_experts.rs AwqExpertPayload;
 * frozen_awq.rs FrozenAwqOps) without printing it; this is the AWQ format's
 * own interleave.  The same order applies to the zero-point words. */
static const int AWQ_NIBBLE_COLUMN[8] = {0, 2, 4, 6, 1, 3, 5, 7};

static int awq_nibble_of_column(int c)
{
    for (int i = 0; i < 8; ++i)
        if (AWQ_NIBBLE_COLUMN[i] == c)
            return i;
    return -1;
}

static unsigned awq_code(uint32_t word, int column_in_group)
{
    int i = awq_nibble_of_column(column_in_group);
    return (word >> (4 * i)) & 0xFu;             /* logical shift of the I32 word */
}

/* packed_experts.rs AwqExpertPayload: qweight I32 [E,K,N/8], qzeros I32
 * [E,K/group,N/8], scales [E,K/group,N] in FP32/FP16/BF16.
 * frozen_awq.rs FrozenAwqOps: the coefficient keeps scale-dtype rounding.
 * Coefficient: (code - zero) * scale, formed exactly in double, rounded once to
 * the scale dtype.  The zero point is the raw 4-bit code. */
double orc_awq_coeff(int K, int N, int g, const int32_t *qweight,
                     const int32_t *qzeros, const void *scales, int sdt,
                     int e, int k, int n)
{
    int words = N / 8;
    int G = K / g;
    uint32_t w = (uint32_t)qweight[((size_t)e * K + k) * words + n / 8];
    uint32_t zw = (uint32_t)qzeros[((size_t)e * G + k / g) * words + n / 8];
    int code = (int)awq_code(w, n % 8);
    int zero = (int)awq_code(zw, n % 8);
    double s = orc_load(scales, sdt, ((size_t)e * G + k / g) * N + n);
    return round_to(sdt, (double)(code - zero) * s);
}

void orc_awq_dequant(int E, int K, int N, int g, const int32_t *qweight,
                     const int32_t *qzeros, const void *scales, int sdt,
                     double *W)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int e = 0; e < E; ++e)
        for (int k = 0; k < K; ++k)
            for (int n = 0; n < N; ++n)
                W[((size_t)e * K + k) * N + n] =
                    orc_awq_coeff(K, N, g, qweight, qzeros, scales, sdt, e, k, n);
}

/* Dense W_e [K,N] of one expert. */
static void awq_expert_dense(int K, int N, int g, const int32_t *qweight,
                             const int32_t *qzeros, const void *scales, int sdt,
                             int e, double *W)
{
#pragma omp parallel for schedule(static)
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n)
            W[(size_t)k * N + n] =
                orc_awq_coeff(K, N, g, qweight, qzeros, scales, sdt, e, k, n);
}

static int expert_has_rows(int A, const uint32_t *row_experts, int e)
{
    if (!row_experts)
        return e == 0 && A > 0;
    for (int p = 0; p < A; ++p)
        if ((int)row_experts[p] == e)
            return 1;
    return 0;
}

/* packed_experts.rs FrozenPackedExpertOps::packed_expert_forward (evaluate only
 * the assigned experts) and frozen_awq.rs FrozenAwqOps::frozen_awq_forward
 * (output keeps the input storage type; optional scale-dtype bias):
 * out[p,n] = round_adt( sum_k in[p,k] * W_e[k,n] + bias[e,n] ), e the row's
 * expert, the sum in double. */
void orc_awq_project(int A, int K, int N, const void *in, int adt,
                     const uint32_t *row_experts, int E, int g,
                     const int32_t *qweight, const int32_t *qzeros,
                     const void *scales, int sdt, const void *bias,
                     void *out, double *out_exact)
{
    double *W = (double *)malloc(sizeof(double) * (size_t)K * N);
    for (int e = 0; e < E; ++e) {
        if (!expert_has_rows(A, row_experts, e))
            continue;                             /* untouched experts: no work */
        awq_expert_dense(K, N, g, qweight, qzeros, scales, sdt, e, W);
#pragma omp parallel for schedule(dynamic, 4)
        for (int p = 0; p < A; ++p) {
            int pe = row_experts ? (int)row_experts[p] : 0;
            if (pe != e)
                continue;
            for (int n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int k = 0; k < K; ++k)
                    acc += orc_load(in, adt, (size_t)p * K + k) * W[(size_t)k * N + n];
                if (bias)
                    acc += orc_load(bias, sdt, (size_t)e * N + n);
                if (out_exact)
                    out_exact[(size_t)p * N + n] = acc;
                orc_store(out, adt, (size_t)p * N + n, acc);
            }
        }
    }
    free(W);
}

/* ------------------------------------------------------------------ */
/* SwiGLU                                                               */
/* ------------------------------------------------------------------ */

/* packed_experts.rs FrozenPackedExpertOps::packed_swiglu_forward: gate/up/down
 * chain with storage-rounded SwiGLU.  h = g' * sigmoid(alpha*g') * (u' + off),
 * g' and u' clamped to [-clamp, clamp] when clamp > 0 (the clamped variant of
 * libmir-metal's clamped_routed engine), in double, rounded once to adt.
 * gate_one_sided != 0 is the variant some MXFP4 models use: the gate is clamped
 * from above only, g' = min(g, clamp), u' as before. */
static double gate_lower(double clamp, int gate_one_sided)
{
    return gate_one_sided ? -INFINITY : -clamp;
}

void orc_swiglu(size_t n, const void *G, const void *U, int adt, double clamp,
                double alpha, double up_offset, int gate_one_sided, void *h)
{
    const double glo = gate_lower(clamp, gate_one_sided);
#pragma omp parallel for schedule(static)
    for (size_t i = 0; i < n; ++i) {
        double g = orc_load(G, adt, i);
        double u = orc_load(U, adt, i);
        if (clamp > 0.0) {
            g = fmin(fmax(g, glo), clamp);
            u = fmin(fmax(u, -clamp), clamp);
        }
        double sig = 1.0 / (1.0 + exp(-alpha * g));
        orc_store(h, adt, i, g * sig * (u + up_offset));
    }
}

/* ------------------------------------------------------------------ */
/* combine and COPY VJP                                                 */
/* ------------------------------------------------------------------ */

/* moe_exchange.rs MoeDispatchOps::moe_combine: the ascending expert-ID combine
 * after the expert rows have returned to their source.  Sorted rows are in
 * expert order, so ascending sorted position = ascending expert ID.  Written
 * in fp32 as acc = fmaf(w, y, acc) from acc = 0, then one rounding to adt. */
void orc_combine(int T, int k, int K, const void *y, int adt,
                 const float *weights, const int32_t *slot_pos, void *out)
{
#pragma omp parallel
    {
        int *order = (int *)malloc(sizeof(int) * (size_t)k);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            for (int j = 0; j < k; ++j)
                order[j] = j;
            for (int a = 1; a < k; ++a) {         /* insertion sort by position */
                int v = order[a], b = a - 1;
                while (b >= 0 && slot_pos[(size_t)t * k + order[b]] >
                                 slot_pos[(size_t)t * k + v]) {
                    order[b + 1] = order[b];
                    --b;
                }
                order[b + 1] = v;
            }
            for (int c = 0; c < K; ++c) {
                float acc = 0.0f;
                for (int a = 0; a < k; ++a) {
                    int j = order[a];
                    size_t p = (size_t)slot_pos[(size_t)t * k + j];
                    float yv = (float)orc_load(y, adt, p * K + c);
                    acc = fmaf(weights[(size_t)t * k + j], yv, acc);
                }
                orc_store(out, adt, (size_t)t * K + c, (double)acc);
            }
        }
        free(order);
    }
}

/* moe_exchange.rs MoeDispatchOps::moe_dispatch_backward: the COPY VJP sums the
 * gradient rows of a token's copies, without multiplying routing weights. */
void orc_copy_vjp(int T, int k, int K, const double *dvalues,
                  const int32_t *slot_pos, double *dx)
{
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += dvalues[(size_t)slot_pos[(size_t)t * k + j] * K + c];
            dx[(size_t)t * K + c] = acc;
        }
}

/* ------------------------------------------------------------------ */
/* input VJP                                                            */
/* ------------------------------------------------------------------ */

/* frozen_awq.rs FrozenAwqOps::frozen_awq_input_backward and packed_experts.rs
 * packed_expert_input_backward: apply the transpose of the same rounded packed
 * coefficients; the result keeps the gradient storage type.
 * grad_in[p,k] = round_gdt( sum_n grad[p,n] * W_e[k,n] ). */
void orc_awq_input_backward(int A, int K, int N, const void *grad, int gdt,
                            const uint32_t *row_experts, int E, int g,
                            const int32_t *qweight, const int32_t *qzeros,
                            const void *scales, int sdt, void *grad_in)
{
    double *W = (double *)malloc(sizeof(double) * (size_t)K * N);
    for (int e = 0; e < E; ++e) {
        if (!expert_has_rows(A, row_experts, e))
            continue;
        awq_expert_dense(K, N, g, qweight, qzeros, scales, sdt, e, W);
#pragma omp parallel for schedule(dynamic, 4)
        for (int p = 0; p < A; ++p) {
            int pe = row_experts ? (int)row_experts[p] : 0;
            if (pe != e)
                continue;
            for (int k = 0; k < K; ++k) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n)
                    acc += orc_load(grad, gdt, (size_t)p * N + n) * W[(size_t)k * N + n];
                orc_store(grad_in, gdt, (size_t)p * K + k, acc);
            }
        }
    }
    free(W);
}

/* ------------------------------------------------------------------ */
/* backward path (first order)                                          */
/* ------------------------------------------------------------------ */

/* Token t's slots in ascending sorted position, which is ascending expert ID
 * (insertion sort; positions of one token are distinct). */
static void slots_by_position(int k, const int32_t *pos_t, int *order)
{
    for (int j = 0; j < k; ++j)
        order[j] = j;
    for (int a = 1; a < k; ++a) {
        int v = order[a], b = a - 1;
        while (b >= 0 && pos_t[order[b]] > pos_t[v]) {
            order[b + 1] = order[b];
            --b;
        }
        order[b + 1] = v;
    }
}

/* moe_exchange.rs MoeDispatchOps::moe_dispatch_backward: the COPY VJP sums the
 * selected expert-row seeds of a token without multiplying routing weights
 * again.  Reading (as for the combine): an fp32 sum in ascending expert ID,
 * i.e. ascending sorted position, from 0, then one rounding to the storage
 * type. */
void orc_dispatch_backward(int T, int k, int K, const void *dvalues, int adt,
                           const int32_t *slot_pos, void *dx)
{
#pragma omp parallel
    {
        int *order = (int *)malloc(sizeof(int) * (size_t)k);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            slots_by_position(k, slot_pos + (size_t)t * k, order);
            for (int c = 0; c < K; ++c) {
                float acc = 0.0f;
                for (int a = 0; a < k; ++a) {
                    size_t p = (size_t)slot_pos[(size_t)t * k + order[a]];
                    acc = acc + (float)orc_load(dvalues, adt, p * K + c);
                }
                orc_store(dx, adt, (size_t)t * K + c, (double)acc);
            }
        }
        free(order);
    }
}

/* moe_exchange.rs MoeDispatchOps::moe_dispatch_weights_backward: the
 * fixed-selection source-logit VJP of the FP32 continuous weights.  With the
 * selection held fixed, w_j is the softmax over the selected scores, so
 * d s_j = w_j * (dw_j - sum_i w_i dw_i), and an unselected logit gets 0 (a
 * discrete selection has no derivative).  Readings: the stored fp32 weights
 * stand for the softmax values; the sum runs over the slots in slot order, in
 * double; one rounding to fp32.  The gradient of the added expert bias is the
 * column sum of dlogits and is not formed here. */
void orc_dispatch_weights_backward(int T, int E, int k, const uint32_t *selected,
                                   const float *weights, const float *dweights,
                                   float *dlogits)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float *w = weights + (size_t)t * k, *dw = dweights + (size_t)t * k;
        double sum = 0.0;
        for (int i = 0; i < k; ++i)
            sum += (double)w[i] * (double)dw[i];
        for (int e = 0; e < E; ++e)
            dlogits[(size_t)t * E + e] = 0.0f;
        for (int j = 0; j < k; ++j)
            dlogits[(size_t)t * E + selected[(size_t)t * k + j]] =
                (float)((double)w[j] * ((double)dw[j] - sum));
    }
}

/* moe_exchange.rs MoeDispatchOps::moe_combine_backward with a
 * MoeCombineSelection: only the requested derivatives are formed (NULL = not
 * requested).  Expert rows: the combine's acc = fma(w, y, acc) has derivative
 * w with respect to y, so dy[p,:] = round_adt(fl32(w[t,j] * dout[t,:])) for
 * the sorted row p of assignment (t,j), one fp32 product (the final storage
 * rounding of the forward passes the gradient through).  FP32 weights:
 * dweights[t,j] = round_fp32(sum_c dout[t,c] * y[p,c]), summed in double. */
void orc_combine_backward(int T, int k, int K, const void *y, int adt,
                          const float *weights, const int32_t *slot_pos,
                          const void *dout, void *dy, float *dweights)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            size_t p = (size_t)slot_pos[(size_t)t * k + j];
            float w = weights[(size_t)t * k + j];
            double acc = 0.0;
            for (int c = 0; c < K; ++c) {
                double g = orc_load(dout, adt, (size_t)t * K + c);
                if (dy)
                    orc_store(dy, adt, p * K + c, (double)(w * (float)g));
                acc += g * orc_load(y, adt, p * K + c);
            }
            if (dweights)
                dweights[(size_t)t * k + j] = (float)acc;
        }
    }
}

/* packed_experts.rs FrozenPackedExpertOps::packed_swiglu_input_backward, the
 * SwiGLU step: derivatives of h = g' * sigmoid(alpha g') * (u' + up_offset)
 * at the storage-rounded G and U of the forward, g' and u' being G and U
 * clamped to [-c, c] when c > 0:
 *   dG = dh * (u' + up_offset) * (s + alpha g' s (1 - s)),  s = sigmoid(alpha g')
 *   dU = dh * g' * s
 * Readings: the storage roundings of the forward pass the gradient through; a
 * clamped value has derivative 1 on the closed interval [-c, c] and 0
 * outside it; dG and dU are evaluated in double and stored in the activation
 * type, like the forward's intermediates. */
void orc_swiglu_backward(size_t n, const void *G, const void *U, const void *dh, int adt,
                         double clamp, double alpha, double up_offset, int gate_one_sided,
                         void *dG, void *dU)
{
    const double glo = gate_lower(clamp, gate_one_sided);
#pragma omp parallel for schedule(static)
    for (size_t i = 0; i < n; ++i) {
        double g = orc_load(G, adt, i), u = orc_load(U, adt, i), d = orc_load(dh, adt, i);
        double gp = g, up = u, gpass = 1.0, upass = 1.0;
        if (clamp > 0.0) {
            gp = fmin(fmax(g, glo), clamp);
            up = fmin(fmax(u, -clamp), clamp);
            gpass = (g >= glo && g <= clamp) ? 1.0 : 0.0;
            upass = (u >= -clamp && u <= clamp) ? 1.0 : 0.0;
        }
        double sg = 1.0 / (1.0 + exp(-alpha * gp));
        orc_store(dG, adt, i, gpass * d * (up + up_offset) * (sg + alpha * gp * sg * (1.0 - sg)));
        orc_store(dU, adt, i, upass * d * gp * sg);
    }
}

/* packed_experts.rs FrozenPackedExpertOps::packed_swiglu_input_backward, the
 * gate/up part of the chain (its down part is orc_awq_input_backward): G and U
 * recomputed as in the forward (storage rounded), dG and dU from
 * orc_swiglu_backward, then the transposes of both rounded packed cubes:
 *   dvalues[p,k] = round_adt( sum_n dG[p,n] Wg_e[k,n] + sum_n dU[p,n] Wu_e[k,n] )
 * in double, gate sum first. */
void orc_awq_swiglu_input_backward(int A, int K, int I, const void *values, int adt,
                                   const uint32_t *row_experts, int E, int g,
                                   const int32_t *gqw, const int32_t *gqz, const void *gs,
                                   const int32_t *uqw, const int32_t *uqz, const void *us,
                                   int sdt, const void *gbias, const void *ubias,
                                   double clamp, double alpha, double up_offset,
                                   int gate_one_sided, const void *dh, void *dvalues)
{
    size_t sz = (adt == ORC_F32 ? 4 : 2) * (size_t)A * I;
    void *G = malloc(sz), *U = malloc(sz), *dG = malloc(sz), *dU = malloc(sz);
    double *Wg = (double *)malloc(sizeof(double) * (size_t)K * I);
    double *Wu = (double *)malloc(sizeof(double) * (size_t)K * I);
    orc_awq_project(A, K, I, values, adt, row_experts, E, g, gqw, gqz, gs, sdt, gbias, G, NULL);
    orc_awq_project(A, K, I, values, adt, row_experts, E, g, uqw, uqz, us, sdt, ubias, U, NULL);
    orc_swiglu_backward((size_t)A * I, G, U, dh, adt, clamp, alpha, up_offset, gate_one_sided,
                        dG, dU);
    for (int e = 0; e < E; ++e) {
        if (!expert_has_rows(A, row_experts, e))
            continue;
        awq_expert_dense(K, I, g, gqw, gqz, gs, sdt, e, Wg);
        awq_expert_dense(K, I, g, uqw, uqz, us, sdt, e, Wu);
#pragma omp parallel for schedule(dynamic, 4)
        for (int p = 0; p < A; ++p) {
            int pe = row_experts ? (int)row_experts[p] : 0;
            if (pe != e)
                continue;
            for (int k = 0; k < K; ++k) {
                double ag = 0.0, au = 0.0;
                for (int n = 0; n < I; ++n) {
                    ag += orc_load(dG, adt, (size_t)p * I + n) * Wg[(size_t)k * I + n];
                    au += orc_load(dU, adt, (size_t)p * I + n) * Wu[(size_t)k * I + n];
                }
                orc_store(dvalues, adt, (size_t)p * K + k, ag + au);
            }
        }
    }
    free(G);
    free(U);
    free(dG);
    free(dU);
    free(Wg);
    free(Wu);
}

/* ------------------------------------------------------------------ */
/* MXFP4 expert bank                                                    */
/* ------------------------------------------------------------------ */

/* OCP Microscaling FP4 E2M1 element: sign bit 3, exponent bits 2..1 (bias 1),
 * mantissa bit 0; exponent 0 is subnormal (0.5 * mantissa). */
double orc_e2m1_value(int nibble)
{
    int sign = (nibble >> 3) & 1;
    int ex = (nibble >> 1) & 3;
    int man = nibble & 1;
    double v = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
    return sign ? -v : v;
}

/* OCP Microscaling E8M0 shared scale: 2^(byte-127); 255 is NaN. */
double orc_e8m0_value(int byte)
{
    return byte == 255 ? NAN : ldexp(1.0, byte - 127);
}

/* libmir-metal clamped_routed/experts/native.rs, ExpertLayout::Native: blocks
 * u8 [E, rows, cols/32, 16] (32 four-bit elements of one row per 16 bytes),
 * scales u8 [E, rows, cols/32] (one E8M0 per 32-element block).  Reading: the
 * even element of a byte pair is the low nibble. */
static double mxfp4_coeff(int R, int C, const uint8_t *blocks,
                          const uint8_t *scales, int e, int r, int c)
{
    int nb = C / 32;
    size_t blk = ((size_t)e * R + r) * nb + c / 32;
    uint8_t byte = blocks[blk * 16 + (c % 32) / 2];
    int nib = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    return orc_e2m1_value(nib) * orc_e8m0_value(scales[blk]); /* exact */
}

void orc_mxfp4_dequant(int E, int R, int C, const uint8_t *blocks,
                       const uint8_t *scales, double *W)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int e = 0; e < E; ++e)
        for (int r = 0; r < R; ++r)
            for (int c = 0; c < C; ++c)
                W[((size_t)e * R + r) * C + c] = mxfp4_coeff(R, C, blocks, scales, e, r, c);
}

/* out[p,r] = round_adt( sum_c in[p,c] * W_e[r,c] + bias[e,r] ): the bank is
 * output-major, so the projection is in . W_e^T; bias is bf16. */
void orc_mxfp4_project(int A, int C, int R, const void *in, int adt,
                       const uint32_t *row_experts, int E, const uint8_t *blocks,
                       const uint8_t *scales, const uint16_t *bias_bf16, void *out)
{
    double *W = (double *)malloc(sizeof(double) * (size_t)R * C);
    for (int e = 0; e < E; ++e) {
        if (!expert_has_rows(A, row_experts, e))
            continue;
#pragma omp parallel for schedule(static)
        for (int r = 0; r < R; ++r)
            for (int c = 0; c < C; ++c)
                W[(size_t)r * C + c] = mxfp4_coeff(R, C, blocks, scales, e, r, c);
#pragma omp parallel for schedule(dynamic, 4)
        for (int p = 0; p < A; ++p) {
            int pe = row_experts ? (int)row_experts[p] : 0;
            if (pe != e)
                continue;
            for (int r = 0; r < R; ++r) {
                double acc = 0.0;
                for (int c = 0; c < C; ++c)
                    acc += orc_load(in, adt, (size_t)p * C + c) * W[(size_t)r * C + c];
                if (bias_bf16)
                    acc += orc_bf16_value(bias_bf16[(size_t)e * R + r]);
                orc_store(out, adt, (size_t)p * R + r, acc);
            }
        }
    }
    free(W);
}

/* ------------------------------------------------------------------ */
/* MXFP8 activations (the block-scaled MFMA variant of the MXFP4 bank)  */
/* ------------------------------------------------------------------ */

/* OCP Microscaling FP8 E4M3 element: sign bit 7, exponent bits 6..3 (bias 7),
 * mantissa bits 2..0; exponent 0 is subnormal (mantissa/8 * 2^-6); S.1111.111 is
 * NaN, so the largest finite magnitude is 1.75 * 2^8 = 448. */
double orc_e4m3_value(int byte)
{
    int sign = (byte >> 7) & 1, ex = (byte >> 3) & 15, man = byte & 7;
    if (ex == 15 && man == 7)
        return NAN;
    double v = ex == 0 ? ldexp(man / 8.0, -6) : ldexp(1.0 + man / 8.0, ex - 7);
    return sign ? -v : v;
}

/* Nearest E4M3 code to v by scanning every finite non-negative code, ties to the
 * even code (mantissa bit 0 clear); |v| beyond the largest code saturates to it.
 * The sign is kept, zero included. */
static uint8_t e4m3_round(double v)
{
    double a = fabs(v);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(orc_e4m3_value(c) - a);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

/* OCP MX quantization of each 32-element block of a row to MXFP8 (E4M3): the
 * shared exponent is floor(log2(max |v|)) minus 8 (the largest E4M3 exponent),
 * kept in the E8M0 range [-127, 127]; each element is v / 2^shared rounded to
 * the nearest E4M3 value, ties to even, saturated to +-448.  A block of zeros
 * gets scale byte 0 (2^-127) and zero elements.  x [rows, K] adt, K % 32 == 0;
 * q [rows, K] codes, s [rows, K/32] scale bytes (shared + 127). */
void orc_mxfp8_quantize(int rows, int K, const void *x, int adt, uint8_t *q, uint8_t *s)
{
    const int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < nb; ++b) {
            size_t base = (size_t)r * K + (size_t)b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i)
                amax = fmax(amax, fabs(orc_load(x, adt, base + i)));
            int shared = -127;
            if (amax > 0.0) {
                int e2;
                frexp(amax, &e2);   /* amax = f 2^e2, f in [0.5, 1): floor(log2) = e2 - 1 */
                shared = e2 - 1 - 8;
                if (shared < -127) shared = -127;
                if (shared > 127) shared = 127;
            }
            s[(size_t)r * nb + b] = (uint8_t)(shared + 127);
            for (int i = 0; i < 32; ++i)
                q[base + i] = e4m3_round(ldexp(orc_load(x, adt, base + i), -shared));
        }
}

/* The projection of MXFP8 rows with an MXFP4 bank, products exact:
 *   out[p, r] = round_adt( sum_c e4m3(q[p,c]) 2^(s[p,c/32]-127) * W_e[r,c] + bias[e,r] )
 * in double. */
void orc_mx8_project(int A, int C, int R, const uint8_t *q, const uint8_t *s,
                     const uint32_t *row_experts, int E, const uint8_t *blocks,
                     const uint8_t *scales, const uint16_t *bias_bf16, int adt, void *out)
{
    const int nb = C / 32;
    double *W = (double *)malloc(sizeof(double) * (size_t)R * C);
    double *xv = (double *)malloc(sizeof(double) * (size_t)(A > 0 ? A : 1) * C);
#pragma omp parallel for schedule(static)
    for (int p = 0; p < A; ++p)
        for (int c = 0; c < C; ++c)
            xv[(size_t)p * C + c] = orc_e4m3_value(q[(size_t)p * C + c]) *
                                    orc_e8m0_value(s[(size_t)p * nb + c / 32]);
    for (int e = 0; e < E; ++e) {
        if (!expert_has_rows(A, row_experts, e))
            continue;
#pragma omp parallel for schedule(static)
        for (int r = 0; r < R; ++r)
            for (int c = 0; c < C; ++c)
                W[(size_t)r * C + c] = mxfp4_coeff(R, C, blocks, scales, e, r, c);
#pragma omp parallel for schedule(dynamic, 4)
        for (int p = 0; p < A; ++p) {
            int pe = row_experts ? (int)row_experts[p] : 0;
            if (pe != e)
                continue;
            for (int r = 0; r < R; ++r) {
                double acc = 0.0;
                for (int c = 0; c < C; ++c)
                    acc += xv[(size_t)p * C + c] * W[(size_t)r * C + c];
                if (bias_bf16)
                    acc += orc_bf16_value(bias_bf16[(size_t)e * R + r]);
                orc_store(out, adt, (size_t)p * R + r, acc);
            }
        }
    }
    free(W);
    free(xv);
}

/* ------------------------------------------------------------------ */
/* whole forward path                                                   */
/* ------------------------------------------------------------------ */

static size_t dsize(int dt) { return dt == ORC_F32 ? 4 : 2; }

int orc_moe_forward(const orc_moe_args *a)
{
    int T = a->T, H = a->H, I = a->I, E = a->E, k = a->k;
    int A = T * k;
    size_t ab = dsize(a->adt);
    uint32_t *sel = a->selected ? a->selected : (uint32_t *)malloc(sizeof(uint32_t) * (size_t)A);
    float *w = a->weights ? a->weights : (float *)malloc(sizeof(float) * (size_t)A);
    int32_t *off = a->offsets ? a->offsets : (int32_t *)malloc(sizeof(int32_t) * ((size_t)E + 1));
    int32_t *src = a->row_src ? a->row_src : (int32_t *)malloc(sizeof(int32_t) * (size_t)A);
    int32_t *pos = a->slot_pos ? a->slot_pos : (int32_t *)malloc(sizeof(int32_t) * (size_t)A);
    uint32_t *rex = a->row_experts ? a->row_experts : (uint32_t *)malloc(sizeof(uint32_t) * (size_t)A);
    void *values = a->values ? a->values : malloc(ab * (size_t)A * H);
    void *h = a->h ? a->h : malloc(ab * (size_t)A * I);
    void *y = a->y ? a->y : malloc(ab * (size_t)A * H);
    void *G = malloc(ab * (size_t)A * I);
    void *U = malloc(ab * (size_t)A * I);

    orc_route(T, E, k, a->logits, a->router_bias, sel, w);
    orc_dispatch_index(T, E, k, sel, off, src, pos, rex);
    orc_copy_rows(A, ab * (size_t)H, a->x, src, values);
    if (a->fmt == 0) {
        orc_awq_project(A, H, I, values, a->adt, rex, E, a->group, a->gate_qw, a->gate_qz,
                        a->gate_s, a->sdt, a->gate_b, G, NULL);
        orc_awq_project(A, H, I, values, a->adt, rex, E, a->group, a->up_qw, a->up_qz,
                        a->up_s, a->sdt, a->up_b, U, NULL);
        orc_swiglu((size_t)A * I, G, U, a->adt, a->clamp, a->alpha, a->up_offset,
                   a->gate_one_sided, h);
        orc_awq_project(A, I, H, h, a->adt, rex, E, a->group, a->down_qw, a->down_qz,
                        a->down_s, a->sdt, a->down_b, y, NULL);
    } else {
        void *GU = malloc(ab * (size_t)A * 2 * I);
        orc_mxfp4_project(A, H, 2 * I, values, a->adt, rex, E, a->gu_blocks, a->gu_scales,
                          a->gu_bias, GU);
        /* interleaved bank: gate feature i is bank row 2i, up feature i row 2i+1 */
        for (size_t p = 0; p < (size_t)A; ++p)
            for (size_t i = 0; i < (size_t)I; ++i) {
                memcpy((char *)G + (p * I + i) * ab, (char *)GU + (p * 2 * I + 2 * i) * ab, ab);
                memcpy((char *)U + (p * I + i) * ab, (char *)GU + (p * 2 * I + 2 * i + 1) * ab, ab);
            }
        free(GU);
        orc_swiglu((size_t)A * I, G, U, a->adt, a->clamp, a->alpha, a->up_offset,
                   a->gate_one_sided, h);
        orc_mxfp4_project(A, I, H, h, a->adt, rex, E, a->dn_blocks, a->dn_scales,
                          a->dn_bias, y);
    }
    orc_combine(T, k, H, y, a->adt, w, pos, a->out);

    free(G);
    free(U);
    if (!a->selected) free(sel);
    if (!a->weights) free(w);
    if (!a->offsets) free(off);
    if (!a->row_src) free(src);
    if (!a->slot_pos) free(pos);
    if (!a->row_experts) free(rex);
    if (!a->values) free(values);
    if (!a->h) free(h);
    if (!a->y) free(y);
    return 0;
}
