/*
 * moe_oracle.c -- plain CPU oracle for one MoE layer's forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header, table or helper with the HIP library.
 *
 * What it computes, step by step, in the order the pages give:
 *   gate       logits z[t,e] = sum_i x[t,i] * Wg[e,i] (+ b[e]) in float32 --
 *              "DeepSeek 中 MoE 的同步税" (wmrh.cn), section 4.1 (gate ->
 *              softmax -> topk -> renormalise) and section 5.1 (compute the
 *              router in float32). The float32 sum is taken in one fixed order:
 *              a single fused-multiply-add chain over i = 0..d-1 starting from
 *              +0.0f. That order is the reading adopted for the bit-exact
 *              routing decision.
 *   top-k      the k experts with the largest logit, ties to the lower expert
 *              id, listed in descending order. Selecting on logits and on
 *              softmax probabilities picks the same set (softmax is strictly
 *              increasing); selecting on the float32 logits avoids exp()
 *              merging two distinct logits.
 *   weights    p = softmax over all E logits (float64), w_j = p_j / sum of the
 *              selected p -- the renormalisation of wmrh.cn section 4.1; the
 *              top-k-then-softmax form of the lpnh.cn deep dive (chapter 1,
 *              top2_gating) gives the same numbers.
 *   dispatch   counts[e], offsets (exclusive prefix sum) and the stable
 *              expert-major, token-ascending placement of every (token, slot)
 *              pair -- the reorder-and-pack step of the DeepEP notes
 *              (zzszmyf.github.io), section 7 "Dispatch", with the saved
 *              indices/locations of section 7.5(2) and no padding (7.5(4)).
 *              With a per-expert cap, assignments beyond it in token order
 *              are dropped (same notes, V3 load balancing part A).
 *   fp8        per-token min/max affine map onto OCP e4m3 -- gsyq.cn,
 *              section 3.1. Reading: centre c = (max+min)/2, half range
 *              r = (max-min)/2, v = (x - c) * (448 / r), clamp to +-448, round
 *              to nearest even; scale s = r / 448; dequantised x = q*s + c.
 *              Taken in float32 because the codes are integers decided by that
 *              arithmetic.
 *   expert FFN SwiGLU FFN_g(v) = W2_g (silu(W1_g v) * (W3_g v)), in float64.
 *   combine    y[t] = sum_s FFN_s(x[t]) + sum_j w_j FFN_{e_j}(xq[t]), float64
 *              -- gsyq.cn section 2.3 and zzszmyf.github.io section 7
 *              "Combine" (weighted sum of the k expert outputs).
 *
 * bf16 values arrive as their 16-bit patterns; a bf16 value is the float32
 * whose upper 16 bits are that pattern and whose lower 16 bits are zero.
 *
 * Every function returns 0 on success and a negative number on bad input.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1 };

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* element i of an activation/weight array stored as float32 or bf16 */
static float elem(const void *p, int dtype, int64_t i)
{
    if (dtype == OR_F32)
        return ((const float *)p)[i];
    return bf16_to_float(((const uint16_t *)p)[i]);
}

float oracle_bf16_to_float(uint16_t b) { return bf16_to_float(b); }

/* ---------------------------------------------------------------- gate ---- */

static float gate_logit(int64_t t, int e, int d, int dtype, const void *x,
                        const void *wg, const float *bias)
{
    float acc = 0.0f;
    for (int i = 0; i < d; ++i)
        acc = fmaf(elem(x, dtype, t * d + i), elem(wg, dtype, (int64_t)e * d + i), acc);
    if (bias)
        acc = acc + bias[e];
    return acc;
}

/* logits[T,E] (float32) */
int oracle_gate_logits(int64_t T, int d, int E, int dtype, const void *x,
                       const void *wg, const float *bias, float *logits,
                       int nthreads)
{
    if (T < 0 || d <= 0 || E <= 0 || (dtype != OR_F32 && dtype != OR_BF16))
        return -1;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e)
            logits[t * E + e] = gate_logit(t, e, d, dtype, x, wg, bias);
    return 0;
}

/* is (za, ia) ranked before (zb, ib)?  larger logit first, then lower id;
 * a NaN logit ranks after every number, NaNs among themselves by id */
static int ranks_before(float za, int ia, float zb, int ib)
{
    int na = isnan(za), nb = isnan(zb);
    if (na || nb)
        return na == nb ? ia < ib : nb;
    return za > zb || (za == zb && ia < ib);
}

/* top-k of one token's logits; idx[k] in rank order, w[k] float64 */
static void select_one(int E, int k, const float *z, int32_t *idx, double *w)
{
    unsigned char taken[1024];
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || ranks_before(z[e], e, z[best], best))
                best = e;
        }
        taken[best] = 1;
        idx[j] = best;
    }
    /* softmax over all E experts, then renormalise over the selected ones;
     * a NaN logit has probability 0 (it counts as -inf) */
    double zmax = -INFINITY;
    for (int e = 0; e < E; ++e)
        if (!isnan(z[e]) && (double)z[e] > zmax)
            zmax = (double)z[e];
    double Z = 0.0;
    for (int e = 0; e < E; ++e)
        if (!isnan(z[e]))
            Z += exp((double)z[e] - zmax);
    double psel = 0.0;
    double p[64];
    for (int j = 0; j < k; ++j) {
        float zj = z[idx[j]];
        p[j] = isnan(zj) ? 0.0 / Z : exp((double)zj - zmax) / Z;
        psel += p[j];
    }
    for (int j = 0; j < k; ++j)
        w[j] = p[j] / psel;
}

int oracle_select_topk(int64_t T, int E, int k, const float *logits,
                       int32_t *topk_idx, double *topk_w)
{
    if (T < 0 || E <= 0 || E > 1024 || k <= 0 || k > E || k > 64)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        select_one(E, k, logits + t * E, topk_idx + t * k, topk_w + t * k);
    return 0;
}

/* ------------------------------------------------------------ dispatch ---- */

int oracle_dispatch(int64_t T, int E, int k, const int32_t *topk_idx,
                    int32_t *counts, int32_t *offsets, int32_t *dest_row,
                    int32_t *src_token)
{
    if (T < 0 || E <= 0 || k <= 0)
        return -1;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = topk_idx[t * k + j];
            if (e < 0 || e >= E)
                return -2;
            for (int jj = 0; jj < j; ++jj)
                if (topk_idx[t * k + jj] == e)
                    return -3; /* a token may pick an expert once only */
            counts[e] += 1;
        }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!seen)
        return -4;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = topk_idx[t * k + j];
            int32_t row = offsets[e] + seen[e];
            seen[e] += 1;
            dest_row[t * k + j] = row;
            src_token[row] = (int32_t)t;
        }
    free(seen);
    return 0;
}

/*
 * Capacity-limited dispatch: the hard per-expert token cap of the DeepEP notes
 * (zzszmyf.github.io), "DeepSeek-V3 ... auxiliary-loss-free load balancing",
 * part A (hard constraint and capacity): the router still picks its top-k,
 * and once an expert holds its cap, later tokens that picked it are turned
 * away -- reassigned to the least-loaded expert of the batch, or dropped.
 *
 * First pass, in token order (ascending t; a token's k slots name distinct
 * experts, so their order within the token does not matter): an assignment
 * to an expert holding fewer than cap rows takes its next row; otherwise it
 * overflows.
 * reassign = 0: every overflowing assignment is dropped.
 * reassign = 1: then, in the same order, each overflowing assignment goes to
 * the expert with the fewest rows at that moment (ties to the lower id),
 * taking its next row, as long as some expert holds fewer than cap rows;
 * once every expert is full the rest are dropped. (Reading: "load" is the
 * rows an expert holds; the reassignment follows the whole first pass.)
 * An expert's rows are its first-pass rows in token order, then its
 * reassigned rows in that order. A dropped assignment gets dest_row = -1
 * and no row; route[t,j] (if not NULL) is the expert whose row it got, or -1.
 * counts[] are the rows per expert and offsets[] their exclusive prefix
 * sums. cap = 0 means no limit (the plain dispatch above).
 */
int oracle_dispatch_capacity(int64_t T, int E, int k, const int32_t *topk_idx,
                             int32_t cap, int reassign, int32_t *counts,
                             int32_t *offsets, int32_t *dest_row,
                             int32_t *src_token, int32_t *route)
{
    if (T < 0 || E <= 0 || k <= 0 || cap < 0)
        return -1;
    int32_t *where = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    if (!where)
        return -4;
    for (int e = 0; e < E; ++e)
        counts[e] = 0; /* rows held so far, then the kept counts */
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = topk_idx[t * k + j];
            if (e < 0 || e >= E)
                return -2;
            for (int jj = 0; jj < j; ++jj)
                if (topk_idx[t * k + jj] == e)
                    return -3;
            if (cap == 0 || counts[e] < cap) {
                dest_row[t * k + j] = counts[e]; /* rank within the expert for now */
                where[t * k + j] = e;
                counts[e] += 1;
            } else {
                dest_row[t * k + j] = -1;
                where[t * k + j] = -2; /* overflowed */
            }
        }
    for (int64_t i = 0; i < T * k; ++i) {
        if (where[i] != -2)
            continue;
        where[i] = -1;
        if (!reassign)
            continue;
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (counts[e] < cap && (best < 0 || counts[e] < counts[best]))
                best = e;
        if (best < 0)
            continue; /* every expert is full */
        dest_row[i] = counts[best];
        where[i] = best;
        counts[best] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            if (route)
                route[t * k + j] = where[t * k + j];
            if (where[t * k + j] < 0)
                continue;
            int32_t row = offsets[where[t * k + j]] + dest_row[t * k + j];
            dest_row[t * k + j] = row;
            src_token[row] = (int32_t)t;
        }
    free(where);
    return 0;
}

/* ----------------------------------------------------------------- fp8 ---- */

/* OCP e4m3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, S.1111.111 is NaN, largest finite 448, subnormals m * 2^-9 */
double oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, ex = (c >> 3) & 15, m = c & 7;
    if (ex == 15 && m == 7)
        return NAN;
    double v = ex == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), ex - 10);
    return s ? -v : v;
}

/* nearest e4m3 code to v (|v| <= 448), ties to the even code */
uint8_t oracle_e4m3_encode(float v)
{
    double a = fabs((double)v);
    int best = 0;
    double bestd = a;
    for (int c = 1; c <= 0x7e; ++c) {
        double dd = fabs(oracle_e4m3_decode((uint8_t)c) - a);
        if (dd < bestd || (dd == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = dd;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

/*
 * The affine map of the range [mn, mx] onto [-448, 448], applied to one row.
 * Per-token mode takes the row's own min/max; the per-expert and global modes
 * of gsyq.cn section 5.2 (the FP8 quantiser's three modes) take the min/max
 * over the expert's rows or over the whole batch, which contain the row.
 */
int oracle_fp8_quantize_row_range(int d, const float *xr, float mn, float mx,
                                  uint8_t *q, float *scale, float *centre)
{
    if (d <= 0 || !(mn <= mx))
        return -1;
    float c = 0.5f * (mx + mn);
    float r = 0.5f * (mx - mn);
    *centre = c;
    if (r == 0.0f) {
        memset(q, 0, (size_t)d);
        *scale = 0.0f;
        return 0;
    }
    float s = r / 448.0f;
    float inv = 448.0f / r;
    *scale = s;
    for (int i = 0; i < d; ++i) {
        float v = (xr[i] - c) * inv;
        if (v > 448.0f)
            v = 448.0f;
        if (v < -448.0f)
            v = -448.0f;
        q[i] = oracle_e4m3_encode(v);
    }
    return 0;
}

int oracle_fp8_quantize_row(int d, const float *xr, uint8_t *q, float *scale,
                            float *centre)
{
    if (d <= 0)
        return -1;
    float mn = xr[0], mx = xr[0];
    for (int i = 1; i < d; ++i) {
        if (xr[i] < mn)
            mn = xr[i];
        if (xr[i] > mx)
            mx = xr[i];
    }
    return oracle_fp8_quantize_row_range(d, xr, mn, mx, q, scale, centre);
}

/* rows [T,d] of x, each with its given range ranges[t] = (min, max); rows
 * are independent, so threads change nothing in the result */
int oracle_fp8_quantize_ranges(int64_t T, int d, int dtype, const void *x,
                               const float *ranges, uint8_t *q, float *qp,
                               int nthreads)
{
    if (T < 0 || d <= 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    int rc = 0;
#pragma omp parallel num_threads(nthreads)
    {
        float *row = (float *)malloc(sizeof(float) * (size_t)d);
#pragma omp for schedule(dynamic, 64)
        for (int64_t t = 0; t < T; ++t) {
            if (!row) {
                rc = -4;
                continue;
            }
            for (int i = 0; i < d; ++i)
                row[i] = elem(x, dtype, t * d + i);
            if (oracle_fp8_quantize_row_range(d, row, ranges[2 * t], ranges[2 * t + 1],
                                              q + t * d, &qp[2 * t], &qp[2 * t + 1]))
                rc = -1;
        }
        free(row);
    }
    return rc;
}

/* quantise rows [T,d] of x (float32 or bf16): codes [T,d], qp [T,2] = (s, c) */
int oracle_fp8_quantize(int64_t T, int d, int dtype, const void *x, uint8_t *q,
                        float *qp, int nthreads)
{
    if (T < 0 || d <= 0 || d > (1 << 20))
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    int rc = 0;
#pragma omp parallel num_threads(nthreads)
    {
        float *row = (float *)malloc(sizeof(float) * (size_t)d);
#pragma omp for schedule(dynamic, 64)
        for (int64_t t = 0; t < T; ++t) {
            if (!row) {
                rc = -4;
                continue;
            }
            for (int i = 0; i < d; ++i)
                row[i] = elem(x, dtype, t * d + i);
            oracle_fp8_quantize_row(d, row, q + t * d, &qp[2 * t], &qp[2 * t + 1]);
        }
        free(row);
    }
    return rc;
}

/* ----------------------------------------------------------- expert FFN --- */

/* out[d] = W2_g (silu(W1_g v) * (W3_g v)); v[d] float64; weights of one group:
 * w1g, w3g [h,d], w2g [d,h]; hbuf scratch [h] */
static void swiglu_ffn(int d, int h, int wdt, const double *v, const void *w1g,
                       const void *w3g, const void *w2g, double *out, double *hbuf)
{
    for (int j = 0; j < h; ++j) {
        double a = 0.0, b = 0.0;
        for (int i = 0; i < d; ++i) {
            a += (double)elem(w1g, wdt, (int64_t)j * d + i) * v[i];
            b += (double)elem(w3g, wdt, (int64_t)j * d + i) * v[i];
        }
        double silu = a / (1.0 + exp(-a));
        hbuf[j] = silu * b;
    }
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int j = 0; j < h; ++j)
            acc += (double)elem(w2g, wdt, (int64_t)i * h + j) * hbuf[j];
        out[i] = acc;
    }
}

static const void *group_ptr(const void *w, int wdt, int64_t g, int64_t elems)
{
    size_t bytes = wdt == OR_F32 ? 4 : 2;
    return (const char *)w + (size_t)(g * elems) * bytes;
}

/* apply expert group g to n rows given in float64: rows [n,d] -> out [n,d] */
int oracle_expert_rows(int d, int h, int wdt, int64_t n, const int32_t *group,
                       const double *rows, const void *w1, const void *w3,
                       const void *w2, double *out, int nthreads)
{
    if (d <= 0 || h <= 0 || n < 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    int rc = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *hbuf = (double *)malloc(sizeof(double) * (size_t)h);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            if (!hbuf) {
                rc = -4;
                continue;
            }
            int64_t g = group[r];
            swiglu_ffn(d, h, wdt, rows + r * d, group_ptr(w1, wdt, g, (int64_t)h * d),
                       group_ptr(w3, wdt, g, (int64_t)h * d),
                       group_ptr(w2, wdt, g, (int64_t)d * h), out + r * d, hbuf);
        }
        free(hbuf);
    }
    return rc;
}

/* ------------------------------------------------------- whole layer ------ */

/*
 * Full layer output for a list of tokens, each computed on its own:
 * gate -> top-k -> weights -> (fp8: quantise/dequantise the token's row for
 * the routed experts) -> y[t] = sum_s FFN_{E+s}(x[t]) + sum_j w_j FFN_{e_j}(xq).
 * route [n,k] (or NULL: the top-k experts themselves) names the expert each
 * slot's row went to under a capacity limit, -1 for a dropped slot, which
 * contributes nothing (its weight is not given to the other slots); a
 * reassigned slot keeps its gate weight. qrange [n,k,2] (or NULL: each
 * token's own min/max) gives the (min, max) range each slot's fp8 row is
 * quantised with (the per-expert or global quantiser modes).
 * Outputs per listed token: topk_idx [n,k], topk_w [n,k], y [n,d] float64.
 */
int oracle_layer_tokens(int d, int E, int k, int S, int h, int dtype, int fp8,
                        int64_t n, const int64_t *tokens, const int32_t *route,
                        const float *qrange, const void *x,
                        const void *wg, const float *bias, const void *w1,
                        const void *w3, const void *w2, int32_t *topk_idx,
                        double *topk_w, double *y, int nthreads)
{
    if (d <= 0 || E <= 0 || E > 1024 || k <= 0 || k > E || k > 64 || S < 0 || h <= 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    int rc = 0;
#pragma omp parallel num_threads(nthreads)
    {
        float *z = (float *)malloc(sizeof(float) * (size_t)E);
        float *xf = (float *)malloc(sizeof(float) * (size_t)d);
        uint8_t *q = (uint8_t *)malloc((size_t)d);
        double *v = (double *)malloc(sizeof(double) * (size_t)d);
        double *vq = (double *)malloc(sizeof(double) * (size_t)d);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        double *hbuf = (double *)malloc(sizeof(double) * (size_t)h);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            if (!z || !xf || !q || !v || !vq || !o || !hbuf) {
                rc = -4;
                continue;
            }
            int64_t t = tokens[r];
            for (int e = 0; e < E; ++e)
                z[e] = gate_logit(t, e, d, dtype, x, wg, bias);
            select_one(E, k, z, topk_idx + r * k, topk_w + r * k);
            for (int i = 0; i < d; ++i) {
                xf[i] = elem(x, dtype, t * d + i);
                v[i] = (double)xf[i];
            }
            if (fp8) {
                float s, c;
                oracle_fp8_quantize_row(d, xf, q, &s, &c);
                for (int i = 0; i < d; ++i)
                    vq[i] = oracle_e4m3_decode(q[i]) * (double)s + (double)c;
            } else {
                memcpy(vq, v, sizeof(double) * (size_t)d);
            }
            double *yr = y + r * d;
            for (int i = 0; i < d; ++i)
                yr[i] = 0.0;
            for (int s = 0; s < S; ++s) {
                int64_t g = E + s;
                swiglu_ffn(d, h, dtype, v, group_ptr(w1, dtype, g, (int64_t)h * d),
                           group_ptr(w3, dtype, g, (int64_t)h * d),
                           group_ptr(w2, dtype, g, (int64_t)d * h), o, hbuf);
                for (int i = 0; i < d; ++i)
                    yr[i] += o[i];
            }
            for (int j = 0; j < k; ++j) {
                if (route && route[r * k + j] < 0)
                    continue; /* dropped by a capacity limit */
                int64_t g = route ? route[r * k + j] : topk_idx[r * k + j];
                if (fp8 && qrange) {
                    /* per-expert or global range for this slot */
                    float s, c;
                    if (oracle_fp8_quantize_row_range(d, xf, qrange[2 * (r * k + j)],
                                                      qrange[2 * (r * k + j) + 1], q, &s, &c)) {
                        rc = -5;
                        continue;
                    }
                    for (int i = 0; i < d; ++i)
                        vq[i] = oracle_e4m3_decode(q[i]) * (double)s + (double)c;
                }
                swiglu_ffn(d, h, dtype, vq, group_ptr(w1, dtype, g, (int64_t)h * d),
                           group_ptr(w3, dtype, g, (int64_t)h * d),
                           group_ptr(w2, dtype, g, (int64_t)d * h), o, hbuf);
                for (int i = 0; i < d; ++i)
                    yr[i] += topk_w[r * k + j] * o[i];
            }
        }
        free(z); free(xf); free(q); free(v); free(vq); free(o); free(hbuf);
    }
    return rc;
}

/*
 * Combine on its own: y[t] = y_sh[t] (if given) + sum_j w[t,j] * Y[dest_row[t,j]],
 * in float64, from rows stored as float32 or bf16.
 */
int oracle_combine(int64_t T, int d, int k, int dtype, const void *y_perm,
                   const void *y_shared, const int32_t *dest_row,
                   const float *topk_w, int64_t rows, double *y)
{
    if (T < 0 || d <= 0 || k <= 0)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        double *yr = y + t * d;
        for (int i = 0; i < d; ++i)
            yr[i] = y_shared ? (double)elem(y_shared, dtype, t * d + i) : 0.0;
        for (int j = 0; j < k; ++j) {
            int64_t p = dest_row[t * k + j];
            if (p < 0 || p >= rows)
                return -2;
            double w = (double)topk_w[t * k + j];
            for (int i = 0; i < d; ++i)
                yr[i] += w * (double)elem(y_perm, dtype, p * d + i);
        }
    }
    return 0;
}

/* ------------------------------------------------------------ backward ---- */
/*
 * Backward of the layer over a list of tokens, for small sizes (every weight
 * gradient is a dense float64 array). The pages describe the backward only
 * as the forward's exchange run in reverse -- gradients return along the
 * forward's routing path (gsyq.cn section 2.4; the DeepEP notes' backward
 * pass section) -- so what it computes is the chain rule of the forward
 * above, with these readings:
 *   - the top-k choice is held fixed (it is not differentiable);
 *   - fp8 rows pass the gradient straight through (d xq / d x = 1);
 *   - a slot dropped by a capacity limit contributes no output, so its
 *     d w is 0, but it stays in the token's softmax;
 *   - the gate bias is a constant.
 * For each listed token, with g = dy[t]:
 *   shared s:  FFN_s backward with upstream g;
 *   slot j:    o_j = FFN_e(xq), d w_j = <g, o_j>, FFN_e backward with w_j g;
 *   weights:   d z_j = w_j (d w_j - sum_i w_i d w_i) for the selected experts;
 *   gate:      dWg[e_j] += d z_j x, dx += d z_j Wg[e_j].
 * FFN backward (v the input, a = W1 v, b = W3 v, s = 1/(1+e^-a),
 * hv = a s b, upstream go): dW2 += go hv^T, dhv = W2^T go,
 * da = dhv b (s + a s (1 - s)), db = dhv a s, dW1 += da v^T, dW3 += db v^T,
 * dv = W1^T da + W3^T db.
 * Outputs: dx [n,d], dtopk_w [n,k]; dwg [E,d], dw1/dw3 [E+S,h,d] and dw2
 * [E+S,d,h] are accumulated (zero them first).
 */
static void swiglu_backward(int d, int h, int wdt, const double *v, const void *w1g,
                            const void *w3g, const void *w2g, const double *go,
                            double *dw1g, double *dw3g, double *dw2g, double *dv,
                            double *a, double *b, double *hv, double *dhv)
{
    for (int j = 0; j < h; ++j) {
        double aa = 0.0, bb = 0.0;
        for (int i = 0; i < d; ++i) {
            aa += (double)elem(w1g, wdt, (int64_t)j * d + i) * v[i];
            bb += (double)elem(w3g, wdt, (int64_t)j * d + i) * v[i];
        }
        a[j] = aa;
        b[j] = bb;
        double sg = 1.0 / (1.0 + exp(-aa));
        hv[j] = aa * sg * bb;
    }
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < h; ++j)
            dw2g[(int64_t)i * h + j] += go[i] * hv[j];
    for (int j = 0; j < h; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i)
            acc += (double)elem(w2g, wdt, (int64_t)i * h + j) * go[i];
        dhv[j] = acc;
    }
    for (int i = 0; i < d; ++i)
        dv[i] = 0.0;
    for (int j = 0; j < h; ++j) {
        double sg = 1.0 / (1.0 + exp(-a[j]));
        double da = dhv[j] * b[j] * (sg + a[j] * sg * (1.0 - sg));
        double db = dhv[j] * a[j] * sg;
        for (int i = 0; i < d; ++i) {
            dw1g[(int64_t)j * d + i] += da * v[i];
            dw3g[(int64_t)j * d + i] += db * v[i];
            dv[i] += (double)elem(w1g, wdt, (int64_t)j * d + i) * da +
                     (double)elem(w3g, wdt, (int64_t)j * d + i) * db;
        }
    }
}

int oracle_layer_backward(int d, int E, int k, int S, int h, int dtype, int fp8,
                          int64_t n, const int64_t *tokens, const int32_t *route,
                          const void *x, const void *wg, const float *bias,
                          const void *w1, const void *w3, const void *w2,
                          const double *dy, double *dx, double *dtopk_w, double *dwg,
                          double *dw1, double *dw3, double *dw2)
{
    if (d <= 0 || E <= 0 || E > 1024 || k <= 0 || k > E || k > 64 || S < 0 || h <= 0)
        return -1;
    float *z = (float *)malloc(sizeof(float) * (size_t)E);
    float *xf = (float *)malloc(sizeof(float) * (size_t)d);
    uint8_t *q = (uint8_t *)malloc((size_t)d);
    double *v = (double *)malloc(sizeof(double) * (size_t)d);
    double *vq = (double *)malloc(sizeof(double) * (size_t)d);
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    double *go = (double *)malloc(sizeof(double) * (size_t)d);
    double *dv = (double *)malloc(sizeof(double) * (size_t)d);
    double *tmp = (double *)malloc(sizeof(double) * (size_t)h * 5);
    int32_t idx[64];
    double w[64], dw[64];
    int rc = 0;
    if (!z || !xf || !q || !v || !vq || !o || !go || !dv || !tmp)
        rc = -4;
    const int64_t hd = (int64_t)h * d;
    for (int64_t r = 0; r < n && rc == 0; ++r) {
        int64_t t = tokens[r];
        for (int e = 0; e < E; ++e)
            z[e] = gate_logit(t, e, d, dtype, x, wg, bias);
        select_one(E, k, z, idx, w);
        for (int i = 0; i < d; ++i) {
            xf[i] = elem(x, dtype, t * d + i);
            v[i] = (double)xf[i];
        }
        if (fp8) {
            float s, c;
            oracle_fp8_quantize_row(d, xf, q, &s, &c);
            for (int i = 0; i < d; ++i)
                vq[i] = oracle_e4m3_decode(q[i]) * (double)s + (double)c;
        } else {
            memcpy(vq, v, sizeof(double) * (size_t)d);
        }
        const double *g = dy + r * d;
        double *dxr = dx + r * d;
        for (int i = 0; i < d; ++i)
            dxr[i] = 0.0;
        for (int s = 0; s < S; ++s) {
            int64_t gi = E + s;
            swiglu_backward(d, h, dtype, v, group_ptr(w1, dtype, gi, hd), group_ptr(w3, dtype, gi, hd),
                            group_ptr(w2, dtype, gi, hd), g, dw1 + gi * hd, dw3 + gi * hd,
                            dw2 + gi * hd, dv, tmp, tmp + h, tmp + 2 * h, tmp + 3 * h);
            for (int i = 0; i < d; ++i)
                dxr[i] += dv[i];
        }
        for (int j = 0; j < k; ++j) {
            dw[j] = 0.0;
            int64_t gi = route ? route[r * k + j] : idx[j];
            if (gi < 0)
                continue; /* dropped: no output, d w = 0 */
            swiglu_ffn(d, h, dtype, vq, group_ptr(w1, dtype, gi, hd), group_ptr(w3, dtype, gi, hd),
                       group_ptr(w2, dtype, gi, hd), o, tmp);
            double acc = 0.0;
            for (int i = 0; i < d; ++i) {
                acc += g[i] * o[i];
                go[i] = w[j] * g[i];
            }
            dw[j] = acc;
            swiglu_backward(d, h, dtype, vq, group_ptr(w1, dtype, gi, hd), group_ptr(w3, dtype, gi, hd),
                            group_ptr(w2, dtype, gi, hd), go, dw1 + gi * hd, dw3 + gi * hd,
                            dw2 + gi * hd, dv, tmp, tmp + h, tmp + 2 * h, tmp + 3 * h);
            for (int i = 0; i < d; ++i)
                dxr[i] += dv[i]; /* straight through the fp8 rows */
        }
        double mean = 0.0;
        for (int j = 0; j < k; ++j) {
            dtopk_w[r * k + j] = dw[j];
            mean += w[j] * dw[j];
        }
        for (int j = 0; j < k; ++j) {
            double dz = w[j] * (dw[j] - mean);
            int e = idx[j];
            for (int i = 0; i < d; ++i) {
                dwg[(int64_t)e * d + i] += dz * v[i];
                dxr[i] += dz * (double)elem(wg, dtype, (int64_t)e * d + i);
            }
        }
    }
    free(z); free(xf); free(q); free(v); free(vq); free(o); free(go); free(dv); free(tmp);
    return rc;
}

/*
 * The backward of combine and of dispatch on their own (the exchanges the
 * pages run in reverse for the gradients: gsyq.cn section 2.4, the DeepEP
 * notes' backward pass section), in float64 from rows stored as float32 or
 * bf16:
 *   combine backward   dy_perm[dest_row[t,j]] = w[t,j] dy[t] and
 *                      dw[t,j] = <dy[t], y_perm[dest_row[t,j]]>;
 *                      the shared experts' upstream gradient is dy itself;
 *   dispatch backward  dx[t] = dx_sh[t] (if given) + sum_j dx_perm[dest_row[t,j]]
 *                      (the transpose of copying row t to k places).
 * Slots with dest_row < 0 (dropped) take and give nothing.
 */
int oracle_combine_backward(int64_t T, int d, int k, int dtype, const void *dy,
                            const void *y_perm, const int32_t *dest_row,
                            const float *topk_w, int64_t rows, double *dy_perm, double *dw)
{
    if (T < 0 || d <= 0 || k <= 0)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int64_t p = dest_row[t * k + j];
            if (p >= rows)
                return -2;
            double acc = 0.0;
            if (p >= 0)
                for (int i = 0; i < d; ++i) {
                    double g = (double)elem(dy, dtype, t * d + i);
                    dy_perm[p * d + i] = (double)topk_w[t * k + j] * g;
                    acc += g * (double)elem(y_perm, dtype, p * d + i);
                }
            dw[t * k + j] = acc;
        }
    return 0;
}

int oracle_dispatch_backward(int64_t T, int d, int k, int dtype, const void *dx_perm,
                             const void *dx_shared, const int32_t *dest_row, int64_t rows,
                             double *dx)
{
    if (T < 0 || d <= 0 || k <= 0)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        double *r = dx + t * d;
        for (int i = 0; i < d; ++i)
            r[i] = dx_shared ? (double)elem(dx_shared, dtype, t * d + i) : 0.0;
        for (int j = 0; j < k; ++j) {
            int64_t p = dest_row[t * k + j];
            if (p >= rows)
                return -2;
            if (p < 0)
                continue;
            for (int i = 0; i < d; ++i)
                r[i] += (double)elem(dx_perm, dtype, p * d + i);
        }
    }
    return 0;
}

/*
 * Backward of the gate with the top-k choice held fixed (the layer backward
 * above, its last step, on its own). The renormalised weights of a token
 * are a softmax over its k chosen logits (the full softmax's normaliser
 * cancels in p_i / sum_K p_l), so for slot j of token t
 *   dz[t,j]      = w[t,j] * (dw[t,j] - sum_l w[t,l] dw[t,l])
 * is the gradient of logit topk_idx[t,j]; every other logit gets zero.
 * Through z = x Wg^T (+ a constant bias):
 *   dx_gate[t]   = sum_j dz[t,j] Wg[topk_idx[t,j]]
 *   dwg[e]      += sum over slots (t,j) with topk_idx[t,j] = e of dz[t,j] x[t]
 * w and dw are float64; x and Wg float32 or bf16; all sums in float64.
 * dwg [E,d] is overwritten.
 */
int oracle_gate_backward(int64_t T, int d, int E, int k, int dtype, const void *x,
                         const void *wg, const int32_t *topk_idx, const double *w,
                         const double *dw, double *dz, double *dx_gate, double *dwg)
{
    if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E)
        return -1;
    for (int64_t i = 0; i < (int64_t)E * d; ++i)
        dwg[i] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        double mean = 0.0;
        for (int j = 0; j < k; ++j)
            mean += w[t * k + j] * dw[t * k + j];
        double *r = dx_gate + t * d;
        for (int i = 0; i < d; ++i)
            r[i] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = topk_idx[t * k + j];
            if (e < 0 || e >= E)
                return -2;
            double g = w[t * k + j] * (dw[t * k + j] - mean);
            dz[t * k + j] = g;
            for (int i = 0; i < d; ++i) {
                r[i] += g * (double)elem(wg, dtype, (int64_t)e * d + i);
                dwg[(int64_t)e * d + i] += g * (double)elem(x, dtype, t * d + i);
            }
        }
    }
    return 0;
}
