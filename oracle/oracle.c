/*
 * oracle.c -- plain double-precision reference convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU baseline leg of
 * the benchmark do.  It shares no code, header or table with the GPU library.
 *
 * What it computes (the canonical convolution, stated in our own words):
 *
 *   executorch PR #25084, "Add triton::convolution and the conv routing
 *   framework", description: one canonical convolution op with explicit
 *   padding_before / padding_after, stride, dilation and groups, and with the
 *   forward and the transposed semantics defined separately.
 *
 *   Forward (torch/_inductor/kernel/conv.py, the LOOP_BODY_2D / LOOP_BODY_3D
 *   template bodies and the group base pointers of conv2d_template): for an
 *   output position o and tap t, the input position in each spatial dimension
 *   is  o*stride - padding + t*dilation,  and the term is dropped (zero
 *   padding) when that position lies outside [0, L).  The padding before the
 *   start (padding_before) is what is subtracted; padding_after only changes
 *   the output length.  Output channel co of group g = co / (C_out/groups)
 *   reads input channels g*Cig .. g*Cig+Cig-1 and weight w[co, c, t].
 *
 *   Transposed (executorch PR #25091, "Run transposed convolutions on the
 *   implicit-GEMM template", description, second paragraph): output o reads,
 *   at tap t, input (o + padding_before - t*dilation) / stride, only when
 *   that quotient is an exact integer inside [0, L).  The weight has shape
 *   [C_in, C_out/groups, k...] and is read with its first two axes swapped,
 *   i.e. output channel j of group g, input channel c uses w[g*Cig + c, j, t].
 *
 * Output lengths (the pages print no formula; the reading used is ATen's):
 *   forward     O = floor((L + pb + pa - dil*(k-1) - 1) / s) + 1
 *   transposed  O = (L-1)*s - pb - pa + dil*(k-1) + op + 1
 *
 * Beside each output value the oracle returns A = sum |x*w| + |b| over the
 * same terms; the parity tests accept |y_gpu - y| <= eps * A.
 *
 * Loops are the definition written out: no blocking, no reordering of a
 * single element's sum beyond the natural (input channel, tap) order.
 * Threads (OpenMP) split independent (n, output channel) pairs only.
 *
 * Gradients (torch/_inductor/kernel/conv.py, convolution_backward: the
 * input, weight and bias gradients of the op).  Both the forward and the
 * transposed op are sums of terms x[n, ci, i] * w(co, c, t) over the pairs
 * (o, t) whose term reads input position i; with gy the gradient of y,
 *   dx[n, ci, i]  = sum over (co of ci's group, t, o whose term reads i) of gy[n, co, o] * w(co, c, t)
 *   dw(co, c, t)  = sum over (n, o whose term at t exists) of gy[n, co, o] * x[n, ci, i(o, t)]
 *   db[co]        = sum over (n, o) of gy[n, co, o]
 * where w(co, c, t) is the weight element the term uses (forward w[co, c, t],
 * transposed w[ci, j, t]).  Beside each gradient element the oracle returns
 * the sum of the absolute values of its terms, the bound the tests use.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct oracle_geom {
    int32_t rank;        /* spatial dims, 1..3 */
    int32_t transposed;  /* 0 forward, 1 transposed */
    int64_t N, C_in, C_out, groups;
    int64_t L[3];        /* input spatial sizes   (unused dims = 1) */
    int64_t K[3];        /* kernel spatial sizes  (unused dims = 1) */
    int64_t O[3];        /* output spatial sizes  (unused dims = 1) */
    int64_t s[3];        /* stride                (unused dims = 1) */
    int64_t pb[3];       /* padding_before        (unused dims = 0) */
    int64_t pa[3];       /* padding_after         (unused dims = 0) */
    int64_t d[3];        /* dilation              (unused dims = 1) */
    int64_t op[3];       /* output_padding        (unused dims = 0) */
} oracle_geom;

/* Output length of one spatial dimension, or -1 when it would be < 1. */
int64_t oracle_out_len(int32_t transposed, int64_t L, int64_t K, int64_t s,
                       int64_t pb, int64_t pa, int64_t d, int64_t op)
{
    int64_t O;
    if (!transposed) {
        int64_t span = L + pb + pa - d * (K - 1) - 1;
        if (span < 0) return -1;
        O = span / s + 1;
    } else {
        O = (L - 1) * s - pb - pa + d * (K - 1) + op + 1;
    }
    return O >= 1 ? O : -1;
}

/* Input position read by output position o at tap t in one dimension, or -1
 * when the term is absent (outside the input, or a non-integer quotient in
 * the transposed case). */
static int64_t src_index(int32_t transposed, int64_t o, int64_t t, int64_t L,
                         int64_t s, int64_t pb, int64_t d)
{
    int64_t i;
    if (!transposed) {
        i = o * s - pb + t * d;
    } else {
        int64_t num = o + pb - t * d;
        if (num < 0) return -1;
        if (num % s != 0) return -1;
        i = num / s;
    }
    return (i >= 0 && i < L) ? i : -1;
}

/* The output position whose term reads input position i at tap t in one
 * dimension, or -1: the exact inverse of src_index (for a forward term
 * i = o*s - pb + t*d, so o = (i + pb - t*d)/s when exact; for a transposed
 * term i = (o + pb - t*d)/s, so o = i*s - pb + t*d), limited to [0, O). */
static int64_t dst_index(int32_t transposed, int64_t i, int64_t t, int64_t O,
                         int64_t s, int64_t pb, int64_t d)
{
    int64_t o;
    if (!transposed) {
        int64_t num = i + pb - t * d;
        if (num < 0) return -1;
        if (num % s != 0) return -1;
        o = num / s;
    } else {
        o = i * s - pb + t * d;
    }
    return (o >= 0 && o < O) ? o : -1;
}

/* One output element y[n, co, o0, o1, o2] and its bound A. */
static void conv_point(const oracle_geom *g, const double *x, const double *w,
                       const double *b, int64_t n, int64_t co,
                       const int64_t o[3], double *y_out, double *a_out)
{
    const int64_t Cig = g->C_in / g->groups;
    const int64_t Cog = g->C_out / g->groups;
    const int64_t grp = co / Cog;
    const int64_t j = co % Cog;
    double sum = 0.0, asum = 0.0;

    for (int64_t c = 0; c < Cig; ++c) {
        const int64_t ci = grp * Cig + c;
        for (int64_t t0 = 0; t0 < g->K[0]; ++t0) {
            int64_t i0 = src_index(g->transposed, o[0], t0, g->L[0], g->s[0], g->pb[0], g->d[0]);
            if (i0 < 0) continue;
            for (int64_t t1 = 0; t1 < g->K[1]; ++t1) {
                int64_t i1 = src_index(g->transposed, o[1], t1, g->L[1], g->s[1], g->pb[1], g->d[1]);
                if (i1 < 0) continue;
                for (int64_t t2 = 0; t2 < g->K[2]; ++t2) {
                    int64_t i2 = src_index(g->transposed, o[2], t2, g->L[2], g->s[2], g->pb[2], g->d[2]);
                    if (i2 < 0) continue;
                    double xv = x[(((n * g->C_in + ci) * g->L[0] + i0) * g->L[1] + i1) * g->L[2] + i2];
                    double wv;
                    if (!g->transposed) /* w: [C_out, Cig, K0, K1, K2] */
                        wv = w[(((co * Cig + c) * g->K[0] + t0) * g->K[1] + t1) * g->K[2] + t2];
                    else                /* w: [C_in, Cog, K0, K1, K2], axes 0/1 swapped on read */
                        wv = w[(((ci * Cog + j) * g->K[0] + t0) * g->K[1] + t1) * g->K[2] + t2];
                    double p = xv * wv;
                    sum += p;
                    asum += fabs(p);
                }
            }
        }
    }
    if (b) {
        sum += b[co];
        asum += fabs(b[co]);
    }
    *y_out = sum;
    *a_out = asum;
}

static int geom_ok(const oracle_geom *g)
{
    if (g->rank < 1 || g->rank > 3) return 0;
    if (g->groups < 1 || g->C_in % g->groups || g->C_out % g->groups) return 0;
    for (int dd = 0; dd < 3; ++dd)
        if (g->s[dd] < 1 || g->d[dd] < 1 || g->K[dd] < 1 || g->L[dd] < 0 || g->O[dd] < 0)
            return 0;
    return 1;
}

/* Full output.  x: [N, C_in, L0, L1, L2] contiguous, y and A: [N, C_out,
 * O0, O1, O2] contiguous, b may be NULL.  nthreads <= 0 keeps OpenMP's
 * default.  Returns 0, or -1 for an inconsistent geometry. */
int oracle_conv_f64(const oracle_geom *g, const double *x, const double *w,
                    const double *b, double *y, double *A, int nthreads)
{
    if (!geom_ok(g)) return -1;
    const int64_t S = g->O[0] * g->O[1] * g->O[2];
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t pairs = g->N * g->C_out;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t n = p / g->C_out, co = p % g->C_out;
        for (int64_t f = 0; f < S; ++f) {
            int64_t o[3];
            o[2] = f % g->O[2];
            o[1] = (f / g->O[2]) % g->O[1];
            o[0] = f / (g->O[2] * g->O[1]);
            conv_point(g, x, w, b, n, co, o, &y[p * S + f], &A[p * S + f]);
        }
    }
    return 0;
}

/* Selected outputs only.  idx holds npts rows of 5 int64 values
 * (n, co, o0, o1, o2); unused spatial entries must be 0. */
int oracle_conv_points_f64(const oracle_geom *g, const double *x, const double *w,
                           const double *b, int64_t npts, const int64_t *idx,
                           double *y, double *A, int nthreads)
{
    if (!geom_ok(g)) return -1;
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t *r = idx + 5 * p;
        if (r[0] < 0 || r[0] >= g->N || r[1] < 0 || r[1] >= g->C_out) return -1;
        for (int dd = 0; dd < 3; ++dd)
            if (r[2 + dd] < 0 || r[2 + dd] >= g->O[dd]) return -1;
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t *r = idx + 5 * p;
        int64_t o[3] = {r[2], r[3], r[4]};
        conv_point(g, x, w, b, r[0], r[1], o, &y[p], &A[p]);
    }
    return 0;
}

/* Index of the weight element w(co, c, t) a term uses: forward
 * w[co, c, t], transposed w[g*Cig + c, j, t] (co = g*Cog + j). */
static int64_t w_index(const oracle_geom *g, int64_t co, int64_t c, int64_t t0, int64_t t1, int64_t t2)
{
    const int64_t Cig = g->C_in / g->groups, Cog = g->C_out / g->groups;
    const int64_t grp = co / Cog, j = co % Cog;
    if (!g->transposed) return (((co * Cig + c) * g->K[0] + t0) * g->K[1] + t1) * g->K[2] + t2;
    return ((((grp * Cig + c) * Cog + j) * g->K[0] + t0) * g->K[1] + t1) * g->K[2] + t2;
}

/* Gradients of the op for a given gradient gy of its output.  x: [N, C_in,
 * L...], w: the op's weight, gy: [N, C_out, O...], all contiguous.  dx, Adx:
 * [N, C_in, L...]; dw, Adw: w's shape; db, Adb: [C_out] (db may be NULL).
 * Returns 0, or -1 for an inconsistent geometry. */
int oracle_conv_backward_f64(const oracle_geom *g, const double *x, const double *w, const double *gy,
                             double *dx, double *Adx, double *dw, double *Adw, double *db, double *Adb,
                             int nthreads)
{
    if (!geom_ok(g)) return -1;
    const int64_t Cig = g->C_in / g->groups, Cog = g->C_out / g->groups;
    const int64_t SL = g->L[0] * g->L[1] * g->L[2];
    const int64_t SO = g->O[0] * g->O[1] * g->O[2];
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    /* dx: each input element gathers the terms that read it. */
    const int64_t xpairs = g->N * g->C_in;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < xpairs; ++p) {
        const int64_t n = p / g->C_in, ci = p % g->C_in;
        const int64_t grp = ci / Cig, c = ci % Cig;
        for (int64_t f = 0; f < SL; ++f) {
            const int64_t i2 = f % g->L[2], i1 = (f / g->L[2]) % g->L[1], i0 = f / (g->L[2] * g->L[1]);
            double sum = 0.0, asum = 0.0;
            for (int64_t j = 0; j < Cog; ++j) {
                const int64_t co = grp * Cog + j;
                for (int64_t t0 = 0; t0 < g->K[0]; ++t0) {
                    const int64_t o0 = dst_index(g->transposed, i0, t0, g->O[0], g->s[0], g->pb[0], g->d[0]);
                    if (o0 < 0) continue;
                    for (int64_t t1 = 0; t1 < g->K[1]; ++t1) {
                        const int64_t o1 = dst_index(g->transposed, i1, t1, g->O[1], g->s[1], g->pb[1], g->d[1]);
                        if (o1 < 0) continue;
                        for (int64_t t2 = 0; t2 < g->K[2]; ++t2) {
                            const int64_t o2 = dst_index(g->transposed, i2, t2, g->O[2], g->s[2], g->pb[2], g->d[2]);
                            if (o2 < 0) continue;
                            const double gv = gy[(((n * g->C_out + co) * g->O[0] + o0) * g->O[1] + o1) * g->O[2] + o2];
                            const double pr = gv * w[w_index(g, co, c, t0, t1, t2)];
                            sum += pr;
                            asum += fabs(pr);
                        }
                    }
                }
            }
            dx[p * SL + f] = sum;
            Adx[p * SL + f] = asum;
        }
    }
    /* dw: each weight element sums its terms over images and output positions. */
    const int64_t wpairs = g->C_out * Cig;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < wpairs; ++p) {
        const int64_t co = p / Cig, c = p % Cig;
        const int64_t ci = (co / Cog) * Cig + c;
        for (int64_t t0 = 0; t0 < g->K[0]; ++t0)
            for (int64_t t1 = 0; t1 < g->K[1]; ++t1)
                for (int64_t t2 = 0; t2 < g->K[2]; ++t2) {
                    double sum = 0.0, asum = 0.0;
                    for (int64_t n = 0; n < g->N; ++n)
                        for (int64_t f = 0; f < SO; ++f) {
                            const int64_t o2 = f % g->O[2], o1 = (f / g->O[2]) % g->O[1], o0 = f / (g->O[2] * g->O[1]);
                            const int64_t i0 = src_index(g->transposed, o0, t0, g->L[0], g->s[0], g->pb[0], g->d[0]);
                            const int64_t i1 = src_index(g->transposed, o1, t1, g->L[1], g->s[1], g->pb[1], g->d[1]);
                            const int64_t i2 = src_index(g->transposed, o2, t2, g->L[2], g->s[2], g->pb[2], g->d[2]);
                            if (i0 < 0 || i1 < 0 || i2 < 0) continue;
                            const double pr = gy[(n * g->C_out + co) * SO + f] *
                                              x[(((n * g->C_in + ci) * g->L[0] + i0) * g->L[1] + i1) * g->L[2] + i2];
                            sum += pr;
                            asum += fabs(pr);
                        }
                    const int64_t wi = w_index(g, co, c, t0, t1, t2);
                    dw[wi] = sum;
                    Adw[wi] = asum;
                }
    }
    /* db: the output gradient summed over images and positions. */
    if (db) {
        for (int64_t co = 0; co < g->C_out; ++co) {
            double sum = 0.0, asum = 0.0;
            for (int64_t n = 0; n < g->N; ++n)
                for (int64_t f = 0; f < SO; ++f) {
                    const double v = gy[(n * g->C_out + co) * SO + f];
                    sum += v;
                    asum += fabs(v);
                }
            db[co] = sum;
            Adb[co] = asum;
        }
    }
    return 0;
}

/* Threads an OpenMP region would use now. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
