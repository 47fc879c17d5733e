/*
 * Oracle for 2-D convolution: a plain, slow, obviously correct CPU
 * implementation, written as the definition (direct convolution).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark use it.  It shares no code, header
 * or constant with the GPU library.
 *
 * What it computes ("Three X's: a new level of working with large convolutions
 * in PyTorch for model training", sections "Where large convolution kernels
 * come from" and "CuBLAS"): a filter bank slides over a multi-channel image;
 * each output value is the sum, over input channels and filter taps, of the
 * filter tap times the image value under it.  Tensors are channel-first, as in
 * PyTorch (the page notes that PyTorch stores tensors channel-first):
 *
 *   x  [batch][C_in][H][W]        input image
 *   w  [C_out][C_in][R][S]        filters
 *   y  [batch][C_out][P][Q]       output
 *
 * with stride (sh, sw), zero padding (ph, pw) and dilation (dh, dw):
 *
 *   P = floor((H + 2 ph - dh (R - 1) - 1) / sh) + 1   (Q likewise)
 *   y[n][co][p][q] = sum_{ci, r, s} x[n][ci][p sh - ph + r dh][q sw - pw + s dw]
 *                                   * w[co][ci][r][s]
 *
 * where image positions outside [0, H) x [0, W) read as zero (the padding).
 * The filter is not flipped (the cross-correlation form that deep-learning
 * frameworks call convolution).
 *
 * The filter gradient, the other product the page's section on large kernels
 * is about (the gradient of a convolution is itself a convolution of the
 * input with the output gradient):
 *
 *   dw[co][ci][r][s] = sum_{n, p, q} dy[n][co][p][q]
 *                                    * x[n][ci][p sh - ph + r dh][q sw - pw + s dw]
 *
 * The convolution matrix of the page's im2col route, for one image: row
 * (ci, r, s) = (ci R + r) S + s, column (p, q) = p Q + q, holds the image value
 * that filter tap (ci, r, s) meets at output position (p, q), or 0 in the
 * padding.  oracle_im2col_* writes it as raw element bits (a copy, no
 * arithmetic).
 *
 * Sums run in the order written (ci, r, s ascending; n, p, q ascending) in
 * double precision; products of two fp32 or two bf16 values are exact in
 * double.  Alongside each sum, S (the same sum of absolute values) is the
 * scale of the tolerance test.
 *
 * Status codes: 0 on success, -1 on an invalid argument, -2 if a thread could
 * not be started.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { IN_F32 = 0, IN_BF16 = 1 };

/* Shape and hyper-parameters, in the order the Python side passes them. */
typedef struct {
    int64_t batch, cin, h, w, cout, r, s, ph, pw, sh, sw, dh, dw;
} conv_shape;

static int64_t out_dim(int64_t in, int64_t pad, int64_t k, int64_t stride, int64_t dil)
{
    int64_t span = in + 2 * pad - dil * (k - 1) - 1;
    if (span < 0) return 0;
    return span / stride + 1;
}

static int check_shape(const conv_shape *c)
{
    if (c->batch < 0 || c->cin < 1 || c->h < 1 || c->w < 1 || c->cout < 1 || c->r < 1 ||
        c->s < 1 || c->ph < 0 || c->pw < 0 || c->sh < 1 || c->sw < 1 || c->dh < 1 || c->dw < 1)
        return -1;
    if (out_dim(c->h, c->ph, c->r, c->sh, c->dh) < 1 || out_dim(c->w, c->pw, c->s, c->sw, c->dw) < 1)
        return -1;
    return 0;
}

static double elem(const void *base, int kind, int64_t idx)
{
    if (kind == IN_F32) return (double)((const float *)base)[idx];
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Image value under tap (r, s) at output (p, q) of channel ci, image n; sets
 * *inside to 0 in the padding (value 0). */
static double image_at(const conv_shape *c, const void *x, int kind, int64_t n, int64_t ci,
                       int64_t p, int64_t q, int64_t r, int64_t s, int *inside)
{
    int64_t y = p * c->sh - c->ph + r * c->dh;
    int64_t xx = q * c->sw - c->pw + s * c->dw;
    if (y < 0 || y >= c->h || xx < 0 || xx >= c->w) {
        *inside = 0;
        return 0.0;
    }
    *inside = 1;
    return elem(x, kind, ((n * c->cin + ci) * c->h + y) * c->w + xx);
}

/* One forward output value and its scale. */
static void fwd_one(const conv_shape *c, int kind, const void *x, const void *w, int64_t n,
                    int64_t co, int64_t p, int64_t q, double *out, double *scale)
{
    double acc = 0.0, sc = 0.0;
    for (int64_t ci = 0; ci < c->cin; ++ci)
        for (int64_t r = 0; r < c->r; ++r)
            for (int64_t s = 0; s < c->s; ++s) {
                int inside;
                double v = image_at(c, x, kind, n, ci, p, q, r, s, &inside);
                if (!inside) continue;
                double f = elem(w, kind, ((co * c->cin + ci) * c->r + r) * c->s + s);
                acc += v * f;
                sc += (v < 0 ? -v : v) * (f < 0 ? -f : f);
            }
    *out = acc;
    *scale = sc;
}

/* One filter-gradient value and its scale. */
static void bwdw_one(const conv_shape *c, int kind, const void *x, const void *dy, int64_t co,
                     int64_t ci, int64_t r, int64_t s, double *out, double *scale)
{
    const int64_t P = out_dim(c->h, c->ph, c->r, c->sh, c->dh);
    const int64_t Q = out_dim(c->w, c->pw, c->s, c->sw, c->dw);
    double acc = 0.0, sc = 0.0;
    for (int64_t n = 0; n < c->batch; ++n)
        for (int64_t p = 0; p < P; ++p)
            for (int64_t q = 0; q < Q; ++q) {
                int inside;
                double v = image_at(c, x, kind, n, ci, p, q, r, s, &inside);
                if (!inside) continue;
                double g = elem(dy, kind, ((n * c->cout + co) * P + p) * Q + q);
                acc += g * v;
                sc += (g < 0 ? -g : g) * (v < 0 ? -v : v);
            }
    *out = acc;
    *scale = sc;
}

/* ---------------------------------------------------------------- threads -- */

typedef struct {
    const conv_shape *c;
    int kind, which; /* which: 0 forward, 1 filter gradient */
    const void *a, *b;
    double *out, *scale;
    int64_t begin, end; /* flat output index range */
} job;

static void run_job(const job *jb)
{
    const conv_shape *c = jb->c;
    const int64_t P = out_dim(c->h, c->ph, c->r, c->sh, c->dh);
    const int64_t Q = out_dim(c->w, c->pw, c->s, c->sw, c->dw);
    for (int64_t t = jb->begin; t < jb->end; ++t) {
        if (jb->which == 0) {
            /* t = ((n * cout + co) * P + p) * Q + q */
            int64_t q = t % Q, rest = t / Q;
            int64_t p = rest % P;
            rest /= P;
            int64_t co = rest % c->cout, n = rest / c->cout;
            fwd_one(c, jb->kind, jb->a, jb->b, n, co, p, q, &jb->out[t], &jb->scale[t]);
        } else {
            /* t = ((co * cin + ci) * R + r) * S + s */
            int64_t s = t % c->s, rest = t / c->s;
            int64_t r = rest % c->r;
            rest /= c->r;
            int64_t ci = rest % c->cin, co = rest / c->cin;
            bwdw_one(c, jb->kind, jb->a, jb->b, co, ci, r, s, &jb->out[t], &jb->scale[t]);
        }
    }
}

static void *job_thread(void *arg)
{
    run_job((const job *)arg);
    return NULL;
}

static int run_parallel(const conv_shape *c, int kind, int which, const void *a, const void *b,
                        double *out, double *scale, int64_t total, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > total) nthreads = (int)(total > 0 ? total : 1);
    job *jobs = (job *)calloc((size_t)nthreads, sizeof(job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -2;
    }
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (job){c, kind, which, a, b, out, scale, total * i / nthreads,
                        total * (i + 1) / nthreads};
        if (i == nthreads - 1) break; /* the caller's thread takes the last share */
        if (pthread_create(&tids[i], NULL, job_thread, &jobs[i]) != 0) {
            rc = -2;
            break;
        }
        ++started;
    }
    if (rc == 0) run_job(&jobs[nthreads - 1]);
    for (int i = 0; i < started; ++i) pthread_join(tids[i], NULL);
    free(jobs);
    free(tids);
    return rc;
}

/* ------------------------------------------------------------- entry points -- */

static int conv_fwd(int kind, const int64_t *shape, const void *x, const void *w, double *y,
                    double *scale, int nthreads)
{
    const conv_shape *c = (const conv_shape *)shape;
    if (check_shape(c) || !y || !scale || (c->batch > 0 && (!x || !w))) return -1;
    const int64_t total = c->batch * c->cout * out_dim(c->h, c->ph, c->r, c->sh, c->dh) *
                          out_dim(c->w, c->pw, c->s, c->sw, c->dw);
    return run_parallel(c, kind, 0, x, w, y, scale, total, nthreads);
}

static int conv_bwd_weight(int kind, const int64_t *shape, const void *x, const void *dy,
                           double *dw, double *scale, int nthreads)
{
    const conv_shape *c = (const conv_shape *)shape;
    if (check_shape(c) || !dw || !scale || (c->batch > 0 && (!x || !dy))) return -1;
    const int64_t total = c->cout * c->cin * c->r * c->s;
    return run_parallel(c, kind, 1, x, dy, dw, scale, total, nthreads);
}

int oracle_conv2d_fwd_f32(const int64_t *shape, const float *x, const float *w, double *y,
                          double *scale, int nthreads)
{
    return conv_fwd(IN_F32, shape, x, w, y, scale, nthreads);
}

int oracle_conv2d_fwd_bf16(const int64_t *shape, const uint16_t *x, const uint16_t *w, double *y,
                           double *scale, int nthreads)
{
    return conv_fwd(IN_BF16, shape, x, w, y, scale, nthreads);
}

int oracle_conv2d_bwd_weight_f32(const int64_t *shape, const float *x, const float *dy,
                                 double *dw, double *scale, int nthreads)
{
    return conv_bwd_weight(IN_F32, shape, x, dy, dw, scale, nthreads);
}

int oracle_conv2d_bwd_weight_bf16(const int64_t *shape, const uint16_t *x, const uint16_t *dy,
                                  double *dw, double *scale, int nthreads)
{
    return conv_bwd_weight(IN_BF16, shape, x, dy, dw, scale, nthreads);
}

/* Forward values at `count` positions (n, co, p, q) given as four index arrays. */
static int conv_fwd_entries(int kind, const int64_t *shape, const void *x, const void *w,
                            int64_t count, const int64_t *n, const int64_t *co, const int64_t *p,
                            const int64_t *q, double *y, double *scale)
{
    const conv_shape *c = (const conv_shape *)shape;
    if (check_shape(c) || count < 0 || (count > 0 && (!x || !w || !n || !co || !p || !q || !y || !scale)))
        return -1;
    const int64_t P = out_dim(c->h, c->ph, c->r, c->sh, c->dh);
    const int64_t Q = out_dim(c->w, c->pw, c->s, c->sw, c->dw);
    for (int64_t t = 0; t < count; ++t) {
        if (n[t] < 0 || n[t] >= c->batch || co[t] < 0 || co[t] >= c->cout || p[t] < 0 || p[t] >= P ||
            q[t] < 0 || q[t] >= Q)
            return -1;
        fwd_one(c, kind, x, w, n[t], co[t], p[t], q[t], &y[t], &scale[t]);
    }
    return 0;
}

int oracle_conv2d_fwd_entries_f32(const int64_t *shape, const float *x, const float *w,
                                  int64_t count, const int64_t *n, const int64_t *co,
                                  const int64_t *p, const int64_t *q, double *y, double *scale)
{
    return conv_fwd_entries(IN_F32, shape, x, w, count, n, co, p, q, y, scale);
}

int oracle_conv2d_fwd_entries_bf16(const int64_t *shape, const uint16_t *x, const uint16_t *w,
                                   int64_t count, const int64_t *n, const int64_t *co,
                                   const int64_t *p, const int64_t *q, double *y, double *scale)
{
    return conv_fwd_entries(IN_BF16, shape, x, w, count, n, co, p, q, y, scale);
}

/* Filter-gradient values at `count` taps (co, ci, r, s). */
static int conv_bwdw_entries(int kind, const int64_t *shape, const void *x, const void *dy,
                             int64_t count, const int64_t *co, const int64_t *ci, const int64_t *r,
                             const int64_t *s, double *dw, double *scale)
{
    const conv_shape *c = (const conv_shape *)shape;
    if (check_shape(c) || count < 0 ||
        (count > 0 && (!co || !ci || !r || !s || !dw || !scale || (c->batch > 0 && (!x || !dy)))))
        return -1;
    for (int64_t t = 0; t < count; ++t) {
        if (co[t] < 0 || co[t] >= c->cout || ci[t] < 0 || ci[t] >= c->cin || r[t] < 0 ||
            r[t] >= c->r || s[t] < 0 || s[t] >= c->s)
            return -1;
        bwdw_one(c, kind, x, dy, co[t], ci[t], r[t], s[t], &dw[t], &scale[t]);
    }
    return 0;
}

int oracle_conv2d_bwd_weight_entries_f32(const int64_t *shape, const float *x, const float *dy,
                                         int64_t count, const int64_t *co, const int64_t *ci,
                                         const int64_t *r, const int64_t *s, double *dw,
                                         double *scale)
{
    return conv_bwdw_entries(IN_F32, shape, x, dy, count, co, ci, r, s, dw, scale);
}

int oracle_conv2d_bwd_weight_entries_bf16(const int64_t *shape, const uint16_t *x,
                                          const uint16_t *dy, int64_t count, const int64_t *co,
                                          const int64_t *ci, const int64_t *r, const int64_t *s,
                                          double *dw, double *scale)
{
    return conv_bwdw_entries(IN_BF16, shape, x, dy, count, co, ci, r, s, dw, scale);
}

/* The convolution matrix of image n: rows (ci, r, s), columns (p, q), leading
 * dimension ld >= P * Q; element bits copied (esize 4 or 2 bytes), zero in the
 * padding.  Columns [P*Q, ld) are left untouched. */
static int conv_im2col(int esize, const int64_t *shape, int64_t n, const void *x, void *cols,
                       int64_t ld)
{
    const conv_shape *c = (const conv_shape *)shape;
    if (check_shape(c) || n < 0 || n >= c->batch || !x || !cols) return -1;
    const int64_t P = out_dim(c->h, c->ph, c->r, c->sh, c->dh);
    const int64_t Q = out_dim(c->w, c->pw, c->s, c->sw, c->dw);
    if (ld < P * Q) return -1;
    for (int64_t ci = 0; ci < c->cin; ++ci)
        for (int64_t r = 0; r < c->r; ++r)
            for (int64_t s = 0; s < c->s; ++s) {
                const int64_t row = (ci * c->r + r) * c->s + s;
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t q = 0; q < Q; ++q) {
                        const int64_t y = p * c->sh - c->ph + r * c->dh;
                        const int64_t xx = q * c->sw - c->pw + s * c->dw;
                        const int inside = y >= 0 && y < c->h && xx >= 0 && xx < c->w;
                        const int64_t src = ((n * c->cin + ci) * c->h + y) * c->w + xx;
                        const int64_t dst = row * ld + p * Q + q;
                        if (esize == 4)
                            ((uint32_t *)cols)[dst] = inside ? ((const uint32_t *)x)[src] : 0u;
                        else
                            ((uint16_t *)cols)[dst] = inside ? ((const uint16_t *)x)[src] : 0u;
                    }
            }
    return 0;
}

int oracle_im2col_f32(const int64_t *shape, int64_t n, const float *x, float *cols, int64_t ld)
{
    return conv_im2col(4, shape, n, x, cols, ld);
}

int oracle_im2col_bf16(const int64_t *shape, int64_t n, const uint16_t *x, uint16_t *cols,
                       int64_t ld)
{
    return conv_im2col(2, shape, n, x, cols, ld);
}

/* Output size along one axis (the formula above); 0 when the filter does not
 * fit. */
int64_t oracle_conv_out_dim(int64_t in, int64_t pad, int64_t k, int64_t stride, int64_t dil)
{
    if (stride < 1 || dil < 1 || k < 1 || pad < 0 || in < 0) return -1;
    return out_dim(in, pad, k, stride, dil);
}
