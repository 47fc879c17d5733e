/*
 * Oracle for N-dimensional convolution (1 to 4 spatial dimensions): a plain,
 * slow, obviously correct CPU implementation of the definition.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark use it.  It shares no code, header
 * or constant with the GPU library.
 *
 * What it computes ("Three X's: a new level of working with large convolutions
 * in PyTorch for model training": the page's aim is convolution in more than
 * three dimensions; its section "CuBLAS" extends the 2-D convolution matrix to
 * 3-D by one more index in the linear index and one more loop over the filter,
 * and says higher dimensions follow the same way).  Channel-first tensors with
 * D spatial dimensions:
 *
 *   x  [batch][C_in][S_1]..[S_D],  w [C_out][C_in][K_1]..[K_D],
 *   y  [batch][C_out][O_1]..[O_D],  O_d = floor((S_d + 2 p_d - l_d (K_d - 1) - 1) / t_d) + 1
 *   y[n][co][o] = sum_{ci, k} x[n][ci][o t - p + k l] * w[co][ci][k]
 *
 * with o, k, t (stride), p (padding) and l (dilation) D-vectors taken
 * element-wise, image positions outside the image reading as zero, and no
 * filter flip.  Filter gradient:
 *
 *   dw[co][ci][k] = sum_{n, o} dy[n][co][o] * x[n][ci][o t - p + k l]
 *
 * Convolution matrix of image n: row (ci, k_1, .., k_D) (row-major), column
 * (o_1, .., o_D) (row-major); written as raw element bits.
 *
 * Index vectors are walked as odometers (last dimension fastest); sums run in
 * that order, ci outermost, in double precision, with S (the same sum of
 * absolute values) beside each.
 *
 * Status codes: 0 on success, -1 on an invalid argument.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { IN_F32 = 0, IN_BF16 = 1, MAXD = 4 };

/* Packed as int64: batch, cin, cout, D, then size[4], kernel[4], pad[4],
 * stride[4], dilation[4] (entries beyond D ignored). */
typedef struct {
    int64_t batch, cin, cout, nd;
    int64_t size[MAXD], kernel[MAXD], pad[MAXD], stride[MAXD], dil[MAXD];
} nd_shape;

static int64_t out_dim(int64_t in, int64_t pad, int64_t k, int64_t stride, int64_t dil)
{
    int64_t span = in + 2 * pad - dil * (k - 1) - 1;
    return span < 0 ? 0 : span / stride + 1;
}

static int check(const nd_shape *c, int64_t *out)
{
    if (c->nd < 1 || c->nd > MAXD || c->batch < 0 || c->cin < 1 || c->cout < 1) return -1;
    for (int d = 0; d < c->nd; ++d) {
        if (c->size[d] < 1 || c->kernel[d] < 1 || c->pad[d] < 0 || c->stride[d] < 1 ||
            c->dil[d] < 1)
            return -1;
        out[d] = out_dim(c->size[d], c->pad[d], c->kernel[d], c->stride[d], c->dil[d]);
        if (out[d] < 1) return -1;
    }
    return 0;
}

static int64_t prod(const int64_t *v, int64_t nd)
{
    int64_t p = 1;
    for (int d = 0; d < nd; ++d) p *= v[d];
    return p;
}

static double elem(const void *base, int kind, int64_t idx)
{
    if (kind == IN_F32) return (double)((const float *)base)[idx];
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Advance an odometer over extents ext[0..nd); returns 0 when it wraps. */
static int next(int64_t *v, const int64_t *ext, int64_t nd)
{
    for (int d = (int)nd - 1; d >= 0; --d) {
        if (++v[d] < ext[d]) return 1;
        v[d] = 0;
    }
    return 0;
}

/* Offset of the image position under tap k at output o within one channel,
 * or -1 in the padding. */
static int64_t image_off(const nd_shape *c, const int64_t *o, const int64_t *k)
{
    int64_t off = 0;
    for (int d = 0; d < c->nd; ++d) {
        const int64_t z = o[d] * c->stride[d] - c->pad[d] + k[d] * c->dil[d];
        if (z < 0 || z >= c->size[d]) return -1;
        off = off * c->size[d] + z;
    }
    return off;
}

static int64_t flat(const int64_t *v, const int64_t *ext, int64_t nd)
{
    int64_t f = 0;
    for (int d = 0; d < nd; ++d) f = f * ext[d] + v[d];
    return f;
}

static void unflat(int64_t f, int64_t *v, const int64_t *ext, int64_t nd)
{
    for (int d = (int)nd - 1; d >= 0; --d) {
        v[d] = f % ext[d];
        f /= ext[d];
    }
}

/* y and S at the positions idx[t] = flat (n, co, o) output indices. */
static int fwd_at(int kind, const int64_t *shape, const void *x, const void *w, int64_t count,
                  const int64_t *idx, double *y, double *scale)
{
    const nd_shape *c = (const nd_shape *)shape;
    int64_t O[MAXD];
    if (check(c, O) || (count > 0 && (!x || !w || !idx || !y || !scale))) return -1;
    const int64_t nd = c->nd, vol_in = prod(c->size, nd), vol_k = prod(c->kernel, nd),
                  vol_o = prod(O, nd);
    for (int64_t t = 0; t < count; ++t) {
        int64_t f = idx[t];
        if (f < 0 || f >= c->batch * c->cout * vol_o) return -1;
        int64_t o[MAXD];
        unflat(f % vol_o, o, O, nd);
        const int64_t co = (f / vol_o) % c->cout, n = f / vol_o / c->cout;
        double acc = 0.0, sc = 0.0;
        for (int64_t ci = 0; ci < c->cin; ++ci) {
            int64_t k[MAXD] = {0, 0, 0, 0};
            do {
                const int64_t off = image_off(c, o, k);
                if (off >= 0) {
                    const double v = elem(x, kind, (n * c->cin + ci) * vol_in + off);
                    const double g = elem(w, kind, (co * c->cin + ci) * vol_k + flat(k, c->kernel, nd));
                    acc += v * g;
                    sc += (v < 0 ? -v : v) * (g < 0 ? -g : g);
                }
            } while (next(k, c->kernel, nd));
        }
        y[t] = acc;
        scale[t] = sc;
    }
    return 0;
}

/* dw and S at the taps idx[t] = flat (co, ci, k) filter indices. */
static int bwdw_at(int kind, const int64_t *shape, const void *x, const void *dy, int64_t count,
                   const int64_t *idx, double *dw, double *scale)
{
    const nd_shape *c = (const nd_shape *)shape;
    int64_t O[MAXD];
    if (check(c, O) || (count > 0 && (!idx || !dw || !scale || (c->batch > 0 && (!x || !dy)))))
        return -1;
    const int64_t nd = c->nd, vol_in = prod(c->size, nd), vol_k = prod(c->kernel, nd),
                  vol_o = prod(O, nd);
    for (int64_t t = 0; t < count; ++t) {
        int64_t f = idx[t];
        if (f < 0 || f >= c->cout * c->cin * vol_k) return -1;
        int64_t k[MAXD];
        unflat(f % vol_k, k, c->kernel, nd);
        const int64_t ci = (f / vol_k) % c->cin, co = f / vol_k / c->cin;
        double acc = 0.0, sc = 0.0;
        for (int64_t n = 0; n < c->batch; ++n) {
            int64_t o[MAXD] = {0, 0, 0, 0};
            do {
                const int64_t off = image_off(c, o, k);
                if (off >= 0) {
                    const double v = elem(x, kind, (n * c->cin + ci) * vol_in + off);
                    const double g = elem(dy, kind, (n * c->cout + co) * vol_o + flat(o, O, nd));
                    acc += g * v;
                    sc += (g < 0 ? -g : g) * (v < 0 ? -v : v);
                }
            } while (next(o, O, nd));
        }
        dw[t] = acc;
        scale[t] = sc;
    }
    return 0;
}

int oracle_convnd_fwd_at_f32(const int64_t *shape, const float *x, const float *w, int64_t count,
                             const int64_t *idx, double *y, double *scale)
{
    return fwd_at(IN_F32, shape, x, w, count, idx, y, scale);
}

int oracle_convnd_fwd_at_bf16(const int64_t *shape, const uint16_t *x, const uint16_t *w,
                              int64_t count, const int64_t *idx, double *y, double *scale)
{
    return fwd_at(IN_BF16, shape, x, w, count, idx, y, scale);
}

int oracle_convnd_bwd_weight_at_f32(const int64_t *shape, const float *x, const float *dy,
                                    int64_t count, const int64_t *idx, double *dw, double *scale)
{
    return bwdw_at(IN_F32, shape, x, dy, count, idx, dw, scale);
}

int oracle_convnd_bwd_weight_at_bf16(const int64_t *shape, const uint16_t *x, const uint16_t *dy,
                                     int64_t count, const int64_t *idx, double *dw, double *scale)
{
    return bwdw_at(IN_BF16, shape, x, dy, count, idx, dw, scale);
}

/* The convolution matrix of image n (element bits), ld >= prod(O). */
static int im2col_nd(int esize, const int64_t *shape, int64_t n, const void *x, void *cols,
                     int64_t ld)
{
    const nd_shape *c = (const nd_shape *)shape;
    int64_t O[MAXD];
    if (check(c, O) || n < 0 || n >= c->batch || !x || !cols) return -1;
    const int64_t nd = c->nd, vol_in = prod(c->size, nd), vol_o = prod(O, nd);
    if (ld < vol_o) return -1;
    int64_t row = 0;
    for (int64_t ci = 0; ci < c->cin; ++ci) {
        int64_t k[MAXD] = {0, 0, 0, 0};
        do {
            int64_t o[MAXD] = {0, 0, 0, 0}, col = 0;
            do {
                const int64_t off = image_off(c, o, k);
                const int64_t src = (n * c->cin + ci) * vol_in + off, dst = row * ld + col;
                if (esize == 4)
                    ((uint32_t *)cols)[dst] = off >= 0 ? ((const uint32_t *)x)[src] : 0u;
                else
                    ((uint16_t *)cols)[dst] = off >= 0 ? ((const uint16_t *)x)[src] : 0u;
                ++col;
            } while (next(o, O, nd));
            ++row;
        } while (next(k, c->kernel, nd));
    }
    return 0;
}

int oracle_convnd_im2col_f32(const int64_t *shape, int64_t n, const float *x, float *cols,
                             int64_t ld)
{
    return im2col_nd(4, shape, n, x, cols, ld);
}

int oracle_convnd_im2col_bf16(const int64_t *shape, int64_t n, const uint16_t *x, uint16_t *cols,
                              int64_t ld)
{
    return im2col_nd(2, shape, n, x, cols, ld);
}
