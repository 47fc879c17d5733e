// 2-D convolution as im2col + GEMM ("Three X's: a new level of working with
// large convolutions in PyTorch for model training", section "CuBLAS"): the
// im2col kernel writes one image's convolution matrix into the caller's
// workspace, then one GEMM of this library finishes the image.  Declared in
// include/conv.h.
//
// The im2col kernel is a copy with zero fill, bound by HBM writes (the matrix
// is C_in R S times larger than a row of outputs per tap).  Consecutive lanes
// write consecutive elements of one matrix row (256 bytes per fp32 store
// instruction, coalesced); each thread keeps the (p, q) decomposition of its
// elements across all S taps of a filter row, so the division by Q happens
// once per element and block, and the image rows it reads stay in the CU's L1
// for the S taps.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "conv.h"
#include "gemm.h"
#include "gemm_internal.hpp"

namespace dg {
namespace {

constexpr int64_t kMaxExtent = int64_t(1) << 30;   // keeps in-kernel int32 math exact
constexpr int64_t kMaxElems = int64_t(1) << 62;
constexpr int kThreads = 256;
constexpr int kEpt = 4;                            // elements per thread and tap
constexpr int64_t kLdAlign = 8;                    // matrix rows padded to 16 bytes (bf16)

struct Im2colArgs {
    const void *x;      // image n: [C_in][H][W]
    void *cols;         // [C_in R S][ld]
    int64_t ld;
    int h, w, r, s;
    int ph, pw, sh, sw, dh, dw;
    int q_out, pq;      // Q and P Q
    uint64_t q_magic;   // floor(j / Q) = (j * q_magic) >> q_shift for j < 2^31
    int q_shift;
    int jblocks;        // blocks per filter row (ci, r)
};

// Word types: the copy moves element bits, never converts.
template <int BYTES>
struct Word;
template <>
struct Word<2> {
    typedef uint16_t T;
};
template <>
struct Word<4> {
    typedef uint32_t T;
};

// Block b covers filter row (ci, r) = b / jblocks and matrix columns
// [jb * kEpt * kThreads, (jb + 1) * kEpt * kThreads), jb = b % jblocks; lane t
// owns columns jb * kEpt * kThreads + e * kThreads + t (e < kEpt), so a wave
// reads and writes 64 consecutive elements per instruction.  The thread keeps
// its columns for all S taps s of the filter row.

// Buffer-load form, used when an image channel spans less than 2 GiB.  For
// each column the taps s whose image column lies inside the image form one
// range [s_lo, s_lo + s_n) (empty when the image row is in the padding); a tap
// outside it reads from an offset past the end of the channel's buffer
// resource, which the hardware answers with zero.  Per element and tap this
// leaves an add, a compare, a select, one load and one store.
template <int ESIZE>
__global__ void __launch_bounds__(kThreads) im2col_buffer_kernel(Im2colArgs a)
{
    typedef typename Word<ESIZE>::T T;
    const int jb = (int)(blockIdx.x % (unsigned)a.jblocks);
    const int cr = (int)(blockIdx.x / (unsigned)a.jblocks);  // ci * R + r
    const int ci = cr / a.r, r = cr - ci * a.r;
    const char *img = static_cast<const char *>(a.x) + (int64_t)ci * a.h * a.w * ESIZE;
    // dword 3: the gfx9 raw-buffer format word (32-bit data format)
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(img), 0, a.h * a.w * ESIZE, 0x00020000);
    char *out = static_cast<char *>(a.cols) + (int64_t)cr * a.s * a.ld * ESIZE;

    int off[kEpt], s_lo[kEpt];
    unsigned s_n[kEpt], jo[kEpt];
    bool ok[kEpt];
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
        const int j = (jb * kEpt + e) * kThreads + (int)threadIdx.x;
        ok[e] = j < a.pq;
        const int jj = min(j, a.pq - 1);
        const int p = (int)(((uint64_t)(uint32_t)jj * a.q_magic) >> a.q_shift);
        const int q = jj - p * a.q_out;
        const int y = p * a.sh - a.ph + r * a.dh;
        const int xb = q * a.sw - a.pw;
        // taps with 0 <= xb + s * dw < w
        int lo = xb >= 0 ? 0 : (-xb + a.dw - 1) / a.dw;
        int hi = xb < a.w ? min(a.s, (a.w - 1 - xb) / a.dw + 1) : 0;
        const bool row_ok = y >= 0 && y < a.h;
        if (!row_ok || hi < lo) hi = lo;
        s_lo[e] = lo;
        s_n[e] = (unsigned)(hi - lo);
        off[e] = row_ok ? (y * a.w + xb) * ESIZE : 0;
        jo[e] = (unsigned)jj * ESIZE;
    }
    const int step = a.dw * ESIZE;
    auto taps = [&](auto check) {
        for (int s = 0; s < a.s; ++s) {
            char *dst = out + (int64_t)s * a.ld * ESIZE;
            T v[kEpt];
#pragma unroll
            for (int e = 0; e < kEpt; ++e) {
                const bool inside = (unsigned)(s - s_lo[e]) < s_n[e];
                const int vo = inside ? off[e] + s * step : (int)0x80000000u;
                if constexpr (ESIZE == 4)
                    v[e] = (T)__builtin_amdgcn_raw_buffer_load_b32(rsrc, vo, 0, 0);
                else
                    v[e] = (T)__builtin_amdgcn_raw_buffer_load_b16(rsrc, vo, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < kEpt; ++e)
                if (!decltype(check)::value || ok[e]) *reinterpret_cast<T *>(dst + jo[e]) = v[e];
        }
    };
    // every block but the last of a filter row stores all its columns
    if ((jb + 1) * kEpt * kThreads <= a.pq)
        taps(std::false_type());
    else
        taps(std::true_type());
}

// Plain-load form for any image size: clamped in-image addresses, zero
// selected in the padding.
template <int ESIZE>
__global__ void __launch_bounds__(kThreads) im2col_kernel(Im2colArgs a)
{
    typedef typename Word<ESIZE>::T T;
    const int jb = (int)(blockIdx.x % (unsigned)a.jblocks);
    const int cr = (int)(blockIdx.x / (unsigned)a.jblocks);  // ci * R + r
    const int ci = cr / a.r, r = cr - ci * a.r;
    const T *img = static_cast<const T *>(a.x) + (int64_t)ci * a.h * a.w;
    T *out = static_cast<T *>(a.cols) + (int64_t)cr * a.s * a.ld;

    int j[kEpt], xb[kEpt];
    int64_t row[kEpt];  // offset of image row y in img, or -1 when y is in the padding
    bool ok[kEpt];
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
        j[e] = (jb * kEpt + e) * kThreads + (int)threadIdx.x;
        ok[e] = j[e] < a.pq;
        // columns past P Q (never stored) take the last column's position,
        // which keeps the index math in range
        const int jj = min(j[e], a.pq - 1);
        const int p = (int)(((uint64_t)(uint32_t)jj * a.q_magic) >> a.q_shift);
        const int q = jj - p * a.q_out;
        const int y = p * a.sh - a.ph + r * a.dh;
        row[e] = (y >= 0 && y < a.h) ? (int64_t)y * a.w : -1;
        xb[e] = q * a.sw - a.pw;
    }
    for (int s = 0; s < a.s; ++s) {
        const int xoff = s * a.dw;
        T *dst = out + (int64_t)s * a.ld;
        T v[kEpt];
#pragma unroll
        for (int e = 0; e < kEpt; ++e) {
            const int x = xb[e] + xoff;
            const bool inside = row[e] >= 0 && x >= 0 && x < a.w;
            const T t = img[inside ? row[e] + x : 0];
            v[e] = inside ? t : T(0);
        }
#pragma unroll
        for (int e = 0; e < kEpt; ++e)
            if (ok[e]) dst[j[e]] = v[e];
    }
}

struct Dims {
    int64_t n, c, h, w, k, r, s, ph, pw, sh, sw, dh, dw, P, Q;
    int64_t pq() const { return P * Q; }
    int64_t crs() const { return c * r * s; }
    int64_t ld() const { return (pq() + kLdAlign - 1) / kLdAlign * kLdAlign; }
};

int64_t out_extent(int64_t in, int64_t pad, int64_t k, int64_t stride, int64_t dil)
{
    const int64_t span = in + 2 * pad - dil * (k - 1) - 1;
    return span < 0 ? 0 : span / stride + 1;
}

// a * b <= limit, for non-negative a and b, without overflow.
bool fits(int64_t a, int64_t b, int64_t limit) { return a == 0 || b <= limit / a; }

int check_dims(const conv2d_params *p, Dims *d)
{
    if (p == nullptr) return GEMM_ERR_INVALID_ARG;
    *d = Dims{p->batch, p->in_channels, p->height, p->width, p->out_channels, p->kernel_h,
              p->kernel_w, p->pad_h, p->pad_w, p->stride_h, p->stride_w, p->dilation_h,
              p->dilation_w, 0, 0};
    if (d->n < 0 || d->c < 1 || d->h < 1 || d->w < 1 || d->k < 1 || d->r < 1 || d->s < 1 ||
        d->ph < 0 || d->pw < 0 || d->sh < 1 || d->sw < 1 || d->dh < 1 || d->dw < 1)
        return GEMM_ERR_INVALID_ARG;
    const int64_t lim = kMaxExtent;
    for (int64_t v : {d->n, d->c, d->h, d->w, d->k, d->r, d->s, d->ph, d->pw, d->sh, d->sw, d->dh,
                      d->dw})
        if (v > lim) return GEMM_ERR_INVALID_ARG;
    // padded extents and dilated filter spans stay within int32 kernel math
    if (d->h + 2 * d->ph > lim || d->w + 2 * d->pw > lim || !fits(d->dh, d->r - 1, lim) ||
        !fits(d->dw, d->s - 1, lim))
        return GEMM_ERR_INVALID_ARG;
    d->P = out_extent(d->h, d->ph, d->r, d->sh, d->dh);
    d->Q = out_extent(d->w, d->pw, d->s, d->sw, d->dw);
    if (d->P < 1 || d->Q < 1) return GEMM_ERR_INVALID_ARG;
    // GEMM extents: C_out, P Q and C_in R S
    if (!fits(d->P, d->Q, lim) || !fits(d->c, d->r, lim) || !fits(d->c * d->r, d->s, lim))
        return GEMM_ERR_INVALID_ARG;
    // tensor sizes
    if (!fits(d->crs(), d->ld(), kMaxElems) || !fits(d->n, d->c, kMaxElems) ||
        !fits(d->n * d->c, d->h, kMaxElems) || !fits(d->n * d->c * d->h, d->w, kMaxElems) ||
        !fits(d->n, d->k, kMaxElems) || !fits(d->n * d->k, d->pq(), kMaxElems) ||
        !fits(d->k, d->crs(), kMaxElems))
        return GEMM_ERR_INVALID_ARG;
    return GEMM_OK;
}

int elem_size(int dtype) { return dtype == GEMM_DTYPE_F32 ? 4 : 2; }
bool valid_dtype(int dtype) { return dtype == GEMM_DTYPE_F32 || dtype == GEMM_DTYPE_BF16; }

// Constants of floor(j / d) = (j * m) >> shift, exact for 0 <= j < 2^31 and
// 1 <= d < 2^31 (the round-up multiplier: m = floor(2^(32+l) / d) + 1 with
// 2^l >= d; its error m d - 2^(32+l) lies in (0, d], and j times that stays
// below 2^(32+l) for j < 2^31).
void div_magic(uint32_t d, uint64_t *m, int *shift)
{
    int l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    *m = (uint64_t(1) << (32 + l)) / d + 1;
    *shift = 32 + l;
}

hipError_t launch_im2col(int esize, const Dims &d, const void *image, void *cols, int64_t ld,
                         hipStream_t stream)
{
    Im2colArgs a;
    a.x = image;
    a.cols = cols;
    a.ld = ld;
    a.h = (int)d.h;
    a.w = (int)d.w;
    a.r = (int)d.r;
    a.s = (int)d.s;
    a.ph = (int)d.ph;
    a.pw = (int)d.pw;
    a.sh = (int)d.sh;
    a.sw = (int)d.sw;
    a.dh = (int)d.dh;
    a.dw = (int)d.dw;
    a.q_out = (int)d.Q;
    a.pq = (int)d.pq();
    div_magic((uint32_t)d.Q, &a.q_magic, &a.q_shift);
    const int64_t per_block = (int64_t)kThreads * kEpt;
    a.jblocks = (int)((d.pq() + per_block - 1) / per_block);
    const int64_t blocks = d.c * d.r * a.jblocks;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(kThreads);
    // buffer offsets are signed 32-bit: the channel must span less than 2 GiB
    const bool buffer = d.h * d.w * esize < (int64_t(1) << 31);
    if (esize == 4) {
        if (buffer)
            hipLaunchKernelGGL(im2col_buffer_kernel<4>, grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL(im2col_kernel<4>, grid, block, 0, stream, a);
    } else {
        if (buffer)
            hipLaunchKernelGGL(im2col_buffer_kernel<2>, grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL(im2col_kernel<2>, grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

// Geometry of the implicit-GEMM loaders; the image of one batch element must
// span less than 2 GiB (buffer offsets are signed 32-bit).
int make_geom(const Dims &d, int esize, ConvGeom *g)
{
    if (d.c * d.h * d.w * esize >= (int64_t(1) << 31)) return GEMM_ERR_INVALID_ARG;
    g->h = (int)d.h;
    g->w = (int)d.w;
    g->r = (int)d.r;
    g->s = (int)d.s;
    g->ph = (int)d.ph;
    g->pw = (int)d.pw;
    g->sh = (int)d.sh;
    g->sw = (int)d.sw;
    g->dh = (int)d.dh;
    g->dw = (int)d.dw;
    g->q = (int)d.Q;
    g->pq = (int)d.pq();
    g->crs = (int)d.crs();
    div_magic((uint32_t)d.Q, &g->q_magic, &g->q_shift);
    div_magic((uint32_t)(d.r * d.s), &g->rs_magic, &g->rs_shift);
    div_magic((uint32_t)d.s, &g->s_magic, &g->s_shift);
    g->img_bytes = (int)(d.c * d.h * d.w * esize);
    return GEMM_OK;
}

int check_workspace(const Dims &d, int dtype, const void *ws, int64_t ws_bytes)
{
    if (ws == nullptr || (uintptr_t)ws % 16 != 0) return GEMM_ERR_INVALID_ARG;
    if (ws_bytes < d.crs() * d.ld() * elem_size(dtype)) return GEMM_ERR_INVALID_ARG;
    return GEMM_OK;
}

bool aligned_to(const void *p, int esize) { return (uintptr_t)p % (uintptr_t)esize == 0; }

int device_ok()
{
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_NO_DEVICE;
    }
    return GEMM_OK;
}

}  // namespace
}  // namespace dg

extern "C" {

int conv2d_output_size(const conv2d_params *p, int64_t *out_h, int64_t *out_w)
{
    dg::Dims d;
    const int rc = dg::check_dims(p, &d);
    if (rc != GEMM_OK) return rc;
    if (out_h) *out_h = d.P;
    if (out_w) *out_w = d.Q;
    return GEMM_OK;
}

int64_t conv2d_workspace_size(int dtype, const conv2d_params *p)
{
    dg::Dims d;
    if (!dg::valid_dtype(dtype)) return GEMM_ERR_INVALID_ARG;
    const int rc = dg::check_dims(p, &d);
    if (rc != GEMM_OK) return rc;
    return d.crs() * d.ld() * dg::elem_size(dtype);
}

int conv2d_im2col(int dtype, const conv2d_params *p, int64_t image, const void *x, void *cols,
                  int64_t ld_cols, hipStream_t stream)
{
    dg::Dims d;
    if (!dg::valid_dtype(dtype)) return GEMM_ERR_INVALID_ARG;
    int rc = dg::check_dims(p, &d);
    if (rc != GEMM_OK) return rc;
    const int es = dg::elem_size(dtype);
    if (image < 0 || image >= d.n || x == nullptr || cols == nullptr || ld_cols < d.pq() ||
        !dg::fits(d.crs(), ld_cols, dg::kMaxElems) || !dg::aligned_to(x, es) ||
        !dg::aligned_to(cols, es))
        return GEMM_ERR_INVALID_ARG;
    if ((rc = dg::device_ok()) != GEMM_OK) return rc;
    const char *img = static_cast<const char *>(x) + image * d.c * d.h * d.w * es;
    return dg::launch_im2col(es, d, img, cols, ld_cols, stream) == hipSuccess ? GEMM_OK
                                                                              : GEMM_ERR_HIP;
}

int conv2d_fwd(int dtype, int dtype_y, const conv2d_params *p, const void *x, const void *w,
               void *y, void *workspace, int64_t workspace_bytes, hipStream_t stream)
{
    dg::Dims d;
    if (!dg::valid_dtype(dtype) || !dg::valid_dtype(dtype_y)) return GEMM_ERR_INVALID_ARG;
    int rc = dg::check_dims(p, &d);
    if (rc != GEMM_OK) return rc;
    if (d.n == 0) return GEMM_OK;
    const int es = dg::elem_size(dtype), esy = dg::elem_size(dtype_y);
    if (x == nullptr || w == nullptr || y == nullptr || !dg::aligned_to(x, es) ||
        !dg::aligned_to(w, es) || !dg::aligned_to(y, esy))
        return GEMM_ERR_INVALID_ARG;
    if ((rc = dg::check_workspace(d, dtype, workspace, workspace_bytes)) != GEMM_OK) return rc;
    if ((rc = dg::device_ok()) != GEMM_OK) return rc;
    const int64_t ld = d.ld();
    for (int64_t n = 0; n < d.n; ++n) {
        const char *img = static_cast<const char *>(x) + n * d.c * d.h * d.w * es;
        if (dg::launch_im2col(es, d, img, workspace, ld, stream) != hipSuccess) return GEMM_ERR_HIP;
        // y[n] (C_out x PQ) = w (C_out x C_in R S) . cols (C_in R S x PQ)
        dg::GemmCall g{dtype, dtype_y, GEMM_OP_N, GEMM_OP_N, d.k, d.pq(), d.crs(), 1.0f, 0.0f,
                       w, d.crs(), workspace, ld,
                       static_cast<char *>(y) + n * d.k * d.pq() * esy, d.pq()};
        if ((rc = dg::gemm_run(g, -1, 0, stream)) != GEMM_OK) return rc;
    }
    return GEMM_OK;
}

int conv2d_bwd_weight(int dtype, const conv2d_params *p, const void *x, const void *dy, float *dw,
                      void *workspace, int64_t workspace_bytes, hipStream_t stream)
{
    dg::Dims d;
    if (!dg::valid_dtype(dtype)) return GEMM_ERR_INVALID_ARG;
    int rc = dg::check_dims(p, &d);
    if (rc != GEMM_OK) return rc;
    const int es = dg::elem_size(dtype);
    if (dw == nullptr || !dg::aligned_to(dw, 4)) return GEMM_ERR_INVALID_ARG;
    if (d.n == 0) {
        // the empty sum: dw := 0 (a GEMM with K == 0)
        dg::GemmCall g{dtype, GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_T, d.k, d.crs(), 0, 1.0f, 0.0f,
                       nullptr, 1, nullptr, 1, dw, d.crs()};
        return dg::gemm_run(g, -1, 0, stream);
    }
    if (x == nullptr || dy == nullptr || !dg::aligned_to(x, es) || !dg::aligned_to(dy, es))
        return GEMM_ERR_INVALID_ARG;
    if ((rc = dg::check_workspace(d, dtype, workspace, workspace_bytes)) != GEMM_OK) return rc;
    if ((rc = dg::device_ok()) != GEMM_OK) return rc;
    const int64_t ld = d.ld();
    for (int64_t n = 0; n < d.n; ++n) {
        const char *img = static_cast<const char *>(x) + n * d.c * d.h * d.w * es;
        if (dg::launch_im2col(es, d, img, workspace, ld, stream) != hipSuccess) return GEMM_ERR_HIP;
        // dw (C_out x C_in R S) (+)= dy[n] (C_out x PQ) . cols^T, cols stored C_in R S x PQ
        dg::GemmCall g{dtype, GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_T, d.k, d.crs(), d.pq(), 1.0f,
                       n == 0 ? 0.0f : 1.0f,
                       static_cast<const char *>(dy) + n * d.k * d.pq() * es, d.pq(),
                       workspace, ld, dw, d.crs()};
        if ((rc = dg::gemm_run(g, -1, 0, stream)) != GEMM_OK) return rc;
    }
    return GEMM_OK;
}

int conv2d_fwd_implicit(int dtype, int dtype_y, const conv2d_params *p, const void *x,
                        const void *w, void *y, hipStream_t stream)
{
    dg::Dims d;
    if (!dg::valid_dtype(dtype) || !dg::valid_dtype(dtype_y)) return GEMM_ERR_INVALID_ARG;
    int rc = dg::check_dims(p, &d);
    if (rc != GEMM_OK) return rc;
    if (d.n == 0) return GEMM_OK;
    const int es = dg::elem_size(dtype), esy = dg::elem_size(dtype_y);
    if (x == nullptr || w == nullptr || y == nullptr || !dg::aligned_to(x, es) ||
        !dg::aligned_to(w, es) || !dg::aligned_to(y, esy))
        return GEMM_ERR_INVALID_ARG;
    dg::ConvGeom geom;
    if ((rc = dg::make_geom(d, es, &geom)) != GEMM_OK) return rc;
    if ((rc = dg::device_ok()) != GEMM_OK) return rc;
    for (int64_t n = 0; n < d.n; ++n) {
        // y[n] (C_out x PQ) = w (C_out x C_in R S) . cols(x[n]), cols formed in the loader
        dg::GemmCall g{dtype, dtype_y, GEMM_OP_N, GEMM_OP_N, d.k, d.pq(), d.crs(), 1.0f, 0.0f,
                       w, d.crs(), static_cast<const char *>(x) + n * d.c * d.h * d.w * es, 1,
                       static_cast<char *>(y) + n * d.k * d.pq() * esy, d.pq(),
                       dg::B_CONV_FWD, &geom};
        if ((rc = dg::gemm_run(g, -1, 0, stream)) != GEMM_OK) return rc;
    }
    return GEMM_OK;
}

int conv2d_bwd_weight_implicit(int dtype, const conv2d_params *p, const void *x, const void *dy,
                               float *dw, hipStream_t stream)
{
    dg::Dims d;
    if (!dg::valid_dtype(dtype)) return GEMM_ERR_INVALID_ARG;
    int rc = dg::check_dims(p, &d);
    if (rc != GEMM_OK) return rc;
    const int es = dg::elem_size(dtype);
    if (dw == nullptr || !dg::aligned_to(dw, 4)) return GEMM_ERR_INVALID_ARG;
    if (d.n == 0) {
        dg::GemmCall g{dtype, GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_T, d.k, d.crs(), 0, 1.0f, 0.0f,
                       nullptr, 1, nullptr, 1, dw, d.crs()};
        return dg::gemm_run(g, -1, 0, stream);
    }
    if (x == nullptr || dy == nullptr || !dg::aligned_to(x, es) || !dg::aligned_to(dy, es))
        return GEMM_ERR_INVALID_ARG;
    dg::ConvGeom geom;
    if ((rc = dg::make_geom(d, es, &geom)) != GEMM_OK) return rc;
    if ((rc = dg::device_ok()) != GEMM_OK) return rc;
    for (int64_t n = 0; n < d.n; ++n) {
        // dw (C_out x C_in R S) (+)= dy[n] (C_out x PQ) . cols(x[n])^T
        dg::GemmCall g{dtype, GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_T, d.k, d.crs(), d.pq(), 1.0f,
                       n == 0 ? 0.0f : 1.0f,
                       static_cast<const char *>(dy) + n * d.k * d.pq() * es, d.pq(),
                       static_cast<const char *>(x) + n * d.c * d.h * d.w * es, 1, dw, d.crs(),
                       dg::B_CONV_WGRAD, &geom};
        if ((rc = dg::gemm_run(g, -1, 0, stream)) != GEMM_OK) return rc;
    }
    return GEMM_OK;
}

}  // extern "C"
