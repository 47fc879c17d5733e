// Convolution in 1 to 4 spatial dimensions as im2col + GEMM ("Three X's: a
// new level of working with large convolutions in PyTorch for model
// training", section "CuBLAS": the convolution matrix of each image is built
// and one GEMM finishes the image; more spatial dimensions add one index to
// the matrix's row and column numbering and one loop over the filter), and
// 2-D convolution as an implicit GEMM (section "CUTLASS": the GEMM's loader
// forms the matrix tiles from the image), in 2-D and, with volume tiles, in
// 1 to 3 dimensions.  Declared in include/conv.h.
//
// The im2col kernel is a copy with zero fill, bound by HBM writes (the matrix
// holds C_in times the filter volume elements per output position).
// Consecutive lanes write consecutive elements of one matrix row (a wave
// store instruction covers 64 consecutive elements); each thread keeps the
// decomposition of its columns into output coordinates across all taps of
// the innermost filter dimension, so the divisions happen once per element
// and block, and the image rows it reads stay in the CU's L1 for those taps.
// 2-D calls run the same kernel with two spatial dimensions.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "conv.h"
#include "gemm.h"
#include "gemm_internal.hpp"

namespace dg {
namespace {

constexpr int kMaxD = 4;
constexpr int64_t kMaxExtent = int64_t(1) << 30;   // keeps in-kernel int32 math exact
constexpr int64_t kMaxElems = int64_t(1) << 62;
constexpr int kThreads = 256;
constexpr int kEpt = 4;                            // elements per thread and tap
constexpr int64_t kLdAlign = 8;                    // matrix rows padded to 16 bytes (bf16)

// Geometry of one image's convolution matrix with D spatial dimensions, the
// last one innermost (contiguous in memory).  Matrix row (ci, k_0 .. k_{D-1})
// and column (o_0 .. o_{D-1}), both numbered row-major.
struct Im2colArgs {
    const void *x;                 // image n: [C_in][size_0]..[size_{D-1}]
    void *cols;                    // [C_in * filter volume][ld]
    int64_t ld;
    int size[kMaxD], kern[kMaxD], pad[kMaxD], stride[kMaxD], dil[kMaxD], out[kMaxD];
    uint64_t out_magic[kMaxD];     // floor(j / out[d]) = (j * out_magic[d]) >> out_shift[d]
    int out_shift[kMaxD];
    int vol_out;                   // product of out: the matrix's columns
    int img_elems;                 // elements of one channel
    int groups_per_ci;             // product of kern[0 .. D-2]
    int jblocks;                   // blocks per row group (ci, k_0 .. k_{D-2})
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

__device__ __forceinline__ int magic_div(int j, uint64_t m, int shift)
{
    return (int)(((uint64_t)(uint32_t)j * m) >> shift);
}

// Row group g = (ci, k_0 .. k_{D-2}) of the block: the channel and the outer
// filter taps (kk[D-1] is unused).
template <int D>
__device__ __forceinline__ int row_group(const Im2colArgs &a, int g, int (&kk)[kMaxD])
{
    const int ci = g / a.groups_per_ci;
    int rest = g - ci * a.groups_per_ci;
#pragma unroll
    for (int d = D - 2; d >= 0; --d) {
        kk[d] = rest % a.kern[d];
        rest /= a.kern[d];
    }
    return ci;
}

// Column j -> output coordinates; for the block's outer taps kk: whether the
// outer image coordinates z_d = o_d t_d - p_d + k_d l_d (d < D-1) lie inside
// the image, the innermost start xb = o_{D-1} t - p (possibly negative), and
// the channel offset of (z_0 .. z_{D-2}, xb) (meaningful when inside; formed
// in wrapping unsigned arithmetic, since xb may be negative).
template <int D>
__device__ __forceinline__ void column_terms(const Im2colArgs &a, const int (&kk)[kMaxD], int j,
                                             bool &row_ok, int &off, int &xb)
{
    int o[kMaxD];
    int rest = j;
#pragma unroll
    for (int d = D - 1; d > 0; --d) {
        const int qd = magic_div(rest, a.out_magic[d], a.out_shift[d]);
        o[d] = rest - qd * a.out[d];
        rest = qd;
    }
    o[0] = rest;
    bool ok = true;
    unsigned u = 0;
#pragma unroll
    for (int d = 0; d < D - 1; ++d) {
        const int z = o[d] * a.stride[d] - a.pad[d] + kk[d] * a.dil[d];
        ok = ok & ((unsigned)z < (unsigned)a.size[d]);
        u = u * (unsigned)a.size[d] + (unsigned)z;
    }
    xb = o[D - 1] * a.stride[D - 1] - a.pad[D - 1];
    u = u * (unsigned)a.size[D - 1] + (unsigned)xb;
    row_ok = ok;
    off = (int)u;
}

// Block b covers row group g = b / jblocks and matrix columns
// [jb * kEpt * kThreads, (jb + 1) * kEpt * kThreads), jb = b % jblocks; lane t
// owns columns jb * kEpt * kThreads + e * kThreads + t (e < kEpt).  The thread
// writes its columns for every tap s of the innermost filter dimension
// (matrix row g * kern[D-1] + s).
//
// Buffer-load form, used when an image channel spans less than 2 GiB.  For
// each column the taps s whose innermost image coordinate lies inside the
// image form one range [s_lo, s_lo + s_n) (empty when an outer coordinate is
// in the padding); a tap outside it reads from an offset past the end of the
// channel's buffer resource, which the hardware answers with zero.  Per
// element and tap this leaves an add, a compare, a select, one load and one
// store.
template <int ESIZE, int D>
__global__ void __launch_bounds__(kThreads) im2col_buffer_kernel(Im2colArgs a)
{
    typedef typename Word<ESIZE>::T T;
    const int jb = (int)(blockIdx.x % (unsigned)a.jblocks);
    const int g = (int)(blockIdx.x / (unsigned)a.jblocks);
    int kk[kMaxD] = {0, 0, 0, 0};
    const int ci = row_group<D>(a, g, kk);
    const char *img = static_cast<const char *>(a.x) + (int64_t)ci * a.img_elems * ESIZE;
    // dword 3: the gfx9 raw-buffer format word (32-bit data format)
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(img), 0, a.img_elems * ESIZE, 0x00020000);
    const int S = a.kern[D - 1], W = a.size[D - 1], dw = a.dil[D - 1];
    char *out = static_cast<char *>(a.cols) + (int64_t)g * S * a.ld * ESIZE;

    int off[kEpt], s_lo[kEpt];
    unsigned s_n[kEpt], jo[kEpt];
    bool ok[kEpt];
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
        const int j = (jb * kEpt + e) * kThreads + (int)threadIdx.x;
        ok[e] = j < a.vol_out;
        const int jj = min(j, a.vol_out - 1);
        bool row_ok;
        int o, xb;
        column_terms<D>(a, kk, jj, row_ok, o, xb);
        // taps with 0 <= xb + s * dw < W
        const int lo = xb >= 0 ? 0 : (-xb + dw - 1) / dw;
        int hi = xb < W ? min(S, (W - 1 - xb) / dw + 1) : 0;
        if (!row_ok || hi < lo) hi = lo;
        s_lo[e] = lo;
        s_n[e] = (unsigned)(hi - lo);
        off[e] = row_ok ? o * ESIZE : 0;
        jo[e] = (unsigned)jj * ESIZE;
    }
    const int step = dw * ESIZE;
    auto taps = [&](auto check) {
        for (int s = 0; s < S; ++s) {
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
    // every block but the last of a row group stores all its columns
    if ((jb + 1) * kEpt * kThreads <= a.vol_out)
        taps(std::false_type());
    else
        taps(std::true_type());
}

// Plain-load form for any channel size: clamped in-image addresses, zero
// selected in the padding.
template <int ESIZE, int D>
__global__ void __launch_bounds__(kThreads) im2col_kernel(Im2colArgs a)
{
    typedef typename Word<ESIZE>::T T;
    const int jb = (int)(blockIdx.x % (unsigned)a.jblocks);
    const int g = (int)(blockIdx.x / (unsigned)a.jblocks);
    int kk[kMaxD] = {0, 0, 0, 0};
    const int ci = row_group<D>(a, g, kk);
    const T *img = static_cast<const T *>(a.x) + (int64_t)ci * a.img_elems;
    const int S = a.kern[D - 1], W = a.size[D - 1], dw = a.dil[D - 1];
    T *out = static_cast<T *>(a.cols) + (int64_t)g * S * a.ld;

    int j[kEpt], xb[kEpt];
    int64_t base[kEpt];  // offset of (z_0 .. z_{D-2}, 0), or -1 when an outer z is in the padding
    bool ok[kEpt];
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
        j[e] = (jb * kEpt + e) * kThreads + (int)threadIdx.x;
        ok[e] = j[e] < a.vol_out;
        bool row_ok;
        int o;
        // columns past the matrix (never stored) take the last column's
        // position, which keeps the index math in range
        column_terms<D>(a, kk, min(j[e], a.vol_out - 1), row_ok, o, xb[e]);
        base[e] = row_ok ? (int64_t)o - xb[e] : -1;
    }
    for (int s = 0; s < S; ++s) {
        T *dst = out + (int64_t)s * a.ld;
        T v[kEpt];
#pragma unroll
        for (int e = 0; e < kEpt; ++e) {
            const int x = xb[e] + s * dw;
            const bool inside = base[e] >= 0 && x >= 0 && x < W;
            const T t = img[inside ? base[e] + x : 0];
            v[e] = inside ? t : T(0);
        }
#pragma unroll
        for (int e = 0; e < kEpt; ++e)
            if (ok[e]) dst[j[e]] = v[e];
    }
}

// Shape of a convolution with nd spatial dimensions (2-D calls have nd = 2).
struct Dims {
    int64_t n, c, k, nd;
    int64_t size[kMaxD], kern[kMaxD], pad[kMaxD], stride[kMaxD], dil[kMaxD], out[kMaxD];
    int64_t vol(const int64_t *v) const
    {
        int64_t p = 1;
        for (int d = 0; d < nd; ++d) p *= v[d];
        return p;
    }
    int64_t vol_out() const { return vol(out); }
    int64_t vol_kern() const { return vol(kern); }
    int64_t img_elems() const { return vol(size); }
    int64_t crs() const { return c * vol_kern(); }
    int64_t ld() const { return (vol_out() + kLdAlign - 1) / kLdAlign * kLdAlign; }
};

int64_t out_extent(int64_t in, int64_t pad, int64_t k, int64_t stride, int64_t dil)
{
    const int64_t span = in + 2 * pad - dil * (k - 1) - 1;
    return span < 0 ? 0 : span / stride + 1;
}

// a * b <= limit, for non-negative a and b, without overflow.
bool fits(int64_t a, int64_t b, int64_t limit) { return a == 0 || b <= limit / a; }

int check_dims(Dims *d)
{
    const int64_t lim = kMaxExtent;
    if (d->nd < 1 || d->nd > kMaxD || d->n < 0 || d->c < 1 || d->k < 1 || d->n > lim ||
        d->c > lim || d->k > lim)
        return GEMM_ERR_INVALID_ARG;
    for (int i = 0; i < d->nd; ++i) {
        if (d->size[i] < 1 || d->kern[i] < 1 || d->pad[i] < 0 || d->stride[i] < 1 ||
            d->dil[i] < 1)
            return GEMM_ERR_INVALID_ARG;
        for (int64_t v : {d->size[i], d->kern[i], d->pad[i], d->stride[i], d->dil[i]})
            if (v > lim) return GEMM_ERR_INVALID_ARG;
        // padded extents and dilated filter spans stay within int32 kernel math
        if (d->size[i] + 2 * d->pad[i] > lim || !fits(d->dil[i], d->kern[i] - 1, lim))
            return GEMM_ERR_INVALID_ARG;
        d->out[i] = out_extent(d->size[i], d->pad[i], d->kern[i], d->stride[i], d->dil[i]);
        if (d->out[i] < 1) return GEMM_ERR_INVALID_ARG;
    }
    // GEMM extents (output volume, C_in times the filter volume) and the
    // elements of one channel stay within the kernels' int32 range
    int64_t vo = 1, vk = d->c, vi = 1;
    for (int i = 0; i < d->nd; ++i) {
        if (!fits(vo, d->out[i], lim) || !fits(vk, d->kern[i], lim) || !fits(vi, d->size[i], lim))
            return GEMM_ERR_INVALID_ARG;
        vo *= d->out[i];
        vk *= d->kern[i];
        vi *= d->size[i];
    }
    // tensor sizes
    if (!fits(d->crs(), d->ld(), kMaxElems) || !fits(d->n * d->c, vi, kMaxElems) ||
        !fits(d->n * d->k, vo, kMaxElems) || !fits(d->k, d->crs(), kMaxElems))
        return GEMM_ERR_INVALID_ARG;
    return GEMM_OK;
}

int dims_2d(const conv2d_params *p, Dims *d)
{
    if (p == nullptr) return GEMM_ERR_INVALID_ARG;
    *d = Dims{p->batch, p->in_channels, p->out_channels, 2,
              {p->height, p->width}, {p->kernel_h, p->kernel_w}, {p->pad_h, p->pad_w},
              {p->stride_h, p->stride_w}, {p->dilation_h, p->dilation_w}, {0, 0}};
    return check_dims(d);
}

int dims_nd(const convnd_params *p, Dims *d)
{
    if (p == nullptr || p->ndim < 1 || p->ndim > kMaxD) return GEMM_ERR_INVALID_ARG;
    *d = Dims{};
    d->n = p->batch;
    d->c = p->in_channels;
    d->k = p->out_channels;
    d->nd = p->ndim;
    for (int i = 0; i < p->ndim; ++i) {
        d->size[i] = p->size[i];
        d->kern[i] = p->kernel[i];
        d->pad[i] = p->pad[i];
        d->stride[i] = p->stride[i];
        d->dil[i] = p->dilation[i];
    }
    return check_dims(d);
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

template <int D>
void launch_d(int esize, bool buffer, dim3 grid, hipStream_t stream, const Im2colArgs &a)
{
    const dim3 block(kThreads);
    if (esize == 4) {
        if (buffer)
            hipLaunchKernelGGL((im2col_buffer_kernel<4, D>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((im2col_kernel<4, D>), grid, block, 0, stream, a);
    } else {
        if (buffer)
            hipLaunchKernelGGL((im2col_buffer_kernel<2, D>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((im2col_kernel<2, D>), grid, block, 0, stream, a);
    }
}

hipError_t launch_im2col(int esize, const Dims &d, const void *image, void *cols, int64_t ld,
                         hipStream_t stream)
{
    Im2colArgs a{};
    a.x = image;
    a.cols = cols;
    a.ld = ld;
    for (int i = 0; i < d.nd; ++i) {
        a.size[i] = (int)d.size[i];
        a.kern[i] = (int)d.kern[i];
        a.pad[i] = (int)d.pad[i];
        a.stride[i] = (int)d.stride[i];
        a.dil[i] = (int)d.dil[i];
        a.out[i] = (int)d.out[i];
        div_magic((uint32_t)d.out[i], &a.out_magic[i], &a.out_shift[i]);
    }
    a.vol_out = (int)d.vol_out();
    a.img_elems = (int)d.img_elems();
    a.groups_per_ci = (int)(d.vol_kern() / d.kern[d.nd - 1]);
    const int64_t per_block = (int64_t)kThreads * kEpt;
    a.jblocks = (int)((d.vol_out() + per_block - 1) / per_block);
    const int64_t blocks = d.c * a.groups_per_ci * a.jblocks;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    // buffer offsets are signed 32-bit: the channel must span less than 2 GiB
    const bool buffer = d.img_elems() * esize < (int64_t(1) << 31);
    const dim3 grid((unsigned)blocks);
    switch (d.nd) {
    case 1: launch_d<1>(esize, buffer, grid, stream, a); break;
    case 2: launch_d<2>(esize, buffer, grid, stream, a); break;
    case 3: launch_d<3>(esize, buffer, grid, stream, a); break;
    default: launch_d<4>(esize, buffer, grid, stream, a); break;
    }
    return hipGetLastError();
}

// Geometry of the implicit-GEMM loaders (2-D only); the image of one batch
// element must span less than 2 GiB (buffer offsets are signed 32-bit).
int make_geom(const Dims &d, int esize, ConvGeom *g)
{
    if (d.nd != 2 || d.c * d.img_elems() * esize >= (int64_t(1) << 31))
        return GEMM_ERR_INVALID_ARG;
    g->h = (int)d.size[0];
    g->w = (int)d.size[1];
    g->r = (int)d.kern[0];
    g->s = (int)d.kern[1];
    g->ph = (int)d.pad[0];
    g->pw = (int)d.pad[1];
    g->sh = (int)d.stride[0];
    g->sw = (int)d.stride[1];
    g->dh = (int)d.dil[0];
    g->dw = (int)d.dil[1];
    g->q = (int)d.out[1];
    g->pq = (int)d.vol_out();
    g->crs = (int)d.crs();
    div_magic((uint32_t)d.out[1], &g->q_magic, &g->q_shift);
    div_magic((uint32_t)(d.kern[0] * d.kern[1]), &g->rs_magic, &g->rs_shift);
    div_magic((uint32_t)d.kern[1], &g->s_magic, &g->s_shift);
    g->img_bytes = (int)(d.c * d.img_elems() * esize);
    return GEMM_OK;
}

// Geometry of the volume implicit-GEMM loaders for 1 to 4 spatial dimensions.
// The loaders see four (u, z, y, x); fewer get leading unit dimensions (size,
// filter, stride and dilation 1, no padding), which changes nothing.  The
// three-dimensional sources read only (z, y, x); the four-dimensional ones
// (nd = 4) also the outermost u.  The image of one batch element must span
// less than 2 GiB.
int make_geom3(const Dims &d, int esize, ConvGeom *g)
{
    if (d.nd > 4 || d.c * d.img_elems() * esize >= (int64_t(1) << 31)) return GEMM_ERR_INVALID_ARG;
    const int lead = 4 - (int)d.nd;
    int64_t size[4], kern[4], pad[4], stride[4], dil[4], out[4];
    for (int i = 0; i < 4; ++i) {
        const bool unit = i < lead;
        const int j = i - lead;
        size[i] = unit ? 1 : d.size[j];
        kern[i] = unit ? 1 : d.kern[j];
        pad[i] = unit ? 0 : d.pad[j];
        stride[i] = unit ? 1 : d.stride[j];
        dil[i] = unit ? 1 : d.dil[j];
        out[i] = unit ? 1 : d.out[j];
    }
    *g = ConvGeom{};
    g->du = (int)size[0];
    g->d = (int)size[1];
    g->h = (int)size[2];
    g->w = (int)size[3];
    g->ku = (int)kern[0];
    g->t = (int)kern[1];
    g->r = (int)kern[2];
    g->s = (int)kern[3];
    g->pu = (int)pad[0];
    g->pz = (int)pad[1];
    g->ph = (int)pad[2];
    g->pw = (int)pad[3];
    g->su = (int)stride[0];
    g->sz = (int)stride[1];
    g->sh = (int)stride[2];
    g->sw = (int)stride[3];
    g->lu = (int)dil[0];
    g->lz = (int)dil[1];
    g->dh = (int)dil[2];
    g->dw = (int)dil[3];
    g->p = (int)out[2];
    g->q = (int)out[3];
    g->pq = (int)(out[2] * out[3]);
    g->opq = (int)(out[1] * out[2] * out[3]);
    g->crs = (int)d.crs();
    div_magic((uint32_t)out[3], &g->q_magic, &g->q_shift);
    div_magic((uint32_t)(out[2] * out[3]), &g->pq_magic, &g->pq_shift);
    div_magic((uint32_t)(out[1] * out[2] * out[3]), &g->opq_magic, &g->opq_shift);
    div_magic((uint32_t)(kern[2] * kern[3]), &g->rs_magic, &g->rs_shift);
    div_magic((uint32_t)(kern[1] * kern[2] * kern[3]), &g->trs_magic, &g->trs_shift);
    div_magic((uint32_t)(kern[0] * kern[1] * kern[2] * kern[3]), &g->ktrs_magic, &g->ktrs_shift);
    div_magic((uint32_t)kern[3], &g->s_magic, &g->s_shift);
    g->img_bytes = (int)(d.c * d.img_elems() * esize);
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

// ------------------------------------------- implicit GEMM: term tables --

// Table of the implicit GEMM's per-k terms, one entry per k: for the forward
// product k is a tap (ci, r, s) with y = r dh, x = s dw and the byte offset of
// (ci, y, x) in the image; for the filter gradient k is an output position
// (p, q) with y = p sh - ph, x = q sw - pw and the (possibly negative) byte
// offset of (y, x).  Entry {y | x << 16, offset} (y and x as signed 16-bit).
__global__ void __launch_bounds__(kThreads) conv_table_kernel(ConvGeom g, int fwd, int esize,
                                                              int count, int2 *tab)
{
    const int k = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (k >= count) return;
    int y, x, off;
    if (fwd) {
        const int ci = k / (g.r * g.s);
        const int rem = k - ci * g.r * g.s;
        const int r = rem / g.s, sx = rem - r * g.s;
        y = r * g.dh;
        x = sx * g.dw;
        off = ((ci * g.h + y) * g.w + x) * esize;
    } else {
        const int p = k / g.q, q = k - p * g.q;
        y = p * g.sh - g.ph;
        x = q * g.sw - g.pw;
        off = (y * g.w + x) * esize;
    }
    tab[k] = make_int2((int)(((unsigned)y & 0xffffu) | ((unsigned)x << 16)), off);
}

// The table's y and x fit in signed 16 bits.
bool table_fits(const Dims &d, bool fwd)
{
    const int64_t lo = -32768, hi = 32767;
    if (fwd)
        return (d.kern[0] - 1) * d.dil[0] <= hi && (d.kern[1] - 1) * d.dil[1] <= hi;
    return -d.pad[0] >= lo && -d.pad[1] >= lo && (d.out[0] - 1) * d.stride[0] - d.pad[0] <= hi &&
           (d.out[1] - 1) * d.stride[1] - d.pad[1] <= hi;
}

// Table addressing of one implicit call: writes the per-k terms into the
// library's table buffer for this stream, points the geometry at it and
// gives the bsrc to launch with.  The caller has checked table_fits.
int table_source(int esize, bool fwd, ConvGeom *geom, hipStream_t stream, int *bsrc)
{
    const int count = fwd ? geom->crs : geom->pq;
    void *buf = nullptr;
    const int rc = conv_table_buffer(stream, (size_t)count * sizeof(int2), &buf);
    if (rc != GEMM_OK) return rc;
    hipLaunchKernelGGL(conv_table_kernel, dim3((unsigned)((count + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, *geom, fwd ? 1 : 0, esize, count,
                       static_cast<int2 *>(buf));
    if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
    geom->tab = static_cast<const int2 *>(buf);
    *bsrc = fwd ? B_CONV_FWD_TAB : B_CONV_WGRAD_TAB;
    return GEMM_OK;
}

int zero_dw(int dtype, const Dims &d, float *dw, hipStream_t stream);

// Spatial dimensions of the padded implicit sources -- outermost (1 below four
// dimensions), depth (1 for 2-D), rows, columns -- their paddings, and the
// padded extents.
struct PadDims {
    int u, d, h, w, pu, pz, ph, pw, up, dp, hp, wp;
};

// Zero-padded copy of one image for the padded implicit sources: dst
// [C][U + 2 pu][D + 2 pz][H + 2 ph][W + 2 pw] (U = 1, pu = 0 below four
// dimensions; D = 1, pz = 0 for 2-D) holds the image with zero borders, so that
// every position a tile touches lies inside it.  One element per thread,
// consecutive threads along the padded rows.
template <int ESIZE>
__global__ void __launch_bounds__(kThreads) conv_pad_kernel(const void *src, void *dst, int total,
                                                            PadDims p)
{
    typedef typename Word<ESIZE>::T T;
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= total) return;
    const int xp = i % p.wp;
    int t = i / p.wp;
    const int yp = t % p.hp;
    t /= p.hp;
    const int zp = t % p.dp;
    t /= p.dp;
    const int up = t % p.up;
    const int c = t / p.up;
    const int u = up - p.pu, z = zp - p.pz, y = yp - p.ph, x = xp - p.pw;
    const bool in = ((unsigned)u < (unsigned)p.u) & ((unsigned)z < (unsigned)p.d) &
                    ((unsigned)y < (unsigned)p.h) & ((unsigned)x < (unsigned)p.w);
    const T *s = static_cast<const T *>(src);
    static_cast<T *>(dst)[i] = in ? s[(((int64_t)(c * p.u + u) * p.d + z) * p.h + y) * p.w + x] : T(0);
}

// Filters with every filter row padded from S to S' taps, for the image-window
// source: dst[co][row][s] = src[co][row][s] for s < S, 0 for S <= s < S'
// (rows = C_in R).  One element per thread.
template <int ESIZE>
__global__ void __launch_bounds__(kThreads) conv_filter_pad_kernel(const void *src, void *dst,
                                                                   int total, int s, int sp)
{
    typedef typename Word<ESIZE>::T T;
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= total) return;
    const int row = i / sp, tap = i - row * sp;
    static_cast<T *>(dst)[i] = tap < s ? static_cast<const T *>(src)[(int64_t)row * s + tap] : T(0);
}

// The inverse for the fp32 filter gradient: dst[row][s] = src[row][s], s < S,
// rows of S' in src, of S in dst.
__global__ void __launch_bounds__(kThreads) conv_filter_unpad_kernel(const float *src, float *dst,
                                                                     int total, int s, int sp)
{
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= total) return;
    const int row = i / s, tap = i - row * s;
    dst[i] = src[(int64_t)row * sp + tap];
}

PadDims pad_dims(const Dims &d)
{
    const int lead = 4 - (int)d.nd;  // 2-D: two leading unit dimensions
    auto at = [&](const int64_t *v, int i, int64_t unit) {
        return (int)(i < lead ? unit : v[i - lead]);
    };
    PadDims p;
    p.u = at(d.size, 0, 1);
    p.d = at(d.size, 1, 1);
    p.h = at(d.size, 2, 1);
    p.w = at(d.size, 3, 1);
    p.pu = at(d.pad, 0, 0);
    p.pz = at(d.pad, 1, 0);
    p.ph = at(d.pad, 2, 0);
    p.pw = at(d.pad, 3, 0);
    p.up = p.u + 2 * p.pu;
    p.dp = p.d + 2 * p.pz;
    p.hp = p.h + 2 * p.ph;
    p.wp = p.w + 2 * p.pw;
    return p;
}

// Bytes of one padded image (C_in times the padded volume), or -1 when it
// would reach 2 GiB (buffer offsets are signed 32-bit).
int64_t padded_bytes(const Dims &d, int esize)
{
    const PadDims p = pad_dims(d);
    const int64_t elems = d.c * (int64_t)p.up * p.dp * p.hp * p.wp;
    return elems * esize < (int64_t(1) << 31) ? elems * esize : -1;
}

// Geometry of the image-window source for a 2-D forward product (see
// ConvWindow in gemm_kernel.hpp), for the tile entry the dispatcher picks for
// C_out output channels.  False when the product does not qualify: it needs
// unit horizontal stride and dilation, S' (S rounded up to a 16-byte slot) must
// divide the k-tile, and one k-tile's window -- NP = BK / S' filter rows of NR
// output rows x W' slots each, rounded up to the thread count -- must fit the
// entry's B stage (BN x BK elements).  *pref: the window pays -- the zero taps
// add at most a quarter to the product (S' <= 5/4 S) and the window is at most
// half the stage (the gather it replaces reads the whole stage per k-tile).
bool window_geom(int dtype, const Dims &d, const PadDims &pd, int64_t pbytes, ConvGeom *g,
                 bool *pref)
{
    *pref = false;
    if (d.nd != 2 || d.stride[1] != 1 || d.dil[1] != 1 || pbytes <= 0) return false;
    const int es = elem_size(dtype), ks = 16 / es;
    int bn = 0, bk = 0, threads = 0;
    if (implicit_tile(dtype, d.k, &bn, &bk, &threads) != GEMM_OK) return false;
    const int64_t S = d.kern[1], sp = (S + ks - 1) / ks * ks;
    if (bk % sp != 0) return false;
    const int64_t P = d.out[0], Q = d.out[1];
    // output rows spanned by one block's BN positions (blocks start at
    // multiples of BN)
    int64_t nr = bn % Q == 0 ? bn / Q : Q % bn == 0 ? 1 : (bn - 1) / Q + 2;
    nr = std::min(nr, P);
    const int64_t np = bk / sp;
    const int64_t nrwp = (nr * pd.wp + threads - 1) / threads * threads;
    const int64_t stage_slots = (int64_t)bn * bk * es / 16;
    if (np * nrwp > stage_slots) return false;
    // K' = C_in R S' a valid k extent; offsets of the rows past the last output
    // row (loaded, never read) still in 32 bits
    const int64_t cr = d.c * d.kern[0];
    if (cr * sp >= (int64_t(1) << 31) ||
        (d.c * pd.hp + (P + nr) * d.stride[0] + d.kern[0] * d.dil[0]) * pd.wp * es >=
            (int64_t(1) << 31))
        return false;
    *g = ConvGeom{};
    g->h = pd.hp;
    g->w = pd.wp;
    g->r = (int)d.kern[0];
    g->s = (int)S;
    g->sh = (int)d.stride[0];
    g->dh = (int)d.dil[0];
    g->q = (int)Q;
    g->pq = (int)(P * Q);
    g->sp = (int)sp;
    g->cr = (int)cr;
    g->nr = (int)nr;
    g->img_bytes = (int)pbytes;
    div_magic((uint32_t)Q, &g->q_magic, &g->q_shift);
    div_magic((uint32_t)sp, &g->sp_magic, &g->sp_shift);
    div_magic((uint32_t)d.kern[0], &g->r_magic, &g->r_shift);
    div_magic((uint32_t)pd.wp, &g->w_magic, &g->w_shift);
    *pref = 4 * sp <= 5 * S && 2 * np * nrwp <= stage_slots;
    return true;
}

// Geometry of the image-window source for a 2-D filter gradient (see
// ConvWindowW in gemm_kernel.hpp), for the entry the dispatcher picks for C_out
// output channels: unit horizontal stride and dilation, S' dividing BN (a
// block's columns are whole filter rows), and per k-tile BN / S' window rows
// of BK + S' - 1 slots, each rounded up to the thread count, within the
// entry's staging registers.  Output rows are padded to Q' = Q rounded up to
// BK.  *pref: bf16 (measured on 31-wide filters: bf16 25% faster than the
// padded gather, fp32 3% slower), the padding adds at most a quarter
// (S' <= 5/4 S, Q' <= 5/4 Q) and the window holds at most half the B stage.
bool window_geom_w(int dtype, const Dims &d, const PadDims &pd, int64_t pbytes, ConvGeom *g,
                   bool *pref)
{
    *pref = false;
    if (d.nd != 2 || d.stride[1] != 1 || d.dil[1] != 1 || pbytes <= 0) return false;
    const int es = elem_size(dtype), ks = 16 / es;
    int bn = 0, bk = 0, threads = 0;
    if (implicit_tile(dtype, d.k, &bn, &bk, &threads) != GEMM_OK) return false;
    const int64_t S = d.kern[1], sp = (S + ks - 1) / ks * ks;
    if (bn % sp != 0) return false;
    const int64_t P = d.out[0], Q = d.out[1], qp = (Q + bk - 1) / bk * bk;
    const int64_t len = bk + sp - 1, vrows = (len + threads - 1) / threads;
    const int64_t stage_slots = (int64_t)bn * bk * es / 16;
    if ((bn / sp) * vrows * threads > stage_slots) return false;
    const int64_t cr = d.c * d.kern[0];
    if (cr * sp >= (int64_t(1) << 31) || P * qp >= (int64_t(1) << 31) ||
        d.k * P * qp * es >= (int64_t(1) << 31) ||
        (d.c * pd.hp * pd.wp + len + bk) * es >= (int64_t(1) << 31))
        return false;
    *g = ConvGeom{};
    g->h = pd.hp;
    g->w = pd.wp;
    g->r = (int)d.kern[0];
    g->s = (int)S;
    g->sh = (int)d.stride[0];
    g->dh = (int)d.dil[0];
    g->q = (int)Q;
    g->sp = (int)sp;
    g->cr = (int)cr;
    g->qp = (int)qp;
    g->img_bytes = (int)pbytes;
    div_magic((uint32_t)sp, &g->sp_magic, &g->sp_shift);
    div_magic((uint32_t)d.kern[0], &g->r_magic, &g->r_shift);
    div_magic((uint32_t)qp, &g->qp_magic, &g->qp_shift);
    *pref = es == 2 && 4 * sp <= 5 * S && 4 * qp <= 5 * Q && 2 * (bn / sp) * len <= stage_slots;
    return true;
}

// One implicit-GEMM convolution call (2-D or volume), forward (a = w, out = y)
// or filter gradient (a = dy, out = dw, fp32): checks, addressing, per-image
// GEMMs.  CONV_ADDR_DEFAULT takes the image-window form where it applies (2-D,
// unit horizontal stride and dilation, window within the B stage) and pays
// (window_geom, window_geom_w), else the padded form when the padded image
// fits, else the analytic one;
// CONV_ADDR_WINDOW runs the padded form where the window does not apply; the
// table form is 2-D only.
int run_implicit(int dtype, int dtype_out, const Dims &d, int addressing, bool fwd, bool vol,
                 const void *x, const void *a, void *out, hipStream_t stream)
{
    const int es = elem_size(dtype), eso = elem_size(dtype_out);
    if (fwd && d.n == 0) return GEMM_OK;
    if (out == nullptr || !aligned_to(out, eso)) return GEMM_ERR_INVALID_ARG;
    if (d.n == 0) return zero_dw(dtype, d, static_cast<float *>(out), stream);
    if (x == nullptr || a == nullptr || !aligned_to(x, es) || !aligned_to(a, es))
        return GEMM_ERR_INVALID_ARG;
    ConvGeom geom{};
    const bool four = vol && d.nd == 4;  // the four-dimensional sources
    int rc = vol ? make_geom3(d, es, &geom) : make_geom(d, es, &geom);
    if (rc != GEMM_OK) return rc;
    const int64_t pbytes = padded_bytes(d, es);
    const PadDims pd = pad_dims(d);
    ConvGeom wgeom;
    bool window_pref = false;
    const bool window =
        !vol && (fwd ? window_geom(dtype, d, pd, pbytes, &wgeom, &window_pref)
                     : window_geom_w(dtype, d, pd, pbytes, &wgeom, &window_pref));
    int mode = addressing;
    if (mode == CONV_ADDR_DEFAULT)
        mode = window_pref ? CONV_ADDR_WINDOW : pbytes > 0 ? CONV_ADDR_PADDED : CONV_ADDR_ANALYTIC;
    if (mode == CONV_ADDR_WINDOW && !window) mode = CONV_ADDR_PADDED;  // where it does not apply
    if ((mode == CONV_ADDR_PADDED && pbytes < 0) ||
        (mode == CONV_ADDR_TABLE && (vol || !table_fits(d, fwd))))
        return GEMM_ERR_INVALID_ARG;
    if ((rc = device_ok()) != GEMM_OK) return rc;
    int bsrc;
    void *padded = nullptr;
    const void *filters = a;
    int64_t kdim = fwd ? d.crs() : d.vol_out();
    void *dyp = nullptr, *dwp = nullptr;  // filter-gradient window: padded dy rows, dw rows
    if (mode == CONV_ADDR_WINDOW && !fwd) {
        if ((rc = conv_padded_buffer(stream, (size_t)pbytes, &padded)) != GEMM_OK) return rc;
        const int64_t P = d.out[0];
        if ((rc = conv_filter_buffer(stream, (size_t)(d.k * P * wgeom.qp * es), &dyp)) != GEMM_OK ||
            (rc = conv_result_buffer(stream, (size_t)(d.k * wgeom.cr * wgeom.sp) * sizeof(float),
                                     &dwp)) != GEMM_OK)
            return rc;
        geom = wgeom;
        bsrc = B_CONV_WGRAD_WIN;
    } else if (mode == CONV_ADDR_WINDOW) {
        if ((rc = conv_padded_buffer(stream, (size_t)pbytes, &padded)) != GEMM_OK) return rc;
        // filters with rows padded to S' taps: K' = C_in R S'
        kdim = (int64_t)wgeom.cr * wgeom.sp;
        const int64_t total = d.k * kdim;
        if (total * es >= (int64_t(1) << 31)) return GEMM_ERR_INVALID_ARG;
        void *fbuf = nullptr;
        if ((rc = conv_filter_buffer(stream, (size_t)(total * es), &fbuf)) != GEMM_OK) return rc;
        const dim3 grid((unsigned)((total + kThreads - 1) / kThreads)), block(kThreads);
        if (es == 4)
            hipLaunchKernelGGL(conv_filter_pad_kernel<4>, grid, block, 0, stream, a, fbuf,
                               (int)total, wgeom.s, wgeom.sp);
        else
            hipLaunchKernelGGL(conv_filter_pad_kernel<2>, grid, block, 0, stream, a, fbuf,
                               (int)total, wgeom.s, wgeom.sp);
        if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
        filters = fbuf;
        geom = wgeom;
        bsrc = B_CONV_FWD_WIN;
    } else if (mode == CONV_ADDR_TABLE) {
        if ((rc = table_source(es, fwd, &geom, stream, &bsrc)) != GEMM_OK) return rc;
    } else if (mode == CONV_ADDR_PADDED) {
        if ((rc = conv_padded_buffer(stream, (size_t)pbytes, &padded)) != GEMM_OK) return rc;
        // the loaders read the padded image: no padding left to apply
        if (vol) {
            geom.du = pd.up;
            geom.pu = 0;
            geom.d = pd.dp;
            geom.pz = 0;
        }
        geom.h = pd.hp;
        geom.w = pd.wp;
        geom.ph = 0;
        geom.pw = 0;
        geom.img_bytes = (int)pbytes;
        geom.tab = nullptr;
        bsrc = four ? (fwd ? B_CONV4_FWD_PAD : B_CONV4_WGRAD_PAD)
               : vol ? (fwd ? B_CONV3_FWD_PAD : B_CONV3_WGRAD_PAD)
                     : (fwd ? B_CONV_FWD_PAD : B_CONV_WGRAD_PAD);
    } else {
        geom.tab = nullptr;
        bsrc = four ? (fwd ? B_CONV4_FWD : B_CONV4_WGRAD)
               : vol ? (fwd ? B_CONV3_FWD : B_CONV3_WGRAD)
                     : (fwd ? B_CONV_FWD : B_CONV_WGRAD);
    }
    const int64_t vo = d.vol_out();
    const int total = (int)(pbytes > 0 ? pbytes / es : 0);
    for (int64_t n = 0; n < d.n; ++n) {
        const void *img = static_cast<const char *>(x) + n * d.c * d.img_elems() * es;
        if (padded != nullptr) {
            const dim3 grid((unsigned)((total + kThreads - 1) / kThreads)), block(kThreads);
            if (es == 4)
                hipLaunchKernelGGL(conv_pad_kernel<4>, grid, block, 0, stream, img, padded, total,
                                   pd);
            else
                hipLaunchKernelGGL(conv_pad_kernel<2>, grid, block, 0, stream, img, padded, total,
                                   pd);
            if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
            img = padded;
        }
        GemmCall g;
        if (fwd)
            // y[n] (C_out x output volume) = w (C_out x C_in filter volume) . cols(x[n])
            // (the window source: filter rows padded to S' taps, K = C_in R S')
            g = GemmCall{dtype, dtype_out, GEMM_OP_N, GEMM_OP_N, d.k, vo, kdim, 1.0f, 0.0f,
                         filters, kdim, img, 1, static_cast<char *>(out) + n * d.k * vo * eso, vo,
                         bsrc, &geom};
        else if (dyp != nullptr) {
            // dw' (C_out x C_in R S') (+)= dy'[n] (C_out x P Q') . cols(x[n])^T, with the
            // rows of dy[n] padded from Q to Q' positions (zeros)
            const int64_t P = d.out[0], rows = d.k * P, total_dy = rows * wgeom.qp;
            const dim3 grid((unsigned)((total_dy + kThreads - 1) / kThreads)), block(kThreads);
            const void *dyn = static_cast<const char *>(a) + n * d.k * vo * es;
            if (es == 4)
                hipLaunchKernelGGL(conv_filter_pad_kernel<4>, grid, block, 0, stream, dyn, dyp,
                                   (int)total_dy, (int)d.out[1], wgeom.qp);
            else
                hipLaunchKernelGGL(conv_filter_pad_kernel<2>, grid, block, 0, stream, dyn, dyp,
                                   (int)total_dy, (int)d.out[1], wgeom.qp);
            if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
            const int64_t ncols = (int64_t)wgeom.cr * wgeom.sp, kp = P * wgeom.qp;
            g = GemmCall{dtype, GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_T, d.k, ncols, kp, 1.0f,
                         n == 0 ? 0.0f : 1.0f, dyp, kp, img, 1, dwp, ncols, bsrc, &geom};
        } else
            // dw (C_out x C_in filter volume) (+)= dy[n] (C_out x output volume) . cols(x[n])^T
            g = GemmCall{dtype, GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_T, d.k, d.crs(), vo, 1.0f,
                         n == 0 ? 0.0f : 1.0f, static_cast<const char *>(a) + n * d.k * vo * es,
                         vo, img, 1, out, d.crs(), bsrc, &geom};
        if ((rc = gemm_run(g, -1, 0, stream)) != GEMM_OK) return rc;
    }
    if (dwp != nullptr) {
        // dw = dw' without the zero-tap columns
        const int64_t total = d.k * d.crs();
        hipLaunchKernelGGL(conv_filter_unpad_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, static_cast<const float *>(dwp),
                           static_cast<float *>(out), (int)total, wgeom.s, wgeom.sp);
        if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
    }
    return GEMM_OK;
}

// ------------------------------------ routines shared by 2-D and N-D calls --

int64_t workspace_bytes(int dtype, int rc, const Dims &d)
{
    if (!valid_dtype(dtype)) return GEMM_ERR_INVALID_ARG;
    if (rc != GEMM_OK) return rc;
    return d.crs() * d.ld() * elem_size(dtype);
}

int im2col(int dtype, const Dims &d, int64_t image, const void *x, void *cols, int64_t ld_cols,
           hipStream_t stream)
{
    if (!valid_dtype(dtype)) return GEMM_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    if (image < 0 || image >= d.n || x == nullptr || cols == nullptr || ld_cols < d.vol_out() ||
        !fits(d.crs(), ld_cols, kMaxElems) || !aligned_to(x, es) || !aligned_to(cols, es))
        return GEMM_ERR_INVALID_ARG;
    const int rc = device_ok();
    if (rc != GEMM_OK) return rc;
    const char *img = static_cast<const char *>(x) + image * d.c * d.img_elems() * es;
    return launch_im2col(es, d, img, cols, ld_cols, stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

int fwd(int dtype, int dtype_y, const Dims &d, const void *x, const void *w, void *y,
        void *workspace, int64_t ws_bytes, hipStream_t stream)
{
    if (!valid_dtype(dtype) || !valid_dtype(dtype_y)) return GEMM_ERR_INVALID_ARG;
    if (d.n == 0) return GEMM_OK;
    const int es = elem_size(dtype), esy = elem_size(dtype_y);
    if (x == nullptr || w == nullptr || y == nullptr || !aligned_to(x, es) || !aligned_to(w, es) ||
        !aligned_to(y, esy))
        return GEMM_ERR_INVALID_ARG;
    int rc = check_workspace(d, dtype, workspace, ws_bytes);
    if (rc != GEMM_OK) return rc;
    if ((rc = device_ok()) != GEMM_OK) return rc;
    const int64_t ld = d.ld(), vo = d.vol_out();
    for (int64_t n = 0; n < d.n; ++n) {
        const char *img = static_cast<const char *>(x) + n * d.c * d.img_elems() * es;
        if (launch_im2col(es, d, img, workspace, ld, stream) != hipSuccess) return GEMM_ERR_HIP;
        // y[n] (C_out x output volume) = w (C_out x C_in filter volume) . cols
        GemmCall g{dtype, dtype_y, GEMM_OP_N, GEMM_OP_N, d.k, vo, d.crs(), 1.0f, 0.0f, w, d.crs(),
                   workspace, ld, static_cast<char *>(y) + n * d.k * vo * esy, vo};
        if ((rc = gemm_run(g, -1, 0, stream)) != GEMM_OK) return rc;
    }
    return GEMM_OK;
}

// dw := 0 through a GEMM with K == 0 (the empty sum over a batch of 0).
int zero_dw(int dtype, const Dims &d, float *dw, hipStream_t stream)
{
    GemmCall g{dtype, GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_T, d.k, d.crs(), 0, 1.0f, 0.0f,
               nullptr, 1, nullptr, 1, dw, d.crs()};
    return gemm_run(g, -1, 0, stream);
}

int bwd_weight(int dtype, const Dims &d, const void *x, const void *dy, float *dw, void *workspace,
               int64_t ws_bytes, hipStream_t stream)
{
    if (!valid_dtype(dtype)) return GEMM_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    if (dw == nullptr || !aligned_to(dw, 4)) return GEMM_ERR_INVALID_ARG;
    if (d.n == 0) return zero_dw(dtype, d, dw, stream);
    if (x == nullptr || dy == nullptr || !aligned_to(x, es) || !aligned_to(dy, es))
        return GEMM_ERR_INVALID_ARG;
    int rc = check_workspace(d, dtype, workspace, ws_bytes);
    if (rc != GEMM_OK) return rc;
    if ((rc = device_ok()) != GEMM_OK) return rc;
    const int64_t ld = d.ld(), vo = d.vol_out();
    for (int64_t n = 0; n < d.n; ++n) {
        const char *img = static_cast<const char *>(x) + n * d.c * d.img_elems() * es;
        if (launch_im2col(es, d, img, workspace, ld, stream) != hipSuccess) return GEMM_ERR_HIP;
        // dw (C_out x C_in filter volume) (+)= dy[n] (C_out x output volume) . cols^T
        GemmCall g{dtype, GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_T, d.k, d.crs(), vo, 1.0f,
                   n == 0 ? 0.0f : 1.0f, static_cast<const char *>(dy) + n * d.k * vo * es, vo,
                   workspace, ld, dw, d.crs()};
        if ((rc = gemm_run(g, -1, 0, stream)) != GEMM_OK) return rc;
    }
    return GEMM_OK;
}

}  // namespace
}  // namespace dg

extern "C" {

// ------------------------------------------------------------------- 2-D --

int conv2d_output_size(const conv2d_params *p, int64_t *out_h, int64_t *out_w)
{
    dg::Dims d;
    const int rc = dg::dims_2d(p, &d);
    if (rc != GEMM_OK) return rc;
    if (out_h) *out_h = d.out[0];
    if (out_w) *out_w = d.out[1];
    return GEMM_OK;
}

int64_t conv2d_workspace_size(int dtype, const conv2d_params *p)
{
    dg::Dims d;
    const int rc = dg::dims_2d(p, &d);
    return dg::workspace_bytes(dtype, rc, d);
}

int conv2d_im2col(int dtype, const conv2d_params *p, int64_t image, const void *x, void *cols,
                  int64_t ld_cols, hipStream_t stream)
{
    dg::Dims d;
    const int rc = dg::dims_2d(p, &d);
    return rc != GEMM_OK ? rc : dg::im2col(dtype, d, image, x, cols, ld_cols, stream);
}

int conv2d_fwd(int dtype, int dtype_y, const conv2d_params *p, const void *x, const void *w,
               void *y, void *workspace, int64_t workspace_bytes, hipStream_t stream)
{
    dg::Dims d;
    const int rc = dg::dims_2d(p, &d);
    return rc != GEMM_OK ? rc
                         : dg::fwd(dtype, dtype_y, d, x, w, y, workspace, workspace_bytes, stream);
}

int conv2d_bwd_weight(int dtype, const conv2d_params *p, const void *x, const void *dy, float *dw,
                      void *workspace, int64_t workspace_bytes, hipStream_t stream)
{
    dg::Dims d;
    const int rc = dg::dims_2d(p, &d);
    return rc != GEMM_OK ? rc
                         : dg::bwd_weight(dtype, d, x, dy, dw, workspace, workspace_bytes, stream);
}

int conv2d_fwd_implicit_ex(int dtype, int dtype_y, const conv2d_params *p, int addressing,
                           const void *x, const void *w, void *y, hipStream_t stream)
{
    dg::Dims d;
    if (!dg::valid_dtype(dtype) || !dg::valid_dtype(dtype_y)) return GEMM_ERR_INVALID_ARG;
    const int rc = dg::dims_2d(p, &d);
    if (rc != GEMM_OK) return rc;
    if (addressing < CONV_ADDR_DEFAULT || addressing > CONV_ADDR_WINDOW) return GEMM_ERR_INVALID_ARG;
    return dg::run_implicit(dtype, dtype_y, d, addressing, true, false, x, w, y, stream);
}

int conv2d_fwd_implicit(int dtype, int dtype_y, const conv2d_params *p, const void *x,
                        const void *w, void *y, hipStream_t stream)
{
    return conv2d_fwd_implicit_ex(dtype, dtype_y, p, CONV_ADDR_DEFAULT, x, w, y, stream);
}

int conv2d_bwd_weight_implicit_ex(int dtype, const conv2d_params *p, int addressing,
                                  const void *x, const void *dy, float *dw, hipStream_t stream)
{
    dg::Dims d;
    if (!dg::valid_dtype(dtype)) return GEMM_ERR_INVALID_ARG;
    const int rc = dg::dims_2d(p, &d);
    if (rc != GEMM_OK) return rc;
    if (addressing < CONV_ADDR_DEFAULT || addressing > CONV_ADDR_WINDOW) return GEMM_ERR_INVALID_ARG;
    return dg::run_implicit(dtype, GEMM_DTYPE_F32, d, addressing, false, false, x, dy, dw, stream);
}

int conv2d_bwd_weight_implicit(int dtype, const conv2d_params *p, const void *x, const void *dy,
                               float *dw, hipStream_t stream)
{
    return conv2d_bwd_weight_implicit_ex(dtype, p, CONV_ADDR_DEFAULT, x, dy, dw, stream);
}

// ------------------------------------------------------------------- N-D --

int convnd_output_size(const convnd_params *p, int64_t *out)
{
    dg::Dims d;
    const int rc = dg::dims_nd(p, &d);
    if (rc != GEMM_OK) return rc;
    if (out)
        for (int i = 0; i < d.nd; ++i) out[i] = d.out[i];
    return GEMM_OK;
}

int64_t convnd_workspace_size(int dtype, const convnd_params *p)
{
    dg::Dims d;
    const int rc = dg::dims_nd(p, &d);
    return dg::workspace_bytes(dtype, rc, d);
}

int convnd_im2col(int dtype, const convnd_params *p, int64_t image, const void *x, void *cols,
                  int64_t ld_cols, hipStream_t stream)
{
    dg::Dims d;
    const int rc = dg::dims_nd(p, &d);
    return rc != GEMM_OK ? rc : dg::im2col(dtype, d, image, x, cols, ld_cols, stream);
}

int convnd_fwd(int dtype, int dtype_y, const convnd_params *p, const void *x, const void *w,
               void *y, void *workspace, int64_t workspace_bytes, hipStream_t stream)
{
    dg::Dims d;
    const int rc = dg::dims_nd(p, &d);
    return rc != GEMM_OK ? rc
                         : dg::fwd(dtype, dtype_y, d, x, w, y, workspace, workspace_bytes, stream);
}

int convnd_bwd_weight(int dtype, const convnd_params *p, const void *x, const void *dy, float *dw,
                      void *workspace, int64_t workspace_bytes, hipStream_t stream)
{
    dg::Dims d;
    const int rc = dg::dims_nd(p, &d);
    return rc != GEMM_OK ? rc
                         : dg::bwd_weight(dtype, d, x, dy, dw, workspace, workspace_bytes, stream);
}

int convnd_fwd_implicit_ex(int dtype, int dtype_y, const convnd_params *p, int addressing,
                           const void *x, const void *w, void *y, hipStream_t stream)
{
    dg::Dims d;
    if (!dg::valid_dtype(dtype) || !dg::valid_dtype(dtype_y)) return GEMM_ERR_INVALID_ARG;
    const int rc = dg::dims_nd(p, &d);
    if (rc != GEMM_OK) return rc;
    if (addressing < CONV_ADDR_DEFAULT || addressing > CONV_ADDR_WINDOW ||
        addressing == CONV_ADDR_TABLE)
        return GEMM_ERR_INVALID_ARG;
    return dg::run_implicit(dtype, dtype_y, d, addressing, true, true, x, w, y, stream);
}

int convnd_fwd_implicit(int dtype, int dtype_y, const convnd_params *p, const void *x,
                        const void *w, void *y, hipStream_t stream)
{
    return convnd_fwd_implicit_ex(dtype, dtype_y, p, CONV_ADDR_DEFAULT, x, w, y, stream);
}

int convnd_bwd_weight_implicit_ex(int dtype, const convnd_params *p, int addressing,
                                  const void *x, const void *dy, float *dw, hipStream_t stream)
{
    dg::Dims d;
    if (!dg::valid_dtype(dtype)) return GEMM_ERR_INVALID_ARG;
    const int rc = dg::dims_nd(p, &d);
    if (rc != GEMM_OK) return rc;
    if (addressing < CONV_ADDR_DEFAULT || addressing > CONV_ADDR_WINDOW ||
        addressing == CONV_ADDR_TABLE)
        return GEMM_ERR_INVALID_ARG;
    return dg::run_implicit(dtype, GEMM_DTYPE_F32, d, addressing, false, true, x, dy, dw, stream);
}

int convnd_bwd_weight_implicit(int dtype, const convnd_params *p, const void *x, const void *dy,
                               float *dw, hipStream_t stream)
{
    return convnd_bwd_weight_implicit_ex(dtype, p, CONV_ADDR_DEFAULT, x, dy, dw, stream);
}

}  // extern "C"
