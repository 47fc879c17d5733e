/*
 * Convolution on MI355X (gfx950) as im2col + GEMM, on one GPU: 2-D, and 1 to
 * 4 spatial dimensions (the convnd_* calls at the end).
 *
 * The operation ("Three X's: a new level of working with large convolutions
 * in PyTorch for model training", sections "Where large convolution kernels
 * come from" and "CuBLAS"): a bank of C_out filters of C_in x R x S taps
 * slides over a batch of C_in-channel images; each output value is the sum
 * over input channels and taps of tap times image value underneath.  With
 * stride (sh, sw), zero padding (ph, pw) and dilation (dh, dw):
 *
 *   P = floor((H + 2 ph - dh (R - 1) - 1) / sh) + 1,   Q likewise from W
 *   y[n][co][p][q] = sum_{ci,r,s} x[n][ci][p sh - ph + r dh][q sw - pw + s dw]
 *                                 * w[co][ci][r][s]
 *
 * (image positions outside the image read as zero; the filter is not flipped:
 * the cross-correlation form that frameworks call convolution).  The filter
 * gradient, the product with large kernels the page is about:
 *
 *   dw[co][ci][r][s] = sum_{n,p,q} dy[n][co][p][q]
 *                                  * x[n][ci][p sh - ph + r dh][q sw - pw + s dw]
 *
 * Route (the page's im2col / GEMM route, section "CuBLAS"): for each image the
 * convolution matrix ("columns") is written to a workspace -- row
 * (ci R + r) S + s, column p Q + q holds the image value that tap (ci, r, s)
 * meets at output (p, q) -- and one GEMM of the library finishes the image:
 *   forward:          y[n] (C_out x PQ)     = w (C_out x C_in R S) . cols
 *   filter gradient:  dw   (C_out x C_in RS) += dy[n] (C_out x PQ) . cols^T
 * (the first image overwrites dw, the next ones accumulate into it in fp32).
 *
 * Layout: every tensor is dense and channel-first, as PyTorch stores it:
 *   x  [batch][C_in][H][W],  w and dw [C_out][C_in][R][S],  y and dy [batch][C_out][P][Q].
 * Types: x, w and dy are all fp32 (dtype GEMM_DTYPE_F32) or all bf16
 * (GEMM_DTYPE_BF16, raw 16-bit patterns).  y is fp32 or bf16 (dtype_y; a bf16
 * y is rounded once, to nearest even); dw is fp32.  Products and sums are fp32
 * (bf16 products are exact).
 *
 * Workspace: the caller provides the device memory for one image's
 * convolution matrix; conv2d_workspace_size gives its size in bytes (C_in R S
 * rows of round_up(P Q, 8) elements).  It must be 16-byte aligned.  Its
 * contents are scratch (overwritten by every call).  Calls that share a
 * workspace must be ordered (same stream, or synchronised).
 *
 * Ownership, streams and errors as for the GEMM (include/gemm.h): caller-owned
 * device memory, work enqueued on `stream`, status codes, no exceptions.
 * GEMM_ERR_INVALID_ARG, with nothing launched, for: a size below 1 (batch may
 * be 0: nothing to do), negative padding, stride or dilation below 1, a
 * filter that does not fit (P or Q below 1), a dimension or product of
 * dimensions beyond the library's range (each GEMM extent and one image
 * channel must stay below 2^30 elements, each tensor below 2^62), a null
 * pointer, a pointer not
 * aligned to its element size, a workspace that is too small or not 16-byte
 * aligned, an unknown dtype.  y must not overlap x, w or the workspace; dw
 * must not overlap x, dy or the workspace.
 */
#ifndef DENSE_GEMM_03_AMD_CONV_H
#define DENSE_GEMM_03_AMD_CONV_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Shape and hyper-parameters of a 2-D convolution. */
typedef struct {
    int64_t batch, in_channels, height, width;
    int64_t out_channels, kernel_h, kernel_w;
    int64_t pad_h, pad_w, stride_h, stride_w, dilation_h, dilation_w;
} conv2d_params;

/* Output extent (P, Q) of a convolution; GEMM_ERR_INVALID_ARG as above.  Host
 * logic only. */
int conv2d_output_size(const conv2d_params *p, int64_t *out_h, int64_t *out_w);

/* Bytes of workspace conv2d_fwd and conv2d_bwd_weight need (one image's
 * convolution matrix); negative (a gemm_status) on invalid arguments.  Host
 * logic only. */
int64_t conv2d_workspace_size(int dtype, const conv2d_params *p);

/* The convolution matrix of image `image` of x into cols (C_in R S rows of
 * ld_cols >= P Q elements of x's type; columns beyond P Q are not written).
 * A pure copy with zero fill: the same bits as x. */
int conv2d_im2col(int dtype, const conv2d_params *p, int64_t image, const void *x, void *cols,
                  int64_t ld_cols, hipStream_t stream);

/* y := conv(x, w).  dtype: of x and w; dtype_y: of y. */
int conv2d_fwd(int dtype, int dtype_y, const conv2d_params *p, const void *x, const void *w,
               void *y, void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* dw := sum over the batch of the filter gradient (fp32).  dtype: of x and
 * dy.  batch == 0 gives dw = 0 (the empty sum). */
int conv2d_bwd_weight(int dtype, const conv2d_params *p, const void *x, const void *dy, float *dw,
                      void *workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * Implicit-GEMM forms of the same two products ("Three X's", section
 * "CUTLASS": the matrix is not built; the GEMM's loader forms each tile of
 * it from the image, from the output coordinates and filter taps, with
 * addresses computed on the fly).  No workspace from the caller (a split of
 * K uses the library's own GEMM workspace).  Same arguments, layouts, types
 * and results as conv2d_fwd / conv2d_bwd_weight; additionally
 * GEMM_ERR_INVALID_ARG when one batch element of x spans 2 GiB or more.
 */
int conv2d_fwd_implicit(int dtype, int dtype_y, const conv2d_params *p, const void *x,
                        const void *w, void *y, hipStream_t stream);
int conv2d_bwd_weight_implicit(int dtype, const conv2d_params *p, const void *x, const void *dy,
                               float *dw, hipStream_t stream);

/*
 * Address generation of the implicit-GEMM loader ("Three X's", section
 * "CUTLASS", which names two iterator kinds: one computes every index and
 * offset on the fly, the other computes them beforehand and reads lookup
 * tables).  Each matrix element's image address is a fixed term per thread
 * plus a term that changes with k (per tap for the forward product, per
 * output position for the filter gradient):
 *   CONV_ADDR_ANALYTIC: the k terms are computed in the loader from k
 *     (integer division by multiply-and-shift);
 *   CONV_ADDR_TABLE: a small kernel first writes one 8-byte entry per k into
 *     a library-owned buffer (one per device and stream, kept for later
 *     calls), and the loader reads its k terms from it, one k-tile ahead.
 *     Needs the y and x terms within signed 16 bits: (R-1) dh and (S-1) dw
 *     for the forward product, ph, pw and the last output's p sh - ph,
 *     q sw - pw for the filter gradient (GEMM_ERR_INVALID_ARG otherwise);
 *   CONV_ADDR_PADDED: before each batch element's product a small kernel
 *     copies its image into a library-owned buffer (one per device and
 *     stream, kept for later calls) with zero borders of the padding's
 *     width, [C_in][H + 2 ph][W + 2 pw]; the loader then reads that copy with
 *     the analytic terms and no padding, so no element needs a range check.
 *     Needs the padded image under 2 GiB (GEMM_ERR_INVALID_ARG otherwise);
 *     costs one extra read and write of the image per call;
 *   CONV_ADDR_WINDOW: with unit horizontal stride and dilation, the padded
 *     copy as above, and each block loads, per k-tile, only the image rows
 *     its filter rows and output rows need into a window in LDS and reads
 *     every B fragment from it with one aligned 16-byte load (instead of
 *     gathering each matrix element).  Filter rows are padded from S to S'
 *     taps (S rounded up to 8 bf16 or 4 fp32 taps): the forward product reads
 *     a library-owned copy of the filters with zero extra taps; the filter
 *     gradient accumulates into a library-owned buffer with S' taps per row
 *     (copied to dw without the extra ones at the end) and reads a copy of
 *     each dy[n] with its output rows padded with zeros to a multiple of the
 *     k-tile.  Applies when one k-tile's window fits the block's staging
 *     (for the filter gradient also S' dividing the block width); other
 *     calls run the padded form.  Same error as CONV_ADDR_PADDED for the
 *     padded image;
 *   CONV_ADDR_DEFAULT: the library's choice (what conv2d_fwd_implicit and
 *     conv2d_bwd_weight_implicit use): the window form where it applies and
 *     pays (the padding adds at most a quarter, S' <= 5/4 S, and the window
 *     is at most half the B stage: wide filters; for the filter gradient,
 *     bf16 only), else the padded form when the padded image fits, else the
 *     analytic one.
 * The analytic, table and padded forms give identical results (same
 * products, same summation order); the window forward product sums the same
 * products (plus zero taps) in a different k order, so its results differ
 * from theirs by rounding only.
 *
 * The library-owned buffers follow the rules of gemm.h ("Memory and
 * ownership", "Graph capture"): kept per (device, stream), grown on demand,
 * replaced buffers kept until gemm_release_buffers(stream); a call that
 * would grow one while its stream is being captured returns
 * GEMM_ERR_CAPTURING.
 */
typedef enum {
    CONV_ADDR_DEFAULT = 0,
    CONV_ADDR_ANALYTIC = 1,
    CONV_ADDR_TABLE = 2,
    CONV_ADDR_PADDED = 3,
    CONV_ADDR_WINDOW = 4
} conv_addressing;

int conv2d_fwd_implicit_ex(int dtype, int dtype_y, const conv2d_params *p, int addressing,
                           const void *x, const void *w, void *y, hipStream_t stream);
int conv2d_bwd_weight_implicit_ex(int dtype, const conv2d_params *p, int addressing,
                                  const void *x, const void *dy, float *dw, hipStream_t stream);

/*
 * Convolution with D = 1 to 4 spatial dimensions ("Three X's", opening and
 * section "CuBLAS": the page's subject is convolution beyond two dimensions;
 * the convolution matrix gains one index per dimension in its row and column
 * numbering and one loop per dimension over the filter taps).  With size
 * S_d, kernel K_d, padding p_d, stride t_d and dilation l_d per dimension
 * (d = 0 .. D-1, the last one innermost):
 *
 *   O_d = floor((S_d + 2 p_d - l_d (K_d - 1) - 1) / t_d) + 1
 *   y[n][co][o] = sum_{ci, k} x[n][ci][o t - p + k l] * w[co][ci][k]
 *
 * with o and k D-vectors and the products element-wise, positions outside
 * the image reading as zero, no filter flip.  The filter gradient is
 * dw[co][ci][k] = sum_{n, o} dy[n][co][o] * x[n][ci][o t - p + k l].
 *
 * Layout (dense, channel-first):  x [batch][C_in][S_0]..[S_{D-1}],
 * w and dw [C_out][C_in][K_0]..[K_{D-1}],  y and dy [batch][C_out][O_0]..[O_{D-1}].
 * Convolution matrix of an image: row (ci, k_0, .., k_{D-1}) and column
 * (o_0, .., o_{D-1}), both numbered row-major; C_in prod(K) rows of
 * round_up(prod(O), 8) elements in the workspace.  D = 2 gives exactly the
 * conv2d_* calls above (kernel_h = K_0, kernel_w = K_1, and so on).
 *
 * Types, workspace, ownership, streams and errors as for the 2-D calls; also
 * GEMM_ERR_INVALID_ARG for ndim outside 1..4.  Entries of the per-dimension
 * arrays at index ndim and beyond are ignored.
 */
typedef struct {
    int64_t batch, in_channels, out_channels, ndim;
    int64_t size[4], kernel[4], pad[4], stride[4], dilation[4];
} convnd_params;

/* Output extents O_0 .. O_{ndim-1} into out[0 .. ndim) (may be NULL).  Host
 * logic only. */
int convnd_output_size(const convnd_params *p, int64_t *out);

/* Bytes of workspace convnd_fwd and convnd_bwd_weight need; negative (a
 * gemm_status) on invalid arguments.  Host logic only. */
int64_t convnd_workspace_size(int dtype, const convnd_params *p);

/* The convolution matrix of image `image` of x into cols (ld_cols >= prod(O));
 * the same bits as x, zero in the padding. */
int convnd_im2col(int dtype, const convnd_params *p, int64_t image, const void *x, void *cols,
                  int64_t ld_cols, hipStream_t stream);

/* y := conv(x, w); dtype of x and w, dtype_y of y. */
int convnd_fwd(int dtype, int dtype_y, const convnd_params *p, const void *x, const void *w,
               void *y, void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* dw := sum over the batch of the filter gradient (fp32); batch == 0 gives
 * dw = 0. */
int convnd_bwd_weight(int dtype, const convnd_params *p, const void *x, const void *dy, float *dw,
                      void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* Implicit-GEMM forms for 1 to 4 spatial dimensions ("Three X's", section
 * "CUTLASS", applied to the N-D matrix): no convolution matrix and no
 * workspace; the GEMM's loader forms each tile from the image with analytic
 * address terms (one to three dimensions run as three with leading unit
 * dimensions; four add the outermost index to those terms).  Same
 * arguments, layouts, types and results as convnd_fwd / convnd_bwd_weight;
 * GEMM_ERR_INVALID_ARG when one batch element of x spans 2 GiB or more.  The _ex forms take the addressing:
 * CONV_ADDR_ANALYTIC, CONV_ADDR_PADDED (the image copied with zero borders
 * in every padded dimension, as for the 2-D calls; CONV_ADDR_WINDOW runs
 * this form here) or CONV_ADDR_DEFAULT (padded when the padded image is
 * under 2 GiB, else analytic; what the plain forms use); CONV_ADDR_TABLE is
 * 2-D only (GEMM_ERR_INVALID_ARG). */
int convnd_fwd_implicit(int dtype, int dtype_y, const convnd_params *p, const void *x,
                        const void *w, void *y, hipStream_t stream);
int convnd_bwd_weight_implicit(int dtype, const convnd_params *p, const void *x, const void *dy,
                               float *dw, hipStream_t stream);
int convnd_fwd_implicit_ex(int dtype, int dtype_y, const convnd_params *p, int addressing,
                           const void *x, const void *w, void *y, hipStream_t stream);
int convnd_bwd_weight_implicit_ex(int dtype, const convnd_params *p, int addressing,
                                  const void *x, const void *dy, float *dw, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_03_AMD_CONV_H */
