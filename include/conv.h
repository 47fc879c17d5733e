/*
 * 2-D convolution on MI355X (gfx950) as im2col + GEMM, on one GPU.
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
 * dimensions beyond the library's range (each GEMM extent must stay below
 * 2^30, each tensor below 2^62 elements), a null pointer, a pointer not
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

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_03_AMD_CONV_H */
