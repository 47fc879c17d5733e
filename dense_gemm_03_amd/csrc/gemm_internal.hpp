// Library-internal entry into the GEMM dispatcher, for the other operations
// built on the GEMM (the im2col convolution).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.hpp"

namespace dg {

// One generalised product C := alpha * op(A) * op(B) + beta * C, with the
// argument meaning of gemm_ex in include/gemm.h.
struct GemmCall {
    int dtype;      // of A and B (GEMM_DTYPE_*)
    int dtype_c;    // of C
    int transa, transb;
    int64_t M, N, K;
    float alpha, beta;
    const void *A;
    int64_t lda;
    const void *B;
    int64_t ldb;
    void *C;
    int64_t ldc;
    // B_MATRIX, or an implicit convolution source: then B is the image of
    // one batch element, ldb is not used, and conv describes the geometry
    int bsrc = B_MATRIX;
    const ConvGeom *conv = nullptr;
};

// Checks the arguments, picks a tile entry (or uses forced_cfg >= 0) and a
// split-K plan (forced_split > 0 forces it), and launches on `stream`.
// Returns a gemm_status.
int gemm_run(const GemmCall &call, int forced_cfg, int forced_split, hipStream_t stream);

// A library-owned device buffer of at least `bytes` for the convolution
// tables of calls on `stream` (current device); it lives until the library is
// unloaded and is reused by the next call on that stream, so the work that
// reads it must be enqueued on `stream`.  Returns a gemm_status.
int conv_table_buffer(hipStream_t stream, size_t bytes, void **out);
// The same for the zero-padded image of the implicit GEMM.
int conv_padded_buffer(hipStream_t stream, size_t bytes, void **out);
// The same for the filters with rows padded to S' taps (image-window source),
// or the output gradient with rows padded to Q' positions.
int conv_filter_buffer(hipStream_t stream, size_t bytes, void **out);
// The same for the filter gradient with rows padded to S' taps.
int conv_result_buffer(hipStream_t stream, size_t bytes, void **out);

// Block width BN, k-tile BK and threads of the entry gemm_run picks for an
// implicit convolution product with M output channels.  Returns a
// gemm_status (GEMM_ERR_INTERNAL if the entry is missing from the table).
int implicit_tile(int dtype, int64_t M, int *bn, int *bk, int *threads);

}  // namespace dg
