/*
 * Dense GEMM for AMD Instinct MI355X (gfx950): C = A . B on one GPU.
 *
 * The operation ("Learning to develop for GPUs through the GEMM operation",
 * section "Matrix product"): A is M x K, B is K x N, C is M x N, and each
 * element of C is the dot product of a row of A with a column of B,
 *
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j].
 *
 * gemm_f32 and gemm_bf16 compute exactly that product: C is overwritten and
 * never read.  gemm_ex computes the generalised product of the page's next
 * section, "Generalized matrix multiplication GEMM":
 *
 *     C := alpha * op(A) * op(B) + beta * C,    op(X) = X or X^T,
 *
 * with C stored as fp32 or bf16 (see gemm_ex below).
 *
 * Layout: every matrix is row-major with a leading dimension, counted in
 * elements, between the starts of consecutive rows (for the plain product):
 *     A[i][k] = A[i*lda + k],  lda >= K
 *     B[k][j] = B[k*ldb + j],  ldb >= N
 *     C[i][j] = C[i*ldc + j],  ldc >= N
 * A column-major caller computes C^T = B^T . A^T with the same call by
 * swapping the operands.  Elements of C outside the M x N window (the ldc
 * padding) are never written.
 *
 * Precision: gemm_f32 multiplies and accumulates in fp32 (true fp32 matrix-core
 * products, no reduced-precision emulation).  gemm_bf16 takes bf16 inputs as
 * raw 16-bit patterns (the upper half of an IEEE binary32), multiplies them
 * exactly and accumulates in fp32; C is fp32.  The order of the k sum is not
 * specified, but a given call on a given device is bitwise reproducible (no
 * atomics are used).
 *
 * Memory and ownership: A, B and C are device pointers owned by the caller
 * (for example tensors allocated by PyTorch).  C must not overlap A or B.  The
 * library never frees caller memory.  It owns a few device buffers per
 * (device, stream): the split-K partial sums of the GEMM, row-aligned copies
 * of bf16 operands (see "Dispatch"), and for the convolution calls of conv.h
 * their term tables, zero-bordered image copies and row-padded filter copies.  A buffer is allocated with hipMalloc on the
 * first call on a stream that needs it and grown (by at least half its size)
 * when a later call on that stream needs more; the buffer it replaces is kept,
 * not freed, until gemm_release_buffers(stream) or library unload, so that a
 * graph captured earlier on that stream stays valid.
 *
 * Graph capture: a call made while `stream` is being captured must not grow a
 * buffer (that would call hipMalloc inside the capture): it returns
 * GEMM_ERR_CAPTURING and enqueues nothing.  Run the same call (or a larger
 * one) once on that stream before capturing, so the buffers already exist.
 * Calls that need no library buffer (no split-K, which the dispatcher picks
 * for most shapes; gemm_split_k tells) capture on any stream.  The operand
 * copies are an optimisation: a call that would copy but whose buffer cannot
 * grow during capture runs on the operands in place instead (same result,
 * slower); gemm_operand_copy_bytes gives the size to warm up.
 *
 * Streams: all work is enqueued on `stream` (NULL is the default stream) and
 * the calls return without waiting for it.  A fault inside a kernel surfaces
 * at the caller's next synchronisation on that stream.
 *
 * Errors: every entry point returns a gemm_status and never throws.
 *   - M, N or K negative; a leading dimension smaller than its row
 *     (lda < max(K,1), ldb < max(N,1), ldc < max(N,1)); a null pointer for a
 *     non-empty operand; a pointer not aligned to its element size:
 *     GEMM_ERR_INVALID_ARG, and nothing is launched.
 *   - M == 0 or N == 0: GEMM_OK, nothing is launched.
 *   - K == 0: C is filled with zeros (the empty sum), GEMM_OK.
 *   - a HIP error while launching or allocating: GEMM_ERR_HIP or
 *     GEMM_ERR_OUT_OF_MEMORY.
 *   - a library buffer would have to grow during stream capture:
 *     GEMM_ERR_CAPTURING (see "Graph capture").
 *   - GEMM_ERR_INTERNAL: the dispatcher names a tile-table entry the build
 *     does not hold (a build error; never returned by a consistent build).
 * Argument checks happen before any HIP call, so an invalid call does not
 * touch the GPU.
 *
 * Threads: the entry points may be called from several host threads; the
 * tile table is read-only and the buffer registry is guarded by a mutex.
 * Library buffers are kept per (device, stream): calls on different streams
 * never share one.  Two threads must not call on the same stream at the same
 * time: their kernels would share that stream's buffers.
 *
 * Dispatch: the tile choice and split-K plan depend on the shape, the operand
 * form and the compute-unit count of the current device (queried once per
 * device; 256, MI355X's count, when no device is visible); the bf16 split-K
 * plan also on whether the operand rows are 16-byte aligned.  bf16 operands
 * whose rows are not all 4-byte aligned (an odd leading dimension, an address
 * that is 2 but not 4 bytes aligned, or an odd M for A^T or N for B) cannot
 * be streamed with the kernels' direct loads.  When K >= 256, the product
 * does at least 2^26 flops, and at least 160 flops per byte of those of its
 * operands that lack 16-byte-aligned rows and are read k-contiguous (A, B^T)
 * plus 56 per byte of those read outer-contiguous (A^T, B), the dispatcher
 * first copies those operands into a library buffer with 16-byte-aligned,
 * zero-padded rows, then runs the product on the copies; other products run
 * on the operands in place.
 * Calls with a forced table entry (the *_with_config entry points) and
 * gemm_ex_noalloc never copy.
 */
#ifndef DENSE_GEMM_03_AMD_GEMM_H
#define DENSE_GEMM_03_AMD_GEMM_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = -1,
    GEMM_ERR_HIP = -2,
    GEMM_ERR_NO_DEVICE = -3,
    GEMM_ERR_OUT_OF_MEMORY = -4,
    GEMM_ERR_INTERNAL = -5,
    GEMM_ERR_CAPTURING = -6,
    GEMM_ERR_SCRATCH_LIMIT = -7
} gemm_status;

typedef enum { GEMM_DTYPE_F32 = 0, GEMM_DTYPE_BF16 = 1 } gemm_dtype;

/* Operand form for gemm_ex: as stored, or transposed. */
typedef enum { GEMM_OP_N = 0, GEMM_OP_T = 1 } gemm_op;

/* C := A . B for fp32 A (M x K), B (K x N) and C (M x N), row-major. */
int gemm_f32(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc,
             hipStream_t stream);

/* C := A . B for bf16 A and B (uint16 bit patterns) and fp32 C, row-major,
 * fp32 accumulation. */
int gemm_bf16(int64_t M, int64_t N, int64_t K,
              const uint16_t *A, int64_t lda,
              const uint16_t *B, int64_t ldb,
              float *C, int64_t ldc,
              hipStream_t stream);

/*
 * C := alpha * op(A) * op(B) + beta * C   ("Generalized matrix multiplication
 * GEMM" on the GEMM page; BLAS's xGEMM with row-major storage).
 *
 * dtype_ab: GEMM_DTYPE_F32 or GEMM_DTYPE_BF16, the type of both A and B
 *   (bf16 as raw 16-bit patterns).  Products are fp32 (fp32 inputs) or exact
 *   (bf16 inputs) and are accumulated in fp32.
 * dtype_c: GEMM_DTYPE_F32 or GEMM_DTYPE_BF16, the type of C on input and
 *   output.  alpha * sum + beta * C is formed in fp32 and, for bf16 C, rounded
 *   once to nearest (ties to even); a NaN stays a NaN.
 * transa, transb: GEMM_OP_N or GEMM_OP_T.  The stored matrices, row-major:
 *   transa == N: A is M x K, op(A)[i][k] = A[i*lda + k], lda >= max(K,1)
 *   transa == T: A is K x M, op(A)[i][k] = A[k*lda + i], lda >= max(M,1)
 *   transb == N: B is K x N, op(B)[k][j] = B[k*ldb + j], ldb >= max(N,1)
 *   transb == T: B is N x K, op(B)[k][j] = B[j*ldb + k], ldb >= max(K,1)
 *   C is M x N, C[i][j] = C[i*ldc + j], ldc >= max(N,1).
 *   (A column-major caller passes its matrices with the transpose flags
 *   flipped and computes C^T.)
 * alpha, beta: fp32 scalars.  When beta == 0, C is not read (it may hold
 *   anything, NaN included).  When alpha == 0 or K == 0, A and B are not read
 *   and C := beta * C (or 0 when beta == 0).
 *
 * Errors as for gemm_f32, and GEMM_ERR_INVALID_ARG for an unknown dtype or
 * transpose flag or for C not aligned to its element size.  Ownership,
 * streams, workspace and threads as above; C must not overlap A or B.
 */
int gemm_ex(int dtype_ab, int dtype_c, int transa, int transb,
            int64_t M, int64_t N, int64_t K,
            float alpha,
            const void *A, int64_t lda,
            const void *B, int64_t ldb,
            float beta,
            void *C, int64_t ldc,
            hipStream_t stream);

/*
 * gemm_ex without any allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, result and errors as gemm_ex, and the
 * same kernels and split-K plan, so its output equals gemm_ex's bit for bit,
 * except for the bf16 calls that gemm_ex runs on row-aligned copies
 * (gemm_operand_copy_bytes > 0): this entry point runs them on the operands
 * in place, where the k sum may be ordered differently (integer-valued
 * operands still give the same result).
 * The split-K partial sums go to a fixed array of 64 MiB in the library's
 * device code (GEMM_SCRATCH_BYTES), one per GPU, held by each GPU the library
 * runs on until the process ends; the library allocates nothing, and the
 * call never calls hipMalloc or hipFree.  The first call on a device looks up
 * that GPU's copy of the array (hipGetSymbolAddress, which may load the
 * library's device code onto it); make that first call outside any capture.
 *   - a call whose split-K plan needs more than GEMM_SCRATCH_BYTES of
 *     partial sums (splits * M * N * 4 bytes; gemm_select_config_ex and
 *     gemm_split_k_ex give the plan) returns GEMM_ERR_SCRATCH_LIMIT and
 *     enqueues nothing;
 *   - every call on one GPU shares that GPU's array: two calls that may run
 *     at the same time on one GPU (different streams, or different host
 *     threads) race on it and give wrong results.  Calls on one stream are
 *     ordered and safe.  The array keeps the last call's partial sums; nothing
 *     in it needs to start at zero.
 */
#define GEMM_SCRATCH_BYTES ((size_t)64 << 20)
int gemm_ex_noalloc(int dtype_ab, int dtype_c, int transa, int transb,
                    int64_t M, int64_t N, int64_t K,
                    float alpha,
                    const void *A, int64_t lda,
                    const void *B, int64_t ldb,
                    float beta,
                    void *C, int64_t ldc,
                    hipStream_t stream);

/* A static, human-readable description of a gemm_status value. */
const char *gemm_status_string(int status);

/*
 * Frees every library buffer (current and retired) that calls on `stream`
 * made on the current device, e.g. before the caller destroys the stream.
 * The next call on that stream allocates afresh.  The caller must ensure no
 * enqueued work and no graph that will still be launched uses them (hipFree
 * waits for the device, so work already enqueued completes first).
 * GEMM_ERR_CAPTURING while `stream` is being captured; GEMM_ERR_NO_DEVICE
 * without a device; GEMM_ERR_HIP if a free failed.
 */
int gemm_release_buffers(hipStream_t stream);

/*
 * Tile-table hooks, for tests and tuning.  The dispatcher of gemm_f32 and
 * gemm_bf16 picks one entry of a per-dtype table of tile configurations by the
 * shape class of (M, N, K) -- how tile sizes must be chosen per task and
 * device is the point of "How to do even better" on the GEMM page.
 *
 * gemm_num_configs: number of table entries for a dtype (negative on a bad
 *   dtype).
 * gemm_select_config: the entry the dispatcher would use for this shape of
 *   the plain product A . B on the current device (host logic; it reads the
 *   device's compute-unit count, 256 without a device); negative on bad
 *   arguments.
 * gemm_select_config_ex: the same for op(A) . op(B) with the given transa,
 *   transb (GEMM_OP_N / GEMM_OP_T): the choice depends on which operands are
 *   read k-contiguous.
 * gemm_config_name: a static string naming an entry ("f32_128x128x32_w2x2"...),
 *   NULL when out of range.
 * gemm_split_k: the number of K slices the dispatcher would use with entry cfg
 *   for this shape of the plain product with 16-byte aligned rows (1 = no
 *   split); negative on bad arguments.  gemm_split_k_ex: the same for the operand form (transa,
 *   transb).
 * gemm_config_layouts: bit (transa * 2 + transb) is set when entry cfg has
 *   kernels for that operand form (the entry the dispatcher chooses for an
 *   operand form always has it); negative on bad arguments.
 * gemm_f32_with_config / gemm_bf16_with_config / gemm_ex_with_config: as
 *   gemm_f32 / gemm_bf16 / gemm_ex but with the table entry forced (an entry
 *   without kernels for the requested operand form is GEMM_ERR_INVALID_ARG);
 *   split_k <= 0 lets the dispatcher choose the number of K slices, a positive
 *   value forces it (clamped so that every slice holds at least one k-tile).
 */
int gemm_num_configs(int dtype);
int gemm_select_config(int dtype, int64_t M, int64_t N, int64_t K);
int gemm_select_config_ex(int dtype, int transa, int transb, int64_t M, int64_t N, int64_t K);
const char *gemm_config_name(int dtype, int cfg);
int gemm_split_k(int dtype, int cfg, int64_t M, int64_t N, int64_t K);
int gemm_split_k_ex(int dtype, int cfg, int transa, int transb, int64_t M, int64_t N, int64_t K);
int gemm_config_layouts(int dtype, int cfg);

/*
 * Bytes of the per-(device, stream) buffer that gemm_ex (and gemm_bf16) would
 * use for row-aligned copies of the operands of this call (see "Dispatch"):
 * 0 when it runs on them in place, GEMM_ERR_INVALID_ARG (negative) for the
 * arguments gemm_ex rejects, apart from C.  A and B are examined for their
 * alignment only, never read; no HIP call is made.  Callers that capture
 * graphs run one such call (or a larger one) on the stream first, so that
 * the buffer exists.
 */
int64_t gemm_operand_copy_bytes(int dtype_ab, int transa, int transb,
                                int64_t M, int64_t N, int64_t K,
                                const void *A, int64_t lda,
                                const void *B, int64_t ldb);

int gemm_f32_with_config(int cfg, int split_k,
                         int64_t M, int64_t N, int64_t K,
                         const float *A, int64_t lda,
                         const float *B, int64_t ldb,
                         float *C, int64_t ldc,
                         hipStream_t stream);

int gemm_bf16_with_config(int cfg, int split_k,
                          int64_t M, int64_t N, int64_t K,
                          const uint16_t *A, int64_t lda,
                          const uint16_t *B, int64_t ldb,
                          float *C, int64_t ldc,
                          hipStream_t stream);

int gemm_ex_with_config(int cfg, int split_k,
                        int dtype_ab, int dtype_c, int transa, int transb,
                        int64_t M, int64_t N, int64_t K,
                        float alpha,
                        const void *A, int64_t lda,
                        const void *B, int64_t ldb,
                        float beta,
                        void *C, int64_t ldc,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_03_AMD_GEMM_H */
