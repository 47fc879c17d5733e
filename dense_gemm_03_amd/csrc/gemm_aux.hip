// The split-K reduce and the scale kernel (K == 0 or alpha == 0), with their
// launchers.  Both finish elements of C the way the GEMM epilogue does:
// alpha * sum + beta * C (C read only when beta != 0), stored as fp32 or bf16.
#include <type_traits>

#include "gemm_configs.hpp"

namespace dg {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float load_c(const void *C, int64_t idx, bool out_bf16)
{
    return out_bf16 ? __uint_as_float((uint32_t) static_cast<const uint16_t *>(C)[idx] << 16)
                    : static_cast<const float *>(C)[idx];
}

__device__ __forceinline__ void store_c(void *C, int64_t idx, float v, bool out_bf16)
{
    if (out_bf16)
        static_cast<uint16_t *>(C)[idx] = f32_to_bf16_rne(v);
    else
        static_cast<float *>(C)[idx] = v;
}

// Sum the split-K partial products in slice order (deterministic) and finish
// each element of C.
__global__ void splitk_reduce_kernel(const float *__restrict__ ws, int splits, int M, int N,
                                     void *__restrict__ C, int64_t ldc, float alpha, float beta,
                                     int out_bf16)
{
    const int64_t total = (int64_t)M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        float s = ws[idx];
        for (int z = 1; z < splits; ++z) s += ws[(int64_t)z * total + idx];
        const int64_t i = idx / N, j = idx - i * N;
        const int64_t c = i * ldc + j;
        float v = alpha * s;
        if (beta != 0.0f) v += beta * load_c(C, c, out_bf16 != 0);
        store_c(C, c, v, out_bf16 != 0);
    }
}

// Vector form of the reduce for fp32 C: 4 consecutive columns per thread
// (N % 4 == 0, ldc % 4 == 0, C 16-byte aligned).
__global__ void splitk_reduce4_kernel(const float *__restrict__ ws, int splits, int M, int N,
                                      float *__restrict__ C, int64_t ldc, float alpha, float beta)
{
    const int64_t total4 = (int64_t)M * N / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const floatx4 *w = reinterpret_cast<const floatx4 *>(ws);
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total4; idx += stride) {
        floatx4 s = w[idx];
        for (int z = 1; z < splits; ++z) s += w[(int64_t)z * total4 + idx];
        const int64_t e = idx * 4;
        const int64_t i = e / N, j = e - i * N;
        floatx4 *c = reinterpret_cast<floatx4 *>(C + i * ldc + j);
        floatx4 v = alpha * s;
        if (beta != 0.0f) v += beta * *c;
        *c = v;
    }
}

// C := beta * C, or 0 when beta == 0 (C not read), over the M x N window.
__global__ void scale_kernel(int M, int N, void *__restrict__ C, int64_t ldc, float beta,
                             int out_bf16)
{
    const int64_t total = (int64_t)M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        const int64_t i = idx / N, j = idx - i * N;
        const int64_t c = i * ldc + j;
        const float v = beta != 0.0f ? beta * load_c(C, c, out_bf16 != 0) : 0.0f;
        store_c(C, c, v, out_bf16 != 0);
    }
}

// Copy of a stored operand, `rows` rows of `cols` elements of ES bytes at a
// pitch of ld_bytes, into dst at a pitch of ldd_bytes (16-byte aligned rows,
// ldd_bytes >= cols * ES rounded up to 16).  Thread (lane l of a row group)
// copies 16-byte chunk c of row r; a block holds 256 >> tpr_shift rows of
// 1 << tpr_shift chunk lanes each, so narrow rows do not leave lanes idle.
// A whole chunk at a source address that is 2 but not 4 bytes aligned comes
// from the five aligned dwords that cover it, shifted into place (each holds
// an element of the chunk, so it lies on a page the source occupies); the
// last chunk of a row is read element by element and padded with zeros.
template <int ES>
__global__ void stage_rows_kernel(const unsigned char *__restrict__ src, int64_t ld_bytes,
                                  int64_t rows, int cols, int cpr, int tpr_shift,
                                  unsigned char *__restrict__ dst, int64_t ldd_bytes)
{
    constexpr int VEC = 16 / ES;
    using E = typename std::conditional<ES == 2, uint16_t, uint32_t>::type;
    const int rpb = (int)blockDim.x >> tpr_shift;
    const int c = (int)blockIdx.x * (1 << tpr_shift) + ((int)threadIdx.x & ((1 << tpr_shift) - 1));
    if (c >= cpr) return;
    const int e0 = c * VEC;
    for (int64_t r = (int64_t)blockIdx.y * rpb + ((int)threadIdx.x >> tpr_shift); r < rows;
         r += (int64_t)gridDim.y * rpb) {
        const unsigned char *s = src + r * ld_bytes + (int64_t)e0 * ES;
        u32x4 v;
        if (e0 + VEC <= cols) {
            const uint32_t mis = (uint32_t)reinterpret_cast<uintptr_t>(s) & 3;   // 0 or 2
            const uint32_t *q = reinterpret_cast<const uint32_t *>(s - mis);
            const uint32_t sh = mis * 8;
            const uint32_t w0 = q[0], w1 = q[1], w2 = q[2], w3 = q[3];
            const uint32_t w4 = q[sh ? 4 : 3];
            v[0] = __builtin_amdgcn_alignbit(w1, w0, sh);
            v[1] = __builtin_amdgcn_alignbit(w2, w1, sh);
            v[2] = __builtin_amdgcn_alignbit(w3, w2, sh);
            v[3] = __builtin_amdgcn_alignbit(w4, w3, sh);
        } else {
            union {
                u32x4 v;
                E e[VEC];
            } u;
            const E *se = reinterpret_cast<const E *>(s);
#pragma unroll
            for (int e = 0; e < VEC; ++e) u.e[e] = e0 + e < cols ? se[e] : E(0);
            v = u.v;
        }
        *reinterpret_cast<u32x4 *>(dst + r * ldd_bytes + (int64_t)e0 * ES) = v;
    }
}

int grid_for(int64_t work, int threads)
{
    int64_t blocks = (work + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;  // grid-stride loops cover the rest
    return blocks < 1 ? 1 : (int)blocks;
}

}  // namespace

hipError_t launch_splitk_reduce(const float *ws, int splits, int M, int N, void *C, int64_t ldc,
                                float alpha, float beta, int out_bf16, hipStream_t stream)
{
    const int threads = 256;
    const bool vec = !out_bf16 && (N % 4 == 0) && (ldc % 4 == 0) && ((uintptr_t)C % 16 == 0);
    if (vec) {
        hipLaunchKernelGGL(splitk_reduce4_kernel, dim3(grid_for((int64_t)M * N / 4, threads)),
                           dim3(threads), 0, stream, ws, splits, M, N, static_cast<float *>(C), ldc,
                           alpha, beta);
    } else {
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid_for((int64_t)M * N, threads)),
                           dim3(threads), 0, stream, ws, splits, M, N, C, ldc, alpha, beta,
                           out_bf16);
    }
    return hipGetLastError();
}

hipError_t launch_stage_rows(const void *src, int64_t ld, int64_t rows, int64_t cols, int esize,
                             void *dst, int64_t ldd, hipStream_t stream)
{
    const int vec = 16 / esize;
    const int64_t cpr = (cols + vec - 1) / vec;
    int shift = 0;
    while ((int64_t(1) << shift) < cpr && shift < 8) ++shift;
    const int64_t rpb = 256 >> shift;
    const int64_t gx = (cpr + (int64_t(1) << shift) - 1) >> shift;
    int64_t gy = (rows + rpb - 1) / rpb;
    if (gy > 32768) gy = 32768;  // the row loop covers the rest
    if (esize == 2)
        hipLaunchKernelGGL(stage_rows_kernel<2>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0,
                           stream, static_cast<const unsigned char *>(src), ld * 2, rows,
                           (int)cols, (int)cpr, shift, static_cast<unsigned char *>(dst), ldd * 2);
    else
        hipLaunchKernelGGL(stage_rows_kernel<4>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0,
                           stream, static_cast<const unsigned char *>(src), ld * 4, rows,
                           (int)cols, (int)cpr, shift, static_cast<unsigned char *>(dst), ldd * 4);
    return hipGetLastError();
}

hipError_t launch_scale(int M, int N, void *C, int64_t ldc, float beta, int out_bf16,
                        hipStream_t stream)
{
    const int threads = 256;
    hipLaunchKernelGGL(scale_kernel, dim3(grid_for((int64_t)M * N, threads)), dim3(threads), 0,
                       stream, M, N, C, ldc, beta, out_bf16);
    return hipGetLastError();
}

}  // namespace dg
