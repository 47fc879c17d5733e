// The split-K reduce and the scale kernel (K == 0 or alpha == 0), with their
// launchers.  Both finish elements of C the way the GEMM epilogue does:
// alpha * sum + beta * C (C read only when beta != 0), stored as fp32 or bf16.
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

hipError_t launch_scale(int M, int N, void *C, int64_t ldc, float beta, int out_bf16,
                        hipStream_t stream)
{
    const int threads = 256;
    hipLaunchKernelGGL(scale_kernel, dim3(grid_for((int64_t)M * N, threads)), dim3(threads), 0,
                       stream, M, N, C, ldc, beta, out_bf16);
    return hipGetLastError();
}

}  // namespace dg
