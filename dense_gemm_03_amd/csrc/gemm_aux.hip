// Launchers of the split-K reduce and of the zero fill (K == 0).
#include "gemm_configs.hpp"

namespace dg {

// Sum the split-K partial products in slice order (deterministic) into C.
__global__ void splitk_reduce_kernel(const float *__restrict__ ws, int splits, int M, int N,
                                     float *__restrict__ C, int64_t ldc)
{
    const int64_t total = (int64_t)M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        float s = ws[idx];
        for (int z = 1; z < splits; ++z) s += ws[(int64_t)z * total + idx];
        const int64_t i = idx / N, j = idx - i * N;
        C[i * ldc + j] = s;
    }
}

// Vector form of the reduce: 4 consecutive columns per thread (N % 4 == 0,
// ldc % 4 == 0, C 16-byte aligned).
__global__ void splitk_reduce4_kernel(const float *__restrict__ ws, int splits, int M, int N,
                                      float *__restrict__ C, int64_t ldc)
{
    typedef float floatx4 __attribute__((ext_vector_type(4)));
    const int64_t total4 = (int64_t)M * N / 4;
    const int64_t plane4 = total4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const floatx4 *w = reinterpret_cast<const floatx4 *>(ws);
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total4; idx += stride) {
        floatx4 s = w[idx];
        for (int z = 1; z < splits; ++z) s += w[(int64_t)z * plane4 + idx];
        const int64_t e = idx * 4;
        const int64_t i = e / N, j = e - i * N;
        *reinterpret_cast<floatx4 *>(C + i * ldc + j) = s;
    }
}

// C := 0 over the M x N window (the empty sum, K == 0).
__global__ void zero_fill_kernel(int M, int N, float *__restrict__ C, int64_t ldc)
{
    const int64_t total = (int64_t)M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        const int64_t i = idx / N, j = idx - i * N;
        C[i * ldc + j] = 0.0f;
    }
}

static int grid_for(int64_t work, int threads)
{
    int64_t blocks = (work + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;  // grid-stride loops cover the rest
    return blocks < 1 ? 1 : (int)blocks;
}

hipError_t launch_splitk_reduce(const float *ws, int splits, int M, int N, float *C, int64_t ldc,
                                hipStream_t stream)
{
    const int threads = 256;
    const bool vec = (N % 4 == 0) && (ldc % 4 == 0) && ((uintptr_t)C % 16 == 0);
    if (vec) {
        hipLaunchKernelGGL(splitk_reduce4_kernel, dim3(grid_for((int64_t)M * N / 4, threads)),
                           dim3(threads), 0, stream, ws, splits, M, N, C, ldc);
    } else {
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid_for((int64_t)M * N, threads)),
                           dim3(threads), 0, stream, ws, splits, M, N, C, ldc);
    }
    return hipGetLastError();
}

hipError_t launch_zero_fill(int M, int N, float *C, int64_t ldc, hipStream_t stream)
{
    const int threads = 256;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(grid_for((int64_t)M * N, threads)), dim3(threads),
                       0, stream, M, N, C, ldc);
    return hipGetLastError();
}

}  // namespace dg
