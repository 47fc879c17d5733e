// Host-side description of the tile table: one entry per compiled kernel
// configuration, with launchers for the aligned (16-byte vector loads) and
// the unaligned (element-wise loads) variant.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.hpp"

namespace dg {

typedef hipError_t (*launch_fn)(const KernelArgs &args, int blocks, hipStream_t stream);

struct TileConfig {
    const char *name;
    int bm, bn, bk;
    int threads;
    int stages;
    int group_m;
    launch_fn aligned;    // needs 16-byte aligned rows of A and B
    launch_fn unaligned;  // element-wise loads, any alignment of the element type
};

template <bool BF16, int BM, int BN, int BK, int WM, int WN, int STAGES, bool ALIGNED>
hipError_t launch_gemm(const KernelArgs &args, int blocks, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_kernel<BF16, BM, BN, BK, WM, WN, STAGES, ALIGNED>), dim3(blocks),
                       dim3(64 * WM * WN), 0, stream, args);
    return hipGetLastError();
}

// One table entry: a name, the tile shape (BM x BN block, BK k-tile), the wave
// grid (WM x WN waves), the number of LDS stages and the raster group height.
#define DG_TILE_CONFIG(NAME, BF16, BM, BN, BK, WM, WN, STAGES, GROUP_M)                     \
    TileConfig                                                                             \
    {                                                                                      \
        NAME, BM, BN, BK, 64 * (WM) * (WN), STAGES, GROUP_M,                               \
            &launch_gemm<BF16, BM, BN, BK, WM, WN, STAGES, true>,                          \
            &launch_gemm<BF16, BM, BN, BK, WM, WN, STAGES, false>                          \
    }

// Tables, defined in gemm_f32.hip and gemm_bf16.hip.
const TileConfig *f32_configs(int *count);
const TileConfig *bf16_configs(int *count);

hipError_t launch_splitk_reduce(const float *ws, int splits, int M, int N, float *C, int64_t ldc,
                                hipStream_t stream);
hipError_t launch_zero_fill(int M, int N, float *C, int64_t ldc, hipStream_t stream);

}  // namespace dg
