// fp32 tile table: v_mfma_f32_32x32x2_f32 kernels.
//
// Shape classes (tile sizes per task, "How to do even better" on the GEMM
// page): square/large blocks for big M and N, a wide-N block with split-K for
// M of a few dozen rows and long K (the im2col weight-gradient shape), a
// tall block for N of a few dozen columns, and a small block when the output
// holds too few large blocks to fill 256 compute units.
#include "gemm_configs.hpp"

namespace dg {

// Host function (not device code), so the table stays on the host.
const TileConfig *f32_configs(int *count)
{
    static const TileConfig table[] = {
        //              name                    bf16   BM   BN  BK WM WN  S  G
        DG_TILE_CONFIG("f32_256x128_w4x2_s2", false, 256, 128, 32, 4, 2, 2, 8),
        DG_TILE_CONFIG("f32_128x128_w2x2_s2", false, 128, 128, 32, 2, 2, 2, 8),
        DG_TILE_CONFIG("f32_256x256_w4x2_s2", false, 256, 256, 32, 4, 2, 2, 8),
        DG_TILE_CONFIG("f32_64x64_w2x2_s2", false, 64, 64, 32, 2, 2, 2, 8),
        DG_TILE_CONFIG("f32_64x64_w2x2_s3", false, 64, 64, 32, 2, 2, 3, 8),
        DG_TILE_CONFIG("f32_64x256_w1x4_s3", false, 64, 256, 32, 1, 4, 3, 1),
        DG_TILE_CONFIG("f32_64x256_w1x4_s4", false, 64, 256, 32, 1, 4, 4, 1),
        DG_TILE_CONFIG("f32_64x128_w1x2_s4", false, 64, 128, 32, 1, 2, 4, 1),
        DG_TILE_CONFIG("f32_256x64_w4x1_s3", false, 256, 64, 32, 4, 1, 3, 8),
        DG_TILE_CONFIG("f32_128x64_w2x1_s2", false, 128, 64, 32, 2, 1, 2, 8),
        DG_TILE_CONFIG("f32_128x64_w2x2_s2", false, 128, 64, 32, 2, 2, 2, 8),
        DG_TILE_CONFIG("f32_128x64_w4x1_s2", false, 128, 64, 32, 4, 1, 2, 8),
        DG_TILE_CONFIG("f32_64x64_w1x1_s2", false, 64, 64, 32, 1, 1, 2, 8),
        DG_TILE_CONFIG("f32_64x64_w1x1_s4", false, 64, 64, 32, 1, 1, 4, 8),
        DG_TILE_CONFIG("f32_64x256_w1x4_s2", false, 64, 256, 32, 1, 4, 2, 1),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
