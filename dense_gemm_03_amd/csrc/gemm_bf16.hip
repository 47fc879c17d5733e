// bf16 tile table: v_mfma_f32_32x32x16_bf16 kernels (fp32 accumulation).
#include "gemm_configs.hpp"

namespace dg {

// Host function (not device code), so the table stays on the host.
const TileConfig *bf16_configs(int *count)
{
    static const TileConfig table[] = {
        //              name                             bf16  BM   BN  BK WM WN  S   G
        DG_TILE_CONFIG("bf16_256x256x64_w2x2_s2", true, 256, 256, 64, 2, 2, 2, 8),
        DG_TILE_CONFIG("bf16_256x256x32_w2x2_s4", true, 256, 256, 32, 2, 2, 4, 8),
        DG_TILE_CONFIG("bf16_256x256x64_w4x2_s2", true, 256, 256, 64, 4, 2, 2, 8),
        DG_TILE_CONFIG("bf16_256x256x64_w2x4_s2", true, 256, 256, 64, 2, 4, 2, 8),
        DG_TILE_CONFIG("bf16_256x256x32_w4x2_s4", true, 256, 256, 32, 4, 2, 4, 4),
        DG_TILE_CONFIG("bf16_128x128x64_w2x2_s2", true, 128, 128, 64, 2, 2, 2, 8),
        DG_TILE_CONFIG("bf16_256x128x64_w2x2_s2", true, 256, 128, 64, 2, 2, 2, 8),
        DG_TILE_CONFIG("bf16_64x64x64_w2x2_s2", true, 64, 64, 64, 2, 2, 2, 8),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
