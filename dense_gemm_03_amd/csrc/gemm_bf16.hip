// bf16 tile table: v_mfma_f32_32x32x16_bf16 kernels (fp32 accumulation).
#include "gemm_configs.hpp"

namespace dg {

// Host function (not device code), so the table stays on the host.
const TileConfig *bf16_configs(int *count)
{
    static const TileConfig table[] = {
        DG_TILE_CONFIG("bf16_256x256_w2x2", true, 256, 256, 2, 2, 8),
        DG_TILE_CONFIG("bf16_128x128_w2x2", true, 128, 128, 2, 2, 8),
        DG_TILE_CONFIG("bf16_256x128_w2x2", true, 256, 128, 2, 2, 8),
        DG_TILE_CONFIG("bf16_64x64_w2x2", true, 64, 64, 2, 2, 8),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
