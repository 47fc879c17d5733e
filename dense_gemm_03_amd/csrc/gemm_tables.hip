// The fp32 (v_mfma_f32_32x32x2_f32) and bf16 (v_mfma_f32_32x32x16_bf16, fp32
// accumulation) tile tables, built from the lists in gemm_configs.hpp.  The
// kernels themselves are instantiated in gemm_instances.hip.
#include "gemm_configs.hpp"

namespace dg {

// Host functions (not device code), so the tables stay on the host.
const TileConfig *f32_configs(int *count)
{
    static const TileConfig table[] = {DG_F32_TABLE(DG_TABLE_ENTRY)};
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

const TileConfig *bf16_configs(int *count)
{
    static const TileConfig table[] = {DG_BF16_TABLE(DG_TABLE_ENTRY)};
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
