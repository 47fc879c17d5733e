// Definition of the kernel launcher and the explicit instantiation of one
// operand layout's kernels from the tile lists.  Included by the per-layout
// source files, each of which defines DG_DTYPE_TABLE (the list), DG_LAYOUT
// (NN, NT, TN, TT, or CF / CW / CFT / CWT / C3F / C3W / CFP / CWP / C3FP /
// C3WP / CFW / CWW / C4F / C4W / C4FP / C4WP for the implicit-GEMM convolution
// kernels: forward / filter gradient, analytic / table-looked-up terms,
// volume, padded image, image windows, four dimensions) and then includes
// this header.
#pragma once

#include "gemm_configs.hpp"

namespace dg {

template <bool BF16, int BM, int BN, int BK, int WM, int WN, int STAGES, int LA, int LB,
          bool ALIGNED, int BSRC>
hipError_t launch_gemm(const KernelArgs &args, int blocks, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_kernel<BF16, BM, BN, BK, WM, WN, STAGES, LA, LB, ALIGNED, BSRC>),
                       dim3(blocks), dim3(64 * WM * WN), 0, stream, args);
    return hipGetLastError();
}

}  // namespace dg

// Explicit instantiation of both alignments of one entry for layout L.
#define DG_INST(BF16, BM, BN, BK, WM, WN, S, L)                                                 \
    template hipError_t dg::launch_gemm<BF16, BM, BN, BK, WM, WN, S, DG_LA_##L, DG_LB_##L,      \
                                        true, ::dg::B_MATRIX>(const dg::KernelArgs &, int,      \
                                                              hipStream_t);                      \
    template hipError_t dg::launch_gemm<BF16, BM, BN, BK, WM, WN, S, DG_LA_##L, DG_LB_##L,      \
                                        false, ::dg::B_MATRIX>(const dg::KernelArgs &, int,     \
                                                               hipStream_t);
// implicit-GEMM slice (CF or CW): two LDS stages
#define DG_IINST(BF16, BM, BN, BK, WM, WN, S, L)                                                \
    template hipError_t dg::launch_gemm<BF16, BM, BN, BK, WM, WN, 2, DG_LA_##L, DG_LB_##L,      \
                                        true, DG_BSRC_##L>(const dg::KernelArgs &, int,         \
                                                           hipStream_t);                         \
    template hipError_t dg::launch_gemm<BF16, BM, BN, BK, WM, WN, 2, DG_LA_##L, DG_LB_##L,      \
                                        false, DG_BSRC_##L>(const dg::KernelArgs &, int,        \
                                                            hipStream_t);
#define DG_INST_ALL_NN(...) DG_INST(__VA_ARGS__, NN)
#define DG_INST_ALL_NT(...) DG_INST(__VA_ARGS__, NT)
#define DG_INST_ALL_TN(...) DG_INST(__VA_ARGS__, TN)
#define DG_INST_ALL_TT(...) DG_INST(__VA_ARGS__, TT)
#define DG_INST_ALL_CF(...)
#define DG_INST_ALL_CW(...)
#define DG_INST_ALL_CFT(...)
#define DG_INST_ALL_CWT(...)
#define DG_INST_ALL_C3F(...)
#define DG_INST_ALL_C3W(...)
#define DG_INST_ALL_CFP(...)
#define DG_INST_ALL_CWP(...)
#define DG_INST_ALL_C3FP(...)
#define DG_INST_ALL_C3WP(...)
#define DG_INST_ALL_CFW(...)
#define DG_INST_ALL_CWW(...)
#define DG_INST_ALL_C4F(...)
#define DG_INST_ALL_C4W(...)
#define DG_INST_ALL_C4FP(...)
#define DG_INST_ALL_C4WP(...)
#define DG_INST_CONV_NN(...) DG_INST(__VA_ARGS__, NN)
#define DG_INST_CONV_NT(...) DG_INST(__VA_ARGS__, NT)
#define DG_INST_CONV_TN(...) DG_INST(__VA_ARGS__, TN)
#define DG_INST_CONV_TT(...) DG_INST(__VA_ARGS__, TT)
#define DG_INST_CONV_CF(...) DG_IINST(__VA_ARGS__, CF)
#define DG_INST_CONV_CW(...) DG_IINST(__VA_ARGS__, CW)
#define DG_INST_CONV_CFT(...) DG_IINST(__VA_ARGS__, CFT)
#define DG_INST_CONV_CWT(...) DG_IINST(__VA_ARGS__, CWT)
#define DG_INST_CONV_C3F(...) DG_IINST(__VA_ARGS__, C3F)
#define DG_INST_CONV_C3W(...) DG_IINST(__VA_ARGS__, C3W)
#define DG_INST_CONV_CFP(...) DG_IINST(__VA_ARGS__, CFP)
#define DG_INST_CONV_CWP(...) DG_IINST(__VA_ARGS__, CWP)
#define DG_INST_CONV_C3FP(...) DG_IINST(__VA_ARGS__, C3FP)
#define DG_INST_CONV_C3WP(...) DG_IINST(__VA_ARGS__, C3WP)
#define DG_INST_CONV_CFW(...) DG_IINST(__VA_ARGS__, CFW)
#define DG_INST_CONV_CWW(...) DG_IINST(__VA_ARGS__, CWW)
#define DG_INST_CONV_C4F(...) DG_IINST(__VA_ARGS__, C4F)
#define DG_INST_CONV_C4W(...) DG_IINST(__VA_ARGS__, C4W)
#define DG_INST_CONV_C4FP(...) DG_IINST(__VA_ARGS__, C4FP)
#define DG_INST_CONV_C4WP(...) DG_IINST(__VA_ARGS__, C4WP)
#define DG_INST_SKINNYC_NN(...) DG_INST(__VA_ARGS__, NN)
#define DG_INST_SKINNYC_NT(...) DG_INST(__VA_ARGS__, NT)
#define DG_INST_SKINNYC_TN(...)
#define DG_INST_SKINNYC_TT(...)
#define DG_INST_SKINNYC_CF(...) DG_IINST(__VA_ARGS__, CF)
#define DG_INST_SKINNYC_CW(...) DG_IINST(__VA_ARGS__, CW)
#define DG_INST_SKINNYC_CFT(...) DG_IINST(__VA_ARGS__, CFT)
#define DG_INST_SKINNYC_CWT(...) DG_IINST(__VA_ARGS__, CWT)
#define DG_INST_SKINNYC_C3F(...) DG_IINST(__VA_ARGS__, C3F)
#define DG_INST_SKINNYC_C3W(...) DG_IINST(__VA_ARGS__, C3W)
#define DG_INST_SKINNYC_CFP(...) DG_IINST(__VA_ARGS__, CFP)
#define DG_INST_SKINNYC_CWP(...) DG_IINST(__VA_ARGS__, CWP)
#define DG_INST_SKINNYC_C3FP(...) DG_IINST(__VA_ARGS__, C3FP)
#define DG_INST_SKINNYC_C3WP(...) DG_IINST(__VA_ARGS__, C3WP)
#define DG_INST_SKINNYC_CFW(...) DG_IINST(__VA_ARGS__, CFW)
#define DG_INST_SKINNYC_CWW(...) DG_IINST(__VA_ARGS__, CWW)
#define DG_INST_SKINNYC_C4F(...) DG_IINST(__VA_ARGS__, C4F)
#define DG_INST_SKINNYC_C4W(...) DG_IINST(__VA_ARGS__, C4W)
#define DG_INST_SKINNYC_C4FP(...) DG_IINST(__VA_ARGS__, C4FP)
#define DG_INST_SKINNYC_C4WP(...) DG_IINST(__VA_ARGS__, C4WP)
#define DG_INST_SKINNY_NN(...) DG_INST(__VA_ARGS__, NN)
#define DG_INST_SKINNY_NT(...) DG_INST(__VA_ARGS__, NT)
#define DG_INST_SKINNY_TN(...)
#define DG_INST_SKINNY_TT(...)
#define DG_INST_SKINNY_CF(...)
#define DG_INST_SKINNY_CW(...)
#define DG_INST_SKINNY_CFT(...)
#define DG_INST_SKINNY_CWT(...)
#define DG_INST_SKINNY_C3F(...)
#define DG_INST_SKINNY_C3W(...)
#define DG_INST_SKINNY_CFP(...)
#define DG_INST_SKINNY_CWP(...)
#define DG_INST_SKINNY_C3FP(...)
#define DG_INST_SKINNY_C3WP(...)
#define DG_INST_SKINNY_CFW(...)
#define DG_INST_SKINNY_CWW(...)
#define DG_INST_SKINNY_C4F(...)
#define DG_INST_SKINNY_C4W(...)
#define DG_INST_SKINNY_C4FP(...)
#define DG_INST_SKINNY_C4WP(...)
#define DG_INST_AK_NN(...) DG_INST(__VA_ARGS__, NN)
#define DG_INST_AK_NT(...) DG_INST(__VA_ARGS__, NT)
#define DG_INST_AK_TN(...)
#define DG_INST_AK_TT(...)
#define DG_INST_AK_CF(...)
#define DG_INST_AK_CW(...)
#define DG_INST_AK_CFT(...)
#define DG_INST_AK_CWT(...)
#define DG_INST_AK_C3F(...)
#define DG_INST_AK_C3W(...)
#define DG_INST_AK_CFP(...)
#define DG_INST_AK_CWP(...)
#define DG_INST_AK_C3FP(...)
#define DG_INST_AK_C3WP(...)
#define DG_INST_AK_CFW(...)
#define DG_INST_AK_CWW(...)
#define DG_INST_AK_C4F(...)
#define DG_INST_AK_C4W(...)
#define DG_INST_AK_C4FP(...)
#define DG_INST_AK_C4WP(...)
#define DG_INST_KK_NN(...)
#define DG_INST_KK_NT(...) DG_INST(__VA_ARGS__, NT)
#define DG_INST_KK_TN(...)
#define DG_INST_KK_TT(...)
#define DG_INST_KK_CF(...)
#define DG_INST_KK_CW(...)
#define DG_INST_KK_CFT(...)
#define DG_INST_KK_CWT(...)
#define DG_INST_KK_C3F(...)
#define DG_INST_KK_C3W(...)
#define DG_INST_KK_CFP(...)
#define DG_INST_KK_CWP(...)
#define DG_INST_KK_C3FP(...)
#define DG_INST_KK_C3WP(...)
#define DG_INST_KK_CFW(...)
#define DG_INST_KK_CWW(...)
#define DG_INST_KK_C4F(...)
#define DG_INST_KK_C4W(...)
#define DG_INST_KK_C4FP(...)
#define DG_INST_KK_C4WP(...)
#define DG_INST_NN_NN(...) DG_INST(__VA_ARGS__, NN)
#define DG_INST_NN_NT(...)
#define DG_INST_NN_TN(...)
#define DG_INST_NN_TT(...)
#define DG_INST_NN_CF(...)
#define DG_INST_NN_CW(...)
#define DG_INST_NN_CFT(...)
#define DG_INST_NN_CWT(...)
#define DG_INST_NN_C3F(...)
#define DG_INST_NN_C3W(...)
#define DG_INST_NN_CFP(...)
#define DG_INST_NN_CWP(...)
#define DG_INST_NN_C3FP(...)
#define DG_INST_NN_C3WP(...)
#define DG_INST_NN_CFW(...)
#define DG_INST_NN_CWW(...)
#define DG_INST_NN_C4F(...)
#define DG_INST_NN_C4W(...)
#define DG_INST_NN_C4FP(...)
#define DG_INST_NN_C4WP(...)
#define DG_INST_SEL2(LAYOUTS, L) DG_INST_##LAYOUTS##_##L
#define DG_INST_SEL(LAYOUTS, L) DG_INST_SEL2(LAYOUTS, L)
#define DG_INST_ENTRY(NAME, BF16, BM, BN, BK, WM, WN, S, G, LAYOUTS)                            \
    DG_INST_SEL(LAYOUTS, DG_LAYOUT)(BF16, BM, BN, BK, WM, WN, S)

DG_DTYPE_TABLE(DG_INST_ENTRY)
