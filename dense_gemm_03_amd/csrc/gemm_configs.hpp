// Host-side description of the tile table: one entry per kernel
// configuration, with launchers for each operand layout it is built for and,
// per layout, an aligned (16-byte vector loads) and an unaligned (element-wise
// loads) variant.
//
// The entries are listed once, in the X-macro lists below.  Each list item is
//   X(NAME, BF16, BM, BN, BK, WM, WN, STAGES, GROUP_M, LAYOUTS)
// with the tile shape (BM x BN block, BK k-tile), the wave grid (WM x WN
// waves), the number of LDS stages, the raster group height, and LAYOUTS =
// ALL (kernels for all four combinations of transposed operands), CONV (ALL,
// plus implicit-GEMM convolution kernels), NN (only A and B as given),
// SKINNY (A . B and A . B^T), SKINNYC (SKINNY plus implicit-GEMM kernels),
// KK (only A . B^T) or AK (A . B and A . B^T: the forms that read A
// k-contiguous, for large blocks).  The kernels of one input type and operand layout are
// instantiated by one compilation of gemm_instances.hip, so the slices compile
// in parallel; the tables (gemm_tables.hip) only take their addresses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.hpp"

namespace dg {

typedef hipError_t (*launch_fn)(const KernelArgs &args, int blocks, hipStream_t stream);

// Operand layout combinations, indexed by transa * 2 + transb.
enum { LAYOUT_NN = 0, LAYOUT_NT = 1, LAYOUT_TN = 2, LAYOUT_TT = 3 };

struct TileConfig {
    const char *name;
    int bm, bn, bk;
    int threads;
    int stages;
    int group_m;
    // fn[layout][0]: needs 16-byte aligned rows of A and B; fn[layout][1]:
    // element-wise loads, any alignment of the element type.  nullptr where
    // the entry has no kernel for that layout.
    launch_fn fn[4][2];
    // implicit-GEMM convolution kernels (B tiles formed from an image),
    // indexed by B source - 1: [0] forward (B = cols), [1] filter gradient
    // (B = cols^T), [2] / [3] the same with table-looked-up per-k terms,
    // [4] / [5] the volume (3-D) forms, [6] .. [9] the 2-D and volume forms
    // reading a zero-padded image, [10] / [11] the 2-D forward product and
    // filter gradient from image windows in LDS, [12] .. [15] the
    // four-dimensional forms (forward, filter gradient; on the image, on its
    // zero-padded copy); [aligned], as fn.  nullptr where the entry has none.
    launch_fn implicit[16][2];
};

// Declared here; defined in gemm_launch.hpp and explicitly instantiated by the
// compilations of gemm_instances.hip.
template <bool BF16, int BM, int BN, int BK, int WM, int WN, int STAGES, int LA, int LB,
          bool ALIGNED, int BSRC>
hipError_t launch_gemm(const KernelArgs &args, int blocks, hipStream_t stream);

// Implicit-GEMM slices: forward (A = filters k-contiguous, B = convolution
// matrix tiles n-contiguous) and filter gradient (A = output gradient
// k-contiguous, B = transposed matrix tiles k-contiguous).  They run the
// register-staged loop, which uses two LDS stages.
#define DG_LA_CF ::dg::KMAJOR
#define DG_LB_CF ::dg::MNMAJOR
#define DG_LA_CW ::dg::KMAJOR
#define DG_LB_CW ::dg::KMAJOR
#define DG_BSRC_CF ::dg::B_CONV_FWD
#define DG_BSRC_CW ::dg::B_CONV_WGRAD
#define DG_LA_CFT ::dg::KMAJOR
#define DG_LB_CFT ::dg::MNMAJOR
#define DG_LA_CWT ::dg::KMAJOR
#define DG_LB_CWT ::dg::KMAJOR
#define DG_BSRC_CFT ::dg::B_CONV_FWD_TAB
#define DG_BSRC_CWT ::dg::B_CONV_WGRAD_TAB
#define DG_LA_C3F ::dg::KMAJOR
#define DG_LB_C3F ::dg::MNMAJOR
#define DG_LA_C3W ::dg::KMAJOR
#define DG_LB_C3W ::dg::KMAJOR
#define DG_BSRC_C3F ::dg::B_CONV3_FWD
#define DG_BSRC_C3W ::dg::B_CONV3_WGRAD
#define DG_LA_CFP ::dg::KMAJOR
#define DG_LB_CFP ::dg::MNMAJOR
#define DG_LA_CWP ::dg::KMAJOR
#define DG_LB_CWP ::dg::KMAJOR
#define DG_LA_C3FP ::dg::KMAJOR
#define DG_LB_C3FP ::dg::MNMAJOR
#define DG_LA_C3WP ::dg::KMAJOR
#define DG_LB_C3WP ::dg::KMAJOR
#define DG_BSRC_CFP ::dg::B_CONV_FWD_PAD
#define DG_BSRC_CWP ::dg::B_CONV_WGRAD_PAD
#define DG_BSRC_C3FP ::dg::B_CONV3_FWD_PAD
#define DG_BSRC_C3WP ::dg::B_CONV3_WGRAD_PAD
#define DG_LA_CFW ::dg::KMAJOR
#define DG_LB_CFW ::dg::MNMAJOR
#define DG_BSRC_CFW ::dg::B_CONV_FWD_WIN
#define DG_LA_CWW ::dg::KMAJOR
#define DG_LB_CWW ::dg::KMAJOR
#define DG_BSRC_CWW ::dg::B_CONV_WGRAD_WIN
#define DG_LA_C4F ::dg::KMAJOR
#define DG_LB_C4F ::dg::MNMAJOR
#define DG_BSRC_C4F ::dg::B_CONV4_FWD
#define DG_LA_C4W ::dg::KMAJOR
#define DG_LB_C4W ::dg::KMAJOR
#define DG_BSRC_C4W ::dg::B_CONV4_WGRAD
#define DG_LA_C4FP ::dg::KMAJOR
#define DG_LB_C4FP ::dg::MNMAJOR
#define DG_BSRC_C4FP ::dg::B_CONV4_FWD_PAD
#define DG_LA_C4WP ::dg::KMAJOR
#define DG_LB_C4WP ::dg::KMAJOR
#define DG_BSRC_C4WP ::dg::B_CONV4_WGRAD_PAD

// Memory orientation of op(A) / op(B) per layout combination: A as given is
// k-contiguous, A^T (stored K x M) outer-contiguous; B as given is
// outer-contiguous, B^T (stored N x K) k-contiguous.
#define DG_LA_NN ::dg::KMAJOR
#define DG_LB_NN ::dg::MNMAJOR
#define DG_LA_NT ::dg::KMAJOR
#define DG_LB_NT ::dg::KMAJOR
#define DG_LA_TN ::dg::MNMAJOR
#define DG_LB_TN ::dg::MNMAJOR
#define DG_LA_TT ::dg::MNMAJOR
#define DG_LB_TT ::dg::KMAJOR

// The tile tables.  The shape classes they serve (tile sizes per task, "How to
// do even better" on the GEMM page): square/large blocks for big M and N; for
// M of a few dozen rows and wide N (the convolution GEMMs), 32- and 64-row
// blocks with split-K, including A . B^T blocks with long k-contiguous rows;
// a tall block for N of a few dozen columns; and a small block when the
// output holds too few large blocks to fill 256 compute units; large bf16
// blocks with 64-deep k-tiles for the forms that read A k-contiguous.
// Entries the dispatcher picks for only some operand forms (SKINNY, SKINNYC,
// KK, AK) are built only for those forms; the others for all four.
#define DG_F32_TABLE(X)                                                     \
    X("f32_256x128_w4x2_s2", false, 256, 128, 32, 4, 2, 2, 8, CONV)         \
    X("f32_128x128_w2x2_s2", false, 128, 128, 32, 2, 2, 2, 8, CONV)         \
    X("f32_256x256_w4x2_s2", false, 256, 256, 32, 4, 2, 2, 8, ALL)          \
    X("f32_64x64_w2x2_s2", false, 64, 64, 32, 2, 2, 2, 8, ALL)              \
    X("f32_64x64_w2x2_s3", false, 64, 64, 32, 2, 2, 3, 8, ALL)              \
    X("f32_64x256_w1x4_s3", false, 64, 256, 32, 1, 4, 3, 1, CONV)           \
    X("f32_64x256_w1x4_s4", false, 64, 256, 32, 1, 4, 4, 1, NN)             \
    X("f32_64x128_w1x2_s4", false, 64, 128, 32, 1, 2, 4, 1, NN)             \
    X("f32_256x64_w4x1_s3", false, 256, 64, 32, 4, 1, 3, 8, NN)             \
    X("f32_128x64_w2x1_s2", false, 128, 64, 32, 2, 1, 2, 8, ALL)            \
    X("f32_128x64_w2x2_s2", false, 128, 64, 32, 2, 2, 2, 8, ALL)            \
    X("f32_128x64_w4x1_s2", false, 128, 64, 32, 4, 1, 2, 8, NN)             \
    X("f32_64x64_w1x1_s2", false, 64, 64, 32, 1, 1, 2, 8, NN)               \
    X("f32_64x64_w1x1_s4", false, 64, 64, 32, 1, 1, 4, 8, NN)               \
    X("f32_64x256_w1x4_s2", false, 64, 256, 32, 1, 4, 2, 1, NN)             \
    X("f32_32x256_w1x4_s2", false, 32, 256, 32, 1, 4, 2, 1, SKINNY)         \
    X("f32_32x256_w1x4_s3", false, 32, 256, 32, 1, 4, 3, 1, SKINNYC)        \
    X("f32_32x128_w1x2_s3", false, 32, 128, 32, 1, 2, 3, 1, SKINNY)         \
    X("f32_32x128_w1x4_s3", false, 32, 128, 32, 1, 4, 3, 1, SKINNYC)        \
    X("f32_32x128x64_w1x4_s2", false, 32, 128, 64, 1, 4, 2, 1, KK)          \
    X("f32_32x128x64_w1x4_s3", false, 32, 128, 64, 1, 4, 3, 1, KK)          \
    X("f32_32x256x64_w1x4_s2", false, 32, 256, 64, 1, 4, 2, 1, KK)          \
    X("f32_64x128x64_w1x4_s2", false, 64, 128, 64, 1, 4, 2, 1, KK)         \
    X("f32_64x64x64_w2x2_s2", false, 64, 64, 64, 2, 2, 2, 1, KK)

#define DG_BF16_TABLE(X)                                                    \
    X("bf16_256x256x32_w4x2_s4", true, 256, 256, 32, 4, 2, 4, 8, ALL)       \
    X("bf16_128x128x64_w2x2_s2", true, 128, 128, 64, 2, 2, 2, 8, CONV)      \
    X("bf16_256x128x64_w2x2_s2", true, 256, 128, 64, 2, 2, 2, 8, CONV)      \
    X("bf16_64x64x64_w2x2_s2", true, 64, 64, 64, 2, 2, 2, 8, ALL)           \
    X("bf16_64x256x64_w1x4_s3", true, 64, 256, 64, 1, 4, 3, 1, CONV)        \
    X("bf16_64x256x64_w1x4_s2", true, 64, 256, 64, 1, 4, 2, 1, NN)         \
    X("bf16_32x256x64_w1x4_s2", true, 32, 256, 64, 1, 4, 2, 1, SKINNY)     \
    X("bf16_32x256x64_w1x4_s3", true, 32, 256, 64, 1, 4, 3, 1, SKINNYC)    \
    X("bf16_32x128x64_w1x2_s3", true, 32, 128, 64, 1, 2, 3, 1, SKINNY)     \
    X("bf16_32x256x128_w1x4_s2", true, 32, 256, 128, 1, 4, 2, 1, KK)       \
    X("bf16_32x128x128_w1x4_s2", true, 32, 128, 128, 1, 4, 2, 1, KK)       \
    X("bf16_32x128x128_w1x4_s3", true, 32, 128, 128, 1, 4, 3, 1, KK)       \
    X("bf16_64x128x128_w1x4_s2", true, 64, 128, 128, 1, 4, 2, 1, KK)       \
    X("bf16_64x64x256_w2x2_s2", true, 64, 64, 256, 2, 2, 2, 1, KK)         \
    X("bf16_64x64x64_w2x2_s4", true, 64, 64, 64, 2, 2, 4, 1, ALL)          \
    X("bf16_256x256x64_w4x2_s2", true, 256, 256, 64, 4, 2, 2, 8, AK)        \
    X("bf16_128x128x64_w2x2_s3", true, 128, 128, 64, 2, 2, 3, 8, ALL)       \
    X("bf16_192x256x64_w2x4_s2", true, 192, 256, 64, 2, 4, 2, 8, AK)

// Launcher pointers of one entry and layout: both alignments, or nullptr.
#define DG_FNS(BF16, BM, BN, BK, WM, WN, S, L)                                               \
    {&launch_gemm<BF16, BM, BN, BK, WM, WN, S, DG_LA_##L, DG_LB_##L, true, ::dg::B_MATRIX>,  \
     &launch_gemm<BF16, BM, BN, BK, WM, WN, S, DG_LA_##L, DG_LB_##L, false, ::dg::B_MATRIX>}
#define DG_IFNS(BF16, BM, BN, BK, WM, WN, L)                                                 \
    {&launch_gemm<BF16, BM, BN, BK, WM, WN, 2, DG_LA_##L, DG_LB_##L, true, DG_BSRC_##L>,     \
     &launch_gemm<BF16, BM, BN, BK, WM, WN, 2, DG_LA_##L, DG_LB_##L, false, DG_BSRC_##L>}
#define DG_NOFNS {nullptr, nullptr}
#define DG_FNS_ALL_NN(...) DG_FNS(__VA_ARGS__, NN)
#define DG_FNS_ALL_NT(...) DG_FNS(__VA_ARGS__, NT)
#define DG_FNS_ALL_TN(...) DG_FNS(__VA_ARGS__, TN)
#define DG_FNS_ALL_TT(...) DG_FNS(__VA_ARGS__, TT)
#define DG_FNS_CONV_NN(...) DG_FNS(__VA_ARGS__, NN)
#define DG_FNS_CONV_NT(...) DG_FNS(__VA_ARGS__, NT)
#define DG_FNS_CONV_TN(...) DG_FNS(__VA_ARGS__, TN)
#define DG_FNS_CONV_TT(...) DG_FNS(__VA_ARGS__, TT)
#define DG_FNS_SKINNYC_NN(...) DG_FNS(__VA_ARGS__, NN)
#define DG_FNS_SKINNYC_NT(...) DG_FNS(__VA_ARGS__, NT)
#define DG_FNS_SKINNYC_TN(...) DG_NOFNS
#define DG_FNS_SKINNYC_TT(...) DG_NOFNS
#define DG_FNS_SKINNY_NN(...) DG_FNS(__VA_ARGS__, NN)
#define DG_FNS_SKINNY_NT(...) DG_FNS(__VA_ARGS__, NT)
#define DG_FNS_SKINNY_TN(...) DG_NOFNS
#define DG_FNS_SKINNY_TT(...) DG_NOFNS
#define DG_FNS_KK_NN(...) DG_NOFNS
#define DG_FNS_KK_NT(...) DG_FNS(__VA_ARGS__, NT)
#define DG_FNS_KK_TN(...) DG_NOFNS
#define DG_FNS_KK_TT(...) DG_NOFNS
#define DG_FNS_AK_NN(...) DG_FNS(__VA_ARGS__, NN)
#define DG_FNS_AK_NT(...) DG_FNS(__VA_ARGS__, NT)
#define DG_FNS_AK_TN(...) DG_NOFNS
#define DG_FNS_AK_TT(...) DG_NOFNS
#define DG_FNS_NN_NN(...) DG_FNS(__VA_ARGS__, NN)
#define DG_FNS_NN_NT(...) DG_NOFNS
#define DG_FNS_NN_TN(...) DG_NOFNS
#define DG_FNS_NN_TT(...) DG_NOFNS

#define DG_IMPL_CONV(BF16, BM, BN, BK, WM, WN)                                                \
    {DG_IFNS(BF16, BM, BN, BK, WM, WN, CF), DG_IFNS(BF16, BM, BN, BK, WM, WN, CW),              \
     DG_IFNS(BF16, BM, BN, BK, WM, WN, CFT), DG_IFNS(BF16, BM, BN, BK, WM, WN, CWT),            \
     DG_IFNS(BF16, BM, BN, BK, WM, WN, C3F), DG_IFNS(BF16, BM, BN, BK, WM, WN, C3W),            \
     DG_IFNS(BF16, BM, BN, BK, WM, WN, CFP), DG_IFNS(BF16, BM, BN, BK, WM, WN, CWP),            \
     DG_IFNS(BF16, BM, BN, BK, WM, WN, C3FP), DG_IFNS(BF16, BM, BN, BK, WM, WN, C3WP),          \
     DG_IFNS(BF16, BM, BN, BK, WM, WN, CFW), DG_IFNS(BF16, BM, BN, BK, WM, WN, CWW),            \
     DG_IFNS(BF16, BM, BN, BK, WM, WN, C4F), DG_IFNS(BF16, BM, BN, BK, WM, WN, C4W),            \
     DG_IFNS(BF16, BM, BN, BK, WM, WN, C4FP), DG_IFNS(BF16, BM, BN, BK, WM, WN, C4WP)}
#define DG_IMPL_NONE                                                                          \
    {DG_NOFNS, DG_NOFNS, DG_NOFNS, DG_NOFNS, DG_NOFNS, DG_NOFNS, DG_NOFNS, DG_NOFNS, DG_NOFNS, \
     DG_NOFNS, DG_NOFNS, DG_NOFNS, DG_NOFNS, DG_NOFNS, DG_NOFNS, DG_NOFNS}
#define DG_IMPL_ALL(...) DG_IMPL_NONE
#define DG_IMPL_NN(...) DG_IMPL_NONE
#define DG_IMPL_SKINNY(...) DG_IMPL_NONE
#define DG_IMPL_SKINNYC(...) DG_IMPL_CONV(__VA_ARGS__)
#define DG_IMPL_KK(...) DG_IMPL_NONE
#define DG_IMPL_AK(...) DG_IMPL_NONE

// One table entry from one list item.
#define DG_TABLE_ENTRY(NAME, BF16, BM, BN, BK, WM, WN, S, G, LAYOUTS)                        \
    TileConfig{NAME, BM, BN, BK, 64 * (WM) * (WN), S, G,                                    \
               {DG_FNS_##LAYOUTS##_NN(BF16, BM, BN, BK, WM, WN, S),                         \
                DG_FNS_##LAYOUTS##_NT(BF16, BM, BN, BK, WM, WN, S),                         \
                DG_FNS_##LAYOUTS##_TN(BF16, BM, BN, BK, WM, WN, S),                         \
                DG_FNS_##LAYOUTS##_TT(BF16, BM, BN, BK, WM, WN, S)},                        \
               DG_IMPL_##LAYOUTS(BF16, BM, BN, BK, WM, WN)},

// Tables, defined in gemm_tables.hip.
const TileConfig *f32_configs(int *count);
const TileConfig *bf16_configs(int *count);

// Split-K reduce: C := alpha * (sum of the slices, in slice order) + beta * C
// (C read only when beta != 0), stored as fp32 or bf16.
hipError_t launch_splitk_reduce(const float *ws, int splits, int M, int N, void *C, int64_t ldc,
                                float alpha, float beta, int out_bf16, hipStream_t stream);
// Copies a stored operand (rows x cols elements of esize bytes at pitch ld,
// any esize-aligned address) into dst (16-byte aligned) at pitch ldd, a
// multiple of 16 bytes no smaller than the row; the columns from cols up to
// the next multiple of 16 bytes are written as zeros.
hipError_t launch_stage_rows(const void *src, int64_t ld, int64_t rows, int64_t cols, int esize,
                             void *dst, int64_t ldd, hipStream_t stream);
// C := beta * C over the M x N window, or C := 0 when beta == 0 (C not read):
// the whole result when K == 0 or alpha == 0.
hipError_t launch_scale(int M, int N, void *C, int64_t ldc, float beta, int out_bf16,
                        hipStream_t stream);

}  // namespace dg
