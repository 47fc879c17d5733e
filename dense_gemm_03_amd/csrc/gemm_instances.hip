// One slice of the kernel instantiations: the kernels of one input type and
// one operand layout.  The build compiles this file once per slice, with
// DG_DTYPE_TABLE set to DG_F32_TABLE or DG_BF16_TABLE and DG_LAYOUT to NN,
// NT, TN, TT, or CF / CW (the implicit-GEMM convolution kernels: forward,
// filter gradient), so the slices compile in parallel.
#if !defined(DG_DTYPE_TABLE) || !defined(DG_LAYOUT)
#error "define DG_DTYPE_TABLE and DG_LAYOUT"
#endif
#include "gemm_launch.hpp"
