// The block-scaled GEMM kernels (gemm_fast_kernel: W4A4 and W4A8) in an object of their
// own.  It is the same source as gemm.hip, built with LLVM's machine sinking off: the
// steady K loop is unrolled by the LDS ring depth so that every ring slot is a constant,
// and machine sinking would move a window's MFMAs past the next window's scale-chunk
// branch, behind that window's barrier, serializing them after its loads.  The other
// GEMM kernels (gemm.hip) keep the pass.
#define MXQ_GEMM_SCALED_OBJECT 1
#include "gemm.hip"
