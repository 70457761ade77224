// The W4A8 (FP8 E4M3 activations x MXFP4 weights) instance of gemm_fast_kernel, in an
// object of its own.  It is the same source, built with LLVM's machine sinking off: its
// steady K loop is unrolled by the LDS ring depth (3) so that every ring slot is a
// constant, and machine sinking would move a window's MFMAs past the next window's
// scale-chunk branch (behind that window's barrier), serializing them after the loads.
// The W4A4 build keeps the pass (without it the W4A4 loop spills), hence two objects.
#define MXQ_GEMM_W4A8_OBJECT 1
#include "gemm.hip"
