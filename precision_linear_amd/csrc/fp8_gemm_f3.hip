// Kernels of the FP8 scaled multiply for A in e5m2 and B in e5m2.
#include "fp8_gemm_kernels.h"

FP8MM_DEFINE_LAUNCH_TABLE(kLaunchF3, 3)
