// Instantiations of the grouped GEMM kernel (gemm_kernel.h), one translation
// unit per group so that the build compiles them in parallel.
#include "gemm_kernel.h"

namespace b12x {

B12X_GEMM_INST(B12X_WEIGHT_NVFP4, kActF16NvRt, MODE_RELU2)
B12X_GEMM_INST(B12X_WEIGHT_NVFP4, kActF16Rt, MODE_RELU2)
B12X_GEMM_INST(B12X_WEIGHT_NVFP4, kActF16, MODE_RELU2)

}  // namespace b12x
