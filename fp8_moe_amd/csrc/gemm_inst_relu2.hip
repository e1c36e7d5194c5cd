// Instantiations of the grouped GEMM kernel (gemm_kernel.h), one translation
// unit per group so that the build compiles them in parallel.
#include "gemm_kernel.h"

namespace b12x {

B12X_GEMM_INST(B12X_WEIGHT_MXFP4, B12X_ACT_MXFP8, MODE_RELU2)
B12X_GEMM_INST(B12X_WEIGHT_NVFP4, kActRt, MODE_RELU2)
B12X_GEMM_INST(B12X_WEIGHT_NVFP4, B12X_ACT_BF16, MODE_RELU2)
B12X_GEMM_INST(B12X_WEIGHT_MXFP4, B12X_ACT_BF16, MODE_RELU2)

}  // namespace b12x
