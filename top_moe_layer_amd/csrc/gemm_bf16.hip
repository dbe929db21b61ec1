// bf16 instantiations of the grouped MFMA GEMM.
#include "gemm_impl.h"

namespace topmoe {

hipError_t launch_gemm_bf16(int kind, GemmShape sh, const GemmParams& p, int64_t mtiles,
                            const Launch& s) {
  return launch_gemm_dtype<bf16_t>(kind, sh, p, mtiles, s);
}

bool gemm_shape_supported_bf16(int kind, const GemmShape& sh) {
  return shape_supported_dtype<bf16_t>(kind, sh);
}

}  // namespace topmoe
