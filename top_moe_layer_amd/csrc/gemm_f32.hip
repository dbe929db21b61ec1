// fp32 instantiations of the grouped MFMA GEMM.
#include "gemm_impl.h"

namespace topmoe {

hipError_t launch_gemm_f32(int kind, GemmShape sh, const GemmParams& p, int64_t mtiles,
                           const Launch& s) {
  return launch_gemm_dtype<float>(kind, sh, p, mtiles, s);
}

bool gemm_shape_supported_f32(int kind, const GemmShape& sh) {
  return shape_supported_dtype<float>(kind, sh);
}

}  // namespace topmoe
