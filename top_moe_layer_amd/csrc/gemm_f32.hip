// fp32 instantiations of the grouped MFMA GEMM.
#include "gemm_impl.h"

namespace topmoe {

hipError_t launch_gemm_f32(int kind, GemmShape sh, const GemmParams& p, int64_t mtiles,
                           const Launch& s) {
  return launch_gemm_dtype<float>(kind, sh, p, mtiles, s);
}

}  // namespace topmoe
