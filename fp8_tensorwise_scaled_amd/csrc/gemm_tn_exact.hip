// FP8 GEMM instances: TN layout, exact-product accumulation.
#include "gemm_kernel.h"

namespace fp8mlp {

hipError_t launch_gemm_tn_exact(const GemmArgs& g, hipStream_t st) {
  return gemm_detail::launch_layout<kLayTN, kAccExact>(g, st);
}

}  // namespace fp8mlp
