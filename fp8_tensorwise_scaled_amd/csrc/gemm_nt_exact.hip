// FP8 GEMM instances: NT layout, exact-product accumulation.
#include "gemm_kernel.h"

namespace fp8mlp {

hipError_t launch_gemm_nt_exact(const GemmArgs& g, hipStream_t st) {
  return gemm_detail::launch_layout<kLayNT, kAccExact>(g, st);
}

}  // namespace fp8mlp
