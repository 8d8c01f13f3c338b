// FP8 GEMM instances: NN layout, FP8 matrix-core accumulation.
#include "gemm_kernel.h"

namespace fp8mlp {

hipError_t launch_gemm_nn_fast(const GemmArgs& g, hipStream_t st) {
  return gemm_detail::launch_layout<kLayNN, kAccFast>(g, st);
}

}  // namespace fp8mlp
