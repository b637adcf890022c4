// gemm_f16.hip — fused GEMM + bias + activation kernels for f16 inputs.
#include "kernels_impl.hpp"

namespace biasact {
int launch_gemm_f16(int dto, int tile, const GemmArgs& a, hipStream_t s) {
  return launch_gemm_in<DT_F16>(dto, tile, a, s);
}
}  // namespace biasact
