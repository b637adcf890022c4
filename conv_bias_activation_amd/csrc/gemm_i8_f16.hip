// gemm_i8_f16.hip — fused GEMM + bias + activation kernels, int8 operands (int32 bias), f16 output.
#include "kernels_impl.hpp"

namespace biasact {
int launch_gemm_i8_f16(int tile, const GemmArgs& a, hipStream_t s) {
  return launch_gemm_tile<DT_I8, DT_F16>(tile, a, s);
}
}  // namespace biasact
