// gemm_i8_bf16.hip — fused GEMM + bias + activation kernels, int8 operands (int32 bias), bf16 output.
#include "kernels_impl.hpp"

namespace biasact {
int launch_gemm_i8_bf16(int tile, const GemmArgs& a, hipStream_t s) {
  return launch_gemm_tile<DT_I8, DT_BF16>(tile, a, s);
}
}  // namespace biasact
