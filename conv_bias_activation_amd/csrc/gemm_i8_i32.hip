// gemm_i8_i32.hip — fused GEMM + bias + activation kernels, int8 operands (int32 bias), i32 output.
#include "kernels_impl.hpp"

namespace biasact {
int launch_gemm_i8_i32(int tile, const GemmArgs& a, hipStream_t s) {
  return launch_gemm_tile<DT_I8, DT_I32>(tile, a, s);
}
}  // namespace biasact
