// gemm_i8_f32.hip — fused GEMM + bias + activation kernels, int8 operands (int32 bias), f32 output.
#include "kernels_impl.hpp"

namespace biasact {
int launch_gemm_i8_f32(int tile, const GemmArgs& a, hipStream_t s) {
  return launch_gemm_tile<DT_I8, DT_F32>(tile, a, s);
}
}  // namespace biasact
