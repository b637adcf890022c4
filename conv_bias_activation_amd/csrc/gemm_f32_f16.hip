// gemm_f32_f16.hip — fused GEMM + bias + activation kernels, f32 operands, f16 output.
#include "kernels_impl.hpp"

namespace biasact {
int launch_gemm_f32_f16(int tile, const GemmArgs& a, hipStream_t s) {
  return launch_gemm_tile<DT_F32, DT_F16>(tile, a, s);
}
}  // namespace biasact
