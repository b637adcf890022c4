// gemm_f32_f32.hip — fused GEMM + bias + activation kernels, f32 operands, f32 output.
#include "kernels_impl.hpp"

namespace biasact {
int launch_gemm_f32_f32(int tile, const GemmArgs& a, hipStream_t s) {
  return launch_gemm_tile<DT_F32, DT_F32>(tile, a, s);
}
}  // namespace biasact
