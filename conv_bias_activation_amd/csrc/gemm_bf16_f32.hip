// gemm_bf16_f32.hip — fused GEMM + bias + activation kernels, bf16 operands, f32 output.
#include "kernels_impl.hpp"

namespace biasact {
int launch_gemm_bf16_f32(int tile, const GemmArgs& a, hipStream_t s) {
  return launch_gemm_tile<DT_BF16, DT_F32>(tile, a, s);
}
}  // namespace biasact
