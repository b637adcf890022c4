// gemm_f16_bf16.hip — fused GEMM + bias + activation kernels, f16 operands, bf16 output.
#include "kernels_impl.hpp"

namespace biasact {
int launch_gemm_f16_bf16(int tile, const GemmArgs& a, hipStream_t s) {
  return launch_gemm_tile<DT_F16, DT_BF16>(tile, a, s);
}
}  // namespace biasact
