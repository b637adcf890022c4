// gemm_f32.hip — fused GEMM + bias + activation kernels for f32 inputs.
#include "kernels_impl.hpp"

namespace biasact {
int launch_gemm_f32(int dto, int tile, const GemmArgs& a, hipStream_t s) {
  return launch_gemm_in<DT_F32>(dto, tile, a, s);
}
}  // namespace biasact
