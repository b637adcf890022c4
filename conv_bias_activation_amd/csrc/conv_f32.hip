// conv_f32.hip — fused implicit-GEMM conv2d + bias + activation kernels for f32 inputs.
#include "kernels_impl.hpp"

namespace biasact {
int launch_conv_f32(int dto, int tile, const ConvArgs& a, hipStream_t s) {
  return launch_conv_in<DT_F32>(dto, tile, a, s);
}
}  // namespace biasact
