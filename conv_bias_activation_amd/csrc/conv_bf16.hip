// conv_bf16.hip — fused implicit-GEMM conv2d + bias + activation kernels for bf16 inputs.
#include "kernels_impl.hpp"

namespace biasact {
int launch_conv_bf16(int dto, int tile, const ConvArgs& a, hipStream_t s) {
  return launch_conv_in<DT_BF16>(dto, tile, a, s);
}
}  // namespace biasact
