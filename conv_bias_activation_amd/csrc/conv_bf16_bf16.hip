// conv_bf16_bf16.hip — fused implicit-GEMM conv2d + bias + activation kernels, bf16 operands, bf16 output.
#include "kernels_impl.hpp"

namespace biasact {
int launch_conv_bf16_bf16(int tile, const ConvArgs& a, hipStream_t s) {
  return launch_conv_tile<DT_BF16, DT_BF16>(tile, a, s);
}
int launch_conv_halo_bf16_bf16(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s) {
  return launch_conv_halo_tile<DT_BF16, DT_BF16>(taps, bm, ks, sn, nw, a, s);
}
}  // namespace biasact
