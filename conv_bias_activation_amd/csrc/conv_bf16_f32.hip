// conv_bf16_f32.hip — fused implicit-GEMM conv2d + bias + activation kernels, bf16 operands, f32 output.
#include "kernels_impl.hpp"

namespace biasact {
int launch_conv_bf16_f32(int tile, const ConvArgs& a, hipStream_t s) {
  return launch_conv_tile<DT_BF16, DT_F32>(tile, a, s);
}
int launch_conv_halo_bf16_f32(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s) {
  return launch_conv_halo_tile<DT_BF16, DT_F32>(taps, bm, ks, sn, nw, a, s);
}
}  // namespace biasact
