// act_cast.hip — second kernel of the two-kernel path (activation + cast).
#include "kernels_impl.hpp"

namespace biasact {
int launch_act_cast(int dto, const float* ws, void* out, uint32_t n, int act, float alpha,
                    const void* res, hipStream_t s) {
  if (n == 0) return 0;
  const uint32_t threads = 256;
  uint32_t blocks = (n + threads * 16 - 1) / (threads * 16);
  if (blocks > 256u * 8u) blocks = 256u * 8u;       // 8 workgroups per CU, then grid-stride
  switch (dto) {
    case DT_F32:
      launch_kernel(act_cast_kernel<DT_F32>, dim3(blocks), dim3(threads), s, ws, out, n, act, alpha, res);
      return 0;
    case DT_F16:
      launch_kernel(act_cast_kernel<DT_F16>, dim3(blocks), dim3(threads), s, ws, out, n, act, alpha, res);
      return 0;
    case DT_BF16:
      launch_kernel(act_cast_kernel<DT_BF16>, dim3(blocks), dim3(threads), s, ws, out, n, act, alpha, res);
      return 0;
    default:
      return -1;
  }
}
}  // namespace biasact
