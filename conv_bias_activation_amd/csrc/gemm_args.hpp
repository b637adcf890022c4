// gemm_args.hpp — kernel argument block of the fused GEMM + bias + activation.
#pragma once

#include <stdint.h>

namespace biasact {

// Kernel argument block of the fused GEMM (passed by value).
struct GemmArgs {
  const void* A;
  const void* B;
  const void* bias;
  void* C;
  const void* R;           // residual [M, N] in C's type, added before the activation; may be null
  uint32_t M, N, K;
  uint32_t a_bytes, b_bytes, bias_bytes, c_bytes;   // R spans c_bytes too
  int bias_dt;             // DT_* of bias, or -1 without bias
  int act;
  float alpha;
  uint32_t tiles_m, tiles_n;
  bool vec_a, vec_b, vec_c;   // 16-byte loads / 4-wide stores allowed
};

}  // namespace biasact
