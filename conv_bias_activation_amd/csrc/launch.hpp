// launch.hpp — host <-> kernel argument blocks, the tile-config table and
// the per-input-type launch entry points of the biasact library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_args.hpp"
#include "mfma_core.hpp"

namespace biasact {

struct ConvArgs {
  const void* x;
  const void* w;
  const void* bias;
  void* y;
  const void* r;            // residual [N, Co, Ho, Wo] in y's type (y_bytes), or null
  ConvGeom geom;
  uint32_t x_bytes, w_bytes, bias_bytes, y_bytes;
  int bias_dt;
  int act;
  float alpha;
  uint32_t tiles_m, tiles_n;
  bool vec_w, vec_y;
};

// Argument block of the halo-staging conv kernel (conv_halo.hpp).
struct HaloArgs {
  const void* x;
  const void* w;
  const void* bias;
  void* y;
  const void* r;            // residual, as in ConvArgs
  ConvGeom geom;
  uint32_t x_bytes, w_bytes, bias_bytes, y_bytes;
  int bias_dt;
  int act;
  float alpha;
  uint32_t PH, PW;          // output rows / columns per workgroup
  uint32_t HR, HC;          // halo rows / columns staged per channel chunk (HC even)
  uint32_t bkc;             // channels per chunk (8, 16, 32 or 64)
  uint32_t co_blocks, w_blocks, h_blocks, blocks;
  uint32_t groups;          // fp32 kernel: workgroups of a resident-filter grid (0: one patch each)
  bool vec_y;               // Wo % 4 == 0 and y aligned for 4-element stores
  // 16-bit kernel: divisions by workgroup-invariant values (FastDiv)
  FastDiv div_cob, div_wb, div_hb, div_pw, div_pairs;
  // fp32 kernel only
  uint32_t hrcp;            // halo floats per channel (HR * HC rounded up to 64)
  FastDiv div_hc;
  uint32_t kpad;            // k-pairs per chunk rounded up to 4
  uint32_t kstr;            // weight row stride in LDS (floats): 2 kpad + 4
  FastDiv div_kstr;
};

// Per-input-type launchers (one translation unit each).  Return 0, or -1 for
// an unknown output type / tile id.
int launch_gemm_f32(int dto, int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_f16(int dto, int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_bf16(int dto, int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_i8(int dto, int tile, const GemmArgs& a, hipStream_t s);
int launch_conv_f32(int dto, int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_f16(int dto, int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_bf16(int dto, int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_halo(int dti, int dto, int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s);
int launch_act_cast(int dto, const float* ws, void* out, uint32_t n, int act, float alpha,
                    const void* res, hipStream_t s);

}  // namespace biasact
