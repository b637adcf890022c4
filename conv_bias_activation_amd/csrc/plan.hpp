// plan.hpp — host-side argument checking and launch planning (no HIP calls,
// no device code): turns the C-ABI arguments into a checked plan or a status.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace biasact {

enum Status : int { kOk = 0, kErrInvalid = 1, kErrUnsupported = 2, kErrHip = 3 };

struct TileShapeDesc {
  int id, bm, bn, waves_m, waves_n;
};
// Must list the same tiles, in the same order, as the launch switch.
constexpr TileShapeDesc kTiles[] = {
    {0, 256, 256, 2, 2},
    {1, 128, 256, 2, 2},
    {2, 128, 128, 2, 2},
    {3, 64, 128, 2, 2},
    {4, 64, 256, 1, 4},
    {5, 64, 64, 2, 2},
    {6, 256, 256, 2, 4},   // 8-wave ping-pong kernel: aligned 16-bit GEMMs only (else as 0)
    {7, 128, 128, 2, 2},   // conv with a channel-last LDS halo: 16-bit square 1x1 to 7x7, fp32 (else as 3)
};
constexpr int kNumTileConfigs = (int)(sizeof(kTiles) / sizeof(kTiles[0]));

struct GemmPlan {
  int dti, dto, bias_dt;           // bias_dt = -1 without bias
  uint32_t M, N, K;
  uint32_t a_bytes, b_bytes, bias_bytes, c_bytes;
  bool vec_a, vec_b, vec_c;
  bool empty;                      // M == 0 or N == 0: nothing to launch
  int tile;
  uint32_t tiles_m, tiles_n;
};

struct ConvPlan {
  int dti, dto, bias_dt;
  uint32_t N, C, H, W, Co, kh, kw, Ho, Wo;
  int32_t sh, sw, pt, pb, pl, pr, dh, dw;
  uint32_t K, P;
  uint32_t x_bytes, w_bytes, bias_bytes, y_bytes;
  bool vec_w, vec_y;
  bool empty;                      // N == 0
  int tile;
  uint32_t tiles_m, tiles_n;
  // halo kernel (tile 7) parameters
  uint32_t h_bm, h_ks, h_sn, h_nw, h_PH, h_PW, h_HR, h_HC, h_bkc, h_co_blocks, h_w_blocks, h_h_blocks, h_blocks;
  uint32_t h_hrcp, h_kpad, h_kstr;   // fp32 halo kernel (see plan_halo32)
  uint32_t h_groups;                 // fp32 halo kernel: resident-filter workgroups, or 0
};

// R (residual, output's type and shape) only enters the alignment decisions.
int plan_gemm(const void* A, const void* B, const void* bias, const void* C, int64_t M, int64_t N,
              int64_t K, uint32_t dtypes, int act, GemmPlan* p, const void* R = nullptr);
int plan_conv(const void* x, const void* w, const void* bias, const void* y, int64_t N, int64_t C,
              int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw, const int32_t* strides,
              const int32_t* pads, const int32_t* dilations, uint32_t dtypes, int act,
              ConvPlan* p, const void* r = nullptr);

// Output size of conv2d with zero padding (floor rounding); kErrInvalid for
// bad strides / pads / dilations or an empty output.
int conv_out_dims(int64_t H, int64_t W, int64_t kh, int64_t kw, const int32_t* strides,
                  const int32_t* pads, const int32_t* dilations, int64_t* Ho, int64_t* Wo);

int select_gemm_tile(int64_t M, int64_t N, int64_t K, int dti);
int select_conv_tile(int64_t N, int64_t Co, int64_t Ho, int64_t Wo, int64_t K, int dti);

// -1 = automatic
int forced_tile();
void set_forced_tile(int id);
// -1 automatic, 0 widest tile, 1 / 2 the two-per-CU variants (see biasact.h)
int forced_halo_variant();
void set_forced_halo_variant(int v);

const char* status_string(int s);

}  // namespace biasact
