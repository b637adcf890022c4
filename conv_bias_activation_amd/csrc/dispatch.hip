// dispatch.hip — (input type, output type) -> kernel translation unit.
#include "launch.hpp"

namespace biasact {

int launch_gemm_f32_f32(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_f32_f16(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_f32_bf16(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_f16_f32(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_f16_f16(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_f16_bf16(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_bf16_f32(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_bf16_f16(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_bf16_bf16(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_i8_f32(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_i8_f16(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_i8_bf16(int tile, const GemmArgs& a, hipStream_t s);
int launch_gemm_i8_i32(int tile, const GemmArgs& a, hipStream_t s);
int launch_conv_f32_f32(int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_f32_f16(int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_f32_bf16(int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_f16_f32(int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_f16_f16(int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_f16_bf16(int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_bf16_f32(int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_bf16_f16(int tile, const ConvArgs& a, hipStream_t s);
int launch_conv_bf16_bf16(int tile, const ConvArgs& a, hipStream_t s);

int launch_gemm_f32(int dto, int tile, const GemmArgs& a, hipStream_t s) {
  switch (dto) {
    case DT_F32: return launch_gemm_f32_f32(tile, a, s);
    case DT_F16: return launch_gemm_f32_f16(tile, a, s);
    case DT_BF16: return launch_gemm_f32_bf16(tile, a, s);
    default: return -1;
  }
}

int launch_gemm_f16(int dto, int tile, const GemmArgs& a, hipStream_t s) {
  switch (dto) {
    case DT_F32: return launch_gemm_f16_f32(tile, a, s);
    case DT_F16: return launch_gemm_f16_f16(tile, a, s);
    case DT_BF16: return launch_gemm_f16_bf16(tile, a, s);
    default: return -1;
  }
}

int launch_gemm_bf16(int dto, int tile, const GemmArgs& a, hipStream_t s) {
  switch (dto) {
    case DT_F32: return launch_gemm_bf16_f32(tile, a, s);
    case DT_F16: return launch_gemm_bf16_f16(tile, a, s);
    case DT_BF16: return launch_gemm_bf16_bf16(tile, a, s);
    default: return -1;
  }
}

int launch_gemm_i8(int dto, int tile, const GemmArgs& a, hipStream_t s) {
  switch (dto) {
    case DT_F32: return launch_gemm_i8_f32(tile, a, s);
    case DT_F16: return launch_gemm_i8_f16(tile, a, s);
    case DT_BF16: return launch_gemm_i8_bf16(tile, a, s);
    case DT_I32: return launch_gemm_i8_i32(tile, a, s);
    default: return -1;
  }
}

int launch_conv_f32(int dto, int tile, const ConvArgs& a, hipStream_t s) {
  switch (dto) {
    case DT_F32: return launch_conv_f32_f32(tile, a, s);
    case DT_F16: return launch_conv_f32_f16(tile, a, s);
    case DT_BF16: return launch_conv_f32_bf16(tile, a, s);
    default: return -1;
  }
}

int launch_conv_f16(int dto, int tile, const ConvArgs& a, hipStream_t s) {
  switch (dto) {
    case DT_F32: return launch_conv_f16_f32(tile, a, s);
    case DT_F16: return launch_conv_f16_f16(tile, a, s);
    case DT_BF16: return launch_conv_f16_bf16(tile, a, s);
    default: return -1;
  }
}

int launch_conv_bf16(int dto, int tile, const ConvArgs& a, hipStream_t s) {
  switch (dto) {
    case DT_F32: return launch_conv_bf16_f32(tile, a, s);
    case DT_F16: return launch_conv_bf16_f16(tile, a, s);
    case DT_BF16: return launch_conv_bf16_bf16(tile, a, s);
    default: return -1;
  }
}

int launch_conv_halo_f32_f32(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s);
int launch_conv_halo_f32_f16(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s);
int launch_conv_halo_f32_bf16(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s);
int launch_conv_halo_f16_f32(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s);
int launch_conv_halo_f16_f16(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s);
int launch_conv_halo_f16_bf16(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s);
int launch_conv_halo_bf16_f32(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s);
int launch_conv_halo_bf16_f16(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s);
int launch_conv_halo_bf16_bf16(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s);

int launch_conv_halo(int dti, int dto, int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s) {
  if (dti == DT_F32 && dto == DT_F32) return launch_conv_halo_f32_f32(taps, bm, ks, sn, nw, a, s);
  if (dti == DT_F32 && dto == DT_F16) return launch_conv_halo_f32_f16(taps, bm, ks, sn, nw, a, s);
  if (dti == DT_F32 && dto == DT_BF16) return launch_conv_halo_f32_bf16(taps, bm, ks, sn, nw, a, s);
  if (dti == DT_F16 && dto == DT_F32) return launch_conv_halo_f16_f32(taps, bm, ks, sn, nw, a, s);
  if (dti == DT_F16 && dto == DT_F16) return launch_conv_halo_f16_f16(taps, bm, ks, sn, nw, a, s);
  if (dti == DT_F16 && dto == DT_BF16) return launch_conv_halo_f16_bf16(taps, bm, ks, sn, nw, a, s);
  if (dti == DT_BF16 && dto == DT_F32) return launch_conv_halo_bf16_f32(taps, bm, ks, sn, nw, a, s);
  if (dti == DT_BF16 && dto == DT_F16) return launch_conv_halo_bf16_f16(taps, bm, ks, sn, nw, a, s);
  if (dti == DT_BF16 && dto == DT_BF16) return launch_conv_halo_bf16_bf16(taps, bm, ks, sn, nw, a, s);
  return -1;
}

}  // namespace biasact
