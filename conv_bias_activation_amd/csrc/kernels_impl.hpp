// kernels_impl.hpp — __global__ kernels built on the main loop of
// mfma_core.hpp: the fused GEMM + bias + activation, the fused implicit-GEMM
// conv2d + bias + activation, and the elementwise activation/cast pass of the
// two-kernel path.  Each translation unit instantiates them for one input
// element type.
#pragma once

#include "conv_halo.hpp"
#include "conv_halo32.hpp"
#include "epilogue.hpp"
#include "gemm_pp.hpp"
#include "launch.hpp"
#include "launch_kernel.hpp"
#include "mfma_core.hpp"

namespace biasact {

// ---------------------------------------------------------------------------
// C[M,N] = act(A[M,K] . B[K,N] + bias[N])   ([MLR] 概述 / 样例规格;
// [FMR] fused_matmul_relu).  One workgroup per BM x BN output tile.  NK > 0:
// the reduction is at most NK k-tiles, all loaded at once (main_loop_allk).
// ---------------------------------------------------------------------------
template <int DTI, int DTO, class TL, int NK = 0>
__global__ __launch_bounds__(TL::threads, 1) void gemm_bias_act_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[(NK > 2 ? NK : 2) * TL::stage_bytes];
  constexpr int BK = kChunks * Elem<DTI>::epc;

  uint32_t tm, tn;
  map_tile(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, tm, tn);
  const uint32_t m0 = tm * TL::BM, n0 = tn * TL::BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_m = wave / TL::WAVES_N, wave_n = wave % TL::WAVES_N;
  const int half = lane >> 5, lrow = lane & 31;

  // accumulator starts at the bias (the extra reduction term), fetched once
  // the first operand loads are in flight
  f32x16 acc[TL::SN][TL::SM];
  auto init_acc = [&]() {
    uint32_t idx[TL::SN * 16];
    float bv[TL::SN * 16];
#pragma unroll
    for (int si = 0; si < TL::SN; ++si)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        idx[si * 16 + r] = n0 + wave_n * TL::WTN + si * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
    load_bias_vec<TL::SN * 16>(a.bias, a.bias_bytes, a.bias_dt, idx, a.N, bv);
#pragma unroll
    for (int si = 0; si < TL::SN; ++si) {
      f32x16 b;
#pragma unroll
      for (int r = 0; r < 16; ++r) b[r] = bv[si * 16 + r];
#pragma unroll
      for (int sj = 0; sj < TL::SM; ++sj) acc[si][sj] = b;
    }
  };

  DenseRowLoader<DTI, TL> la;
  DenseColLoader<DTI, TL> lb;
  la.init(a.A, a.a_bytes, a.M, a.K, m0, a.vec_a);
  lb.init(a.B, a.b_bytes, a.K, a.N, n0, a.vec_b);
  const int ktiles = (int)((a.K + BK - 1) / BK);
  if constexpr (NK > 0)
    main_loop_allk<DTI, TL, NK>(acc, la, lb, smem, ktiles, init_acc);
  else
    main_loop<DTI, TL>(acc, la, lb, smem, ktiles, init_acc);

  // epilogue: activation, cast, one store per element
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.C, a.c_bytes);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.R, a.R ? a.c_bytes : 0u);
  with_act(a.act, [&](auto act_c) __attribute__((always_inline)) {
  constexpr int ACT = decltype(act_c)::value;
  with_residual(a.R != nullptr, [&](auto res_c) __attribute__((always_inline)) {
  constexpr bool HAS_R = decltype(res_c)::value;
  if (a.vec_c) {
    // N % 4 == 0 and C (and R) 16-byte aligned: the sums leave through LDS
    // (StagedOut), whole 128-byte row runs per store
    using SO = StagedOut<TL>;
    static_assert(SO::bytes <= (NK > 2 ? NK : 2) * TL::stage_bytes, "staged column block exceeds the LDS tile");
    const SO so;
#pragma unroll
    for (int si = 0; si < TL::SN; ++si) {
      __syncthreads();      // the main loop's (or the previous pass's) LDS reads are done
      SO::put(acc, smem, si);
      __syncthreads();
      const uint32_t n = n0 + so.col(si);
#pragma unroll
      for (int k = 0; k < SO::CPT; ++k) {
        const uint32_t m = m0 + so.row(k);
        const f32x4 v = so.get(smem, k);
        float z[4] = {v[0], v[1], v[2], v[3]};
        const bool ok = m < a.M && n < a.N;
        if constexpr (HAS_R && DTI != DT_I8) {
          float rv[4];
          load4<DTO>(rr, m * a.N + n, ok, rv);
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] += rv[e];
        }
        store4<DTO>(rc, m * a.N + n, ok, out_value<DTI, DTO, ACT>(z[0], a.alpha),
                    out_value<DTI, DTO, ACT>(z[1], a.alpha), out_value<DTI, DTO, ACT>(z[2], a.alpha),
                    out_value<DTI, DTO, ACT>(z[3], a.alpha));
      }
    }
    return;
  }
#pragma unroll
  for (int si = 0; si < TL::SN; ++si)
#pragma unroll
    for (int sj = 0; sj < TL::SM; ++sj) {
      const uint32_t m = m0 + wave_m * TL::WTM + sj * 32 + lrow;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t n = n0 + wave_n * TL::WTN + si * 32 + 8 * g + 4 * half;
        const bool mok = m < a.M;
        float z[4] = {acc[si][sj][4 * g + 0], acc[si][sj][4 * g + 1], acc[si][sj][4 * g + 2],
                      acc[si][sj][4 * g + 3]};
        if constexpr (HAS_R && DTI != DT_I8) {
          if (a.vec_c) {
            float rv[4];
            load4<DTO>(rr, m * a.N + n, mok && n < a.N, rv);
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] += rv[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] += load1<DTO>(rr, m * a.N + n + e, mok && n + e < a.N);
          }
        }
        const float y0 = out_value<DTI, DTO, ACT>(z[0], a.alpha);
        const float y1 = out_value<DTI, DTO, ACT>(z[1], a.alpha);
        const float y2 = out_value<DTI, DTO, ACT>(z[2], a.alpha);
        const float y3 = out_value<DTI, DTO, ACT>(z[3], a.alpha);
        if (a.vec_c) {
          store4<DTO>(rc, m * a.N + n, mok && n < a.N, y0, y1, y2, y3);
        } else {
          store1<DTO>(rc, m * a.N + n + 0, mok && n + 0 < a.N, y0);
          store1<DTO>(rc, m * a.N + n + 1, mok && n + 1 < a.N, y1);
          store1<DTO>(rc, m * a.N + n + 2, mok && n + 2 < a.N, y2);
          store1<DTO>(rc, m * a.N + n + 3, mok && n + 3 < a.N, y3);
        }
      }
    }
  });
  });
}

// ---------------------------------------------------------------------------
// y[N,Co,Ho,Wo] = act(conv2d(x, w) + bias[Co]) as an implicit GEMM:
// j = co (weights [Co, C*kh*kw]), i = p = (n, oh, ow) gathered from x
// ([FCT] "这个算子到底在算什么" and "双 Kernel 是怎么分工的").
// ---------------------------------------------------------------------------
template <int DTI, int DTO, class TL>
__global__ __launch_bounds__(TL::threads, 1) void conv_bias_act_kernel(ConvArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TL::stage_bytes];
  constexpr int BK = kChunks * Elem<DTI>::epc;
  const ConvGeom& G = a.geom;

  uint32_t tm, tn;
  map_tile(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, tm, tn);
  const uint32_t m0 = tm * TL::BM, p0 = tn * TL::BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_m = wave / TL::WAVES_N, wave_n = wave % TL::WAVES_N;
  const int half = lane >> 5, lrow = lane & 31;

  f32x16 acc[TL::SN][TL::SM];
  auto init_acc = [&]() {
    uint32_t idx[TL::SM];
    float bv[TL::SM];
#pragma unroll
    for (int sj = 0; sj < TL::SM; ++sj) idx[sj] = m0 + wave_m * TL::WTM + sj * 32 + lrow;
    load_bias_vec<TL::SM>(a.bias, a.bias_bytes, a.bias_dt, idx, G.Co, bv);
#pragma unroll
    for (int sj = 0; sj < TL::SM; ++sj)
#pragma unroll
      for (int si = 0; si < TL::SN; ++si)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[si][sj][r] = bv[sj];
  };

  DenseRowLoader<DTI, TL> la;
  ConvGatherLoader<DTI, TL> lb;
  la.init(a.w, a.w_bytes, G.Co, G.K, m0, a.vec_w);
  lb.init(a.x, a.x_bytes, G, p0);
  const int ktiles = (int)((G.K + BK - 1) / BK);
  main_loop<DTI, TL>(acc, la, lb, smem, ktiles, init_acc);

  const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, a.y_bytes);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.r, a.r ? a.y_bytes : 0u);
  const uint32_t howo = G.Ho * G.Wo;
  with_act(a.act, [&](auto act_c) __attribute__((always_inline)) {
  constexpr int ACT = decltype(act_c)::value;
  with_residual(a.r != nullptr, [&](auto res_c) __attribute__((always_inline)) {
  constexpr bool HAS_R = decltype(res_c)::value;
  if (a.vec_y) {
    // Ho*Wo % 4 == 0: every group of four positions lies in one image; the
    // pre-activations leave through LDS (StagedOut)
    using SO = StagedOut<TL>;
    static_assert(SO::bytes <= 2 * TL::stage_bytes, "staged column block exceeds the LDS tile");
    const SO so;
#pragma unroll
    for (int si = 0; si < TL::SN; ++si) {
      __syncthreads();      // the main loop's (or the previous pass's) LDS reads are done
      SO::put(acc, smem, si);
      __syncthreads();
      const uint32_t p = p0 + so.col(si);
      const uint32_t img = fdiv(p, G.div_howo);
      const uint32_t base = img * G.Co * howo + (p - img * howo);
      const bool pok = p < G.P;
#pragma unroll
      for (int k = 0; k < SO::CPT; ++k) {
        const uint32_t co = m0 + so.row(k);
        const f32x4 v = so.get(smem, k);
        float z[4] = {v[0], v[1], v[2], v[3]};
        const uint32_t off = base + co * howo;
        const bool ok = pok && co < G.Co;
        if constexpr (HAS_R) {
          float rv[4];
          load4<DTO>(rr, off, ok, rv);
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] += rv[e];
        }
        store4<DTO>(ry, off, ok, act_fn<ACT, DTO>(z[0], a.alpha), act_fn<ACT, DTO>(z[1], a.alpha),
                    act_fn<ACT, DTO>(z[2], a.alpha), act_fn<ACT, DTO>(z[3], a.alpha));
      }
    }
    return;
  }
#pragma unroll
  for (int si = 0; si < TL::SN; ++si)
#pragma unroll
    for (int sj = 0; sj < TL::SM; ++sj) {
      const uint32_t co = m0 + wave_m * TL::WTM + sj * 32 + lrow;
      const bool cok = co < G.Co;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t p = p0 + wave_n * TL::WTN + si * 32 + 8 * g + 4 * half;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t pe = p + e;
          const uint32_t img = fdiv(pe, G.div_howo);
          const uint32_t q = pe - img * howo;
          const uint32_t off = (img * G.Co + co) * howo + q;
          const bool ok = cok && pe < G.P;
          float ze = acc[si][sj][4 * g + e];
          if constexpr (HAS_R) ze += load1<DTO>(rr, off, ok);
          store1<DTO>(ry, off, ok, act_fn<ACT, DTO>(ze, a.alpha));
        }
      }
    }
  });
  });
}

// ---------------------------------------------------------------------------
// Second kernel of the two-kernel path: out[i] = cast(act(ws[i] (+ res[i])))
// over a packed fp32 workspace that already holds A.B + bias (GEMM, [M,N]) or
// conv + bias (conv, NCHW); res, if given, is the residual in out's type.
// Each thread handles 16 elements per pass, as four groups of 4 consecutive
// ones, with four 16-byte loads issued before any is used (64 bytes in
// flight per lane); grid-stride over the array with a grid that fills every
// CU.
// ---------------------------------------------------------------------------
template <int DTO>
__global__ __launch_bounds__(256) void act_cast_kernel(const float* ws, void* out, uint32_t n,
                                                       int act, float alpha, const void* res) {
  constexpr uint32_t EPT = 16, WT = 64 * EPT;       // elements per thread, per wave tile
  const __amdgpu_buffer_rsrc_t ri = make_rsrc(ws, n * 4u);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(out, n * (uint32_t)Elem<DTO>::bytes);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(res, res ? n * (uint32_t)Elem<DTO>::bytes : 0u);
  // A wave takes tiles of 1024 consecutive elements; its q-th access covers
  // elements [q * 256, q * 256 + 256) of the tile, four per lane, so every
  // load and store instruction moves one contiguous run across the wave.
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const uint32_t stride = ((gridDim.x * blockDim.x) >> 6) * WT;
  auto run = [&](auto act_c, auto res_c) __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool HAS_R = decltype(res_c)::value;
    for (uint32_t tile = wave * WT; tile < n; tile += stride) {
      const bool full = tile + WT <= n;
      uint32_t first[EPT / 4];                       // this lane's first element of access q
#pragma unroll
      for (uint32_t q = 0; q < EPT / 4; ++q) first[q] = tile + q * 256 + lane * 4;
      float z[EPT];
      if (full) {
        u32x4 v[EPT / 4];
#pragma unroll
        for (uint32_t q = 0; q < EPT / 4; ++q) v[q] = ld_b128(ri, first[q] * 4u);
#pragma unroll
        for (uint32_t q = 0; q < EPT / 4; ++q) {
          z[4 * q + 0] = __uint_as_float(v[q].x);
          z[4 * q + 1] = __uint_as_float(v[q].y);
          z[4 * q + 2] = __uint_as_float(v[q].z);
          z[4 * q + 3] = __uint_as_float(v[q].w);
        }
      } else {
#pragma unroll
        for (uint32_t q = 0; q < EPT / 4; ++q)
#pragma unroll
          for (uint32_t e = 0; e < 4; ++e) {
            const uint32_t i = first[q] + e;
            z[4 * q + e] = __uint_as_float(ld_b32(ri, i < n ? i * 4u : kOOB));
          }
      }
      if constexpr (HAS_R) {
        // the residual joins the pre-activation (A.B + bias) before act
        if (full) {
#pragma unroll
          for (uint32_t q = 0; q < EPT / 4; ++q) {
            float rv[4];
            load4<DTO>(rr, first[q], true, rv);
#pragma unroll
            for (int e = 0; e < 4; ++e) z[4 * q + e] += rv[e];
          }
        } else {
#pragma unroll
          for (uint32_t q = 0; q < EPT / 4; ++q)
#pragma unroll
            for (uint32_t e = 0; e < 4; ++e) z[4 * q + e] += load1<DTO>(rr, first[q] + e, first[q] + e < n);
        }
      }
      float y[EPT];
#pragma unroll
      for (uint32_t e = 0; e < EPT; ++e) y[e] = act_fn<ACT, DTO>(z[e], alpha);
      if (full) {
#pragma unroll
        for (uint32_t q = 0; q < EPT / 4; ++q)
          store4<DTO>(ro, first[q], true, y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
      } else {
#pragma unroll
        for (uint32_t q = 0; q < EPT / 4; ++q)
#pragma unroll
          for (uint32_t e = 0; e < 4; ++e) store1<DTO>(ro, first[q] + e, first[q] + e < n, y[4 * q + e]);
      }
    }
  };
  // activation and residual dispatched once per thread
  with_act(act, [&](auto act_c) __attribute__((always_inline)) {
    with_residual(res != nullptr, [&](auto res_c) __attribute__((always_inline)) { run(act_c, res_c); });
  });
}

// ---------------------------------------------------------------------------
// Host-side launch helpers (instantiated per input type in its own TU).
// ---------------------------------------------------------------------------
template <int DTI, int DTO, class TL, int NK = 0>
inline void launch_gemm_t(const GemmArgs& a, hipStream_t s) {
  const uint32_t nblk = a.tiles_m * a.tiles_n;
  note_launch("gemm %dx%d/%dx%d%s", TL::BM, TL::BN, TL::WAVES_M, TL::WAVES_N,
              NK > 0 ? " all-k" : "");
  launch_kernel(gemm_bias_act_kernel<DTI, DTO, TL, NK>, dim3(nblk), dim3(TL::threads), s, a);
}

template <int DTI, int DTO, class TL>
inline void launch_conv_t(const ConvArgs& a, hipStream_t s) {
  const uint32_t nblk = a.tiles_m * a.tiles_n;
  note_launch("conv %dx%d/%dx%d", TL::BM, TL::BN, TL::WAVES_M, TL::WAVES_N);
  launch_kernel(conv_bias_act_kernel<DTI, DTO, TL>, dim3(nblk), dim3(TL::threads), s, a);
}

// The tile table (same ids and order as kTiles in plan.hpp).
using T0 = Tile<256, 256, 2, 2>;
using T1 = Tile<128, 256, 2, 2>;
using T2 = Tile<128, 128, 2, 2>;
using T3 = Tile<64, 128, 2, 2>;
using T4 = Tile<64, 256, 1, 4>;
using T5 = Tile<64, 64, 2, 2>;

template <int DTI, int DTO>
inline int launch_gemm_tile(int tile, const GemmArgs& a, hipStream_t s) {
  switch (tile) {
    case 0: launch_gemm_t<DTI, DTO, T0>(a, s); return 0;
    case 1: launch_gemm_t<DTI, DTO, T1>(a, s); return 0;
    case 2: launch_gemm_t<DTI, DTO, T2>(a, s); return 0;
    case 3: launch_gemm_t<DTI, DTO, T3>(a, s); return 0;
    case 4: launch_gemm_t<DTI, DTO, T4>(a, s); return 0;
    case 5:
      // a reduction of at most 4 k-tiles has no steady state to pipeline:
      // load all of it at once
      if (a.K <= 4u * (kChunks * Elem<DTI>::epc))
        launch_gemm_t<DTI, DTO, T5, 4>(a, s);
      else
        launch_gemm_t<DTI, DTO, T5>(a, s);
      return 0;
    case 6:
      if constexpr (DTI == DT_F16 || DTI == DT_BF16 || DTI == DT_I8) {
        if (a.vec_a && a.vec_b && a.vec_c) {
          launch_gemm_pp<DTI, DTO>(a, s);
          return 0;
        }
      }
      launch_gemm_t<DTI, DTO, T0>(a, s);
      return 0;
    default: return -1;
  }
}

template <int DTI, int DTO>
inline int launch_conv_tile(int tile, const ConvArgs& a, hipStream_t s) {
  switch (tile) {
    case 0: launch_conv_t<DTI, DTO, T0>(a, s); return 0;
    case 1: launch_conv_t<DTI, DTO, T1>(a, s); return 0;
    case 2: launch_conv_t<DTI, DTO, T2>(a, s); return 0;
    case 3: launch_conv_t<DTI, DTO, T3>(a, s); return 0;
    case 4: launch_conv_t<DTI, DTO, T4>(a, s); return 0;
    case 5: launch_conv_t<DTI, DTO, T5>(a, s); return 0;
    default: return -1;
  }
}

template <int DTI, int DTO, int T, int BM>
inline int launch_conv_halo_ks_small(int ks, int sn, int nw, const HaloArgs& a, hipStream_t s) {
  // a wave keeps KS * BM / 64 weight-fragment sets of a chunk in registers (at
  // most 4); the one-tile-per-wave variants exist only where two workgroups
  // share a CU, or in the eight-wave 64-channel variants (two fragment sets)
  if (nw == 8) {
    if constexpr (BM == 64) {
      if (ks == 2 && sn == 1) { launch_conv_halo_t<DTI, DTO, T, BM, 2, 1, 8>(a, s); return 0; }
      if (ks == 2 && sn == 2) { launch_conv_halo_t<DTI, DTO, T, BM, 2, 2, 8>(a, s); return 0; }
    }
    return -1;
  }
  if (nw != 4) return -1;
  if (sn == 2) {
    switch (ks) {
      case 1: launch_conv_halo_t<DTI, DTO, T, BM, 1, 2>(a, s); return 0;
      case 2: launch_conv_halo_t<DTI, DTO, T, BM, 2, 2>(a, s); return 0;
      case 4:
        if constexpr (BM == 64) {
          launch_conv_halo_t<DTI, DTO, T, BM, 4, 2>(a, s);
          return 0;
        } else {
          return -1;
        }
      default: return -1;
    }
  }
  if (sn == 1) {
    if (ks == 1) { launch_conv_halo_t<DTI, DTO, T, BM, 1, 1>(a, s); return 0; }
    if constexpr (BM == 64) {
      if (ks == 2) { launch_conv_halo_t<DTI, DTO, T, BM, 2, 1>(a, s); return 0; }
    }
  }
  return -1;
}

template <int DTI, int DTO, int T, int BM>
inline int launch_conv_halo_ks(int ks, int sn, int nw, const HaloArgs& a, hipStream_t s) {
  if constexpr (T > 9) {
    // larger filters: one k-step per chunk, two position tiles per wave, four waves
    if (BM == 64 && ks == 1 && sn == 2 && nw == 4) {
      launch_conv_halo_t<DTI, DTO, T, 64, 1, 2, 4>(a, s);
      return 0;
    }
    return -1;
  } else {
    return launch_conv_halo_ks_small<DTI, DTO, T, BM>(ks, sn, nw, a, s);
  }
}

template <int DTI, int DTO>
inline int launch_conv_halo_tile(int taps, int bm, int ks, int sn, int nw, const HaloArgs& a, hipStream_t s) {
  if constexpr (DTI == DT_F32) {
    (void)taps;
    (void)ks;
    (void)sn;
    (void)nw;
    if (bm == 64) { launch_conv32_halo_t<DTO, 64>(a, s); return 0; }
    if (bm == 128) { launch_conv32_halo_t<DTO, 128>(a, s); return 0; }
    return -1;
  } else {
    if (taps == 9 && bm == 64) return launch_conv_halo_ks<DTI, DTO, 9, 64>(ks, sn, nw, a, s);
    if (taps == 9 && bm == 128) return launch_conv_halo_ks<DTI, DTO, 9, 128>(ks, sn, nw, a, s);
    if (taps == 1 && bm == 64) return launch_conv_halo_ks<DTI, DTO, 1, 64>(ks, sn, nw, a, s);
    if (taps == 1 && bm == 128) return launch_conv_halo_ks<DTI, DTO, 1, 128>(ks, sn, nw, a, s);
    if (taps == 25 && bm == 64) return launch_conv_halo_ks<DTI, DTO, 25, 64>(ks, sn, nw, a, s);
    if (taps == 49 && bm == 64) return launch_conv_halo_ks<DTI, DTO, 49, 64>(ks, sn, nw, a, s);
    return -1;
  }
}

}  // namespace biasact
