// conv_halo32.hpp — implicit-GEMM conv2d + bias + activation for fp32
// operands, any filter larger than 1x1, stride, padding and dilation ([FCT]
// "这个算子到底在算什么": y = act(conv2d(x, filter, bias)); "双 Kernel 是怎么
// 分工的": weights as the co x k operand, input features as the k x spatial
// operand).
//
// v_mfma_f32_32x32x2_f32 takes one value per lane from each operand: lane l
// gives row l % 32 at reduction index k0 + l / 32.  Both operands are therefore
// read from LDS one float per lane, and the reduction keeps the filter's own
// order, k = c * T + t (t = r * kw + s), so a shallow stem (C = 3, 7x7) wastes
// no MFMA lanes on padding.
//
// Workgroup: 256 threads (2 x 2 waves), BM output channels x a patch of PH
// output rows x PW output columns of one image (at most 128 positions).  A
// channel chunk of bkc channels is staged as
//   halo   [c][row][col] : input rows ih = oh0*sh - pt + row, columns
//                          iw = ow0*sw - pl + col; HR*HC floats per channel,
//                          rounded up to 64
//   wts    [co][h][kp]   : filter value k = 2 kp + h of the chunk for each
//                          output channel; rows KSTR = 2 KPAD + 4 floats
//                          apart (16-byte reads of 16 rows hit all banks)
// both by direct loads: one wave instruction moves 64 consecutive floats of
// one channel's halo, or of the weight block (padding, rows
// past Co, channels past C and positions outside the image arrive as zeros).
// Chunks alternate between two LDS arrays, so the next chunk's copy overlaps
// the multiply of the current one and the multiply's reads carry no wait on
// it; when all C channels form one chunk (a shallow stem: C = 3), its halo
// takes one array and its weights the other.  With one chunk and one
// output-channel block, a resident-filter grid of 512 workgroups stages the
// weight block once per workgroup and streams its patches' halos through two
// halo arrays.  Either layout and the offset table fit 80 KB, so two
// workgroups share a CU.  A table of the halo offset of every reduction index
// of a chunk lets a lane fetch the offsets of 4 steps with one read.
#pragma once

#include <utility>

#include "epilogue.hpp"
#include "launch.hpp"
#include "launch_kernel.hpp"
#include "mfma_core.hpp"

namespace biasact {

namespace halo32 {
constexpr int THREADS = 256;
constexpr int KOFF_MAX = 256;               // reduction-offset table: 2 x (k-pairs per chunk)
// Classic layout: two chunk buffers (and a 16-byte unused third array), 80 KB in all
constexpr int BUF_FLOATS = (80 * 1024 - KOFF_MAX * 4 - 16) / 8 / 4 * 4;
// Resident-filter layout: a weight block and two halo buffers, 80 KB in all
constexpr int RES_W_FLOATS = 10240, RES_H_FLOATS = (80 * 1024 - KOFF_MAX * 4) / 4 / 2 - RES_W_FLOATS / 2;
constexpr int WTN = 64;                     // positions per wave (two 32-wide MFMA tiles)
}  // namespace halo32

// BM = output channels per workgroup (64 or 128); RES: the resident-filter grid.
// Every region that a direct load may fill while another is read is its own
// __shared__ array, addressed through pointers the compiler can resolve: it
// then knows the multiply's reads do not touch the LDS an in-flight direct load
// writes, and does not drain the loads before them.
template <int DTO, int BM, bool RES>
__global__ __launch_bounds__(256, 2) void conv32_halo_kernel(HaloArgs a) {
  constexpr int WTM = BM / 2, SM = WTM / 32, SN = halo32::WTN / 32;
  // classic: chunk buffers 0 and 1; resident: weights, halo buffers 1 and 2
  __shared__ __attribute__((aligned(16))) float s_buf0[RES ? halo32::RES_W_FLOATS : halo32::BUF_FLOATS];
  __shared__ __attribute__((aligned(16))) float s_buf1[RES ? halo32::RES_H_FLOATS : halo32::BUF_FLOATS];
  __shared__ __attribute__((aligned(16))) float s_buf2[RES ? halo32::RES_H_FLOATS : 4];
  __shared__ __attribute__((aligned(16))) uint32_t s_koff[halo32::KOFF_MAX];
  const ConvGeom& G = a.geom;

  // Patches are numbered (image, output-row block, output-column block), the
  // column block fastest.  Workgroup -> (co block, one patch); with a resident
  // filter (a.groups > 0, one co block, one chunk) workgroup b takes patches
  // [b P / groups, (b + 1) P / groups) of the P = N * h_blocks * w_blocks.
  // (Numbering the workgroups so that each XCD takes a contiguous range of
  // patches, as the 16-bit kernel does, measured 1.3 % slower on the fp32
  // stem in alternating runs, although it cut the input's re-reads from HBM
  // from 2.0x to 1.2x: at this kernel's 0.3 TB/s they limit nothing.)
  const uint32_t wg = blockIdx.x;
  uint32_t cb = 0, p_first, p_end;
  if (a.groups) {
    const uint32_t P = G.N * a.h_blocks * a.w_blocks;
    p_first = (uint32_t)((uint64_t)wg * P / a.groups);
    p_end = (uint32_t)((uint64_t)(wg + 1) * P / a.groups);
  } else {
    p_first = fdiv(wg, a.div_cob);
    cb = wg - p_first * a.co_blocks;
    p_end = p_first + 1;
  }
  const uint32_t co0 = cb * BM;
  // patch pi -> image, first output row and column
  // (divisions by the grid's invariant counts through FastDiv: a runtime
  // integer division costs tens of instructions)
  auto patch = [&](uint32_t pi, uint32_t& img, uint32_t& oh0, uint32_t& ow0) {
    const uint32_t r = fdiv(pi, a.div_wb);
    ow0 = (pi - r * a.w_blocks) * a.PW;
    img = fdiv(r, a.div_hb);
    oh0 = (r - img * a.h_blocks) * a.PH;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_m = wave >> 1, wave_n = wave & 1;
  const int half = lane >> 5, lrow = lane & 31;

  const uint32_t HR = a.HR, HC = a.HC, HRC = a.hrcp;       // halo rows, columns, floats per channel
  const uint32_t T = G.kh * G.kw, KSTR = a.kstr, BKC = a.bkc;
  const uint32_t KPAD = a.kpad;                             // k-pairs per chunk, multiple of 4
  const uint32_t wofs = BKC * HRC;                          // several chunks: weights follow the halo
  const uint32_t nchunks = (G.C + BKC - 1) / BKC;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);

  // ---- reduction offsets: s_koff[h * KPAD + kp] = halo offset of k = 2 kp + h
  // (k = c*T + r*kw + s -> c*HRC + r*dh*HC + s*dw; 0 past the chunk's indices,
  // where the weights are zero and the input is a finite value of the patch)
  for (uint32_t idx = threadIdx.x; idx < 2 * KPAD; idx += halo32::THREADS) {
    const uint32_t h = idx >= KPAD, kp = idx - h * KPAD, k = 2 * kp + h;
    uint32_t off = 0;
    if (k < BKC * T) {
      const uint32_t c = k / T, t = k - c * T, r = t / G.kw, sx = t - r * G.kw;
      off = c * HRC + r * G.dh * HC + sx * G.dw;
    }
    s_koff[idx] = off;
  }

  // ---- one chunk into LDS (direct loads, 64 floats per instruction)
  // halo of the patch at (img, oh0, ow0) into sh: channel cl, floats
  // [64 pb, 64 pb + 64) of its HR x HC positions; position f = (row, col)
  // reads x at (ih_lo + row, iw_lo + col).
  const uint32_t npi = HRC / 64;                            // instructions per channel
  const uint32_t n_halo = BKC * npi;
  const uint32_t n_wts = (BM * KSTR + 63) / 64;             // weight instructions
  auto halo_to_lds = [&](float* sh, uint32_t c0, uint32_t img, uint32_t oh0, uint32_t ow0) {
    const int32_t ih_lo = (int32_t)oh0 * G.sh - G.pt;
    const int32_t iw_lo = (int32_t)ow0 * G.sw - G.pl;
    const uint32_t bc = G.C - c0 < BKC ? G.C - c0 : BKC;  // channels in this chunk
    uint32_t cl = 0, pbk = (uint32_t)wave;                  // instruction wave + 4j = (cl, pbk)
    while (pbk >= npi) { pbk -= npi; ++cl; }
    for (uint32_t i = wave; i < n_halo; i += 4) {
      const uint32_t f = pbk * 64 + lane;
      const uint32_t row = fdiv(f, a.div_hc), col = f - row * HC;
      const int32_t ih = ih_lo + (int32_t)row;
      const int32_t iw = iw_lo + (int32_t)col;
      const bool ok = cl < bc && row < HR && (uint32_t)ih < G.H && (uint32_t)iw < G.W;
      const uint32_t src = ok ? (((img * G.C + c0 + cl) * G.H + (uint32_t)ih) * G.W + (uint32_t)iw) * 4u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(sh + cl * HRC + pbk * 64), 4, src, 0, 0, 0);
      pbk += 4;
      while (pbk >= npi) { pbk -= npi; ++cl; }
    }
  };
  // weight block of the chunk into sw: [row][h][kp] = w[co0 + row][c0*T + 2 kp + h]; rows KSTR apart
  auto weights_to_lds = [&](float* sw, uint32_t c0) {
    const uint32_t bc = G.C - c0 < BKC ? G.C - c0 : BKC;
    const uint32_t kc = bc * T;
    for (uint32_t i = wave; i < n_wts; i += 4) {
      const uint32_t f = i * 64 + lane;
      const uint32_t row = fdiv(f, a.div_kstr), rem = f - row * KSTR;
      const uint32_t h = rem >= KPAD, kp = rem - h * KPAD, k = 2 * kp + h;
      const bool ok = row < BM && co0 + row < G.Co && rem < 2 * KPAD && k < kc;
      const uint32_t src = ok ? ((co0 + row) * G.C * T + c0 * T + k) * 4u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(sw + i * 64), 4, src, 0, 0, 0);
    }
  };

  // ---- per-lane read offsets (floats) ----------------------------------------
  uint32_t pb[SN];                     // halo offset of this lane's positions (tap 0, channel 0)
#pragma unroll
  for (int si = 0; si < SN; ++si) {
    const uint32_t q = wave_n * halo32::WTN + si * 32 + lrow;
    const uint32_t qh = fdiv(q, a.div_pw), qw = q - qh * a.PW;
    // lanes past the patch read position 0 (in range); their results are never stored
    pb[si] = q < a.PH * a.PW ? qh * G.sh * HC + qw * G.sw : 0u;
  }
  uint32_t wrow[SM];                   // this lane's weights: row, parity half (from the block start)
#pragma unroll
  for (int sj = 0; sj < SM; ++sj)
    wrow[sj] = (uint32_t)(wave_m * WTM + sj * 32 + lrow) * KSTR + (uint32_t)half * KPAD;
  const uint32_t krow = (uint32_t)half * KPAD;

  f32x16 acc[SN][SM];
  auto zero_acc = [&]() {
#pragma unroll
    for (int si = 0; si < SN; ++si)
#pragma unroll
      for (int sj = 0; sj < SM; ++sj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[si][sj][r] = 0.0f;
  };

  // Multiply one chunk in groups of 4 k-pairs: one 16-byte read gives a lane
  // its 4 reduction offsets, one per row tile its 4 weights, then 4 * SN input
  // reads; the next group's reads are issued before this group's MFMAs.
  struct Group {
    float b[4][SN];
    u32x4 w[SM];
  };
  auto load_group = [&](const float* sh, const float* sw, uint32_t g, Group& G4) {
    const u32x4 ko = *reinterpret_cast<const u32x4*>(s_koff + krow + 4 * g);
#pragma unroll
    for (int sj = 0; sj < SM; ++sj) G4.w[sj] = *reinterpret_cast<const u32x4*>(sw + wrow[sj] + 4 * g);
    const uint32_t kos[4] = {ko.x, ko.y, ko.z, ko.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int si = 0; si < SN; ++si) G4.b[j][si] = sh[pb[si] + kos[j]];
  };
  auto mma_group = [&](const Group& G4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int si = 0; si < SN; ++si)
#pragma unroll
        for (int sj = 0; sj < SM; ++sj)
          acc[si][sj] = __builtin_amdgcn_mfma_f32_32x32x2f32(G4.b[j][si], __uint_as_float(G4.w[sj][j]),
                                                             acc[si][sj], 0, 0, 0);
  };
  // the halo at sh, the weight block at sw
  auto multiply = [&](const float* sh, const float* sw, uint32_t kc) {
    const uint32_t ngroups = ((kc + 1) / 2 + 3) / 4;
    Group g0, g1;
    load_group(sh, sw, 0, g0);
    uint32_t g = 0;
    for (; g + 2 <= ngroups; g += 2) {
      load_group(sh, sw, g + 1, g1);
      mma_group(g0);
      if (g + 2 < ngroups) load_group(sh, sw, g + 2, g0);
      mma_group(g1);
    }
    if (g < ngroups) mma_group(g0);
  };

  // raw bias words of this lane's output channels, converted in the epilogue
  uint32_t braw[SM];
  auto load_bias = [&]() {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.bias, a.bias_bytes);
    const bool b32 = a.bias_dt == DT_F32;
#pragma unroll
    for (int sj = 0; sj < SM; ++sj) {
      const uint32_t co = co0 + wave_m * WTM + sj * 32 + lrow;
      const uint32_t off = co < G.Co ? co * (b32 ? 4u : 2u) : kOOB;
      braw[sj] = b32 ? ld_b32(rb, off) : (uint32_t)ld_b16(rb, off);
    }
  };
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, a.y_bytes);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.r, a.r ? a.y_bytes : 0u);
  const uint32_t howo = G.Ho * G.Wo;
  const uint32_t npos = a.PH * a.PW;
  uint32_t img = 0, oh0 = 0, ow0 = 0;                       // the patch the epilogue stores
  auto epilogue = [&](auto act_c, auto res_c) __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool HAS_R = decltype(res_c)::value;
    float bvv[SM];
#pragma unroll
    for (int sj = 0; sj < SM; ++sj)
      bvv[sj] = a.bias_dt == DT_F32 ? __uint_as_float(braw[sj])
                : a.bias_dt == DT_F16 ? widen<DT_F16>(braw[sj]) : widen<DT_BF16>(braw[sj]);
#pragma unroll
    for (int si = 0; si < SN; ++si)
#pragma unroll
      for (int sj = 0; sj < SM; ++sj) {
        const uint32_t co = co0 + wave_m * WTM + sj * 32 + lrow;
        const bool cok = co < G.Co;
        const uint32_t ybase = (img * G.Co + co) * howo;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t q = wave_n * halo32::WTN + si * 32 + 8 * g + 4 * half;
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = acc[si][sj][4 * g + e] + bvv[sj];
          if (a.vec_y) {
            // PW % 4 == 0 and Wo % 4 == 0: positions q..q+3 share an output row
            const uint32_t qh = fdiv(q, a.div_pw), qw = q - qh * a.PW;
            const uint32_t oh = oh0 + qh, ow = ow0 + qw;
            const bool ok = cok && q < npos && oh < G.Ho && ow < G.Wo;
            if constexpr (HAS_R) {
              float rv[4];
              load4<DTO>(rr, ybase + oh * G.Wo + ow, ok, rv);
#pragma unroll
              for (int e = 0; e < 4; ++e) z[e] += rv[e];
            }
            store4<DTO>(ry, ybase + oh * G.Wo + ow, ok, act_fn<ACT, DTO>(z[0], a.alpha),
                        act_fn<ACT, DTO>(z[1], a.alpha), act_fn<ACT, DTO>(z[2], a.alpha),
                        act_fn<ACT, DTO>(z[3], a.alpha));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t qe = q + e;
              const uint32_t qh = fdiv(qe, a.div_pw), qw = qe - qh * a.PW;
              const uint32_t oh = oh0 + qh, ow = ow0 + qw;
              const bool ok = cok && qe < npos && oh < G.Ho && ow < G.Wo;
              float ze = z[e];
              if constexpr (HAS_R) ze += load1<DTO>(rr, ybase + oh * G.Wo + ow, ok);
              store1<DTO>(ry, ybase + oh * G.Wo + ow, ok, act_fn<ACT, DTO>(ze, a.alpha));
            }
          }
        }
      }
  };
  // activation and residual dispatched once per patch
  auto store_patch = [&]() {
    with_act(a.act, [&](auto act_c) __attribute__((always_inline)) {
      with_residual(a.r != nullptr,
                    [&](auto res_c) __attribute__((always_inline)) { epilogue(act_c, res_c); });
    });
  };

  if constexpr (RES) {
    // ---- resident filter (one chunk, one co block): the weight block is
    // staged once; the halo of the next patch streams into the other halo
    // buffer while this one multiplies
    (void)s_buf2;
    patch(p_first, img, oh0, ow0);
    weights_to_lds(s_buf0, 0);
    halo_to_lds(s_buf1, 0, img, oh0, ow0);
    load_bias();
    // patch pi from halo buffer `cur`, the next one into `nxt`
    auto step = [&](uint32_t pi, float* cur, float* nxt) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x0F70);    // this thread's loads of this patch (and earlier stores) done
      __syncthreads();                       // everyone's; the other halo buffer's last reader is done
      uint32_t nimg = 0, noh0 = 0, now0 = 0;
      if (pi + 1 < p_end) {
        patch(pi + 1, nimg, noh0, now0);
        halo_to_lds(nxt, 0, nimg, noh0, now0);
      }
      zero_acc();
      multiply(cur, s_buf0, G.C * T);
      store_patch();
      img = nimg;
      oh0 = noh0;
      ow0 = now0;
    };
    for (uint32_t pi = p_first; pi < p_end; pi += 2) {
      step(pi, s_buf1, s_buf2);
      if (pi + 1 < p_end) step(pi + 1, s_buf2, s_buf1);
    }
  } else {
    (void)s_buf2;
    patch(p_first, img, oh0, ow0);
    load_bias();
    zero_acc();
    if (nchunks == 1) {
      // ---- one chunk: the halo in buffer 0, the weight block in buffer 1
      halo_to_lds(s_buf0, 0, img, oh0, ow0);
      weights_to_lds(s_buf1, 0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      multiply(s_buf0, s_buf1, G.C * T);
    } else {
      // ---- chunk ck in buffer ck % 2 (its halo, then its weight block)
      halo_to_lds(s_buf0, 0, img, oh0, ow0);
      weights_to_lds(s_buf0 + wofs, 0);
      for (uint32_t ck = 0; ck < nchunks; ++ck) {
        const uint32_t c0 = ck * BKC;
        const uint32_t bc = G.C - c0 < BKC ? G.C - c0 : BKC;
        __builtin_amdgcn_s_waitcnt(0x0F70);            // this thread's direct loads of chunk ck have landed
        __syncthreads();                               // ... everyone's, and chunk ck-1's buffer is free
        if (ck & 1) {
          if (ck + 1 < nchunks) {
            halo_to_lds(s_buf0, c0 + BKC, img, oh0, ow0);
            weights_to_lds(s_buf0 + wofs, c0 + BKC);
          }
          multiply(s_buf1, s_buf1 + wofs, bc * T);
        } else {
          if (ck + 1 < nchunks) {
            halo_to_lds(s_buf1, c0 + BKC, img, oh0, ow0);
            weights_to_lds(s_buf1 + wofs, c0 + BKC);
          }
          multiply(s_buf0, s_buf0 + wofs, bc * T);
        }
      }
    }
    store_patch();
  }
}

template <int DTO, int BM>
inline void launch_conv32_halo_t(const HaloArgs& a, hipStream_t s) {
  note_launch("conv-halo fp32, %d co x %ux%u positions%s", BM, a.PH, a.PW,
              a.groups ? ", resident filter" : "");
  if (a.groups)
    launch_kernel(conv32_halo_kernel<DTO, BM, true>, dim3(a.blocks), dim3(halo32::THREADS), s, a);
  else
    launch_kernel(conv32_halo_kernel<DTO, BM, false>, dim3(a.blocks), dim3(halo32::THREADS), s, a);
}

}  // namespace biasact
