// conv_halo.hpp — implicit-GEMM conv2d + bias + activation for fp16 / bf16
// operands that stages the input footprint ("halo") of a patch of output
// rows in LDS, channel-last ([FCT] "这个算子到底在算什么": y = act(conv2d(x,
// filter, bias)); "双 Kernel 是怎么分工的": weights as the co x k operand, input
// features as the k x spatial operand).
//
// The reduction index is ordered (tap, channel): k = t * C + c with
// t = r * kw + s.  For one tap and 8 consecutive channels, both operands are
// 16 contiguous bytes in LDS:
//   halo  [row][col][c] : input rows  ih = oh*sh - pt + r*dh of the patch,
//                         columns iw = iw_lo + col (iw_lo even, <= ow0*sw - pl)
//   wts   [t][co][c]
// Channels are staged in chunks of BKC = 64, 32 or 16 (zero-filled past C).
// so every MFMA fragment is one ds_read_b128 whatever the stride, padding or
// dilation, and each input element is fetched from memory once per channel
// chunk instead of once per tap.
//
// Workgroup: 256 threads (2 x 2 waves), BM output channels x a patch of PH
// output rows x PW output columns (positions q = row * PW + col, BN = PH * PW
// rounded up to 32 per wave column).  Channel chunks of BKC are staged with
// register-transposed 4-byte input loads (two columns x 8 channels -> two
// 16-byte LDS writes) and 16-byte weight loads (8 channels x T taps -> T
// 16-byte LDS writes).  Each 16-byte chunk of an LDS row sits at slot
// chunk ^ (row % 8) (rows of 8 chunks) so 8 consecutive rows hit 8 slots.
#pragma once

#include "epilogue.hpp"
#include "launch.hpp"
#include "mfma_core.hpp"

namespace biasact {

namespace halo {
constexpr int THREADS = 256;
constexpr int LDS_BYTES = 144 * 1024;
}  // namespace halo

// Slot of 16-byte chunk `c` in a row `row` holding `nch` chunks (power of 2).
__device__ __forceinline__ uint32_t halo_slot(uint32_t row, uint32_t c, uint32_t nch) {
  return c ^ (row & (nch - 1) & 7);
}

// T = taps (kh*kw) known at compile time (1, 9, ...): 16-byte weight loads.
// BM: output channels per workgroup (64 or 128); WTN: positions per wave (multiple of 32).
template <int DTI, int DTO, int T, int BM, int WTN>
__global__ __launch_bounds__(256, 1) void conv16_halo_kernel(HaloArgs a) {
  static_assert(DTI == DT_F16 || DTI == DT_BF16, "16-bit operands only");
  constexpr int WTM = BM / 2, SM = WTM / 32, SN = WTN / 32;
  __shared__ __attribute__((aligned(16))) uint8_t smem[halo::LDS_BYTES];
  const ConvGeom& G = a.geom;

  // workgroup -> (co block, image, output-row block, output-column block)
  uint32_t bid = blockIdx.x;
  const uint32_t cb = bid % a.co_blocks;  bid /= a.co_blocks;
  const uint32_t wb = bid % a.w_blocks;   bid /= a.w_blocks;
  const uint32_t hb = bid % a.h_blocks;   bid /= a.h_blocks;
  const uint32_t img = bid;
  const uint32_t co0 = cb * BM, oh0 = hb * a.PH, ow0 = wb * a.PW;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_m = wave >> 1, wave_n = wave & 1;
  const int half = lane >> 5, lrow = lane & 31;

  // halo geometry of this patch
  const int32_t ih_lo = (int32_t)oh0 * G.sh - G.pt;
  const int32_t iw_first = (int32_t)ow0 * G.sw - G.pl;
  const int32_t iw_lo = iw_first & ~1;                 // even (floor) so column pairs are 4-byte aligned
  const uint32_t col_shift = (uint32_t)(iw_first - iw_lo);
  const uint32_t BKC = a.bkc, NCH = BKC / 8;
  const uint32_t HR = a.HR, HC = a.HC;                 // halo rows, columns (HC even)
  const uint32_t halo_bytes = HR * HC * BKC * 2;
  uint8_t* s_halo = smem;
  uint8_t* s_wts = smem + halo_bytes;                  // T * BM * BKC * 2 bytes

  // ---- accumulators start at the bias ------------------------------------
  f32x16 acc[SN][SM];
  {
    uint32_t idx[SM];
    float bv[SM];
#pragma unroll
    for (int sj = 0; sj < SM; ++sj) idx[sj] = co0 + wave_m * WTM + sj * 32 + lrow;
    load_bias_vec<SM>(a.bias, a.bias_bytes, a.bias_dt, idx, G.Co, bv);
#pragma unroll
    for (int sj = 0; sj < SM; ++sj)
#pragma unroll
      for (int si = 0; si < SN; ++si)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[si][sj][r] = bv[sj];
  }

  // ---- per-lane B-fragment positions (position -> halo row/col) -----------
  uint32_t pos_rowcol[SN];     // halo (row, col) of tap (0, 0) as row * HC + col
  bool pos_ok[SN];
#pragma unroll
  for (int si = 0; si < SN; ++si) {
    const uint32_t q = wave_n * WTN + si * 32 + lrow;
    const uint32_t qh = q / a.PW, qw = q - qh * a.PW;
    pos_ok[si] = q < a.PH * a.PW;
    // lanes past the patch read halo position 0 (in range); their results are never stored
    pos_rowcol[si] = pos_ok[si] ? (qh * G.sh) * HC + qw * G.sw + col_shift : 0u;
  }

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
  const uint32_t HW = G.H * G.W;
  const uint32_t nchunks = (G.C + BKC - 1) / BKC;

  for (uint32_t ck = 0; ck < nchunks; ++ck) {
    const uint32_t c0 = ck * BKC;
    if (ck > 0) __syncthreads();                       // previous chunk fully consumed
    // ---- stage the input halo: item = (row, column pair, 8-channel group)
    {
      const uint32_t pairs = HC / 2, items = HR * pairs * NCH;
      for (uint32_t it = threadIdx.x; it < items; it += halo::THREADS) {
        const uint32_t g = it % NCH;
        const uint32_t rp = it / NCH;
        const uint32_t pr = rp % pairs, hr = rp / pairs;
        const int32_t ih = ih_lo + (int32_t)hr;
        const int32_t iw = iw_lo + 2 * (int32_t)pr;
        const bool rok = (uint32_t)ih < G.H && (uint32_t)iw < G.W;   // W even: iw+1 < W too
        uint32_t d[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t c = c0 + g * 8 + e;
          const uint32_t off = (img * G.C + c) * HW + (uint32_t)ih * G.W + (uint32_t)iw;
          d[e] = ld_b32(rx, (rok && c < G.C) ? off * 2u : kOOB);
        }
        // d[e] = (col 2pr: channel e | col 2pr+1: channel e); transpose to two channel chunks
        u32x4 lo, hi;
        lo.x = (d[0] & 0xffffu) | (d[1] << 16);
        lo.y = (d[2] & 0xffffu) | (d[3] << 16);
        lo.z = (d[4] & 0xffffu) | (d[5] << 16);
        lo.w = (d[6] & 0xffffu) | (d[7] << 16);
        hi.x = (d[0] >> 16) | (d[1] & 0xffff0000u);
        hi.y = (d[2] >> 16) | (d[3] & 0xffff0000u);
        hi.z = (d[4] >> 16) | (d[5] & 0xffff0000u);
        hi.w = (d[6] >> 16) | (d[7] & 0xffff0000u);
        const uint32_t p0 = hr * HC + 2 * pr, p1 = p0 + 1;
        *reinterpret_cast<u32x4*>(s_halo + (p0 * NCH + halo_slot(p0, g, NCH)) * 16) = lo;
        *reinterpret_cast<u32x4*>(s_halo + (p1 * NCH + halo_slot(p1, g, NCH)) * 16) = hi;
      }
    }
    // ---- stage the weights: item = (co, 8-channel group); 8*T contiguous values
    {
      const uint32_t items = BM * NCH;
      for (uint32_t it = threadIdx.x; it < items; it += halo::THREADS) {
        const uint32_t g = it % NCH, col = it / NCH;
        const uint32_t co = co0 + col;
        const uint32_t cbase = c0 + g * 8;
        const bool ok = co < G.Co && cbase < G.C;     // C % 8 == 0: whole group in or out
        const uint32_t base = (co * G.C + cbase) * T * 2u;
        uint32_t v[4 * T];
#pragma unroll
        for (int j = 0; j < T; ++j) {
          const u32x4 q = ld_b128(rw, ok ? base + 16u * j : kOOB);
          v[4 * j + 0] = q.x; v[4 * j + 1] = q.y; v[4 * j + 2] = q.z; v[4 * j + 3] = q.w;
        }
        // element (channel e, tap t) is value e*T + t of the run
#pragma unroll
        for (int t = 0; t < T; ++t) {
          uint32_t w16[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int p = e * T + t;
            w16[e] = (v[p >> 1] >> (16 * (p & 1))) & 0xffffu;
          }
          u32x4 o;
          o.x = w16[0] | (w16[1] << 16);
          o.y = w16[2] | (w16[3] << 16);
          o.z = w16[4] | (w16[5] << 16);
          o.w = w16[6] | (w16[7] << 16);
          const uint32_t row = t * BM + col;
          *reinterpret_cast<u32x4*>(s_wts + (row * NCH + halo_slot(row, g, NCH)) * 16) = o;
        }
      }
    }
    __syncthreads();
    // ---- multiply: every tap, every 16-channel step ---------------------------
    const uint32_t ksteps = BKC / 16;
    for (int t = 0; t < T; ++t) {
      const uint32_t r = t / G.kw, s = t - r * G.kw;
      const uint32_t tap_rc = (r * G.dh) * HC + s * G.dw;
      for (uint32_t ks = 0; ks < ksteps; ++ks) {
        const uint32_t ch = 2 * ks + half;                 // 16-byte chunk of this lane
        u32x4 fi[SN], fj[SM];
#pragma unroll
        for (int si = 0; si < SN; ++si) {
          const uint32_t p = pos_rowcol[si] + tap_rc;
          fi[si] = *reinterpret_cast<const u32x4*>(s_halo + (p * NCH + halo_slot(p, ch, NCH)) * 16);
        }
#pragma unroll
        for (int sj = 0; sj < SM; ++sj) {
          const uint32_t row = t * BM + wave_m * WTM + sj * 32 + lrow;
          fj[sj] = *reinterpret_cast<const u32x4*>(s_wts + (row * NCH + halo_slot(row, ch, NCH)) * 16);
        }
#pragma unroll
        for (int si = 0; si < SN; ++si)
#pragma unroll
          for (int sj = 0; sj < SM; ++sj) mfma_chunk<DTI>(acc[si][sj], fi[si], fj[sj]);
      }
    }
  }

  // ---- epilogue: activation, cast, one store per element -------------------
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, a.y_bytes);
  const uint32_t howo = G.Ho * G.Wo;
#pragma unroll
  for (int si = 0; si < SN; ++si)
#pragma unroll
    for (int sj = 0; sj < SM; ++sj) {
      const uint32_t co = co0 + wave_m * WTM + sj * 32 + lrow;
      const bool cok = co < G.Co;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t q = wave_n * WTN + si * 32 + 8 * g + 4 * half + e;
          const uint32_t qh = q / a.PW, qw = q - qh * a.PW;
          const uint32_t oh = oh0 + qh, ow = ow0 + qw;
          const bool ok = cok && q < a.PH * a.PW && oh < G.Ho && ow < G.Wo;
          const float v = apply_act(a.act, acc[si][sj][4 * g + e], a.alpha);
          store1<DTO>(ry, (img * G.Co + co) * howo + oh * G.Wo + ow, ok, v);
        }
      }
    }
}

template <int DTI, int DTO, int T, int BM, int WTN>
inline void launch_conv_halo_t(const HaloArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((conv16_halo_kernel<DTI, DTO, T, BM, WTN>), dim3(a.blocks), dim3(halo::THREADS), 0,
                     s, a);
}

}  // namespace biasact
