// conv_halo.hpp — implicit-GEMM conv2d + bias + activation for fp16 / bf16
// operands that stages the input footprint ("halo") of a patch of output
// rows in LDS, channel-last ([FCT] "这个算子到底在算什么": y = act(conv2d(x,
// filter, bias)); "双 Kernel 是怎么分工的": weights as the co x k operand, input
// features as the k x spatial operand).
//
// The reduction index is ordered (tap, channel): k = t * C + c with
// t = r * kw + s.  For one tap and 8 consecutive channels the input operand
// is 16 contiguous bytes of the LDS halo
//   halo  [row][col][c] : input rows  ih = oh*sh - pt + r*dh of the patch,
//                         columns iw = iw_lo + col (iw_lo even, <= ow0*sw - pl)
// so every input fragment is one ds_read_b128 whatever the stride, padding or
// dilation, and each input element is fetched from memory once per channel
// chunk instead of once per tap.  The weight fragments (8 channels of one tap
// per lane) are regrouped in registers from the chunk's raw OIHW rows in LDS
// (below).  Channels are staged in chunks of BKC = 16 * KS (KS = 1, 2, 4 MFMA
// k-steps per tap; zero-filled past C).
//
// Workgroup: NW = 4 or 8 waves as 2 (output-channel halves) x NW / 2
// (position groups), BM output channels x a patch of PH output rows x PW
// output columns (positions q = row * PW + col, at most 32 * SN * NW / 2).
// Four-wave variants small enough for two workgroups per CU (80 KB of LDS,
// two fragment sets per wave) let one workgroup's staging and epilogue
// overlap another's MFMAs; the eight-wave variants have their CU alone with
// two waves per SIMD, which fetches each weight chunk once per CU.  Square
// filters up to 7x7: beyond 3x3 (T = 25, 49 taps) one four-wave configuration
// (64 channels, one 16-channel k-step per chunk) whose wave holds the 4 T
// fragment registers of a chunk in the accumulation registers.
// Staging items: input (halo row, column pair, 8 channels) — eight 4-byte
// loads transposed in registers into two 16-byte LDS writes; weights — the
// chunk's raw OIHW rows (8 channels x T taps are contiguous) copied into LDS
// by 16-byte direct loads, then regrouped in each wave's registers into MFMA
// fragments.  The first HB input items of each thread form a batch whose
// offsets are computed once; the batch and weights of chunk 0 are issued
// before anything waits, and those of chunk ck + 1 are spread over the MFMA
// steps of chunk ck.  Items beyond the batch (large halos) are staged with
// their own loads before the multiply.  The multiply is unrolled over its
// T * KS (tap, k-step) steps; a step's input fragments are read two steps
// ahead.
//
// Halo rows (one position) hold NCH = 2 * KS chunks of 16 bytes; chunk c of
// row p sits at slot c ^ ((p >> S) % NCH) with 2^S = 16 / NCH rows per 256
// bytes, so the 16 lanes of a read phase that take 16 consecutive rows hit
// all 64 banks once.  Raw weight rows carry one 16-byte pad piece each, so 16
// consecutive rows start in 16 different bank groups.  The bias is fetched as
// raw words after the first staging loads and added in the epilogue.
#pragma once

#include <utility>

#include "epilogue.hpp"
#include "launch.hpp"
#include "launch_kernel.hpp"
#include "mfma_core.hpp"
#include "tile_map.hpp"

namespace biasact {

namespace halo {
constexpr int LDS_ONE = 144 * 1024;     // LDS of a workgroup that has its CU alone
constexpr int LDS_TWO = 80 * 1024;      // LDS of a workgroup that shares its CU with another
constexpr int HB = 4;     // input items per thread in the precomputed batch (2 with two workgroups
                          // per CU, eight waves, or filters beyond 3x3)
constexpr uint32_t kNone = 0xffffffffu;   // "no LDS write" marker of an item
constexpr uint32_t kFar = 1u << 30;       // channel offset that fails every c < C test

// Row -> slot-mask shift for rows of NCH 16-byte chunks.
template <int NCH>
constexpr int row_shift() { return NCH == 8 ? 1 : (NCH == 4 ? 2 : 3); }

template <int NCH>
__device__ __forceinline__ uint32_t slot(uint32_t row, uint32_t c) {
  return c ^ ((row >> row_shift<NCH>()) & (NCH - 1));
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order.
template <class F, int... I>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

// Scheduling groups of one multiply step: NM MFMAs, with the ND LDS reads and
// NV global loads of the step spread evenly behind them.
template <int NM, int ND, int NV, int I = 0>
__device__ __forceinline__ void interleave() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int d = (I + 1) * ND / NM - I * ND / NM;
    if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);
    constexpr int v = (I + 1) * NV / NM - I * NV / NM;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
    interleave<NM, ND, NV, I + 1>();
  }
}
}  // namespace halo

// Two four-wave workgroups share a CU when a wave holds at most two
// weight-fragment sets of at most 9 taps and two accumulator tiles (then 256
// registers per lane suffice); an eight-wave workgroup has its CU alone (two
// waves per SIMD), and so has a four-wave one with a larger filter (its wave
// holds 4 T fragment registers: up to 512 registers per lane with the
// accumulation registers).
template <int BM, int KS, int SN, int NW = 4, int T = 9>
constexpr int occupancy() {
  return NW == 4 && T <= 9 && KS * (BM / 64) <= 2 && SN * (BM / 64) <= 2 ? 2 : 1;
}

// T = taps (kh*kw: a square 1x1, 3x3, 5x5 or 7x7 filter), BM = output
// channels per workgroup (64 or 128),
// KS = 16-channel k-steps per tap and chunk (1, 2 or 4; KS * BM / 64 <= 4),
// SN = 32-position MFMA tiles per wave, NW = waves (4 or 8) as a grid of 2
// (output-channel halves) x NW / 2 (position groups): NW / 2 x SN x 32
// positions per workgroup.
template <int DTI, int DTO, int T, int BM, int KS, int SN, int NW>
__global__ __launch_bounds__(NW * 64, (occupancy<BM, KS, SN, NW, T>())) void conv16_halo_kernel(HaloArgs a) {
  static_assert(DTI == DT_F16 || DTI == DT_BF16, "16-bit operands only");
  static_assert(T == 1 || T == 9 || T == 25 || T == 49, "square 1x1, 3x3, 5x5 or 7x7 filters");
  static_assert(T <= 9 || (KS == 1 && BM == 64 && NW == 4), "larger filters: one k-step, 64 channels, four waves");
  constexpr uint32_t KW = T == 49 ? 7 : T == 25 ? 5 : T == 9 ? 3 : 1;   // filter width
  constexpr int WTM = BM / 2, SM = WTM / 32, WTN = 32 * SN;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  constexpr int LDS = occupancy<BM, KS, SN, NW, T>() == 2 ? halo::LDS_TWO : halo::LDS_ONE;
  constexpr int WGN = NW / 2;                           // position groups
  static_assert(KS * SM <= 4, "weight fragments of a chunk must fit in registers");
  constexpr int BKC = 16 * KS, NCH = 2 * KS, ROWB = NCH * 16;
  constexpr int NSTEP = T * KS;
  constexpr int HB = occupancy<BM, KS, SN, NW, T>() == 2 || NW == 8 || T > 9 ? 2 : halo::HB, NTH = NW * 64;
  constexpr int RP = BKC * T / 8;                       // 16-byte pieces of one weight row
  constexpr int RSTR = (RP + 1) * 16;                   // row stride: the pieces and a pad
  constexpr int NPIECE = BM * (RP + 1);
  constexpr int NDMA = (NPIECE + 63) / 64;              // direct loads of one chunk (all waves)
  constexpr int NPF = HB * 8;                           // input loads of one batch
  constexpr int PER = (NPF + NSTEP - 1) / NSTEP;        // batch loads per multiply step
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[NDMA * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t s_halo[LDS - NDMA * 1024];
  const ConvGeom& G = a.geom;

  // workgroup -> (co block, output-column block, output-row block, image),
  // numbered so that each XCD takes a contiguous range: neighbouring row
  // blocks, whose halos share input rows, then share an L2
  uint32_t bid = xcd_contiguous(blockIdx.x, gridDim.x);
  // (divisions by the grid's invariant block counts through FastDiv: a
  // runtime integer division costs tens of VALU instructions)
  uint32_t qd = fdiv(bid, a.div_cob);
  const uint32_t cb = bid - qd * a.co_blocks;  bid = qd;
  qd = fdiv(bid, a.div_wb);
  const uint32_t wb = bid - qd * a.w_blocks;   bid = qd;
  qd = fdiv(bid, a.div_hb);
  const uint32_t hb = bid - qd * a.h_blocks;   bid = qd;
  const uint32_t img = bid;
  const uint32_t co0 = cb * BM, oh0 = hb * a.PH, ow0 = wb * a.PW;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_m = wave / WGN, wave_n = wave % WGN;
  const int half = lane >> 5, lrow = lane & 31;

  // halo geometry of this patch
  const int32_t ih_lo = (int32_t)oh0 * G.sh - G.pt;
  const int32_t iw_first = (int32_t)ow0 * G.sw - G.pl;
  const int32_t iw_lo = iw_first & ~1;                 // even (floor) so column pairs are 4-byte aligned
  const uint32_t col_shift = (uint32_t)(iw_first - iw_lo);
  const uint32_t HC = a.HC;                            // halo columns (even)

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
  const uint32_t HW2 = G.H * G.W * 2u;                 // bytes between channels of x
  const uint32_t nchunks = (G.C + BKC - 1) / BKC;
  const uint32_t pairs = HC / 2;
  const uint32_t h_items = a.HR * pairs * NCH;

  // ---- weights: raw OIHW rows of a chunk, copied straight into LDS ---------
  // Piece P of the chunk = (row P / (RP+1), piece P % (RP+1)); the last piece
  // of a row is padding so rows start in different banks.  Padding, rows past
  // Co and channel groups past C are filled with zeros (out-of-range loads).
  // Wave w issues the direct loads w, w + 4, ...
  constexpr int KWL = (NDMA + NW - 1) / NW;             // direct weight loads per wave
  // Direct load k of this wave (load i = wave + NW k covers pieces 64i .. 64i+63).
  // Each lane's offset within the chunk is computed once (kOOB for pad
  // pieces and rows past Co), its low bits (zero in a 16-byte offset) holding
  // the piece's 8-channel group; a chunk at channel c0 then passes c0 * T * 2
  // as the scalar offset of the load, and a lane whose channels lie past C (a
  // partial last chunk) passes kOOB.  The
  // issue of these loads is bound by the vector instructions of their
  // addresses (a probe of this copy moved 20 B/clk per CU with the addresses
  // computed per load and 52 B/clk with them computed beforehand).
  static_assert(BKC / 8 <= 8, "the channel group must fit the offset's low bits");
  uint32_t wofs[KWL];
#pragma unroll
  for (int k = 0; k < KWL; ++k) {
    const uint32_t P = (uint32_t)(wave + NW * k) * 64 + lane;
    const uint32_t row = P / (RP + 1), pc = P - row * (RP + 1);
    const bool ok = pc < RP && row < BM && co0 + row < G.Co;
    wofs[k] = ok ? ((co0 + row) * G.C * T * 2u + pc * 16u) | (pc / T) : kOOB;
  }
  // lim = channels left from c0 (0: issue the loads but fetch nothing)
  auto weight_load = [&](auto k_c, uint32_t c0, uint32_t lim) {
    constexpr int k = decltype(k_c)::value;
    const int li = wave + NW * k;
    if (k + 1 < KWL || li < NDMA) {                    // only the last load can be past the chunk
      const uint32_t src = 8u * (wofs[k] & 7u) < lim ? wofs[k] & ~15u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(s_raw + li * 1024), 16, src, c0 * T * 2u, 0, 0);
    }
  };
  auto weights_to_lds = [&](uint32_t c0, uint32_t lim) {
    halo::unroll<KWL>([&](auto k_c) { weight_load(k_c, c0, lim); });
  };

  // ---- input halo: item it = (halo row, channel group, column pair) --------
  // x offset of channel 8g of chunk 0 (kOOB outside the image), channel offset
  // 8g (kFar when the item does not exist), LDS addresses of its two columns.
  // The column pair varies fastest across lanes, so each of an item's eight
  // 4-byte loads (one channel each) reads consecutive column pairs of one
  // input row: a wave's load covers a few cache lines, not one line per lane.
  auto halo_item = [&](uint32_t it, uint32_t& src, uint32_t& g8, uint32_t& lo, uint32_t& hi) {
    const uint32_t rg = fdiv(it, a.div_pairs), pr = it - rg * pairs;
    const uint32_t g = rg % NCH, hr = rg / NCH;
    const int32_t ih = ih_lo + (int32_t)hr, iw = iw_lo + 2 * (int32_t)pr;
    const bool exists = it < h_items;
    // W even: iw + 1 < W too
    src = (uint32_t)ih < G.H && (uint32_t)iw < G.W
              ? ((img * G.C + g * 8) * G.H * G.W + (uint32_t)ih * G.W + (uint32_t)iw) * 2u
              : kOOB;
    g8 = exists ? g * 8 : halo::kFar;
    const uint32_t p0 = hr * HC + 2 * pr, p1 = p0 + 1;
    lo = exists ? p0 * ROWB + halo::slot<NCH>(p0, g) * 16 : halo::kNone;
    hi = p1 * ROWB + halo::slot<NCH>(p1, g) * 16;
  };
  uint32_t hreg[HB][8];
  auto halo_load1 = [&](uint32_t (&d)[8], uint32_t src, uint32_t g8, uint32_t c0) {
    const bool ok = src != kOOB && c0 + g8 < G.C;    // C % 8 == 0: the group is all in or all out
    const uint32_t off = src + c0 * HW2;
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = ld_b32(rx, ok ? off + e * HW2 : kOOB);
  };
  auto halo_store1 = [&](const uint32_t (&d)[8], uint32_t lo, uint32_t hi) {
    if (lo == halo::kNone) return;
    // d[e] = (column 2pr: channel e | column 2pr+1: channel e); transpose into two chunks
    u32x4 vlo, vhi;
    vlo.x = __builtin_amdgcn_perm(d[1], d[0], 0x05040100u);
    vlo.y = __builtin_amdgcn_perm(d[3], d[2], 0x05040100u);
    vlo.z = __builtin_amdgcn_perm(d[5], d[4], 0x05040100u);
    vlo.w = __builtin_amdgcn_perm(d[7], d[6], 0x05040100u);
    vhi.x = __builtin_amdgcn_perm(d[1], d[0], 0x07060302u);
    vhi.y = __builtin_amdgcn_perm(d[3], d[2], 0x07060302u);
    vhi.z = __builtin_amdgcn_perm(d[5], d[4], 0x07060302u);
    vhi.w = __builtin_amdgcn_perm(d[7], d[6], 0x07060302u);
    *reinterpret_cast<u32x4*>(s_halo + lo) = vlo;
    *reinterpret_cast<u32x4*>(s_halo + hi) = vhi;
  };
  // batch descriptors (fixed for the whole workgroup)
  uint32_t hd_src[HB], hd_g8[HB], hd_lo[HB], hd_hi[HB];
#pragma unroll
  for (int b = 0; b < HB; ++b) halo_item(b * NTH + threadIdx.x, hd_src[b], hd_g8[b], hd_lo[b], hd_hi[b]);
  // Batch of the chunk at channel c0 with lim channels left from c0 (0: fetch
  // nothing): per item the x offset of its channel group at chunk 0, or kOOB
  // (set once per chunk); load e of the item adds (c0 + e) * HW2 as the scalar
  // offset of the load.  (kOOB plus a scalar offset below 2^31 stays past
  // every buffer: all tensors are smaller than 2^31 bytes.)
  uint32_t hbase[HB];
  auto batch_bases = [&](uint32_t lim) {
#pragma unroll
    for (int b = 0; b < HB; ++b) hbase[b] = hd_g8[b] < lim ? hd_src[b] : kOOB;
  };
  auto batch_load = [&](auto i_c, uint32_t c0) {
    constexpr int b = decltype(i_c)::value / 8, e = decltype(i_c)::value % 8;
    hreg[b][e] = __builtin_amdgcn_raw_buffer_load_b32(rx, hbase[b], (c0 + e) * HW2, 0);
  };

  // ---- fragment addresses --------------------------------------------------
  // input (k-step 0; k-step ks flips slot bits by 2*ks): tap t, MFMA tile si.
  // Up to 9 taps the addresses are kept (T * SN registers); larger filters
  // form them per step from the tap's offset, a scalar.
  constexpr bool KEEP = T <= 9;
  uint32_t pos[SN];
#pragma unroll
  for (int si = 0; si < SN; ++si) {
    const uint32_t q = wave_n * WTN + si * 32 + lrow;
    const uint32_t qh = fdiv(q, a.div_pw), qw = q - qh * a.PW;
    // lanes past the patch read halo position 0 (in range); their results are never stored
    pos[si] = q < a.PH * a.PW ? (qh * G.sh) * HC + qw * G.sw + col_shift : 0u;
  }
  // halo position of tap (r, s) for tile si: prow[r][si] + s * dw
  uint32_t prow[KW][SN];
#pragma unroll
  for (uint32_t r = 0; r < KW; ++r)
#pragma unroll
    for (int si = 0; si < SN; ++si) prow[r][si] = pos[si] + r * G.dh * HC;
  auto frag_addr = [&](uint32_t t, int si) {
    const uint32_t r = t / KW, s = t - r * KW;
    const uint32_t p = prow[r][si] + s * G.dw;
    return p * ROWB + halo::slot<NCH>(p, (uint32_t)half) * 16;
  };
  uint32_t h_addr[KEEP ? T : 1][SN];
  if constexpr (KEEP) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int si = 0; si < SN; ++si) h_addr[t][si] = frag_addr((uint32_t)t, si);
  }
  // weights: this lane's rows (output channels) in the raw chunk
  uint32_t w_row[SM];
#pragma unroll
  for (int sj = 0; sj < SM; ++sj) w_row[sj] = (uint32_t)(wave_m * WTM + sj * 32 + lrow) * RSTR;

  // Weight fragments of a chunk: for k-step ks and row tile sj, this lane's
  // 8 channels (8 * (2 ks + half) ...) of every tap, regrouped from the raw run
  // (channel e, tap t at element e * T + t); channels past C arrive as zeros.
  // Up to 9 taps the whole run (T 16-byte reads) is read into registers at
  // once; larger filters read the 8 words of each fragment one by one, so
  // that only the fragments stay live.
  auto sel_of = [](int p0, int p1) {
    return (uint32_t)((p0 & 1) * 2) | ((uint32_t)((p0 & 1) * 2 + 1) << 8) |
           ((uint32_t)(4 + (p1 & 1) * 2) << 16) | ((uint32_t)(5 + (p1 & 1) * 2) << 24);
  };
  u32x4 afr[KS][T][SM];
  auto build_weights = [&]() {
    if constexpr (!KEEP) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int sj = 0; sj < SM; ++sj) {
          const uint32_t g = 2 * ks + half;
          const uint8_t* base = s_raw + w_row[sj] + g * 16 * T;
#pragma unroll
          for (int t = 0; t < T; ++t) {
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int p0 = (2 * k) * T + t, p1 = (2 * k + 1) * T + t;
              const uint32_t d0 = *reinterpret_cast<const uint32_t*>(base + (p0 >> 1) * 4);
              const uint32_t d1 = *reinterpret_cast<const uint32_t*>(base + (p1 >> 1) * 4);
              o[k] = __builtin_amdgcn_perm(d1, d0, sel_of(p0, p1));
            }
            afr[ks][t][sj] = u32x4{o[0], o[1], o[2], o[3]};
            // a few fragments at a time: the scheduler would otherwise issue
            // every read first and hold all their words in registers
            if (t % 4 == 3) __builtin_amdgcn_sched_barrier(0);
          }
        }
      return;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int sj = 0; sj < SM; ++sj) {
        const uint32_t g = 2 * ks + half;
        const uint8_t* base = s_raw + w_row[sj] + g * 16 * T;
        uint32_t v[4 * T];
#pragma unroll
        for (int j = 0; j < T; ++j) {
          const u32x4 q = *reinterpret_cast<const u32x4*>(base + 16 * j);
          v[4 * j + 0] = q.x;
          v[4 * j + 1] = q.y;
          v[4 * j + 2] = q.z;
          v[4 * j + 3] = q.w;
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          uint32_t o[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int p0 = (2 * k) * T + t, p1 = (2 * k + 1) * T + t;
            o[k] = __builtin_amdgcn_perm(v[p1 >> 1], v[p0 >> 1], sel_of(p0, p1));
          }
          afr[ks][t][sj] = u32x4{o[0], o[1], o[2], o[3]};
        }
      }
  };

  auto load_b = [&](auto st_c, u32x4 (&fi)[SN]) {
    constexpr int st = decltype(st_c)::value;
    constexpr int ks = st / T, t = st % T;
    constexpr uint32_t flip = (uint32_t)(2 * ks) << 4;
#pragma unroll
    for (int si = 0; si < SN; ++si) {
      uint32_t ad;
      if constexpr (KEEP) ad = h_addr[t][si];
      else ad = frag_addr((uint32_t)t, si);
      fi[si] = *reinterpret_cast<const u32x4*>(s_halo + (ad ^ flip));
    }
  };

  // Accumulators.  A wave with a single 32x32 tile alternates two of them
  // between consecutive steps: an MFMA that waits for the previous one's
  // result issues about a third slower than one that does not.
  constexpr int NACC = SN * SM == 1 ? 2 : 1;
  f32x16 acc[NACC][SN][SM];
#pragma unroll
  for (int c = 0; c < NACC; ++c)
#pragma unroll
    for (int si = 0; si < SN; ++si)
#pragma unroll
      for (int sj = 0; sj < SM; ++sj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][si][sj][r] = 0.0f;

  // All KS * T steps of one chunk (k-step major).  The weight copy and the
  // input batch of the chunk at channel c1 (lim1 channels left from c1; 0 past
  // the last chunk: then the loads fetch nothing) ride along, WPS direct loads
  // and PER input loads per step, so their issue, which waits whenever the
  // memory pipeline is full, stays behind the MFMAs.  One instance of the
  // step sequence for every chunk keeps the accumulators in the same
  // registers throughout.
  constexpr int WPS = (KWL + NSTEP - 1) / NSTEP;
  constexpr int PD = NSTEP >= 3 ? 2 : 1, NB = PD + 1;
  auto multiply = [&](uint32_t c1, uint32_t lim1) {
    batch_bases(lim1);
    // fragments are read PD steps ahead: one step's MFMAs are too short to
    // cover the latency of an LDS read
    u32x4 fi[NB][SN];
    halo::unroll<PD>([&](auto j_c) { load_b(j_c, fi[decltype(j_c)::value]); });
    halo::unroll<NSTEP>([&](auto st_c) {
      constexpr int st = decltype(st_c)::value;
      constexpr int cur = st % NB, ks = st / T, t = st % T;
      if constexpr (st + PD < NSTEP) load_b(std::integral_constant<int, st + PD>{}, fi[(st + PD) % NB]);
      constexpr int w0 = st * WPS < KWL ? st * WPS : KWL;
      constexpr int w1 = (st + 1) * WPS < KWL ? (st + 1) * WPS : KWL;
      halo::unroll<w1 - w0>([&](auto k_c) {
        weight_load(std::integral_constant<int, w0 + decltype(k_c)::value>{}, c1, lim1);
      });
      constexpr int v0 = st * PER < NPF ? st * PER : NPF;
      constexpr int v1 = (st + 1) * PER < NPF ? (st + 1) * PER : NPF;
      halo::unroll<v1 - v0>([&](auto k_c) {
        batch_load(std::integral_constant<int, v0 + decltype(k_c)::value>{}, c1);
      });
#pragma unroll
      for (int si = 0; si < SN; ++si)
#pragma unroll
        for (int sj = 0; sj < SM; ++sj) mfma_chunk<DTI>(acc[st % NACC][si][sj], fi[cur][si], afr[ks][t][sj]);
      halo::interleave<SN * SM, st + PD < NSTEP ? SN : 0, (v1 - v0) + (w1 - w0)>();
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- chunk loop ------------------------------------------------------------
  weights_to_lds(0u, G.C);
  batch_bases(G.C);
  halo::unroll<NPF>([&](auto i_c) { batch_load(i_c, 0u); });
  // raw bias words of this lane's output channels, converted in the epilogue
  uint32_t braw[SM];
  {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.bias, a.bias_bytes);
    const bool b32 = a.bias_dt == DT_F32;
#pragma unroll
    for (int sj = 0; sj < SM; ++sj) {
      const uint32_t co = co0 + wave_m * WTM + sj * 32 + lrow;
      const uint32_t off = co < G.Co ? co * (b32 ? 4u : 2u) : kOOB;
      braw[sj] = b32 ? ld_b32(rb, off) : (uint32_t)ld_b16(rb, off);
    }
  }
  for (uint32_t ck = 0; ck < nchunks; ++ck) {
    const uint32_t c0 = ck * BKC, c1 = c0 + BKC;
    if (ck > 0) __syncthreads();                       // the previous multiply is done with the halo
#pragma unroll
    for (int b = 0; b < HB; ++b) halo_store1(hreg[b], hd_lo[b], hd_hi[b]);
    // input items past the batch (large halos)
    for (uint32_t f = HB * NTH; f < h_items; f += NTH) {
      uint32_t src, g8, lo, hi;
      halo_item(f + threadIdx.x, src, g8, lo, hi);
      halo_load1(hreg[0], src, g8, c0);
      halo_store1(hreg[0], lo, hi);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);                // this thread's direct weight loads have landed
    __syncthreads();
    build_weights();
    __syncthreads();                                   // every wave has its fragments: reuse the raw rows
    multiply(c1, c1 < G.C ? G.C - c1 : 0u);            // copies the next chunk's weights as it goes
  }

  // the last multiply issued loads that fetch nothing (past the last chunk):
  // let them land before the workgroup can end
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if constexpr (NACC == 2) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][0][0][r] += acc[1][0][0][r];
  }

  // ---- epilogue: bias, activation, cast, store -------------------------------
  float bv[SM];
#pragma unroll
  for (int sj = 0; sj < SM; ++sj)
    bv[sj] = a.bias_dt == DT_F32 ? __uint_as_float(braw[sj])
             : a.bias_dt == DT_F16 ? widen<DT_F16>(braw[sj]) : widen<DT_BF16>(braw[sj]);
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, a.y_bytes);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.r, a.r ? a.y_bytes : 0u);
  const uint32_t howo = G.Ho * G.Wo;
  const uint32_t npos = a.PH * a.PW;

  // Staged epilogue.  The accumulator layout gives a lane 4 consecutive
  // positions of one output channel, and the 32 lanes of a store hold 32
  // channels: direct stores scatter 8-byte pieces over 32 rows of y.  When a
  // patch spans whole output rows (PW == Wo) its positions are one contiguous
  // run of y per channel, so the pre-activations (accumulator + bias, fp32)
  // go through LDS as [channel][position] rows, and each thread then takes 8
  // consecutive positions of one channel: one 16-byte load of the residual,
  // the activation, one 16-byte store (two of each for fp32 outputs).  The
  // same fp32 operations in the same order as the direct path: the same bits.
  constexpr int ZSTR = WGN * 32 * SN + 4;               // floats per channel row (+16 B: no bank conflicts)
  static_assert(BM * ZSTR * 4 <= LDS - NDMA * 1024, "the staged tile must fit the halo buffer");
  constexpr uint32_t E16 = 16 / Elem<DTO>::bytes;       // outputs per 16 bytes
  const bool staged = a.PW == G.Wo && (a.PH * G.Wo) % E16 == 0 && howo % E16 == 0 &&
                      ((reinterpret_cast<uintptr_t>(a.y) | reinterpret_cast<uintptr_t>(a.r)) & 15u) == 0;
  if (staged) {
    __syncthreads();                                   // every wave is done with the halo
    float* zt = reinterpret_cast<float*>(s_halo);
#pragma unroll
    for (int si = 0; si < SN; ++si)
#pragma unroll
      for (int sj = 0; sj < SM; ++sj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t col = wave_m * WTM + sj * 32 + lrow;
          const uint32_t q = wave_n * WTN + si * 32 + 8 * g + 4 * half;
          f32x4 v;
          v.x = acc[0][si][sj][4 * g + 0] + bv[sj];
          v.y = acc[0][si][sj][4 * g + 1] + bv[sj];
          v.z = acc[0][si][sj][4 * g + 2] + bv[sj];
          v.w = acc[0][si][sj][4 * g + 3] + bv[sj];
          *reinterpret_cast<f32x4*>(zt + col * ZSTR + q) = v;
        }
    __syncthreads();
    const uint32_t rows_here = G.Ho - oh0 < a.PH ? G.Ho - oh0 : a.PH;
    const uint32_t nvalid = rows_here * G.Wo;          // this patch's positions, contiguous from (oh0, 0)
    constexpr uint32_t CPR = WGN * 32 * SN / 8;        // groups of 8 positions per channel row
    with_act(a.act, [&](auto act_c) __attribute__((always_inline)) {
      constexpr int ACT = decltype(act_c)::value;
      with_residual(a.r != nullptr, [&](auto res_c) __attribute__((always_inline)) {
        constexpr bool HAS_R = decltype(res_c)::value;
        for (uint32_t i = threadIdx.x; i < (uint32_t)BM * CPR; i += NTH) {
          const uint32_t col = i / CPR, q0 = 8 * (i - col * CPR);
          const uint32_t co = co0 + col;
          if (co >= G.Co || q0 >= nvalid) continue;
          const float* zp = zt + col * ZSTR + q0;
          const f32x4 z0 = *reinterpret_cast<const f32x4*>(zp);
          const f32x4 z1 = *reinterpret_cast<const f32x4*>(zp + 4);
          float z[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
          const uint32_t base = (img * G.Co + co) * howo + oh0 * G.Wo + q0;
          if (q0 + 8 <= nvalid) {
            if constexpr (Elem<DTO>::bytes == 4) {
              if constexpr (HAS_R) {
                const u32x4 r0 = ld_b128(rr, base * 4u), r1 = ld_b128(rr, base * 4u + 16u);
                z[0] += __uint_as_float(r0.x); z[1] += __uint_as_float(r0.y);
                z[2] += __uint_as_float(r0.z); z[3] += __uint_as_float(r0.w);
                z[4] += __uint_as_float(r1.x); z[5] += __uint_as_float(r1.y);
                z[6] += __uint_as_float(r1.z); z[7] += __uint_as_float(r1.w);
              }
              u32x4 o0, o1;
              o0.x = __float_as_uint(act_fn<ACT, DTO>(z[0], a.alpha));
              o0.y = __float_as_uint(act_fn<ACT, DTO>(z[1], a.alpha));
              o0.z = __float_as_uint(act_fn<ACT, DTO>(z[2], a.alpha));
              o0.w = __float_as_uint(act_fn<ACT, DTO>(z[3], a.alpha));
              o1.x = __float_as_uint(act_fn<ACT, DTO>(z[4], a.alpha));
              o1.y = __float_as_uint(act_fn<ACT, DTO>(z[5], a.alpha));
              o1.z = __float_as_uint(act_fn<ACT, DTO>(z[6], a.alpha));
              o1.w = __float_as_uint(act_fn<ACT, DTO>(z[7], a.alpha));
              st_b128(ry, base * 4u, o0);
              st_b128(ry, base * 4u + 16u, o1);
            } else {
              if constexpr (HAS_R) {
                const u32x4 rv = ld_b128(rr, base * 2u);
                const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  z[2 * e] += widen<DTO>(rw[e] & 0xffffu);
                  z[2 * e + 1] += widen<DTO>(rw[e] >> 16);
                }
              }
              uint32_t o[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                o[e] = narrow<DTO>(act_fn<ACT, DTO>(z[2 * e], a.alpha)) |
                       (narrow<DTO>(act_fn<ACT, DTO>(z[2 * e + 1], a.alpha)) << 16);
              st_b128(ry, base * 2u, u32x4{o[0], o[1], o[2], o[3]});
            }
          } else {
            // the last rows of the image end inside this group
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const bool ok = q0 + e < nvalid;
              float ze = z[e];
              if constexpr (HAS_R) ze += load1<DTO>(rr, base + e, ok);
              store1<DTO>(ry, base + e, ok, act_fn<ACT, DTO>(ze, a.alpha));
            }
          }
        }
      });
    });
    return;
  }

  auto epilogue = [&](auto act_c, auto res_c) __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool HAS_R = decltype(res_c)::value;
#pragma unroll
    for (int si = 0; si < SN; ++si)
#pragma unroll
      for (int sj = 0; sj < SM; ++sj) {
        const uint32_t co = co0 + wave_m * WTM + sj * 32 + lrow;
        const bool cok = co < G.Co;
        const uint32_t ybase = (img * G.Co + co) * howo;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t q = wave_n * WTN + si * 32 + 8 * g + 4 * half;
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = acc[0][si][sj][4 * g + e] + bv[sj];
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
  // activation and residual dispatched once per workgroup
  with_act(a.act, [&](auto act_c) __attribute__((always_inline)) {
    with_residual(a.r != nullptr,
                  [&](auto res_c) __attribute__((always_inline)) { epilogue(act_c, res_c); });
  });
}

template <int DTI, int DTO, int T, int BM, int KS, int SN, int NW = 4>
inline void launch_conv_halo_t(const HaloArgs& a, hipStream_t s) {
  note_launch("conv-halo %d taps, %d co x %ux%u positions, %d chunk set%s, %d waves", T, BM, a.PH, a.PW, KS,
              KS > 1 ? "s" : "", NW);
  launch_kernel(conv16_halo_kernel<DTI, DTO, T, BM, KS, SN, NW>, dim3(a.blocks), dim3(NW * 64), s, a);
}

}  // namespace biasact
