// mfma_core.hpp — the fused contraction + bias + activation main loop for
// gfx950: LDS double-buffered operand tiles, 32x32 MFMA accumulation in fp32,
// and the epilogue's output staging (activation, output cast, one store per
// element).
//
// Orientation.  The MFMA "row" index i runs over the output's contiguous
// dimension (GEMM column n, conv spatial position p) and the MFMA "column"
// index j over the other one (GEMM row m, conv output channel co).  With the
// 32x32 accumulator layout (lane l, register r <-> i = 8*(r/4) + 4*(l/32) +
// r%4, j = l%32) each lane then owns four consecutive output elements per
// register group.  Where output rows allow 4-wide accesses the kernels pass
// them through the LDS tile first (StagedOut, at the end of this file), so
// that a store covers 128-byte runs of 8 rows; otherwise each lane stores
// its elements one by one.
//
// LDS layout.  Both operand tiles are stored k-contiguous: one 128-byte LDS
// row per i (or j) index holding 8 chunks of 16 bytes (BK = 64 16-bit values
// or 32 fp32 values).  Chunk c of row r sits at physical slot
// c ^ (r & 7) ^ ((r >> 3) & 7): eight consecutive rows read at the same chunk
// hit eight different slots, and the transposing B-store (rows 8 apart) also
// spreads over eight slots.
//
// The bias enters the contraction as one more reduction term: the
// accumulator starts at the bias value, which is the contribution of an extra
// k column holding the bias against an all-ones row ([FCT] "双 Kernel 是怎么
// 分工的"), so the main loop's result is already act's argument.
#pragma once

#include "device_common.hpp"
#include "tile_map.hpp"

namespace biasact {

constexpr int kChunks = 8;          // chunks per LDS row
constexpr int kRowBytes = 128;

__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  const int phys = chunk ^ (row & 7) ^ ((row >> 3) & 7);
  return (uint32_t)(row * kRowBytes + phys * 16);
}

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int threads = WAVES_M * WAVES_N * 64;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int SM = WTM / 32, SN = WTN / 32;
  static constexpr int a_bytes = BM * kRowBytes;     // j-side tile (A / weights)
  static constexpr int b_bytes = BN * kRowBytes;     // i-side tile (B / gathered input)
  static constexpr int stage_bytes = a_bytes + b_bytes;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");
};

// Pack EPC loaded elements (each in the low bits of a dword) into a chunk.
template <int DT>
__device__ __forceinline__ u32x4 pack_chunk(const uint32_t (&w)[Elem<DT>::epc]) {
  u32x4 v;
  if constexpr (Elem<DT>::bytes == 4) {
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
  } else if constexpr (Elem<DT>::bytes == 1) {
    v.x = (w[0] & 0xffu) | ((w[1] & 0xffu) << 8) | ((w[2] & 0xffu) << 16) | (w[3] << 24);
    v.y = (w[4] & 0xffu) | ((w[5] & 0xffu) << 8) | ((w[6] & 0xffu) << 16) | (w[7] << 24);
    v.z = (w[8] & 0xffu) | ((w[9] & 0xffu) << 8) | ((w[10] & 0xffu) << 16) | (w[11] << 24);
    v.w = (w[12] & 0xffu) | ((w[13] & 0xffu) << 8) | ((w[14] & 0xffu) << 16) | (w[15] << 24);
  } else {
    v.x = (w[0] & 0xffffu) | (w[1] << 16);
    v.y = (w[2] & 0xffffu) | (w[3] << 16);
    v.z = (w[4] & 0xffffu) | (w[5] << 16);
    v.w = (w[6] & 0xffffu) | (w[7] << 16);
  }
  return v;
}

template <int DT>
__device__ __forceinline__ uint32_t ld_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (Elem<DT>::bytes == 4) return ld_b32(r, off);
  else if constexpr (Elem<DT>::bytes == 1) return (uint32_t)ld_b8(r, off);
  else return (uint32_t)ld_b16(r, off);
}

// One element at vector offset voff plus the wave-uniform scalar offset soff.
template <int DT>
__device__ __forceinline__ uint32_t ld_elem_so(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (Elem<DT>::bytes == 4) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  else if constexpr (Elem<DT>::bytes == 1) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
  else return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// ---------------------------------------------------------------------------
// j-side loader: a dense row-major [rows, K] matrix, k contiguous (GEMM A,
// conv weights viewed as [Co, C*kh*kw]).  Each thread moves RA chunks per
// k-tile; with `vec` the chunk is one 16-byte load, otherwise EPC element
// loads (K not a multiple of the chunk, or a misaligned base).
// ---------------------------------------------------------------------------
template <int DT, class TL>
struct DenseRowLoader {
  static constexpr int EPC = Elem<DT>::epc, ES = Elem<DT>::bytes, BK = kChunks * EPC;
  static constexpr int RA = TL::BM * kChunks / TL::threads;
  static_assert(RA >= 1 && TL::BM * kChunks % TL::threads == 0, "A tile / thread mismatch");

  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t K, row_off[RA];    // byte offset of the row start (kOOB if the row is out of range)
  int chunk[RA];
  bool vec;
  u32x4 reg[RA];

  __device__ __forceinline__ void init(const void* p, uint32_t nbytes, uint32_t rows, uint32_t K_, uint32_t r0,
                       bool vec_) {
    rsrc = make_rsrc(p, nbytes);
    K = K_;
    vec = vec_;
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int q = threadIdx.x + i * TL::threads;
      const uint32_t row = r0 + (q >> 3);
      chunk[i] = q & 7;
      row_off[i] = row < rows ? row * K * ES : kOOB;
    }
  }

  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const uint32_t k = (uint32_t)kt * BK + chunk[i] * EPC;
      if (vec) {
        const uint32_t off = (row_off[i] != kOOB && k < K) ? row_off[i] + k * ES : kOOB;
        reg[i] = ld_b128(rsrc, off);
      } else {
        uint32_t w[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const uint32_t kk = k + e;
          w[e] = ld_elem<DT>(rsrc, (row_off[i] != kOOB && kk < K) ? row_off[i] + kk * ES : kOOB);
        }
        reg[i] = pack_chunk<DT>(w);
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* s) const {
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int q = threadIdx.x + i * TL::threads;
      *reinterpret_cast<u32x4*>(s + lds_off(q >> 3, chunk[i])) = reg[i];
    }
  }
};

// ---------------------------------------------------------------------------
// i-side loader for a dense row-major [K, N] matrix (GEMM B, n contiguous).
// The MFMA wants k contiguous per lane, so each thread loads an EPC x EPC
// block (EPC k-rows of one 16-byte n-chunk) and transposes it in registers
// into EPC k-chunks, one per n.
// ---------------------------------------------------------------------------
template <int DT, class TL>
struct DenseColLoader {
  static constexpr int EPC = Elem<DT>::epc, ES = Elem<DT>::bytes, BK = kChunks * EPC;
  static constexpr int NB_N = TL::BN / EPC;              // blocks across n
  static constexpr int NBLK = kChunks * NB_N;            // blocks per k-tile
  static constexpr int RB = (NBLK + TL::threads - 1) / TL::threads;

  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t K, N, n0, col[RB];      // first n of the block (global), or N (out of range)
  int kb[RB], nb[RB];
  bool active[RB];
  bool vec;
  u32x4 reg[RB][EPC];

  __device__ __forceinline__ void init(const void* p, uint32_t nbytes, uint32_t K_, uint32_t N_, uint32_t n0_,
                       bool vec_) {
    rsrc = make_rsrc(p, nbytes);
    K = K_;
    N = N_;
    n0 = n0_;
    vec = vec_;
    rebase(0);
  }
  // Blocks to threads, starting at thread `first` (mod the workgroup): with
  // fewer blocks than threads, the all-k loop starts each k-tile's blocks
  // where the previous one's ended, so every wave takes a share of the loads
  // and register transposes instead of the first wave taking them all.
  __device__ __forceinline__ void rebase(int first) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int q = ((int)threadIdx.x + TL::threads - first) % TL::threads + i * TL::threads;
      active[i] = q < NBLK;
      kb[i] = q / NB_N;
      nb[i] = q % NB_N;
      col[i] = n0 + nb[i] * EPC;
    }
  }

  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (!active[i]) continue;
#pragma unroll
      for (int r = 0; r < EPC; ++r) {
        const uint32_t k = (uint32_t)kt * BK + kb[i] * EPC + r;
        if (vec) {
          const uint32_t off = (k < K && col[i] < N) ? (k * N + col[i]) * ES : kOOB;
          reg[i][r] = ld_b128(rsrc, off);
        } else {
          uint32_t w[EPC];
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            const uint32_t n = col[i] + e;
            w[e] = ld_elem<DT>(rsrc, (k < K && n < N) ? (k * N + n) * ES : kOOB);
          }
          reg[i][r] = pack_chunk<DT>(w);
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* s) const {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (!active[i]) continue;
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        u32x4 o;
        if constexpr (ES == 4) {
          o.x = reg[i][0][j]; o.y = reg[i][1][j]; o.z = reg[i][2][j]; o.w = reg[i][3][j];
        } else if constexpr (ES == 1) {
          // byte j % 4 of dword j / 4 of rows 4q .. 4q+3 form dword q of chunk j
          const int d = j >> 2, b = j & 3;
          const uint32_t sel = (uint32_t)b | ((uint32_t)(4 + b) << 8) | 0x0c0c0000u;
          uint32_t q4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = __builtin_amdgcn_perm(reg[i][4 * q + 1][d], reg[i][4 * q + 0][d], sel);
            const uint32_t hi = __builtin_amdgcn_perm(reg[i][4 * q + 3][d], reg[i][4 * q + 2][d], sel);
            q4[q] = lo | (hi << 16);
          }
          o.x = q4[0]; o.y = q4[1]; o.z = q4[2]; o.w = q4[3];
        } else {
          // element (row r, column j) is half (j & 1) of dword j/2 of row r
          const int d = j >> 1;
          const uint32_t a0 = reg[i][0][d], a1 = reg[i][1][d], a2 = reg[i][2][d], a3 = reg[i][3][d];
          const uint32_t a4 = reg[i][4][d], a5 = reg[i][5][d], a6 = reg[i][6][d], a7 = reg[i][7][d];
          if (j & 1) {
            o.x = (a0 >> 16) | (a1 & 0xffff0000u);
            o.y = (a2 >> 16) | (a3 & 0xffff0000u);
            o.z = (a4 >> 16) | (a5 & 0xffff0000u);
            o.w = (a6 >> 16) | (a7 & 0xffff0000u);
          } else {
            o.x = (a0 & 0xffffu) | (a1 << 16);
            o.y = (a2 & 0xffffu) | (a3 << 16);
            o.z = (a4 & 0xffffu) | (a5 << 16);
            o.w = (a6 & 0xffffu) | (a7 << 16);
          }
        }
        *reinterpret_cast<u32x4*>(s + lds_off(nb[i] * EPC + j, kb[i])) = o;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// i-side loader for conv2d as an implicit GEMM ([FCT] "双 Kernel 是怎么分工
// 的": weights are the co x k operand, input features the k x spatial one).
// Row p of the tile is output position (n, oh, ow); chunk c holds EPC
// consecutive k = (c_in, r, s) values of the gathered input
//   x[n, c_in, oh*sh - pt + r*dh, ow*sw - pl + s*dw]  (0 outside the image).
// Every thread owns one output position and TL::BN*8/threads chunks whose k
// range is the same for the whole wave, so the k -> (c_in, r, s) decode runs
// on scalar registers.
// ---------------------------------------------------------------------------
struct ConvGeom {
  uint32_t N, C, H, W, Co, kh, kw, Ho, Wo;
  int32_t sh, sw, pt, pl, dh, dw;
  uint32_t K, P;                 // K = C*kh*kw, P = N*Ho*Wo
  FastDiv div_wo, div_howo;
  FastDiv div_khkw, div_kw;      // the k -> (c_in, r, s) decode
};

template <int DT, class TL>
struct ConvGatherLoader {
  static constexpr int EPC = Elem<DT>::epc, ES = Elem<DT>::bytes, BK = kChunks * EPC;
  static_assert(TL::threads % TL::BN == 0 || TL::BN % TL::threads == 0, "tile/thread mismatch");
  static constexpr int CPT = TL::BN * kChunks / TL::threads;   // chunks per thread per k-tile
  static_assert(CPT >= 1, "conv tile too small for the thread count");
  static constexpr int PPT = TL::BN > TL::threads ? TL::BN / TL::threads : 1;  // positions/thread
  static constexpr int CPP = CPT / PPT;                        // chunks per position

  __amdgpu_buffer_rsrc_t rsrc;
  ConvGeom g;
  int32_t pbase[PPT], ih0[PPT], iw0[PPT];
  uint32_t pofs[PPT];           // 1x1 filters: the position's byte offset, or kOOB
  int prow[PPT];
  uint32_t c0;                  // first chunk index of this wave (wave-uniform)
  u32x4 reg[PPT][CPP];

  __device__ __forceinline__ void init(const void* x, uint32_t nbytes, const ConvGeom& geom, uint32_t p0) {
    rsrc = make_rsrc(x, nbytes);
    g = geom;
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int t = threadIdx.x + u * TL::threads;
      prow[u] = t % TL::BN;
      const uint32_t p = p0 + prow[u];
      if (p < geom.P) {
        const uint32_t img = fdiv(p, geom.div_howo);
        const uint32_t q = p - img * geom.Ho * geom.Wo;
        const uint32_t oh = fdiv(q, geom.div_wo);
        const uint32_t ow = q - oh * geom.Wo;
        ih0[u] = (int32_t)oh * geom.sh - geom.pt;
        iw0[u] = (int32_t)ow * geom.sw - geom.pl;
        pbase[u] = (int32_t)(img * geom.C * geom.H * geom.W) + ih0[u] * (int32_t)geom.W + iw0[u];
      } else {
        ih0[u] = -(1 << 30);        // every tap fails the row range check
        iw0[u] = 0;
        pbase[u] = 0;
      }
      const bool inside = (uint32_t)ih0[u] < geom.H && (uint32_t)iw0[u] < geom.W;
      pofs[u] = inside ? (uint32_t)pbase[u] * ES : kOOB;
    }
    c0 = __builtin_amdgcn_readfirstlane((uint32_t)(threadIdx.x / TL::BN));
  }

  // 1x1 filter, any stride and padding: k is the input channel and a
  // position reads the same spatial offset for every k.  A position in the
  // padding or past P got kOOB once in init(); each element load then takes
  // its channel's offset as the scalar offset and costs no vector
  // instruction (pofs + that offset stays below 2^32: both are < 2^31).
  __device__ __forceinline__ void load_1x1(int kt) {
    const uint32_t cstep = TL::threads >= TL::BN ? TL::threads / TL::BN : 1;
    const uint32_t plane = g.H * g.W * ES;
#pragma unroll
    for (int v = 0; v < CPP; ++v) {
      const uint32_t kc = (uint32_t)kt * BK + (c0 + v * cstep) * EPC;   // wave-uniform
      uint32_t w[PPT][EPC];
      if (kc + EPC <= g.K) {
#pragma unroll
        for (int e = 0; e < EPC; ++e)
#pragma unroll
          for (int u = 0; u < PPT; ++u) w[u][e] = ld_elem_so<DT>(rsrc, pofs[u], (kc + e) * plane);
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e)
#pragma unroll
          for (int u = 0; u < PPT; ++u)
            w[u][e] = kc + e < g.K ? ld_elem_so<DT>(rsrc, pofs[u], (kc + e) * plane) : 0u;
      }
#pragma unroll
      for (int u = 0; u < PPT; ++u) reg[u][v] = pack_chunk<DT>(w[u]);
    }
  }

  __device__ __forceinline__ void load(int kt) {
    if (g.kh == 1 && g.kw == 1) {
      load_1x1(kt);
      return;
    }
    const ConvGeom& G = g;
    const uint32_t cstep = TL::threads >= TL::BN ? TL::threads / TL::BN : 1;
#pragma unroll
    for (int v = 0; v < CPP; ++v) {
      // k range of this chunk: wave-uniform
      // (scalar divisions through FastDiv: a runtime division is tens of
      // scalar instructions, and this runs for every chunk of every k-tile)
      const uint32_t kc = (uint32_t)kt * BK + (c0 + v * cstep) * EPC;
      uint32_t cin = fdiv(kc, G.div_khkw);
      uint32_t rs = kc - cin * G.kh * G.kw;
      uint32_t r = fdiv(rs, G.div_kw);
      uint32_t s = rs - r * G.kw;
      uint32_t w[PPT][EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const bool kval = kc + e < G.K;
        const int32_t rh = (int32_t)(r * G.dh), sw = (int32_t)(s * G.dw);
        const int32_t koff = (int32_t)(cin * G.H * G.W) + rh * (int32_t)G.W + sw;
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
          const bool ok = kval && (uint32_t)(ih0[u] + rh) < G.H && (uint32_t)(iw0[u] + sw) < G.W;
          w[u][e] = ld_elem<DT>(rsrc, ok ? (uint32_t)(pbase[u] + koff) * ES : kOOB);
        }
        // advance (cin, r, s) to the next k
        if (++s == G.kw) {
          s = 0;
          if (++r == G.kh) {
            r = 0;
            ++cin;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < PPT; ++u) reg[u][v] = pack_chunk<DT>(w[u]);
    }
  }

  __device__ __forceinline__ void store(uint8_t* s) const {
    const uint32_t cstep = TL::threads >= TL::BN ? TL::threads / TL::BN : 1;
#pragma unroll
    for (int u = 0; u < PPT; ++u)
#pragma unroll
      for (int v = 0; v < CPP; ++v)
        *reinterpret_cast<u32x4*>(s + lds_off(prow[u], c0 + v * cstep)) = reg[u][v];
  }
};

// ---------------------------------------------------------------------------
// The main loop.  acc[si][sj] is the 32x32 block (i-subtile si, j-subtile sj)
// of this wave.  Double-buffered: the global loads of k-tile kt+1 are in
// flight while k-tile kt is multiplied out of LDS.
// ---------------------------------------------------------------------------
// One k-tile from LDS stage (sA, sB): 4 k-steps of 16-byte chunks.
template <int DT, class TL>
__device__ __forceinline__ void tile_mma(f32x16 (&acc)[TL::SN][TL::SM], const uint8_t* sA, const uint8_t* sB) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_m = wave / TL::WAVES_N, wave_n = wave % TL::WAVES_N;
  const int half = lane >> 5, lrow = lane & 31;
#pragma unroll
  for (int ks = 0; ks < kChunks / 2; ++ks) {
    const int ch = 2 * ks + half;
    u32x4 fi[TL::SN], fj[TL::SM];
#pragma unroll
    for (int si = 0; si < TL::SN; ++si)
      fi[si] = *reinterpret_cast<const u32x4*>(sB + lds_off(wave_n * TL::WTN + si * 32 + lrow, ch));
#pragma unroll
    for (int sj = 0; sj < TL::SM; ++sj)
      fj[sj] = *reinterpret_cast<const u32x4*>(sA + lds_off(wave_m * TL::WTM + sj * 32 + lrow, ch));
#pragma unroll
    for (int si = 0; si < TL::SN; ++si)
#pragma unroll
      for (int sj = 0; sj < TL::SM; ++sj) mfma_chunk<DT>(acc[si][sj], fi[si], fj[sj]);
  }
}

// Double-buffered main loop: the loads of k-tile kt+1 are in flight while
// k-tile kt is multiplied.  init_acc() runs once the first loads are issued,
// so its own loads (the bias) do not delay them.
template <int DT, class TL, class LA, class LB, class F>
__device__ __forceinline__ void main_loop(f32x16 (&acc)[TL::SN][TL::SM], LA& la, LB& lb,
                                          uint8_t* smem, int ktiles, F&& init_acc) {
  if (ktiles <= 0) {
    init_acc();
    return;
  }
  la.load(0);
  lb.load(0);
  init_acc();
  la.store(smem);
  lb.store(smem + TL::a_bytes);
  __syncthreads();

  for (int kt = 0; kt < ktiles; ++kt) {
    uint8_t* cur = smem + (kt & 1) * TL::stage_bytes;
    uint8_t* nxt = smem + ((kt + 1) & 1) * TL::stage_bytes;
    const bool more = kt + 1 < ktiles;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
    tile_mma<DT, TL>(acc, cur, cur + TL::a_bytes);
    if (more) {
      la.store(nxt);
      lb.store(nxt + TL::a_bytes);
    }
    __syncthreads();
  }
}

// Short reduction (ktiles <= NK): every k-tile's loads are issued before any
// is stored, so the operands cost one memory round trip, then NK LDS stages.
template <int DT, class TL, int NK, class LA, class LB, class F>
__device__ __forceinline__ void main_loop_allk(f32x16 (&acc)[TL::SN][TL::SM], const LA& la0,
                                               const LB& lb0, uint8_t* smem, int ktiles, F&& init_acc) {
  LA la[NK];
  LB lb[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    la[k] = la0;
    lb[k] = lb0;
    if constexpr (LB::NBLK < TL::threads) lb[k].rebase((k * LB::NBLK) % TL::threads);
    if (k < ktiles) {
      la[k].load(k);
      lb[k].load(k);
    }
  }
  init_acc();
#pragma unroll
  for (int k = 0; k < NK; ++k)
    if (k < ktiles) {
      la[k].store(smem + k * TL::stage_bytes);
      lb[k].store(smem + k * TL::stage_bytes + TL::a_bytes);
    }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NK; ++k)
    if (k < ktiles) tile_mma<DT, TL>(acc, smem + k * TL::stage_bytes, smem + k * TL::stage_bytes + TL::a_bytes);
}

// ---------------------------------------------------------------------------
// Output staging.  The accumulator layout gives a lane 4 consecutive
// outputs of one row (GEMM row m, conv output channel co) per register group,
// so a store straight from it covers 16- (or 8-) byte pieces of 32 rows.
// Instead, one 32-wide column block (si) of every wave goes through the LDS
// tile per pass: row j (0 .. BM-1) holds WAVES_N runs of 32 outputs, the
// 16-byte chunk c of a run at slot c ^ (j & 7), so 8 consecutive rows spread
// over all banks both when written in the accumulator layout and when read
// by rows.  Thread t then owns chunk c = t % 8 of run rn = (t / 8) % WAVES_N
// in rows r0, r0 + RSTEP, ... : a store instruction covers 128-byte runs of
// 8 rows.
// ---------------------------------------------------------------------------
template <class TL>
struct StagedOut {
  static constexpr int RUNS = TL::WAVES_N, ROWB = RUNS * 128;
  static constexpr int RSTEP = TL::threads / (8 * RUNS);   // rows between a thread's chunks
  static constexpr int CPT = TL::BM / RSTEP;                // chunks per thread per pass
  static constexpr int bytes = TL::BM * ROWB;
  uint32_t c, rn, r0;

  __device__ __forceinline__ StagedOut()
      : c(threadIdx.x & 7), rn((threadIdx.x >> 3) % RUNS), r0((threadIdx.x >> 3) / RUNS) {}

  // column (within the tile) of this thread's first output in pass si
  __device__ __forceinline__ uint32_t col(int si) const { return rn * TL::WTN + si * 32 + 4 * c; }
  // row (within the tile) of this thread's chunk k
  __device__ __forceinline__ uint32_t row(int k) const { return r0 + (uint32_t)(k * RSTEP); }

  // column block si of this wave's accumulators into the staging area (the
  // caller has a barrier before, so the area is free, and one after)
  __device__ __forceinline__ static void put(const f32x16 (&acc)[TL::SN][TL::SM], uint8_t* smem, int si) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wave_m = wave / TL::WAVES_N, wave_n = wave % TL::WAVES_N;
    const int half = lane >> 5, lrow = lane & 31;
#pragma unroll
    for (int sj = 0; sj < TL::SM; ++sj) {
      const uint32_t j = wave_m * TL::WTM + sj * 32 + lrow;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t slot = (uint32_t)(2 * g + half) ^ (j & 7u);
        const f32x4 v = {acc[si][sj][4 * g + 0], acc[si][sj][4 * g + 1], acc[si][sj][4 * g + 2],
                         acc[si][sj][4 * g + 3]};
        *reinterpret_cast<f32x4*>(smem + j * ROWB + wave_n * 128 + slot * 16) = v;
      }
    }
  }
  // this thread's chunk k of the staged block
  __device__ __forceinline__ f32x4 get(const uint8_t* smem, int k) const {
    const uint32_t j = row(k);
    return *reinterpret_cast<const f32x4*>(smem + j * ROWB + rn * 128 + ((c ^ (j & 7u)) * 16));
  }
};

}  // namespace biasact
