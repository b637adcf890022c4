// gemm_pp.hpp — the large-tile fused GEMM + bias + activation for fp16 / bf16
// operands on gfx950 ("ping-pong" kernel).
//
//   C[M,N] = act(A[M,K] . B[K,N] + bias[N])   ([MLR] 概述 / 样例规格; [FMR]
//   fused_matmul_relu: the intermediate never leaves the chip, one HBM read of
//   the operands and one write of C)
//
// Workgroup: 512 threads = 8 waves, output tile 256 (m) x 256 (n), k-tile 64.
// Waves 0-3 form cluster 0 and waves 4-7 cluster 1; wave w owns the 128 (m) x
// 64 (n) sub-tile at m = 128*(w/4), n = 64*(w%4), i.e. 4 x 2 accumulator
// blocks of 32x32 (128 fp32 values per lane).  Each SIMD runs one wave of
// each cluster.  The clusters alternate phases between workgroup barriers:
// while one wave of a SIMD multiplies (16 MFMAs, one half k-tile, already in
// registers), the other reads its next fragments from LDS and issues global
// loads, so the matrix core is fed without waiting on LDS latency.
//
// Operands reach LDS without passing through registers: 16-byte buffer loads
// with the LDS-destination bit write each lane's 16 bytes at base + 16*lane
// (out-of-range lanes write zeros, which covers ragged M, N and the K tail).
// The swizzle is applied by choosing which global chunk each lane fetches.
//   A stage: 256 rows (m) x 64 k = 128 B per row, 16-byte chunk c of row r at
//            slot c ^ (r & 7) ^ ((r >> 3) & 1); fragments via ds_read_b128.
//   B stage: 64 rows (k) x 256 n = 512 B per row (n contiguous, as in memory),
//            chunk c of row k at slot c ^ 4*(k & 3); fragments via the
//            transposing ds_read_b64_tr_b16, two per 32x32x16 operand: lane L
//            addresses row 8*(L/32) + (L%16)/4 (+4 for the second read),
//            columns 16*((L/16)%2) + 4*(L%4) .. +3, and receives the 8
//            consecutive k of column L%32 that the MFMA expects.
// Two stages (128 KB of the 160 KB LDS): A0 | A1 | B0 | B1, so every stage /
// subtile / k-step displacement of an LDS address is an instruction immediate.
#pragma once

#include "epilogue.hpp"
#include "launch.hpp"
#include "mfma_core.hpp"

namespace biasact {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

namespace pp {
constexpr int BM = 256, BN = 256, BK = 64, THREADS = 512;
constexpr int A_STAGE = BM * 128;            // 32 KB
constexpr int B_STAGE = BK * BN * 2;         // 32 KB
constexpr int A_OFF = 0, B_OFF = 2 * A_STAGE;
constexpr int LDS_BYTES = 2 * (A_STAGE + B_STAGE);

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int WAIT_LGKM0 = 0xC07F;
constexpr int WAIT_VM0 = 0x0F70;

__device__ __forceinline__ int swz_a(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz_b(int k) { return 4 * (k & 3); }
}  // namespace pp

template <int DTI, int DTO>
__global__ __launch_bounds__(512, 1) void gemm16_pp_kernel(GemmArgs a) {
  static_assert(DTI == DT_F16 || DTI == DT_BF16, "16-bit operands only");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[pp::LDS_BYTES];

  uint32_t tm, tn;
  map_tile(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, tm, tn);
  const uint32_t m0 = tm * pp::BM, n0 = tn * pp::BN;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 2, wn = w & 3;          // cluster == wm
  const int half = lane >> 5, lrow = lane & 31;

  // ---- accumulators start at the bias (the extra reduction term) --------
  f32x16 acc[2][4];
  {
    uint32_t idx[32];
    float bv[32];
#pragma unroll
    for (int si = 0; si < 2; ++si)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        idx[si * 16 + r] = n0 + wn * 64 + si * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
    load_bias_vec<32>(a.bias, a.bias_bytes, a.bias_dt, idx, a.N, bv);
#pragma unroll
    for (int si = 0; si < 2; ++si) {
      f32x16 b;
#pragma unroll
      for (int r = 0; r < 16; ++r) b[r] = bv[si * 16 + r];
#pragma unroll
      for (int sj = 0; sj < 4; ++sj) acc[si][sj] = b;
    }
  }

  // ---- per-lane global offsets of this wave's direct loads --------------
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, a.a_bytes);
  const __amdgpu_buffer_rsrc_t rbm = make_rsrc(a.B, a.b_bytes);
  uint32_t a_off[4], a_k[4], b_off[4], b_k[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = w * 32 + i * 8 + (lane >> 3);           // A stage row
    const int c = (lane & 7) ^ pp::swz_a(row);               // logical k-chunk for slot lane&7
    const uint32_t gm = m0 + row;
    a_off[i] = gm < a.M ? (gm * a.K + c * 8) * 2 : kOOB;
    a_k[i] = c * 8;
    const int k = w * 8 + 2 * i + (lane >> 5);               // B stage row
    const int cb = (lane & 31) ^ pp::swz_b(k);               // logical n-chunk for slot lane&31
    const uint32_t gn = n0 + cb * 8;
    b_off[i] = (gn < a.N && (uint32_t)k < a.K) ? ((uint32_t)k * a.N + gn) * 2 : kOOB;
    b_k[i] = k;
  }
  const uint32_t b_kstep = 64u * a.N * 2u;                  // bytes per k-tile of B

  auto issue_loads = [&](int kt, int stage) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t kk = (uint32_t)kt * 64u;
      const uint32_t ao = (a_off[i] != kOOB && kk + a_k[i] < a.K) ? a_off[i] + kk * 2u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_void*)(smem + pp::A_OFF + stage * pp::A_STAGE + w * 4096 + i * 1024), 16, ao, 0, 0, 0);
      const uint32_t bo = (b_off[i] != kOOB && kk + b_k[i] < a.K) ? b_off[i] + (uint32_t)kt * b_kstep : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rbm, (lds_void*)(smem + pp::B_OFF + stage * pp::B_STAGE + w * 4096 + i * 1024), 16, bo, 0, 0, 0);
    }
  };

  // ---- LDS fragment addresses -------------------------------------------
  // A (m side): row wm*128 + sj*32 + lrow, chunk 2*ks + half.
  const int xa = pp::swz_a(lrow);
  uint32_t a_rd[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    a_rd[ks] = pp::A_OFF + (wm * 128 + lrow) * 128 + (((2 * ks + half) ^ xa) * 16);
  // B (n side): k = 8*half + (lane%16)/4 (+ 16*ks + 4*q), n = wn*64 + si*32 + 16*((lane/16)%2) + 4*(lane%4)
  uint32_t b_rd[2];
#pragma unroll
  for (int si = 0; si < 2; ++si) {
    const int k = 8 * half + ((lane & 15) >> 2);
    const int n = wn * 64 + si * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int phys = (n >> 3) ^ pp::swz_b(k);
    b_rd[si] = pp::B_OFF + k * 512 + phys * 16 + (n & 7) * 2;
  }

  const int ktiles = (int)((a.K + pp::BK - 1) / pp::BK);

  // ---- prologue: tile 0 --------------------------------------------------
  if (ktiles > 0) {
    issue_loads(0, 0);
    __builtin_amdgcn_s_waitcnt(pp::WAIT_VM0);
  }
  __builtin_amdgcn_s_barrier();
  if (wm == 1) __builtin_amdgcn_s_barrier();      // cluster 1 runs one phase behind

  u32x4 fa[4][2];        // [sj][ks within the half]
  u32x4 fb[2][2];        // [si][ks within the half]
  for (int kt = 0; kt < ktiles; ++kt) {
    const int stage = kt & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // ---- memory phase: fragments of this half, next tile's loads -------
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ks = 2 * h + kk;
#pragma unroll
        for (int sj = 0; sj < 4; ++sj)
          fa[sj][kk] = *reinterpret_cast<const u32x4*>(smem + a_rd[ks] + stage * pp::A_STAGE + sj * 4096);
#pragma unroll
        for (int si = 0; si < 2; ++si) {
          const uint32_t base = b_rd[si] + stage * pp::B_STAGE + ks * 16 * 512;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(smem + base));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(smem + base + 4 * 512));
          u32x4 f;
          f.x = __builtin_bit_cast(u32x2, lo).x;
          f.y = __builtin_bit_cast(u32x2, lo).y;
          f.z = __builtin_bit_cast(u32x2, hi).x;
          f.w = __builtin_bit_cast(u32x2, hi).y;
          fb[si][kk] = f;
        }
      }
      if (h == 0 && kt + 1 < ktiles) issue_loads(kt + 1, stage ^ 1);
      if (h == 1) __builtin_amdgcn_s_waitcnt(pp::WAIT_VM0);
      __builtin_amdgcn_s_waitcnt(pp::WAIT_LGKM0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // ---- compute phase: 16 MFMAs from registers ------------------------
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int si = 0; si < 2; ++si)
#pragma unroll
          for (int sj = 0; sj < 4; ++sj) mfma_chunk<DTI>(acc[si][sj], fb[si][kk], fa[sj][kk]);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
    }
  }
  if (wm == 0) __builtin_amdgcn_s_barrier();      // same barrier count for both clusters

  // ---- epilogue: activation, cast, one store per element -----------------
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.C, a.c_bytes);
#pragma unroll
  for (int si = 0; si < 2; ++si)
#pragma unroll
    for (int sj = 0; sj < 4; ++sj) {
      const uint32_t m = m0 + wm * 128 + sj * 32 + lrow;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t n = n0 + wn * 64 + si * 32 + 8 * g + 4 * half;
        const float y0 = apply_act(a.act, acc[si][sj][4 * g + 0], a.alpha);
        const float y1 = apply_act(a.act, acc[si][sj][4 * g + 1], a.alpha);
        const float y2 = apply_act(a.act, acc[si][sj][4 * g + 2], a.alpha);
        const float y3 = apply_act(a.act, acc[si][sj][4 * g + 3], a.alpha);
        store4<DTO>(rc, m * a.N + n, m < a.M && n < a.N, y0, y1, y2, y3);
      }
    }
}

template <int DTI, int DTO>
inline void launch_gemm_pp(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gemm16_pp_kernel<DTI, DTO>), dim3(a.tiles_m * a.tiles_n), dim3(pp::THREADS), 0, s, a);
}

}  // namespace biasact
