// gemm_pp.hpp — the large-tile fused GEMM + bias + activation for fp16 / bf16
// and int8 operands on gfx950 ("ping-pong" kernel).
//
//   C[M,N] = act(A[M,K] . B[K,N] + bias[N])   ([MLR] 概述 / 样例规格; [FMR]
//   fused_matmul_relu: the intermediate never leaves the chip, one HBM read of
//   the operands and one write of C)
//
// Workgroup: 512 threads = 8 waves, output tile 256 (m) x 256 (n), k-tile of
// 64 bytes per row of A (32 16-bit values, 64 int8 values).
// Waves 0-3 form cluster 0 and waves 4-7 cluster 1; wave w owns the 128 (m) x
// 64 (n) sub-tile at m = 128*(w/4), n = 64*(w%4), i.e. 4 x 2 accumulator
// blocks of 32x32 (128 fp32 values per lane).  Each SIMD runs one wave of
// each cluster.  The clusters alternate phases between workgroup barriers:
// while one wave of a SIMD multiplies one k-tile (16 MFMAs from registers),
// the other reads its fragments of the next k-tile from LDS and, between
// those reads, issues its global loads of the k-tile three ahead, so the LDS
// pipeline (fragment reads) and the texture path (global loads) work side by
// side under the matrix-core work of the partner wave.
//
// Operands reach LDS without passing through registers: 16-byte buffer loads
// with the LDS-destination bit write each lane's 16 bytes at base + 16*lane
// (out-of-range lanes write zeros, which covers ragged M, N and the K tail).
// The swizzle is applied by choosing which global chunk each lane fetches.
//   A stage: 256 rows (m) x 32 k = 64 B per row, 16-byte chunk c of row r at
//            slot c ^ ((r >> 2) & 3); fragments via ds_read_b128.
//   B stage: 32 rows (k) x 256 n = 512 B per row (n contiguous, as in memory),
//            chunk c of row k at slot c ^ 4*(k & 3); fragments via the
//            transposing ds_read_b64_tr_b16, two per 32x32x16 operand: lane L
//            addresses row 8*(L/32) + (L%16)/4 (+4 for the second read),
//            columns 16*((L/16)%2) + 4*(L%4) .. +3, and receives the 8
//            consecutive k of column L%32 that the MFMA expects.
//   int8 B:  64 rows (k) x 256 B, chunk c of row k at slot c ^ 2*(k & 7) (the
//            32 reads of a half-wave cover all 64 banks); ds_read_b64_tr_b8
//            (in each 16-lane group, lane i receives byte i%8 of the 8-byte
//            rows addressed by lanes i/8 + 2r, r = 0..7): lane L addresses row
//            16*(L/32) + (L%16)/2 (+8 for the second read), columns
//            16*((L/16)%2) + 8*(L%2) .. +7, and receives 8 consecutive k of
//            column L%32; with the A chunk of the same 16 k this feeds
//            v_mfma_i32_32x32x32_i8, whose int32 sums (bias included) are exact.
//            The LDS displacements of the second read (+2048) and of the next
//            k-step (+8192) are the 16-bit kernel's.
// Four stages (128 KB of the 160 KB LDS): A0..A3 | B0..B3; stage, subtile and
// k-step displacements of LDS addresses are instruction immediates.
//
// Epilogue.  A 16-bit output tile (256 x 256 x 2 B) fills the LDS exactly, so
// once the last k-tile is consumed each lane writes its activated, rounded
// values into LDS (row r = m, 16-byte chunk c of the 512-byte row at slot
// c ^ (r & 31), which spreads the 32 rows one register group covers over
// every bank), and the waves then store whole rows: each half-wave writes one
// 512-byte row with 16-byte stores.  The accumulator layout itself gives only
// 16 contiguous bytes in each of 32 rows per store instruction; stored that
// way a 4096^3 bf16 output costs 1.56x its size in HBM writes.  A residual is
// read the same way (whole rows into LDS, then added in the accumulator
// layout).  32-bit outputs (fp32, int32) leave in two passes of 128 rows.  C
// or R not on a 16-byte boundary store from the accumulator layout directly.
#pragma once

#include "epilogue.hpp"
#include "gemm_args.hpp"
#include "launch_kernel.hpp"
#include "tile_map.hpp"

namespace biasact {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

namespace pp {
constexpr int BM = 256, BN = 256, THREADS = 512, STAGES = 4;
constexpr int A_STAGE = BM * 64;             // 16 KB: 64 bytes of k per row
constexpr int B_STAGE = BN * 64;             // 16 KB: 32 rows of 16-bit n, or 64 rows of int8 n
constexpr int A_OFF = 0, B_OFF = STAGES * A_STAGE;
constexpr int LDS_BYTES = STAGES * (A_STAGE + B_STAGE);
constexpr int LOADS_PER_TILE = 4;            // direct loads per wave per k-tile

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int WAIT_LGKM0 = 0xC07F;
constexpr int wait_vm(int n) { return 0x0F70 | (n & 0xF) | ((n >> 4) << 14); }

__device__ __forceinline__ int swz_a(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int swz_b(int k) { return 4 * (k & 3); }
__device__ __forceinline__ int swz_b8(int k) { return 2 * (k & 7); }

// Transposing 8-byte LDS read (see the header comment for the lane layout).
// Issued as inline assembly: the compiler cannot tell that it does not touch
// the LDS stages the in-flight direct loads are filling and would otherwise
// drain every outstanding load before it.  Its completion is covered by the
// explicit lgkmcnt(0) wait that ends every memory phase.
template <int OFFSET>
__device__ __forceinline__ u32x2 ds_read_tr16_b64(uint32_t lds_addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(lds_addr), "i"(OFFSET));
  return v;
}
template <int OFFSET>
__device__ __forceinline__ u32x2 ds_read_tr8_b64(uint32_t lds_addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v) : "v"(lds_addr), "i"(OFFSET));
  return v;
}
// B fragment of k-step KS of the stage at lds_addr (16 k per lane: two transposing reads)
template <int DTI, int KS>
__device__ __forceinline__ u32x4 read_b_frag(uint32_t lds_addr) {
  u32x2 lo, hi;
  if constexpr (DTI == DT_I8) {
    lo = ds_read_tr8_b64<KS * 8192>(lds_addr);
    hi = ds_read_tr8_b64<KS * 8192 + 2048>(lds_addr);
  } else {
    lo = ds_read_tr16_b64<KS * 8192>(lds_addr);
    hi = ds_read_tr16_b64<KS * 8192 + 2048>(lds_addr);
  }
  u32x4 f;
  f.x = lo.x;
  f.y = lo.y;
  f.z = hi.x;
  f.w = hi.y;
  return f;
}

}  // namespace pp

template <int DTI, int DTO>
__global__ __launch_bounds__(512, 1) void gemm16_pp_kernel(GemmArgs a) {
  static_assert(DTI == DT_F16 || DTI == DT_BF16 || DTI == DT_I8, "16-bit or int8 operands");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[pp::LDS_BYTES];
  constexpr uint32_t ES = Elem<DTI>::bytes, EPC = Elem<DTI>::epc;   // bytes per value, values per chunk
  constexpr uint32_t BK = 64 / ES;                                   // k values per k-tile
  constexpr int BRPI = DTI == DT_I8 ? 4 : 2;                         // B rows per 1 KB direct load
  constexpr int BCPR = 64 / BRPI;                                    // 16-byte chunks per B row

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
    // 4 consecutive columns per (si, r / 4), all in or all out (N % 8 == 0):
    // one 16-byte (32-bit bias) or 8-byte (16-bit bias) load each when the
    // bias is aligned for it, so the 8 loads are in flight together
    const int bbytes = a.bias_dt == DT_F32 || a.bias_dt == DT_I32 ? 4 : 2;
    if (a.bias_dt >= 0 && (reinterpret_cast<uintptr_t>(a.bias) & (4u * bbytes - 1u)) == 0) {
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.bias, a.bias_bytes);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t n = idx[4 * q];
        const bool ok = n < a.N;
        if (bbytes == 4) {
          const u32x4 v = ld_b128(rb, ok ? n * 4u : kOOB);
          bv[4 * q + 0] = __uint_as_float(v.x);
          bv[4 * q + 1] = __uint_as_float(v.y);
          bv[4 * q + 2] = __uint_as_float(v.z);
          bv[4 * q + 3] = __uint_as_float(v.w);
        } else {
          const u32x2 v = ld_b64(rb, ok ? n * 2u : kOOB);
          const bool f16 = a.bias_dt == DT_F16;
          bv[4 * q + 0] = f16 ? widen<DT_F16>(v.x & 0xffffu) : widen<DT_BF16>(v.x & 0xffffu);
          bv[4 * q + 1] = f16 ? widen<DT_F16>(v.x >> 16) : widen<DT_BF16>(v.x >> 16);
          bv[4 * q + 2] = f16 ? widen<DT_F16>(v.y & 0xffffu) : widen<DT_BF16>(v.y & 0xffffu);
          bv[4 * q + 3] = f16 ? widen<DT_F16>(v.y >> 16) : widen<DT_BF16>(v.y >> 16);
        }
      }
    } else {
      load_bias_vec<32>(a.bias, a.bias_bytes, a.bias_dt, idx, a.N, bv);
    }
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
  // A: instruction i covers stage rows (2w + i)*16 .. +16 (16 rows x 64 B);
  // B: instruction i covers stage rows (k) (2w + i)*BRPI .. +BRPI (1 KB).
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, a.a_bytes);
  const __amdgpu_buffer_rsrc_t rbm = make_rsrc(a.B, a.b_bytes);
  uint32_t a_off[2], a_k[2], b_off[2], b_k[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (2 * w + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ pp::swz_a(row);               // logical k-chunk for slot lane&3
    const uint32_t gm = m0 + row;
    a_off[i] = gm < a.M ? (gm * a.K + c * EPC) * ES : kOOB;
    a_k[i] = c * EPC;
    const int k = (2 * w + i) * BRPI + lane / BCPR;
    const int slot = lane % BCPR;
    const int cb = slot ^ (DTI == DT_I8 ? pp::swz_b8(k) : pp::swz_b(k));   // logical n-chunk for the slot
    const uint32_t gn = n0 + cb * EPC;
    b_off[i] = (gn < a.N && (uint32_t)k < a.K) ? ((uint32_t)k * a.N + gn) * ES : kOOB;
    b_k[i] = k;
  }
  const uint32_t b_kstep = BK * a.N * ES;                   // bytes of B per k-tile

  // One direct load j (0..3) of k-tile kt: even j = A rows, odd j = B rows.
  // K-tiles at or beyond K read as zeros (every offset fails the K test), so
  // the loop can issue its loads unconditionally into the stage it frees.
  auto issue_one = [&](int kt, int j) {
    const int stage = kt & (pp::STAGES - 1);
    const uint32_t kk = (uint32_t)kt * BK;
    const int i = j >> 1;
    if ((j & 1) == 0) {
      const uint32_t ao = (a_off[i] != kOOB && kk + a_k[i] < a.K) ? a_off[i] + kk * ES : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_void*)(smem + pp::A_OFF + stage * pp::A_STAGE + (2 * w + i) * 1024), 16, ao, 0, 0, 0);
    } else {
      const uint32_t bo = (b_off[i] != kOOB && kk + b_k[i] < a.K) ? b_off[i] + (uint32_t)kt * b_kstep : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rbm, (lds_void*)(smem + pp::B_OFF + stage * pp::B_STAGE + (2 * w + i) * 1024), 16, bo, 0, 0, 0);
    }
  };

  // ---- LDS fragment addresses -------------------------------------------
  // A (m side): row wm*128 + sj*32 + lrow, chunk 2*ks + half (ks = 0, 1).
  const int xa = pp::swz_a(lrow);          // (row >> 2) & 3 depends on lrow only
  uint32_t a_rd[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    a_rd[ks] = pp::A_OFF + (wm * 128 + lrow) * 64 + (((2 * ks + half) ^ xa) * 16);
  // B (n side), 16-bit: k = 8*half + (lane%16)/4 (+ 16*ks + 4*q),
  //   n = wn*64 + si*32 + 16*((lane/16)%2) + 4*(lane%4);
  // int8: k = 16*half + (lane%16)/2 (+ 32*ks + 8*q), n = wn*64 + si*32 + 16*((lane/16)%2) + 8*(lane%2)
  uint32_t b_rd[2];
#pragma unroll
  for (int si = 0; si < 2; ++si) {
    if constexpr (DTI == DT_I8) {
      const int k = 16 * half + ((lane & 15) >> 1);
      const int n = wn * 64 + si * 32 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
      const int phys = (n >> 4) ^ pp::swz_b8(k);
      b_rd[si] = pp::B_OFF + k * 256 + phys * 16 + (n & 15);
    } else {
      const int k = 8 * half + ((lane & 15) >> 2);
      const int n = wn * 64 + si * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      const int phys = (n >> 3) ^ pp::swz_b(k);
      b_rd[si] = pp::B_OFF + k * 512 + phys * 16 + (n & 7) * 2;
    }
  }

  const int ktiles = (int)((a.K + BK - 1) / BK);
  // LDS byte address of smem (an address-space-3 pointer converts to its offset)
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)smem;

  // ---- prologue: k-tiles 0 .. 2 in flight, k-tile 0 landed ----------------
  for (int t = 0; t < pp::STAGES - 1; ++t)
#pragma unroll
    for (int j = 0; j < pp::LOADS_PER_TILE; ++j) issue_one(t, j);
  __builtin_amdgcn_s_waitcnt(pp::wait_vm(2 * pp::LOADS_PER_TILE));
  __builtin_amdgcn_s_barrier();
  if (wm == 1) __builtin_amdgcn_s_barrier();      // cluster 1 runs one phase behind

  // Interval schedule (cluster 0 / cluster 1): M(t) at 2t / 2t+1, C(t) at
  // 2t+1 / 2t+2.  M(t) loads k-tile t+3 into stage (t+3)%4 = (t-1)%4, whose
  // last reader, M(t-1), ended by interval 2t-1.  M(t) also waits for its own
  // loads of k-tile t+1 (issued in M(t-2); k-tiles t+2 and t+3 may remain in
  // flight) before the barrier that precedes the first read of t+1 at
  // interval 2t+2.
  u32x4 fa[4][2];        // [sj][ks]
  u32x4 fb[2][2];        // [si][ks]
  for (int kt = 0; kt < ktiles; ++kt) {
    const int stage = kt & (pp::STAGES - 1);
    // ---- memory phase: fragments of k-tile kt, loads of k-tile kt + 3 -------
    const int kn = kt + pp::STAGES - 1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int sj = 0; sj < 4; ++sj) {
        fa[sj][ks] = *reinterpret_cast<const u32x4*>(smem + a_rd[ks] + stage * pp::A_STAGE + sj * 2048);
        if (sj & 1) {              // one direct load after every second A-fragment read
          __builtin_amdgcn_sched_barrier(0);
          issue_one(kn, ks * 2 + (sj >> 1));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int si = 0; si < 2; ++si) {
        const uint32_t base = lds_base + b_rd[si] + stage * pp::B_STAGE;
        fb[si][ks] = ks == 0 ? pp::read_b_frag<DTI, 0>(base) : pp::read_b_frag<DTI, 1>(base);
      }
    }
    // k-tile kt+1 landed for this wave (k-tiles kt+2 and kt+3 may be in flight)
    __builtin_amdgcn_s_waitcnt(pp::wait_vm(2 * pp::LOADS_PER_TILE));
    __builtin_amdgcn_s_waitcnt(pp::WAIT_LGKM0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // ---- compute phase: 16 MFMAs from registers ------------------------------
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int si = 0; si < 2; ++si)
#pragma unroll
        for (int sj = 0; sj < 4; ++sj) mfma_chunk<DTI>(acc[si][sj], fb[si][ks], fa[sj][ks]);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
  }
  // no direct load may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(pp::wait_vm(0));
  if (wm == 0) __builtin_amdgcn_s_barrier();      // same barrier count for both clusters

  // ---- epilogue: activation, cast, one store per element -----------------
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.C, a.c_bytes);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.R, a.R ? a.c_bytes : 0u);
  bool staged = false;
  if constexpr (Elem<DTO>::bytes == 2)
    staged = ((reinterpret_cast<uintptr_t>(a.C) | reinterpret_cast<uintptr_t>(a.R)) & 15u) == 0;
  if (staged) {
    __syncthreads();     // every wave's direct loads have landed and its fragment reads are done
    auto slot = [](int r, int c) { return (uint32_t)(r * 512 + ((c ^ (r & 31)) << 4)); };
    // rows 16*it + rrow, chunk rchunk; N % 8 == 0 here, so a chunk is wholly inside or outside C
    const int rrow = 2 * w + (lane >> 5), rchunk = lane & 31;
    with_act(a.act, [&](auto act_c) __attribute__((always_inline)) {
      constexpr int ACT = decltype(act_c)::value;
      with_residual(a.R != nullptr, [&](auto res_c) __attribute__((always_inline)) {
        constexpr bool HAS_R = decltype(res_c)::value;
        if constexpr (HAS_R && DTI != DT_I8) {     // int8 GEMMs take no residual
#pragma unroll
          for (int it = 0; it < 16; ++it) {
            const int r = it * 16 + rrow;
            const uint32_t m = m0 + r, n = n0 + rchunk * 8;
            *reinterpret_cast<u32x4*>(smem + slot(r, rchunk)) =
                ld_b128(rr, (m < a.M && n < a.N) ? (m * a.N + n) * 2u : kOOB);
          }
          __syncthreads();
        }
        // each lane reads (residual) and writes the same 8 bytes: no other lane touches them
#pragma unroll
        for (int si = 0; si < 2; ++si)
#pragma unroll
          for (int sj = 0; sj < 4; ++sj) {
            const int r = wm * 128 + sj * 32 + lrow;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              u32x2* p = reinterpret_cast<u32x2*>(smem + slot(r, wn * 8 + si * 4 + g) + half * 8);
              float z[4] = {acc[si][sj][4 * g + 0], acc[si][sj][4 * g + 1], acc[si][sj][4 * g + 2],
                            acc[si][sj][4 * g + 3]};
              if constexpr (HAS_R && DTI != DT_I8) {
                const u32x2 rv = *p;
                z[0] += widen<DTO>(rv.x & 0xffffu);
                z[1] += widen<DTO>(rv.x >> 16);
                z[2] += widen<DTO>(rv.y & 0xffffu);
                z[3] += widen<DTO>(rv.y >> 16);
              }
              u32x2 o;
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = out_value<DTI, DTO, ACT>(z[e], a.alpha);
              o.x = narrow<DTO>(v[0]) | (narrow<DTO>(v[1]) << 16);
              o.y = narrow<DTO>(v[2]) | (narrow<DTO>(v[3]) << 16);
              *p = o;
            }
          }
      });
    });
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int r = it * 16 + rrow;
      const uint32_t m = m0 + r, n = n0 + rchunk * 8;
      st_b128(rc, (m < a.M && n < a.N) ? (m * a.N + n) * 2u : kOOB,
              *reinterpret_cast<const u32x4*>(smem + slot(r, rchunk)));
    }
    return;
  }
  bool staged32 = false;
  if constexpr (Elem<DTO>::bytes == 4)
    staged32 = ((reinterpret_cast<uintptr_t>(a.C) | reinterpret_cast<uintptr_t>(a.R)) & 15u) == 0;
  if (staged32) {
    // 32-bit outputs: the 256 KB tile leaves in two passes of 128 rows (one
    // cluster's rows each) through 128 KB of LDS: 1 KB rows, 16-byte chunk c
    // of row r at slot c ^ 2*(r & 31); each wave then stores whole rows.
    auto slot = [](int r, int c) { return (uint32_t)(r * 1024 + ((c ^ (2 * (r & 31))) << 4)); };
    with_act(a.act, [&](auto act_c) __attribute__((always_inline)) {
      constexpr int ACT = decltype(act_c)::value;
      with_residual(a.R != nullptr, [&](auto res_c) __attribute__((always_inline)) {
        constexpr bool HAS_R = decltype(res_c)::value && DTI != DT_I8;   // int8 GEMMs take no residual
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
          // pass 0: every direct load has landed and every fragment read is done;
          // pass 1: the rows of pass 0 have left LDS
          __syncthreads();
          if constexpr (HAS_R) {
#pragma unroll
            for (int it = 0; it < 16; ++it) {
              const int r = it * 8 + w;
              const uint32_t m = m0 + pass * 128 + r, n = n0 + lane * 4;
              *reinterpret_cast<u32x4*>(smem + slot(r, lane)) =
                  ld_b128(rr, (m < a.M && n < a.N) ? (m * a.N + n) * 4u : kOOB);
            }
            __syncthreads();
          }
          if (wm == pass) {
#pragma unroll
            for (int si = 0; si < 2; ++si)
#pragma unroll
              for (int sj = 0; sj < 4; ++sj) {
                const int r = sj * 32 + lrow;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  u32x4* p = reinterpret_cast<u32x4*>(smem + slot(r, wn * 16 + si * 8 + 2 * g + half));
                  float z[4] = {acc[si][sj][4 * g + 0], acc[si][sj][4 * g + 1], acc[si][sj][4 * g + 2],
                                acc[si][sj][4 * g + 3]};
                  if constexpr (HAS_R) {
                    const u32x4 rv = *p;
                    z[0] += __uint_as_float(rv.x);
                    z[1] += __uint_as_float(rv.y);
                    z[2] += __uint_as_float(rv.z);
                    z[3] += __uint_as_float(rv.w);
                  }
                  u32x4 o;
                  o.x = narrow<DTO>(out_value<DTI, DTO, ACT>(z[0], a.alpha));
                  o.y = narrow<DTO>(out_value<DTI, DTO, ACT>(z[1], a.alpha));
                  o.z = narrow<DTO>(out_value<DTI, DTO, ACT>(z[2], a.alpha));
                  o.w = narrow<DTO>(out_value<DTI, DTO, ACT>(z[3], a.alpha));
                  *p = o;
                }
              }
          }
          __syncthreads();
#pragma unroll
          for (int it = 0; it < 16; ++it) {
            const int r = it * 8 + w;
            const uint32_t m = m0 + pass * 128 + r, n = n0 + lane * 4;   // N % 8 == 0: 4 values all in or out
            st_b128(rc, (m < a.M && n < a.N) ? (m * a.N + n) * 4u : kOOB,
                    *reinterpret_cast<const u32x4*>(smem + slot(r, lane)));
          }
        }
      });
    });
    return;
  }
  with_act(a.act, [&](auto act_c) __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_c)::value;
    with_residual(a.R != nullptr, [&](auto res_c) __attribute__((always_inline)) {
      constexpr bool HAS_R = decltype(res_c)::value;
#pragma unroll
      for (int si = 0; si < 2; ++si)
#pragma unroll
        for (int sj = 0; sj < 4; ++sj) {
          const uint32_t m = m0 + wm * 128 + sj * 32 + lrow;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint32_t n = n0 + wn * 64 + si * 32 + 8 * g + 4 * half;
            const bool ok = m < a.M && n < a.N;
            float z[4] = {acc[si][sj][4 * g + 0], acc[si][sj][4 * g + 1], acc[si][sj][4 * g + 2],
                          acc[si][sj][4 * g + 3]};
            if constexpr (HAS_R && DTI != DT_I8) {
              float rv[4];
              load4<DTO>(rr, m * a.N + n, ok, rv);
#pragma unroll
              for (int e = 0; e < 4; ++e) z[e] += rv[e];
            }
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = out_value<DTI, DTO, ACT>(z[e], a.alpha);
            store4<DTO>(rc, m * a.N + n, ok, v[0], v[1], v[2], v[3]);
          }
        }
    });
  });
}

template <int DTI, int DTO>
inline void launch_gemm_pp(const GemmArgs& a, hipStream_t s) {
  note_launch(DTI == DT_I8 ? "gemm 256x256/2x4 ping-pong int8" : "gemm 256x256/2x4 ping-pong");
  launch_kernel(gemm16_pp_kernel<DTI, DTO>, dim3(a.tiles_m * a.tiles_n), dim3(pp::THREADS), s, a);
}

}  // namespace biasact
