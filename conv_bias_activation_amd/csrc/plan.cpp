// plan.cpp — argument checking, tile selection and launch planning for the
// biasact C ABI.  Plain C++: no HIP call happens here, so every error path is
// reachable on a machine without a GPU.
#include "plan.hpp"

#include <atomic>

namespace biasact {

namespace {

constexpr int kF32 = 0, kF16 = 1, kBF16 = 2, kI8 = 3, kI32 = 4;
constexpr int64_t kMaxBytes = (int64_t)1 << 31;   // every tensor < 2 GiB (32-bit buffer offsets)
// int8 GEMMs: K * 128 * 128 < 2^31, so the product sum alone fits int32
constexpr int64_t kMaxKInt8 = 131071;

int elem_bytes(int dt) { return dt == kI8 ? 1 : (dt == kF32 || dt == kI32) ? 4 : 2; }
int chunk_elems(int dt) { return 16 / elem_bytes(dt); }   // 16 bytes of one type
bool valid_float_dt(int dt) { return dt == kF32 || dt == kF16 || dt == kBF16; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

std::atomic<int> g_forced_tile{-1};
std::atomic<int> g_forced_halo{-1};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shared dtype decoding: A/x and B/w share one type.  Floating-point operands:
// bias fp32 or the operand type, output fp32, fp16 or bf16.  int8 operands:
// bias int32 (the only bias type the MatmulLeakyRelu page allows for int8),
// output int32 or a floating-point type.
int decode_dtypes(uint32_t dtypes, bool has_bias, int* dti, int* dto, int* dtb) {
  const int a = (int)(dtypes & 0xffu), b = (int)((dtypes >> 8) & 0xffu);
  const int bias = (int)((dtypes >> 16) & 0xffu), out = (int)((dtypes >> 24) & 0xffu);
  if (b != a) return kErrUnsupported;
  if (a == kI8) {
    if (!(valid_float_dt(out) || out == kI32)) return kErrUnsupported;
    if (has_bias && bias != kI32) return kErrUnsupported;
  } else {
    if (!valid_float_dt(a) || !valid_float_dt(out)) return kErrUnsupported;
    if (has_bias && !(bias == kF32 || bias == a)) return kErrUnsupported;
  }
  *dti = a;
  *dto = out;
  *dtb = has_bias ? bias : -1;
  return kOk;
}

// Pick the first tile (in preference order) that yields at least `want`
// workgroups; otherwise the one with the most workgroups.
int pick_tile(const int* order, int n_order, int64_t rows_j, int64_t rows_i, int64_t want) {
  int best = order[n_order - 1];
  int64_t best_tiles = -1;
  for (int k = 0; k < n_order; ++k) {
    const TileShapeDesc& t = kTiles[order[k]];
    const int64_t tiles = ceil_div(rows_j, t.bm) * ceil_div(rows_i, t.bn);
    if (tiles >= want) return order[k];
    if (tiles > best_tiles) {
      best_tiles = tiles;
      best = order[k];
    }
  }
  return best;
}

// Halo-kernel parameters for an fp32 conv (any filter larger than 1x1, any
// stride, padding and dilation).  All C channels form one chunk when their
// halo (HR x HC positions per channel, rounded up to 64) and their weight
// block (bm rows of 2 kpad + 4 floats) each fit a chunk buffer; otherwise the
// chunk is the widest whose halo and weights share one buffer, evened out over
// the chunks it takes.  Returns false when a single channel does not fit.
bool plan_halo32(ConvPlan* p, const void* x, const void* w) {
  // A 1x1 filter is a strided GEMM: the generic kernel stages exactly the
  // operands it reads and measures faster there.
  if (p->kh * p->kw == 1) return false;
  if (!aligned(x, 4) || !aligned(w, 4)) return false;
  const uint64_t T = (uint64_t)p->kh * p->kw;
  const uint32_t bm = p->Co <= 64 ? 64 : 128;
  const uint32_t bn = 128;
  const uint32_t PW = p->Wo < bn ? p->Wo : bn;
  const uint32_t PH = bn / PW < p->Ho ? bn / PW : p->Ho;      // rows of one image only
  const uint64_t HR = (uint64_t)(PH - 1) * p->sh + (uint64_t)(p->kh - 1) * p->dh + 1;
  const uint64_t HC = (uint64_t)(PW - 1) * p->sw + (uint64_t)(p->kw - 1) * p->dw + 1;
  const uint64_t HRCP = (HR * HC + 63) / 64 * 64;
  // LDS layouts of conv32_halo_kernel (80 KB each, with the 256-entry offset
  // table): two chunk buffers of 10108 floats, or (resident filter) a
  // 10240-float weight block and two 4992-float halo buffers
  const uint64_t limit = 10108, res_w = 10240, res_h = 4992;
  auto kpad = [&](uint64_t b) { return ((b * T + 1) / 2 + 3) / 4 * 4; };
  auto kstr = [&](uint64_t b) { return 2 * kpad(b) + 4; };
  auto wsz = [&](uint64_t b) { return (bm * kstr(b) + 63) / 64 * 64; };
  auto fits = [&](uint64_t b) { return kpad(b) <= 128 && b * HRCP + wsz(b) <= limit; };
  uint64_t lo;
  if (kpad(p->C) <= 128 && p->C * HRCP <= limit && wsz(p->C) <= limit) {
    lo = p->C;                     // one chunk: its halo in one buffer, its weights in the other
  } else {
    if (!fits(1)) return false;
    lo = 1;
    uint64_t hi = p->C;            // largest chunk whose halo and weights share one buffer
    while (lo < hi) {
      const uint64_t mid = (lo + hi + 1) / 2;
      if (fits(mid)) lo = mid;
      else hi = mid - 1;
    }
    const uint64_t n = (p->C + lo - 1) / lo;                  // same chunk count, even split
    lo = (p->C + n - 1) / n;
  }
  p->h_bm = bm;
  p->h_ks = 0;
  p->h_sn = 2;
  p->h_nw = 4;
  p->h_PH = PH;
  p->h_PW = PW;
  p->h_HR = (uint32_t)HR;
  p->h_HC = (uint32_t)HC;
  p->h_hrcp = (uint32_t)HRCP;
  p->h_bkc = (uint32_t)lo;
  p->h_kpad = (uint32_t)kpad(lo);
  p->h_kstr = (uint32_t)kstr(lo);
  p->h_co_blocks = (p->Co + bm - 1) / bm;
  p->h_w_blocks = (p->Wo + PW - 1) / PW;
  p->h_h_blocks = (p->Ho + PH - 1) / PH;
  const uint64_t blocks = (uint64_t)p->h_co_blocks * p->h_w_blocks * p->h_h_blocks * p->N;
  if (blocks >= (1u << 31)) return false;
  p->h_blocks = (uint32_t)blocks;
  // Resident filter: with one chunk and one co block every patch multiplies
  // the same weight block.  When it fits the resident layout's weight block
  // and a patch's halo its halo buffers, and there are more patches than
  // workgroup slots (two per CU on 256 CUs), 512 workgroups each stage the
  // weights once and stream their patches' halos through the two buffers.
  constexpr uint64_t kSlots = 512;
  p->h_groups = 0;
  if (lo == p->C && p->h_co_blocks == 1 && wsz(lo) <= res_w && lo * HRCP <= res_h && blocks > kSlots) {
    p->h_groups = (uint32_t)kSlots;
    p->h_blocks = (uint32_t)kSlots;
  }
  return true;
}

// Halo-kernel parameters for a conv (16-bit operands, C % 8 == 0, even W,
// square 1x1, 3x3, 5x5 or 7x7 filters, aligned x / w; fp32 operands go to
// plan_halo32).
// Returns false when it does not apply.
bool plan_halo(ConvPlan* p, const void* x, const void* w) {
  p->h_hrcp = 0;
  p->h_kpad = 0;
  p->h_kstr = 0;
  p->h_groups = 0;
  if (p->dti == kF32) return plan_halo32(p, x, w);
  if (p->C % 8 != 0 || p->W % 2 != 0) return false;
  const uint32_t T = p->kh * p->kw;
  if (p->kh != p->kw || (p->kh != 1 && p->kh != 3 && p->kh != 5 && p->kh != 7)) return false;   // square 1, 3, 5, 7
  const bool large = T > 9;         // 5x5, 7x7: one configuration (64 channels, 4 waves, chunks of 16)
  if (!aligned(x, 4) || !aligned(w, 16)) return false;
  // One configuration = (bm output channels, 2 x 32 sn positions, LDS budget).
  // LDS: the halo (HR x HC positions x bkc channels) and one raw weight chunk
  // (bm rows of bkc*T values plus a 16-byte pad, rounded up to whole 1 KiB
  // direct loads).  One MFMA k-step consumes 16 channels: chunks of 64, 32 or
  // 16 (zero-filled past C), with at most four (k-step, 32-row) weight-fragment
  // sets per wave held in registers -- two where two workgroups share a CU.
  struct Cfg {
    uint32_t bm, sn, nw, ks, PH, PW, HR, HC, bkc, co_blocks, w_blocks, h_blocks;
    uint64_t blocks;
    bool ok;
  };
  // shared: two four-wave workgroups per CU; nw = 8: one eight-wave workgroup
  // per CU (two waves per SIMD, at most 256 registers per lane each)
  auto make = [&](uint32_t bm, uint32_t sn, bool shared, uint32_t nw = 4) {
    Cfg c{};
    c.bm = bm;
    c.sn = sn;
    c.nw = nw;
    const uint32_t bn = 32 * sn * (nw / 2);
    c.PW = p->Wo < bn ? p->Wo : bn;
    c.PH = bn / c.PW < p->Ho ? bn / c.PW : p->Ho;            // rows of one image only
    c.PH = (p->Ho + (p->Ho + c.PH - 1) / c.PH - 1) / ((p->Ho + c.PH - 1) / c.PH);   // as even as the block count allows
    c.HR = (c.PH - 1) * p->sh + (p->kh - 1) * p->dh + 1;
    // a patch whose first input column ow0*sw - pl is odd starts one column
    // into its (even-aligned) halo: one more column; when every patch starts
    // on an even column (pl even, and one column block or an even PW*sw) none
    const uint32_t wblk = (p->Wo + c.PW - 1) / c.PW;
    const bool even_starts = p->pl % 2 == 0 && (wblk == 1 || (c.PW * p->sw) % 2 == 0);
    c.HC = (c.PW - 1) * p->sw + (p->kw - 1) * p->dw + (even_starts ? 1 : 2);
    c.HC += c.HC & 1;
    // the kernel's occupancy rule: two workgroups per CU (80 KB of LDS each)
    // when a wave holds at most two fragment sets and two accumulator tiles
    auto limit = [&](uint64_t b) {
      const bool two = nw == 4 && !large && (b / 16) * (bm / 64) <= 2 && sn * (bm / 64) <= 2;
      return (uint64_t)(two ? 80 : 144) * 1024;
    };
    auto lds_bytes = [&](uint64_t b) {
      const uint64_t raw = ((uint64_t)bm * (b * T / 8 + 1) + 63) / 64 * 1024;
      return (uint64_t)c.HR * c.HC * b * 2 + raw;
    };
    const uint32_t max_sets = large ? 1 : shared || nw == 8 ? 2 : 4;   // k-steps x 32-row tiles per wave
    uint32_t bkc = 16 * (max_sets / (bm / 64));
    if (bkc > 64) bkc = 64;
    while (bkc > 16 && bkc / 2 >= p->C) bkc /= 2;            // no wider than the channel count needs
    while (bkc > 16 && lds_bytes(bkc) > limit(bkc)) bkc /= 2;
    c.ok = lds_bytes(bkc) <= limit(bkc) && (!shared || sn * (bm / 64) <= 2);
    c.bkc = bkc;
    c.ks = bkc / 16;
    c.co_blocks = (p->Co + bm - 1) / bm;
    c.w_blocks = (p->Wo + c.PW - 1) / c.PW;
    c.h_blocks = (p->Ho + c.PH - 1) / c.PH;
    c.blocks = (uint64_t)c.co_blocks * c.w_blocks * c.h_blocks * p->N;
    c.ok = c.ok && c.blocks < (1u << 31);
    return c;
  };
  // Eight-wave variants (one workgroup of 64 channels per CU, two waves per
  // SIMD, chunks of 32 channels): 64 channels x 128 positions up to 64 output
  // channels; 64 x 256 positions beyond, when that still gives 200 or more
  // workgroups.  Otherwise a four-wave workgroup per CU with the widest tile,
  // unless that leaves fewer than two workgroups per CU: then tiles half as
  // wide in channels (or positions) that two workgroups can share a CU with,
  // when they give 1.5x the workgroups.
  Cfg c = make(p->Co <= 64 || large ? 64 : 128, 2, false);
  const Cfg alt[4] = {make(64, 2, true), make(64, 1, true), make(64, 1, false, 8), make(64, 2, false, 8)};
  auto eight_ok = [&](const Cfg& e) { return e.ok && e.ks == 2; };
  const int forced = forced_halo_variant();
  if (large) {
    // larger filters have the one configuration
  } else if (forced >= 1 && forced <= 4) {
    const Cfg& f = alt[forced - 1];
    if (forced <= 2 ? f.ok : eight_ok(f)) c = f;
  } else if (forced < 0 && p->Co <= 64 && eight_ok(alt[2])) {
    c = alt[2];
  } else if (forced < 0 && p->Co > 64 && eight_ok(alt[3]) && alt[3].blocks >= 200) {
    c = alt[3];
  } else if (forced < 0 && c.ok && c.blocks < 512) {
    for (int i = 0; i < 2; ++i)
      if (alt[i].ok && alt[i].blocks * 2 >= c.blocks * 3) {
        c = alt[i];
        break;
      }
  }
  if (!c.ok) return false;
  p->h_bm = c.bm;
  p->h_ks = c.ks;                                              // k-steps of 16 channels per tap
  p->h_sn = c.sn;
  p->h_nw = c.nw;
  p->h_PH = c.PH;
  p->h_PW = c.PW;
  p->h_HR = c.HR;
  p->h_HC = c.HC;
  p->h_bkc = c.bkc;
  p->h_co_blocks = c.co_blocks;
  p->h_w_blocks = c.w_blocks;
  p->h_h_blocks = c.h_blocks;
  p->h_blocks = (uint32_t)c.blocks;
  return true;
}

}  // namespace

int forced_tile() { return g_forced_tile.load(std::memory_order_relaxed); }
int forced_halo_variant() { return g_forced_halo.load(std::memory_order_relaxed); }
void set_forced_halo_variant(int v) { g_forced_halo.store(v, std::memory_order_relaxed); }
void set_forced_tile(int id) { g_forced_tile.store(id, std::memory_order_relaxed); }

int select_gemm_tile(int64_t M, int64_t N, int64_t /*K*/, int dti) {
  // Largest tiles first while the grid still covers all 256 compute units.
  // int8 skips 256x256: its 16x16-byte register transposes of B do not fit
  // beside 256 accumulators per lane.
  static const int order[] = {0, 1, 2, 3, 5};
  if (dti == kI8) return pick_tile(order + 1, 4, M, N, 256);
  return pick_tile(order, 5, M, N, 256);
}

// Among the tiles (in preference order) that give at least 256 workgroups,
// the one whose busiest CU computes the fewest outputs: a grid of `tiles`
// workgroups puts ceil(tiles / 256) of them on some CU.  A later (smaller)
// tile must cut that load by at least an eighth to be taken, since its
// per-workgroup costs (operand round trip, epilogue) weigh more.  With no
// tile reaching 256 workgroups, pick_tile's choice.
int pick_tile_balanced(const int* order, int n_order, int64_t rows_j, int64_t rows_i) {
  int best = -1;
  int64_t best_load = 0;
  for (int k = 0; k < n_order; ++k) {
    const TileShapeDesc& t = kTiles[order[k]];
    const int64_t tiles = ceil_div(rows_j, t.bm) * ceil_div(rows_i, t.bn);
    if (tiles < 256) continue;
    const int64_t load = ceil_div(tiles, 256) * t.bm * t.bn;
    if (best < 0 || load * 8 <= best_load * 7) {
      best = order[k];
      best_load = load;
    }
  }
  return best >= 0 ? best : pick_tile(order, n_order, rows_j, rows_i, 256);
}

int select_conv_tile(int64_t N, int64_t Co, int64_t Ho, int64_t Wo, int64_t /*K*/, int /*dti*/) {
  const int64_t P = N * Ho * Wo;
  if (Co <= 64) {
    static const int order[] = {4, 3, 5};
    return pick_tile_balanced(order, 3, Co, P);
  }
  static const int order[] = {0, 1, 2, 3, 5};
  return pick_tile_balanced(order, 5, Co, P);
}

int plan_gemm(const void* A, const void* B, const void* bias, const void* C, int64_t M, int64_t N,
              int64_t K, uint32_t dtypes, int act, GemmPlan* p, const void* R) {
  if (!p) return kErrInvalid;
  if (M < 0 || N < 0 || K < 0) return kErrInvalid;
  if (act < 0 || act > 5) return kErrInvalid;
  int dti, dto, dtb;
  int rc = decode_dtypes(dtypes, bias != nullptr, &dti, &dto, &dtb);
  if (rc) return rc;
  if (dti == kI8) {
    if (K > kMaxKInt8) return kErrUnsupported;
    // an int32 output holds integers: no activation with a non-integer result
    if (dto == kI32 && act != 0 && act != 1) return kErrUnsupported;
    if (R) return kErrUnsupported;                      // no residual on int8 GEMMs
  }
  const int64_t es = elem_bytes(dti);
  const int64_t a_bytes = M * K * es, b_bytes = K * N * es, c_bytes = M * N * elem_bytes(dto);
  const int64_t bias_bytes = bias ? N * elem_bytes(dtb) : 0;
  if (M >= kMaxBytes || N >= kMaxBytes || K >= kMaxBytes) return kErrUnsupported;
  if (a_bytes >= kMaxBytes || b_bytes >= kMaxBytes || c_bytes >= kMaxBytes) return kErrUnsupported;
  if ((a_bytes > 0 && !A) || (b_bytes > 0 && !B) || (c_bytes > 0 && !C)) return kErrInvalid;
  p->dti = dti;
  p->dto = dto;
  p->bias_dt = dtb;
  p->M = (uint32_t)M;
  p->N = (uint32_t)N;
  p->K = (uint32_t)K;
  p->a_bytes = (uint32_t)a_bytes;
  p->b_bytes = (uint32_t)b_bytes;
  p->bias_bytes = (uint32_t)bias_bytes;
  p->c_bytes = (uint32_t)c_bytes;
  const int epc = chunk_elems(dti);
  p->vec_a = K % epc == 0 && aligned(A, 16);
  p->vec_b = N % epc == 0 && aligned(B, 16);
  p->vec_c = N % 4 == 0 && aligned(C, 4 * (uintptr_t)elem_bytes(dto)) &&
             (!R || aligned(R, 4 * (uintptr_t)elem_bytes(dto)));
  p->empty = M == 0 || N == 0;
  int tile = forced_tile();
  if (tile < 0 || tile >= kNumTileConfigs) tile = select_gemm_tile(M, N, K, dti);
  // the ping-pong kernel takes 16-bit or int8 operands with 16-byte aligned
  // rows; int8 takes it wherever its 256x256 grid still covers every CU
  const bool pp_ok = (dti == kF16 || dti == kBF16 || dti == kI8) && p->vec_a && p->vec_b && p->vec_c;
  if (pp_ok && forced_tile() < 0 &&
      (tile == 0 || (dti == kI8 && ceil_div(M, 256) * ceil_div(N, 256) >= 256)))
    tile = 6;
  if (tile == 6 && !pp_ok) tile = dti == kI8 ? 1 : 0;
  if (tile == 7) tile = 2;                              // the halo tile is conv-only
  p->tile = tile;
  p->tiles_m = (uint32_t)ceil_div(M, kTiles[tile].bm);
  p->tiles_n = (uint32_t)ceil_div(N, kTiles[tile].bn);
  return kOk;
}

int conv_out_dims(int64_t H, int64_t W, int64_t kh, int64_t kw, const int32_t* strides,
                  const int32_t* pads, const int32_t* dilations, int64_t* Ho, int64_t* Wo) {
  if (!strides || !pads || !dilations || !Ho || !Wo) return kErrInvalid;
  if (H <= 0 || W <= 0 || kh <= 0 || kw <= 0) return kErrInvalid;
  if (H >= kMaxBytes || W >= kMaxBytes || kh >= kMaxBytes || kw >= kMaxBytes) return kErrUnsupported;
  const int32_t sh = strides[0], sw = strides[1], dh = dilations[0], dw = dilations[1];
  const int32_t pt = pads[0], pb = pads[1], pl = pads[2], pr = pads[3];
  if (sh < 1 || sw < 1 || dh < 1 || dw < 1) return kErrInvalid;
  if (pt < 0 || pb < 0 || pl < 0 || pr < 0) return kErrInvalid;
  // floor((in + pad_lo + pad_hi - dil * (k - 1) - 1) / stride) + 1 per axis
  const int64_t span_h = H + pt + pb - (int64_t)dh * (kh - 1) - 1;
  const int64_t span_w = W + pl + pr - (int64_t)dw * (kw - 1) - 1;
  if (span_h < 0 || span_w < 0) return kErrInvalid;  // empty output
  *Ho = span_h / sh + 1;
  *Wo = span_w / sw + 1;
  return kOk;
}

int plan_conv(const void* x, const void* w, const void* bias, const void* y, int64_t N, int64_t C,
              int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw, const int32_t* strides,
              const int32_t* pads, const int32_t* dilations, uint32_t dtypes, int act,
              ConvPlan* p, const void* r) {
  if (!p || !strides || !pads || !dilations) return kErrInvalid;
  if (N < 0 || C <= 0 || H <= 0 || W <= 0 || Co <= 0 || kh <= 0 || kw <= 0) return kErrInvalid;
  if (act < 0 || act > 5) return kErrInvalid;
  if (act == 2) return kErrUnsupported;                 // no alpha argument on this entry point
  const int32_t sh = strides[0], sw = strides[1], dh = dilations[0], dw = dilations[1];
  const int32_t pt = pads[0], pb = pads[1], pl = pads[2], pr = pads[3];
  int64_t Ho, Wo;
  const int dims_rc = conv_out_dims(H, W, kh, kw, strides, pads, dilations, &Ho, &Wo);
  if (dims_rc) return dims_rc;
  int dti, dto, dtb;
  int rc = decode_dtypes(dtypes, bias != nullptr, &dti, &dto, &dtb);
  if (rc) return rc;
  if (dti == kI8) return kErrUnsupported;              // int8 is a GEMM-only path
  const int64_t es = elem_bytes(dti);
  const int64_t K = C * kh * kw, P = N * Ho * Wo;
  const int64_t x_bytes = N * C * H * W * es, w_bytes = Co * K * es;
  const int64_t y_bytes = N * Co * Ho * Wo * elem_bytes(dto);
  const int64_t bias_bytes = bias ? Co * elem_bytes(dtb) : 0;
  if (C >= kMaxBytes || H >= kMaxBytes || W >= kMaxBytes || Co >= kMaxBytes || K >= kMaxBytes ||
      P >= kMaxBytes || Ho * Wo >= kMaxBytes || H + pt + pb >= kMaxBytes || W + pl + pr >= kMaxBytes)
    return kErrUnsupported;
  if (x_bytes >= kMaxBytes || w_bytes >= kMaxBytes || y_bytes >= kMaxBytes) return kErrUnsupported;
  if ((x_bytes > 0 && !x) || !w || (y_bytes > 0 && !y)) return kErrInvalid;
  p->dti = dti;
  p->dto = dto;
  p->bias_dt = dtb;
  p->N = (uint32_t)N; p->C = (uint32_t)C; p->H = (uint32_t)H; p->W = (uint32_t)W;
  p->Co = (uint32_t)Co; p->kh = (uint32_t)kh; p->kw = (uint32_t)kw;
  p->Ho = (uint32_t)Ho; p->Wo = (uint32_t)Wo;
  p->sh = sh; p->sw = sw; p->pt = pt; p->pb = pb; p->pl = pl; p->pr = pr; p->dh = dh; p->dw = dw;
  p->K = (uint32_t)K;
  p->P = (uint32_t)P;
  p->x_bytes = (uint32_t)x_bytes;
  p->w_bytes = (uint32_t)w_bytes;
  p->bias_bytes = (uint32_t)bias_bytes;
  p->y_bytes = (uint32_t)y_bytes;
  p->vec_w = K % chunk_elems(dti) == 0 && aligned(w, 16);
  p->vec_y = (Ho * Wo) % 4 == 0 && aligned(y, 4 * (uintptr_t)elem_bytes(dto)) &&
             (!r || aligned(r, 4 * (uintptr_t)elem_bytes(dto)));
  p->empty = N == 0;
  int tile = forced_tile();
  const bool auto_tile = tile < 0 || tile >= kNumTileConfigs;
  if (auto_tile) tile = select_conv_tile(N, Co, Ho, Wo, K, dti);
  if (tile == 6) tile = 0;                              // no ping-pong conv kernel
  const bool halo_ok = plan_halo(p, x, w);
  if (halo_ok && (auto_tile || tile == 7)) tile = 7;
  if (tile == 7 && !halo_ok) tile = 3;
  p->tile = tile;
  p->tiles_m = (uint32_t)ceil_div(Co, kTiles[tile].bm);
  p->tiles_n = (uint32_t)ceil_div(P, kTiles[tile].bn);
  return kOk;
}

const char* status_string(int s) {
  switch (s) {
    case kOk: return "ok";
    case kErrInvalid:
      return "invalid argument (null pointer, negative or empty dimension, bad activation, "
             "stride/dilation < 1, pad < 0, empty conv output, or workspace too small)";
    case kErrUnsupported:
      return "unsupported (element types: A = B in {f32, f16, bf16}, bias in {f32, input type}, "
             "output in {f32, f16, bf16}; conv has no LeakyReLU; every tensor < 2^31 bytes)";
    case kErrHip: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

}  // namespace biasact
