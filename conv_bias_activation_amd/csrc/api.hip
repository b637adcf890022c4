// api.hip — the extern "C" entry points declared in include/biasact.h.
// Each call checks its arguments (plan.cpp), then queues one kernel (fused
// path) or two kernels (two-kernel path) on the caller's stream.  Nothing is
// allocated and nothing is synchronised here.
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <vector>

#include "biasact.h"
#include "launch.hpp"
#include "launch_kernel.hpp"
#include "plan.hpp"

using namespace biasact;

namespace biasact {
thread_local hipError_t t_launch_error = hipSuccess;
thread_local char t_launch_desc[kLaunchDescBytes] = "none";
}

namespace {

// the HIP error behind the most recent BA_ERR_HIP on this thread
thread_local hipError_t t_last_hip = hipSuccess;

// Status of the launches queued since the last call (launch_kernel records
// the first refusal).
int launch_status() {
  const hipError_t e = t_launch_error;
  t_launch_error = hipSuccess;
  if (e == hipSuccess) return kOk;
  t_last_hip = e;
  return kErrHip;
}

int out_bytes(int dt) { return (dt == DT_F32 || dt == DT_I32) ? 4 : 2; }

// aligned for 4-element (16- or 8-byte) accesses of an output-type tensor
bool aligned_for(const void* p, int dt) { return ((uintptr_t)p % (4u * out_bytes(dt))) == 0; }

int launch_gemm_plan(const GemmPlan& p, const void* A, const void* B, const void* bias, void* C,
                     const void* R, int dto, int act, float alpha, hipStream_t s) {
  GemmArgs a;
  a.A = A;
  a.B = B;
  a.bias = bias;
  a.C = C;
  a.R = R;
  a.M = p.M;
  a.N = p.N;
  a.K = p.K;
  a.a_bytes = p.a_bytes;
  a.b_bytes = p.b_bytes;
  a.bias_bytes = p.bias_bytes;
  a.c_bytes = p.M * p.N * (uint32_t)out_bytes(dto);
  a.bias_dt = p.bias_dt;
  a.act = act;
  a.alpha = alpha;
  a.tiles_m = p.tiles_m;
  a.tiles_n = p.tiles_n;
  a.vec_a = p.vec_a;
  a.vec_b = p.vec_b;
  a.vec_c = p.N % 4 == 0 && aligned_for(C, dto) && (!R || aligned_for(R, dto));
  int rc;
  switch (p.dti) {
    case DT_F32: rc = launch_gemm_f32(dto, p.tile, a, s); break;
    case DT_F16: rc = launch_gemm_f16(dto, p.tile, a, s); break;
    case DT_BF16: rc = launch_gemm_bf16(dto, p.tile, a, s); break;
    case DT_I8: rc = launch_gemm_i8(dto, p.tile, a, s); break;
    default: return kErrUnsupported;
  }
  if (rc) return kErrUnsupported;
  return launch_status();
}

int launch_conv_plan(const ConvPlan& p, const void* x, const void* w, const void* bias, void* y,
                     const void* r, int dto, int act, hipStream_t s) {
  ConvArgs a;
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.y = y;
  a.r = r;
  ConvGeom& g = a.geom;
  g.N = p.N; g.C = p.C; g.H = p.H; g.W = p.W; g.Co = p.Co; g.kh = p.kh; g.kw = p.kw;
  g.Ho = p.Ho; g.Wo = p.Wo;
  g.sh = p.sh; g.sw = p.sw; g.pt = p.pt; g.pl = p.pl; g.dh = p.dh; g.dw = p.dw;
  g.K = p.K;
  g.P = p.P;
  g.div_wo = make_fastdiv(p.Wo);
  g.div_howo = make_fastdiv(p.Ho * p.Wo);
  g.div_khkw = make_fastdiv(p.kh * p.kw);
  g.div_kw = make_fastdiv(p.kw);
  a.x_bytes = p.x_bytes;
  a.w_bytes = p.w_bytes;
  a.bias_bytes = p.bias_bytes;
  a.y_bytes = p.N * p.Co * p.Ho * p.Wo * (dto == DT_F32 ? 4u : 2u);
  a.bias_dt = p.bias_dt;
  a.act = act;
  a.alpha = 0.0f;
  a.tiles_m = p.tiles_m;
  a.tiles_n = p.tiles_n;
  a.vec_w = p.vec_w;
  a.vec_y = (p.Ho * p.Wo) % 4 == 0 && aligned_for(y, dto) && (!r || aligned_for(r, dto));
  int rc;
  if (p.tile == 7) {
    HaloArgs h;
    h.x = x;
    h.w = w;
    h.bias = bias;
    h.y = y;
    h.r = r;
    h.geom = a.geom;
    h.x_bytes = a.x_bytes;
    h.w_bytes = a.w_bytes;
    h.bias_bytes = a.bias_bytes;
    h.y_bytes = a.y_bytes;
    h.bias_dt = a.bias_dt;
    h.act = act;
    h.alpha = 0.0f;
    h.PH = p.h_PH;
    h.PW = p.h_PW;
    h.HR = p.h_HR;
    h.HC = p.h_HC;
    h.bkc = p.h_bkc;
    h.co_blocks = p.h_co_blocks;
    h.w_blocks = p.h_w_blocks;
    h.h_blocks = p.h_h_blocks;
    h.blocks = p.h_blocks;
    h.vec_y = p.Wo % 4 == 0 && aligned_for(y, dto) && (!r || aligned_for(r, dto));
    h.hrcp = p.h_hrcp;
    h.div_hc = make_fastdiv(p.h_HC ? p.h_HC : 1u);
    h.kstr = p.h_kstr;
    h.kpad = p.h_kpad;
    h.div_kstr = make_fastdiv(p.h_kstr ? p.h_kstr : 1u);
    h.groups = p.h_groups;
    h.div_cob = make_fastdiv(p.h_co_blocks ? p.h_co_blocks : 1u);
    h.div_wb = make_fastdiv(p.h_w_blocks ? p.h_w_blocks : 1u);
    h.div_hb = make_fastdiv(p.h_h_blocks ? p.h_h_blocks : 1u);
    h.div_pw = make_fastdiv(p.h_PW ? p.h_PW : 1u);
    h.div_pairs = make_fastdiv(p.h_HC >= 2 ? p.h_HC / 2 : 1u);
    rc = launch_conv_halo(p.dti, dto, (int)(p.kh * p.kw), (int)p.h_bm, (int)p.h_ks, (int)p.h_sn, (int)p.h_nw, h, s);
    if (rc) return kErrUnsupported;
    return launch_status();
  }
  switch (p.dti) {
    case DT_F32: rc = launch_conv_f32(dto, p.tile, a, s); break;
    case DT_F16: rc = launch_conv_f16(dto, p.tile, a, s); break;
    case DT_BF16: rc = launch_conv_bf16(dto, p.tile, a, s); break;
    default: return kErrUnsupported;
  }
  if (rc) return kErrUnsupported;
  return launch_status();
}

int launch_second_kernel(int dto, const void* ws, void* out, uint64_t n, int act, float alpha,
                         const void* res, hipStream_t s) {
  if (launch_act_cast(dto, static_cast<const float*>(ws), out, (uint32_t)n, act, alpha, res, s))
    return kErrUnsupported;
  return launch_status();
}

// Shared bodies of the entry points; R / r is the residual or null.
int gemm_impl(const void* A, const void* B, const void* bias, const void* R, void* C, int64_t M,
              int64_t N, int64_t K, uint32_t dtypes, int act, float alpha, hipStream_t stream) {
  GemmPlan p;
  int rc = plan_gemm(A, B, bias, C, M, N, K, dtypes, act, &p, R);
  if (rc || p.empty) return rc;
  return launch_gemm_plan(p, A, B, bias, C, R, p.dto, act, alpha, stream);
}

// dtypes with the output code replaced by fp32 (kernel 1 of the two-kernel
// path writes the fp32 workspace)
uint32_t with_f32_out(uint32_t dtypes) { return (dtypes & 0x00ffffffu) | (BA_F32 << 24); }

// The description of the call's first kernel, marked as the two-kernel path.
void note_two_kernel() {
  char first[kLaunchDescBytes];
  snprintf(first, sizeof(first), "%s", t_launch_desc);
  note_launch("two-kernel: %s", first);
}

int gemm_2k_impl(const void* A, const void* B, const void* bias, const void* R, void* C, int64_t M,
                 int64_t N, int64_t K, uint32_t dtypes, int act, float alpha, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  GemmPlan p;
  int rc = plan_gemm(A, B, bias, C, M, N, K, dtypes, act, &p, R);
  if (rc || p.empty) return rc;
  if (p.dti == DT_I8) return kErrUnsupported;         // int8 runs the fused path only
  const uint64_t need = (uint64_t)M * (uint64_t)N * 4u;
  if (need >= (1ull << 31)) return kErrUnsupported;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 16) != 0) return kErrInvalid;
  // kernel 1: the contraction, fp32 pre-activation (A.B + bias) to the
  // workspace; its tile is planned for the buffer it writes (the output's and
  // the residual's alignment only concern kernel 2)
  GemmPlan p1;
  rc = plan_gemm(A, B, bias, workspace, M, N, K, with_f32_out(dtypes), BA_ACT_NONE, &p1);
  if (rc) return rc;
  rc = launch_gemm_plan(p1, A, B, bias, workspace, nullptr, DT_F32, BA_ACT_NONE, 0.0f, stream);
  if (rc) return rc;
  note_two_kernel();
  // kernel 2: residual, activation and cast
  return launch_second_kernel(p.dto, workspace, C, need / 4u, act, alpha, R, stream);
}

int conv_impl(const void* x, const void* w, const void* bias, const void* r, void* y, int64_t N,
              int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw,
              const int32_t strides[2], const int32_t pads[4], const int32_t dilations[2],
              uint32_t dtypes, int act, hipStream_t stream) {
  ConvPlan p;
  int rc = plan_conv(x, w, bias, y, N, C, H, W, Co, kh, kw, strides, pads, dilations, dtypes, act,
                     &p, r);
  if (rc || p.empty) return rc;
  return launch_conv_plan(p, x, w, bias, y, r, p.dto, act, stream);
}

int conv_2k_impl(const void* x, const void* w, const void* bias, const void* r, void* y, int64_t N,
                 int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw,
                 const int32_t strides[2], const int32_t pads[4], const int32_t dilations[2],
                 uint32_t dtypes, int act, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  ConvPlan p;
  int rc = plan_conv(x, w, bias, y, N, C, H, W, Co, kh, kw, strides, pads, dilations, dtypes, act,
                     &p, r);
  if (rc || p.empty) return rc;
  const uint64_t need = (uint64_t)p.N * p.Co * p.Ho * p.Wo * 4u;
  if (need >= (1ull << 31)) return kErrUnsupported;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 16) != 0) return kErrInvalid;
  rc = launch_conv_plan(p, x, w, bias, workspace, nullptr, DT_F32, BA_ACT_NONE, stream);
  if (rc) return rc;
  note_two_kernel();
  return launch_second_kernel(p.dto, workspace, y, need / 4u, act, 0.0f, r, stream);
}

// ---- the two-kernel GEMM without allocation -------------------------------
// Callers that cannot allocate (graph capture, serving loops) get the
// two-kernel path with its fp32 workspace in this fixed device array: 64 MiB,
// the workspace of a 4096 x 4096 output.  Each GPU the library runs on holds
// its own copy until the process ends; calls on one GPU share it.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

// Device address of `scratch` on each device, looked up once per device with
// that device current.  In host code `scratch` itself is only a host-side
// stand-in for the symbol: kernels get these addresses.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    t_last_hip = e;
    return kErrHip;
  }
  if (dev < 0 || dev >= kMaxDevices) return kErrUnsupported;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      t_last_hip = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return kErrHip;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return kOk;
}

// ---- fused-vs-two-kernel selection --------------------------------------
// Decisions recorded by the tuning calls, per problem (kind, sizes, types,
// activation); the auto entry points look them up.
std::mutex g_path_mu;
std::map<std::vector<int64_t>, int> g_paths;

std::vector<int64_t> gemm_key(int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act) {
  return {0, M, N, K, (int64_t)dtypes, act};
}

std::vector<int64_t> conv_key(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh,
                              int64_t kw, const int32_t* st, const int32_t* pd, const int32_t* dl,
                              uint32_t dtypes, int act) {
  return {1, N, C, H, W, Co, kh, kw, st[0], st[1], pd[0], pd[1], pd[2], pd[3], dl[0], dl[1],
          (int64_t)dtypes, act};
}

int lookup_path(const std::vector<int64_t>& key) {
  std::lock_guard<std::mutex> g(g_path_mu);
  auto it = g_paths.find(key);
  return it == g_paths.end() ? BA_PATH_FUSED : it->second;
}

void record_path(const std::vector<int64_t>& key, int path) {
  std::lock_guard<std::mutex> g(g_path_mu);
  if (path < 0) g_paths.erase(key);
  else g_paths[key] = path;
}

// The static choice for a GEMM nobody has tuned.  The fused kernel's
// epilogue must leave from the registers that hold the accumulators; the
// 256x256 ping-pong kernel's epilogue (whole 16-byte rows through LDS, or
// 4-wide stores) needs an output (and residual) aligned for 4-element
// accesses, and without it the fused call drops to a slower main loop.  The
// two-kernel path keeps the ping-pong main loop, writing its own aligned fp32
// workspace, and moves the misaligned accesses into the element-wise second
// kernel: chosen when that is the case and a large enough workspace is given.
int static_gemm_path(const void* A, const void* B, const void* bias, const void* C, int64_t M,
                     int64_t N, int64_t K, uint32_t dtypes, int act, const void* workspace,
                     size_t workspace_bytes) {
  GemmPlan pf, p1;
  if (plan_gemm(A, B, bias, C, M, N, K, dtypes, act, &pf) || pf.empty) return BA_PATH_FUSED;
  if (pf.tile == 6 || pf.dti == DT_I8) return BA_PATH_FUSED;
  if (!workspace || workspace_bytes < (uint64_t)M * (uint64_t)N * 4u ||
      ((uintptr_t)workspace % 16) != 0)
    return BA_PATH_FUSED;
  if (plan_gemm(A, B, bias, workspace, M, N, K, with_f32_out(dtypes), BA_ACT_NONE, &p1))
    return BA_PATH_FUSED;
  return p1.tile == 6 ? BA_PATH_TWO_KERNEL : BA_PATH_FUSED;
}

// The recorded path, or -1.
int recorded_path(const std::vector<int64_t>& key) {
  std::lock_guard<std::mutex> g(g_path_mu);
  auto it = g_paths.find(key);
  return it == g_paths.end() ? -1 : it->second;
}

// Mean milliseconds per call of `run` over `reps` calls on `stream`, after
// one untimed call; negative status on a launch or runtime error.
template <class F>
int time_calls(F&& run, int reps, hipStream_t stream, float* ms) {
  int rc = run();
  if (rc) return rc;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return kErrHip;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return kErrHip;
  }
  rc = hipEventRecord(e0, stream) == hipSuccess ? kOk : kErrHip;
  for (int i = 0; i < reps && rc == kOk; ++i) rc = run();
  if (rc == kOk && hipEventRecord(e1, stream) != hipSuccess) rc = kErrHip;
  if (rc == kOk && hipEventSynchronize(e1) != hipSuccess) rc = kErrHip;
  float t = 0.0f;
  if (rc == kOk && hipEventElapsedTime(&t, e0, e1) != hipSuccess) rc = kErrHip;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  *ms = t / (float)reps;
  return rc;
}

// Times the fused call and, where it runs, the two-kernel call; records and
// returns the faster path (or a negative-free error status through *path).
template <class FF, class FT>
int tune_paths(FF&& fused, FT&& two, bool two_ok, int reps, hipStream_t stream,
               const std::vector<int64_t>& key, int* path) {
  if (reps < 1) return kErrInvalid;
  float t_fused = 0.0f, t_two = 0.0f;
  int rc = time_calls(fused, reps, stream, &t_fused);
  if (rc) return rc;
  int best = BA_PATH_FUSED;
  if (two_ok) {
    rc = time_calls(two, reps, stream, &t_two);
    if (rc) return rc;
    if (t_two < t_fused) best = BA_PATH_TWO_KERNEL;
  }
  record_path(key, best);
  *path = best;
  return kOk;
}

}  // namespace

extern "C" {

int gemm_bias_act(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N,
                  int64_t K, uint32_t dtypes, int act, float alpha, hipStream_t stream) {
  return gemm_impl(A, B, bias, nullptr, C, M, N, K, dtypes, act, alpha, stream);
}

size_t gemm_bias_act_workspace_size(int64_t M, int64_t N) {
  if (M < 0 || N < 0) return 0;
  return (size_t)M * (size_t)N * 4u;
}

int gemm_bias_act_2k(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N,
                     int64_t K, uint32_t dtypes, int act, float alpha, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  return gemm_2k_impl(A, B, bias, nullptr, C, M, N, K, dtypes, act, alpha, workspace,
                      workspace_bytes, stream);
}

int gemm_bias_act_2k_noalloc(const void* A, const void* B, const void* bias, void* C, int64_t M,
                             int64_t N, int64_t K, uint32_t dtypes, int act, float alpha,
                             hipStream_t stream) {
  // every check that needs no HIP call comes first
  GemmPlan p;
  int rc = plan_gemm(A, B, bias, C, M, N, K, dtypes, act, &p);
  if (rc || p.empty) return rc;
  if (p.dti == DT_I8) return kErrUnsupported;
  if ((uint64_t)M * (uint64_t)N * 4u > kScratchBytes) return kErrUnsupported;
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc) return rc;
  // kernel 1 writes every workspace element kernel 2 reads, in stream order:
  // nothing needs clearing
  return gemm_2k_impl(A, B, bias, nullptr, C, M, N, K, dtypes, act, alpha, ws, kScratchBytes,
                      stream);
}

int gemm_bias_add_act(const void* A, const void* B, const void* bias, const void* R, void* C,
                      int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act, float alpha,
                      hipStream_t stream) {
  if (!R && M > 0 && N > 0) return kErrInvalid;
  return gemm_impl(A, B, bias, R, C, M, N, K, dtypes, act, alpha, stream);
}

int gemm_bias_add_act_2k(const void* A, const void* B, const void* bias, const void* R, void* C,
                         int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act, float alpha,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!R && M > 0 && N > 0) return kErrInvalid;
  return gemm_2k_impl(A, B, bias, R, C, M, N, K, dtypes, act, alpha, workspace, workspace_bytes,
                      stream);
}

int conv2d_bias_act(const void* x, const void* w, const void* bias, void* y, int64_t N, int64_t C,
                    int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw,
                    const int32_t strides[2], const int32_t pads[4], const int32_t dilations[2],
                    uint32_t dtypes, int act, hipStream_t stream) {
  return conv_impl(x, w, bias, nullptr, y, N, C, H, W, Co, kh, kw, strides, pads, dilations,
                   dtypes, act, stream);
}

size_t conv2d_bias_act_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co,
                                      int64_t kh, int64_t kw, const int32_t strides[2],
                                      const int32_t pads[4], const int32_t dilations[2]) {
  ConvPlan p;
  // geometry only: any valid element types and non-null placeholders
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  if (plan_conv(dummy, dummy, nullptr, dummy, N, C, H, W, Co, kh, kw, strides, pads, dilations,
                BA_DTYPES(BA_F32, BA_F32, BA_F32, BA_F32), BA_ACT_NONE, &p))
    return 0;
  return (size_t)p.N * p.Co * p.Ho * p.Wo * 4u;
}

int conv2d_bias_act_2k(const void* x, const void* w, const void* bias, void* y, int64_t N,
                       int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw,
                       const int32_t strides[2], const int32_t pads[4],
                       const int32_t dilations[2], uint32_t dtypes, int act, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return conv_2k_impl(x, w, bias, nullptr, y, N, C, H, W, Co, kh, kw, strides, pads, dilations,
                      dtypes, act, workspace, workspace_bytes, stream);
}

int conv2d_bias_add_act(const void* x, const void* w, const void* bias, const void* r, void* y,
                        int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh,
                        int64_t kw, const int32_t strides[2], const int32_t pads[4],
                        const int32_t dilations[2], uint32_t dtypes, int act, hipStream_t stream) {
  if (!r && N > 0) return kErrInvalid;
  return conv_impl(x, w, bias, r, y, N, C, H, W, Co, kh, kw, strides, pads, dilations, dtypes,
                   act, stream);
}

int conv2d_bias_add_act_2k(const void* x, const void* w, const void* bias, const void* r, void* y,
                           int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh,
                           int64_t kw, const int32_t strides[2], const int32_t pads[4],
                           const int32_t dilations[2], uint32_t dtypes, int act, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!r && N > 0) return kErrInvalid;
  return conv_2k_impl(x, w, bias, r, y, N, C, H, W, Co, kh, kw, strides, pads, dilations, dtypes,
                      act, workspace, workspace_bytes, stream);
}

int biasact_gemm_path(int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act) {
  return lookup_path(gemm_key(M, N, K, dtypes, act));
}

int biasact_conv_path(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh,
                      int64_t kw, const int32_t strides[2], const int32_t pads[4],
                      const int32_t dilations[2], uint32_t dtypes, int act) {
  if (!strides || !pads || !dilations) return -kErrInvalid;
  return lookup_path(conv_key(N, C, H, W, Co, kh, kw, strides, pads, dilations, dtypes, act));
}

int biasact_set_gemm_path(int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act, int path) {
  if (path < -1 || path > BA_PATH_TWO_KERNEL) return kErrInvalid;
  record_path(gemm_key(M, N, K, dtypes, act), path);
  return kOk;
}

int biasact_set_conv_path(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh,
                          int64_t kw, const int32_t strides[2], const int32_t pads[4],
                          const int32_t dilations[2], uint32_t dtypes, int act, int path) {
  if (!strides || !pads || !dilations) return kErrInvalid;
  if (path < -1 || path > BA_PATH_TWO_KERNEL) return kErrInvalid;
  record_path(conv_key(N, C, H, W, Co, kh, kw, strides, pads, dilations, dtypes, act), path);
  return kOk;
}

int biasact_gemm_static_path(const void* A, const void* B, const void* bias, const void* C,
                             int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act,
                             const void* workspace, size_t workspace_bytes) {
  return static_gemm_path(A, B, bias, C, M, N, K, dtypes, act, workspace, workspace_bytes);
}

int conv2d_bias_act_out_dims(int64_t H, int64_t W, int64_t kh, int64_t kw, const int32_t strides[2],
                             const int32_t pads[4], const int32_t dilations[2], int64_t* Ho,
                             int64_t* Wo) {
  return conv_out_dims(H, W, kh, kw, strides, pads, dilations, Ho, Wo);
}

int biasact_tune_gemm(const void* A, const void* B, const void* bias, void* C, int64_t M,
                      int64_t N, int64_t K, uint32_t dtypes, int act, float alpha, void* workspace,
                      size_t workspace_bytes, int reps, hipStream_t stream, int* path) {
  if (!path) return kErrInvalid;
  GemmPlan p;
  int rc = plan_gemm(A, B, bias, C, M, N, K, dtypes, act, &p);
  if (rc) return rc;
  const bool two_ok = p.dti != DT_I8 && workspace &&
                      workspace_bytes >= (uint64_t)M * (uint64_t)N * 4u;
  return tune_paths(
      [&]() { return gemm_impl(A, B, bias, nullptr, C, M, N, K, dtypes, act, alpha, stream); },
      [&]() {
        return gemm_2k_impl(A, B, bias, nullptr, C, M, N, K, dtypes, act, alpha, workspace,
                            workspace_bytes, stream);
      },
      two_ok, reps, stream, gemm_key(M, N, K, dtypes, act), path);
}

int biasact_tune_conv(const void* x, const void* w, const void* bias, void* y, int64_t N,
                      int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw,
                      const int32_t strides[2], const int32_t pads[4], const int32_t dilations[2],
                      uint32_t dtypes, int act, void* workspace, size_t workspace_bytes, int reps,
                      hipStream_t stream, int* path) {
  if (!path) return kErrInvalid;
  ConvPlan p;
  int rc = plan_conv(x, w, bias, y, N, C, H, W, Co, kh, kw, strides, pads, dilations, dtypes, act,
                     &p);
  if (rc) return rc;
  const bool two_ok = workspace && workspace_bytes >= (uint64_t)p.N * p.Co * p.Ho * p.Wo * 4u;
  return tune_paths(
      [&]() {
        return conv_impl(x, w, bias, nullptr, y, N, C, H, W, Co, kh, kw, strides, pads, dilations,
                         dtypes, act, stream);
      },
      [&]() {
        return conv_2k_impl(x, w, bias, nullptr, y, N, C, H, W, Co, kh, kw, strides, pads,
                            dilations, dtypes, act, workspace, workspace_bytes, stream);
      },
      two_ok, reps, stream, conv_key(N, C, H, W, Co, kh, kw, strides, pads, dilations, dtypes, act),
      path);
}

int gemm_bias_act_auto(const void* A, const void* B, const void* bias, void* C, int64_t M,
                       int64_t N, int64_t K, uint32_t dtypes, int act, float alpha, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  int path = recorded_path(gemm_key(M, N, K, dtypes, act));
  if (path < 0)
    path = static_gemm_path(A, B, bias, C, M, N, K, dtypes, act, workspace, workspace_bytes);
  if (path == BA_PATH_TWO_KERNEL && workspace && workspace_bytes >= (uint64_t)M * N * 4u)
    return gemm_2k_impl(A, B, bias, nullptr, C, M, N, K, dtypes, act, alpha, workspace,
                        workspace_bytes, stream);
  return gemm_impl(A, B, bias, nullptr, C, M, N, K, dtypes, act, alpha, stream);
}

int conv2d_bias_act_auto(const void* x, const void* w, const void* bias, void* y, int64_t N,
                         int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw,
                         const int32_t strides[2], const int32_t pads[4],
                         const int32_t dilations[2], uint32_t dtypes, int act, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!strides || !pads || !dilations) return kErrInvalid;
  const int path =
      lookup_path(conv_key(N, C, H, W, Co, kh, kw, strides, pads, dilations, dtypes, act));
  if (path == BA_PATH_TWO_KERNEL && workspace &&
      workspace_bytes >= conv2d_bias_act_workspace_size(N, C, H, W, Co, kh, kw, strides, pads,
                                                        dilations))
    return conv_2k_impl(x, w, bias, nullptr, y, N, C, H, W, Co, kh, kw, strides, pads, dilations,
                        dtypes, act, workspace, workspace_bytes, stream);
  return conv_impl(x, w, bias, nullptr, y, N, C, H, W, Co, kh, kw, strides, pads, dilations,
                   dtypes, act, stream);
}

const char* biasact_status_string(int status) { return status_string(status); }

int biasact_last_tile_config(char* buf, size_t n) {
  if (!buf || n == 0) return kErrInvalid;
  snprintf(buf, n, "%s", t_launch_desc);
  return kOk;
}

int biasact_last_hip_error(void) { return (int)t_last_hip; }

const char* biasact_last_hip_error_string(void) {
  return t_last_hip == hipSuccess ? "no HIP error" : hipGetErrorString(t_last_hip);
}

int biasact_num_tile_configs(void) { return kNumTileConfigs; }

int biasact_tile_config_name(int id, char* buf, size_t n) {
  if (id < 0 || id >= kNumTileConfigs || !buf || n == 0) return kErrInvalid;
  const TileShapeDesc& t = kTiles[id];
  const char* kind = id == 6 ? " ping-pong" : (id == 7 ? " conv-halo" : "");
  snprintf(buf, n, "%dx%d/%dx%d%s", t.bm, t.bn, t.waves_m, t.waves_n, kind);
  return kOk;
}

int biasact_gemm_tile_config(int64_t M, int64_t N, int64_t K, uint32_t dtypes) {
  // the choice gemm_bias_act makes for 16-byte aligned operands
  GemmPlan p;
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  if (plan_gemm(dummy, dummy, nullptr, dummy, M, N, K, dtypes, BA_ACT_NONE, &p)) return -1;
  return p.tile;
}

int biasact_conv_tile_config(int64_t N, int64_t Co, int64_t Ho, int64_t Wo, int64_t K_total,
                             uint32_t dtypes) {
  int f = forced_tile();
  if (f < 0) f = select_conv_tile(N, Co, Ho, Wo, K_total, (int)(dtypes & 0xffu));
  return f == 6 ? 0 : f;   // the halo tile (7) depends on the filter and alignment: see conv2d_bias_act
}

int biasact_force_tile_config(int id) {
  if (id < -1 || id >= kNumTileConfigs) return kErrInvalid;
  set_forced_tile(id);
  return kOk;
}

int biasact_force_halo_variant(int v) {
  if (v < -1 || v > 4) return kErrInvalid;
  set_forced_halo_variant(v);
  return kOk;
}

}  // extern "C"
