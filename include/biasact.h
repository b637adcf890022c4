/*
 * biasact.h — C ABI of the MI355X (gfx950) fused contraction + bias +
 * activation library (libbiasact.so).
 *
 * Computes, in one kernel and one store per output element,
 *     C = act(A . B + bias)                       (GEMM)
 *     y = act(conv2d(x, w) + bias)                (conv2d as an implicit GEMM)
 * with act in {identity, ReLU, LeakyReLU(alpha), tanh, GELU, Sigmoid}.  Sources
 * (web pages, cited by title and section):
 *   - "CANN pyasc MatmulLeakyRelu 融合算子实战" (lshu.cn/news/76032): section
 *     概述 (C = A x B + Bias, then LeakyReLU: non-negative values unchanged,
 *     negative values times alpha), section 样例规格 (operand shapes and types:
 *     fp16 A/B, fp32 bias [1,N], fp32 alpha, fp32 C), section 补充说明 (bias
 *     may be fp16 or fp32 for fp16 operands).
 *   - ops-nn fused_matmul_relu article (mlqm.cn/news/1824): sections
 *     "fused_matmul_relu底层到底做了什么" (fused matmul + ReLU on caller-owned
 *     device buffers, one HBM read of the operands and one write of C; the
 *     two-step matmul-then-activation fallback through a device temporary).
 *     Section ops-nn的融合算子分类与适用场景: the matmul + activation class
 *     covers ReLU, GELU, Sigmoid and tanh, all element-wise.
 *   - multimodal-ops "Fused ConvTanh" article (wmrh.cn/news/81139): sections
 *     这个算子到底在算什么 (y = tanh(conv2d(x, filter, bias)) with strides,
 *     pads and dilations), 双 Kernel 是怎么分工的 (implicit GEMM with the
 *     weights as the co x k operand; bias as one extra k column; the two-kernel
 *     split through an fp32 workspace), 快速上手 (the Python entry point
 *     fused_conv_tanh(x, conv_filter, bias, strides, pads, dilations)).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees, or synchronises.  Work is enqueued on `stream`
 *     (0 = the null stream) and runs asynchronously; the call returns once the
 *     kernels are queued.
 *   - Tensors are packed and contiguous: A[M,K], B[K,N], C[M,N] row-major;
 *     x[N,C,H,W], w[Co,C,kh,kw], y[N,Co,Ho,Wo] (NCHW / OIHW); bias is a vector
 *     of N (GEMM) or Co (conv) elements added to every row / every spatial
 *     position.  bias == NULL means no bias.
 *   - Every tensor must be smaller than 2^31 bytes.
 *   - Accumulation is fp32.  The bias is the first term of the sum (the
 *     contribution of an extra k column of bias against a row of ones), the
 *     activation runs in fp32, and the result is rounded once to the output
 *     type (round to nearest, ties to even).
 *   - Return value: BA_OK, or an error code below; nothing is launched when an
 *     error is returned.  No exception crosses the ABI.
 */
#ifndef BIASACT_H
#define BIASACT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type codes (storage size: 4, 2, 2, 1, 4 bytes) */
#define BA_F32 0u
#define BA_F16 1u
#define BA_BF16 2u
#define BA_I8 3u            /* two's complement int8: GEMM operands only */
#define BA_I32 4u           /* two's complement int32: bias / output of int8 GEMMs */

/* dtypes argument: one 8-bit code per operand.
 *   a   : A (GEMM) or x (conv)
 *   b   : B (GEMM) or w (conv)      — must equal a
 *   bias: bias element type         — fp32, or the same type as a (ignored when bias == NULL)
 *   out : C (GEMM) or y (conv)      — fp32, fp16 or bf16
 * int8 GEMMs ("CANN pyasc MatmulLeakyRelu 融合算子实战", section 补充说明: with
 * int8 A and B the bias must be int32): a = b = BA_I8, bias BA_I32, out BA_I32
 * or a floating-point type.  The sum A.B + bias is exact in int32 (K is
 * limited to 131071 so that the product sum alone fits; the bias must keep
 * the total in range, else it wraps); an int32 output takes act NONE or RELU
 * only, a floating-point output the integer rounded to fp32 and then any
 * activation.  gemm_bias_act only: the conv, two-kernel and residual entry
 * points return BA_ERR_UNSUPPORTED for int8. */
#define BA_DTYPES(a, b, bias, out) \
  ((uint32_t)(a) | ((uint32_t)(b) << 8) | ((uint32_t)(bias) << 16) | ((uint32_t)(out) << 24))

/* activation codes */
#define BA_ACT_NONE 0
#define BA_ACT_RELU 1       /* z > 0 ? z : +0 */
#define BA_ACT_LEAKY_RELU 2 /* z >= 0 ? z : alpha * z */
#define BA_ACT_TANH 3       /* tanh(z) */
#define BA_ACT_GELU 4       /* z * Phi(z), Phi the standard normal CDF (exact erf form) */
#define BA_ACT_SIGMOID 5    /* 1 / (1 + e^-z) */

/* status codes */
#define BA_OK 0
#define BA_ERR_INVALID 1     /* null pointer, negative dimension, bad act, stride/dilation < 1,
                                pad < 0, empty conv output, workspace too small */
#define BA_ERR_UNSUPPORTED 2 /* dtype combination, act for this op, tensor >= 2^31 bytes */
#define BA_ERR_HIP 3         /* the HIP runtime refused the launch */

/* C[M,N] = act(A[M,K] . B[K,N] + bias[N]).
 * M, N, K >= 0 (M or N == 0: nothing to do; K == 0: C = act(bias)).
 * alpha is read only for BA_ACT_LEAKY_RELU (fp32, as in the MatmulLeakyRelu
 * spec).  Fast path: K and N multiples of 8 (fp16/bf16) or 4 (fp32) and
 * 16-byte aligned pointers; other shapes are correct but slower. */
int gemm_bias_act(const void* A, const void* B, const void* bias, void* C,
                  int64_t M, int64_t N, int64_t K, uint32_t dtypes,
                  int act, float alpha, hipStream_t stream);

/* y = act(conv2d(x, w) + bias): cross-correlation, zero padding, groups = 1.
 * strides = {sh, sw} >= 1, pads = {top, bottom, left, right} >= 0,
 * dilations = {dh, dw} >= 1, all HOST pointers to int32.
 *   Ho = floor((H + top + bottom - dh*(kh-1) - 1) / sh) + 1, likewise Wo;
 * both must be >= 1.  N >= 0 (N == 0: nothing to do).  This entry point has
 * no alpha, so BA_ACT_LEAKY_RELU returns BA_ERR_UNSUPPORTED. */
int conv2d_bias_act(const void* x, const void* w, const void* bias, void* y,
                    int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co,
                    int64_t kh, int64_t kw, const int32_t strides[2],
                    const int32_t pads[4], const int32_t dilations[2],
                    uint32_t dtypes, int act, hipStream_t stream);

/* Output size of conv2d_bias_act for an H x W input and a kh x kw filter
 * (the output-size formula of "PyAsc與Ascend-C算子開發實戰", section 3.1,
 * with dilation): Ho = floor((H + top + bottom - dh*(kh-1) - 1) / sh) + 1,
 * likewise Wo.  strides, pads, dilations as for conv2d_bias_act (HOST int32
 * pointers); *Ho and *Wo are host pointers written on success.  Returns
 * BA_ERR_INVALID for null pointers, H, W, kh or kw < 1, a stride or dilation
 * < 1, a pad < 0 or an empty output; BA_ERR_UNSUPPORTED for a dimension of
 * 2^31 or more. */
int conv2d_bias_act_out_dims(int64_t H, int64_t W, int64_t kh, int64_t kw,
                             const int32_t strides[2], const int32_t pads[4],
                             const int32_t dilations[2], int64_t* Ho, int64_t* Wo);

/* Two-kernel variants (the ablation of the fused path): kernel 1 runs the
 * contraction and stores the fp32 pre-activation (A.B + bias, or conv + bias)
 * to `workspace` ([M,N], or NCHW for conv); kernel 2 reads it back and applies
 * the residual (if any), the activation and the output cast.  Kernel 1's tile
 * is planned for the workspace it writes, so a GEMM whose output or residual
 * is not aligned for 4-element accesses still runs the 256x256 ping-pong main
 * loop here.  With the same main loop (aligned outputs) the results are
 * bitwise identical to the fused entry points; across main loops each result
 * is still one rounding of an fp32 sum in ascending k.  `workspace` is a
 * caller-owned, 16-byte aligned device buffer of at least *_workspace_size()
 * bytes (BA_ERR_INVALID otherwise). */
size_t gemm_bias_act_workspace_size(int64_t M, int64_t N);
int gemm_bias_act_2k(const void* A, const void* B, const void* bias, void* C,
                     int64_t M, int64_t N, int64_t K, uint32_t dtypes,
                     int act, float alpha, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* gemm_bias_act_2k without a caller workspace and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The fp32
 * workspace is a fixed 64 MiB device array inside the library, one per GPU,
 * held from the library's first use of that GPU until the process ends; the
 * calling thread's current device must be the stream's device.  Limit:
 * M * N * 4 <= 64 MiB (e.g. a 4096 x 4096 output), else BA_ERR_UNSUPPORTED
 * with nothing launched; int8 operands: BA_ERR_UNSUPPORTED.  Kernel 1 writes
 * every workspace element that kernel 2 reads, so nothing needs clearing.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other threads) race and give undefined results;
 * serialise them on one stream.  Results are bitwise those of
 * gemm_bias_act_2k with a 16-byte aligned workspace.  Other arguments, checks
 * and return codes as gemm_bias_act. */
int gemm_bias_act_2k_noalloc(const void* A, const void* B, const void* bias, void* C,
                             int64_t M, int64_t N, int64_t K, uint32_t dtypes,
                             int act, float alpha, hipStream_t stream);

size_t conv2d_bias_act_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co,
                                      int64_t kh, int64_t kw, const int32_t strides[2],
                                      const int32_t pads[4], const int32_t dilations[2]);
int conv2d_bias_act_2k(const void* x, const void* w, const void* bias, void* y,
                       int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co,
                       int64_t kh, int64_t kw, const int32_t strides[2],
                       const int32_t pads[4], const int32_t dilations[2],
                       uint32_t dtypes, int act, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Residual epilogue: the same contraction with an extra input R of the
 * output's type and shape (C's [M,N] row-major, or y's [N,Co,Ho,Wo]) joining
 * the sum before the activation:
 *     C = act(A . B + bias + R)        y = act(conv2d(x, w) + bias + R)
 * the "matmul + add + bias" fusion of residual networks in the ops-nn article
 * (mlqm.cn/news/1824), section ops-nn的融合算子分类与适用场景 (math class).
 * R is a device pointer owned by the caller, read once per output element;
 * it may be the output buffer itself (in place: each element is read before
 * it is written, by the same thread), but must not overlap it otherwise.
 * R == NULL with a non-empty output returns BA_ERR_INVALID.  The other
 * arguments, limits and return codes are those of the entry points above;
 * the _2k variants add R in their second kernel and match the fused results
 * bit for bit. */
int gemm_bias_add_act(const void* A, const void* B, const void* bias, const void* R, void* C,
                      int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act, float alpha,
                      hipStream_t stream);
int gemm_bias_add_act_2k(const void* A, const void* B, const void* bias, const void* R, void* C,
                         int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act, float alpha,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);
int conv2d_bias_add_act(const void* x, const void* w, const void* bias, const void* R, void* y,
                        int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh,
                        int64_t kw, const int32_t strides[2], const int32_t pads[4],
                        const int32_t dilations[2], uint32_t dtypes, int act, hipStream_t stream);
int conv2d_bias_add_act_2k(const void* x, const void* w, const void* bias, const void* R, void* y,
                           int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh,
                           int64_t kw, const int32_t strides[2], const int32_t pads[4],
                           const int32_t dilations[2], uint32_t dtypes, int act, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Fused or two-kernel path, chosen per problem.  The pages decide at run
 * time whether to fuse: ops-nn (mlqm.cn/news/1824, sections
 * "fused_matmul_relu底层到底做了什么" and 融合不是万能的) checks that the
 * tiles and the activation's buffer fit the on-chip budget and otherwise runs
 * the two steps; the Fused ConvTanh article (wmrh.cn/news/81139, section
 * 核心问题) measures first.  Here the fused epilogue needs no on-chip space
 * beyond the accumulators, but the 256x256 ping-pong GEMM's epilogue needs
 * an output (and residual) aligned for 4-element accesses.  The static rule
 * for a problem nobody tuned: the two-kernel path when the fused call would
 * lose the ping-pong main loop to the output's alignment while kernel 1,
 * writing the aligned workspace, keeps it (and a workspace is given);
 * otherwise fused.  Convs are always fused statically.  biasact_tune_*
 * measure both paths on the caller's buffers and record the faster for that
 * problem (sizes, attributes, dtypes, act); biasact_set_*_path record a
 * choice directly (e.g. from an earlier tuning run; -1 forgets it); the
 * *_auto entry points follow the record, else the static rule.
 *   biasact_gemm_path / biasact_conv_path: the recorded path, else
 *     BA_PATH_FUSED (the static choice for aligned buffers); negative
 *     -BA_ERR_INVALID for null attribute arrays.
 *   biasact_gemm_static_path: the static rule for these buffers (no launch;
 *     BA_PATH_FUSED for invalid arguments).
 *   biasact_set_gemm_path / biasact_set_conv_path: record `path`
 *     (BA_PATH_FUSED, BA_PATH_TWO_KERNEL, or -1 to forget); BA_ERR_INVALID for
 *     another value or null attribute arrays.
 *   biasact_tune_gemm / biasact_tune_conv: run the fused call once plus
 *     `reps` timed calls, then the two-kernel call likewise (only with a
 *     workspace of *_workspace_size bytes, and never for int8), SYNCHRONISING
 *     `stream` (the only library calls that do); the output buffer is
 *     overwritten; the chosen path goes to *path.  Returns a status code.
 *     The record is process-wide and guarded by a lock.
 *   gemm_bias_act_auto / conv2d_bias_act_auto: the recorded path, else the
 *     static rule; the two-kernel path only when its workspace is given and
 *     large enough, else the fused path. */
#define BA_PATH_FUSED 0
#define BA_PATH_TWO_KERNEL 1
int biasact_gemm_path(int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act);
int biasact_conv_path(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh,
                      int64_t kw, const int32_t strides[2], const int32_t pads[4],
                      const int32_t dilations[2], uint32_t dtypes, int act);
int biasact_gemm_static_path(const void* A, const void* B, const void* bias, const void* C,
                             int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act,
                             const void* workspace, size_t workspace_bytes);
int biasact_set_gemm_path(int64_t M, int64_t N, int64_t K, uint32_t dtypes, int act, int path);
int biasact_set_conv_path(int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh,
                          int64_t kw, const int32_t strides[2], const int32_t pads[4],
                          const int32_t dilations[2], uint32_t dtypes, int act, int path);
int biasact_tune_gemm(const void* A, const void* B, const void* bias, void* C, int64_t M,
                      int64_t N, int64_t K, uint32_t dtypes, int act, float alpha, void* workspace,
                      size_t workspace_bytes, int reps, hipStream_t stream, int* path);
int biasact_tune_conv(const void* x, const void* w, const void* bias, void* y, int64_t N,
                      int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw,
                      const int32_t strides[2], const int32_t pads[4], const int32_t dilations[2],
                      uint32_t dtypes, int act, void* workspace, size_t workspace_bytes, int reps,
                      hipStream_t stream, int* path);
int gemm_bias_act_auto(const void* A, const void* B, const void* bias, void* C, int64_t M,
                       int64_t N, int64_t K, uint32_t dtypes, int act, float alpha, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);
int conv2d_bias_act_auto(const void* x, const void* w, const void* bias, void* y, int64_t N,
                         int64_t C, int64_t H, int64_t W, int64_t Co, int64_t kh, int64_t kw,
                         const int32_t strides[2], const int32_t pads[4],
                         const int32_t dilations[2], uint32_t dtypes, int act, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Introspection and tuning. */
const char* biasact_status_string(int status);  /* static string, never NULL */
/* The hipError_t behind the most recent BA_ERR_HIP returned on the calling
 * thread (hipSuccess = 0 if there was none), and its hipGetErrorString text
 * (static, never NULL).  Other calls leave it unchanged. */
int biasact_last_hip_error(void);
const char* biasact_last_hip_error_string(void);
int biasact_num_tile_configs(void);
/* Describe tile config `id` ("BMxBN/waves_mxwaves_n") into buf (NUL-terminated,
 * truncated to n bytes); BA_ERR_INVALID for an unknown id. */
int biasact_tile_config_name(int id, char* buf, size_t n);
/* Describes into buf (NUL-terminated, truncated to n bytes) the main kernel
 * that the calling thread queued last (the most recent entry-point call that
 * launched anything):
 * its kind and tile, e.g. "gemm 64x64/2x2 all-k", "gemm 256x256/2x4
 * ping-pong", "conv-halo 9 taps, 64 co x 8x56 positions, 2 chunk sets";
 * "none" before the first launch.  A two-kernel call (*_2k, or *_auto taking
 * that path) reports "two-kernel: " followed by its first kernel.
 * BA_ERR_INVALID for a null buf or n == 0. */
int biasact_last_tile_config(char* buf, size_t n);
/* Tile config the library picks for a GEMM / conv problem (no launch). */
int biasact_gemm_tile_config(int64_t M, int64_t N, int64_t K, uint32_t dtypes);
int biasact_conv_tile_config(int64_t N, int64_t Co, int64_t Ho, int64_t Wo, int64_t K_total,
                             uint32_t dtypes);
/* Process-wide override of the tile choice for tuning (-1 restores the
 * automatic choice).  Not synchronised: set it before launching from other
 * threads.  Returns BA_ERR_INVALID for an unknown id. */
int biasact_force_tile_config(int id);
/* Process-wide override of the fp16/bf16 conv-halo variant, for tests and
 * tuning: -1 automatic; 0 the widest tile, one four-wave workgroup per CU;
 * 1 64 output channels x 128 positions and 2 64 output channels x 64
 * positions, both small enough for two four-wave workgroups per CU; 3 and 4
 * 64 output channels x 128 and x 256 positions in one eight-wave workgroup
 * per CU (chunks of 32 channels only).  A variant that does not apply to a
 * problem falls back to the widest tile.  Not synchronised, like the tile
 * override.  Returns BA_ERR_INVALID outside -1..4. */
int biasact_force_halo_variant(int v);

#ifdef __cplusplus
}
#endif
#endif /* BIASACT_H */
