/*
 * oracle.h — plain, slow, fp64 CPU reference for the fused
 * contraction + bias + activation, and for conv2d + bias + activation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * includes, links or calls anything here, and this file includes nothing
 * from it.
 *
 * Sources (web pages; cited by title and section):
 *   [MLR]  "CANN pyasc MatmulLeakyRelu 融合算子实战" (lshu.cn/news/76032)
 *   [PYA]  "PyAsc與Ascend-C算子開發實戰" (jh158.com/news/60091)
 *   [FMR]  ops-nn fused_matmul_relu article, "前言 …" (mlqm.cn/news/1824)
 *   [FCT]  multimodal-ops "Fused ConvTanh" article (wmrh.cn/news/81139)
 *
 * Every floating-point input is first decoded exactly to double (fp16,
 * bf16 and fp32 values are all representable in binary64), and every sum is
 * formed in double in ascending reduction-index order.
 */
#ifndef BIASACT_ORACLE_H
#define BIASACT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element-type codes of the encoded inputs. */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_I8 = 3, ORC_I32 = 4 };

/* Activation codes. */
enum { ORC_ACT_NONE = 0, ORC_ACT_RELU = 1, ORC_ACT_LEAKY = 2, ORC_ACT_TANH = 3,
       ORC_ACT_GELU = 4, ORC_ACT_SIGMOID = 5 };

/* Exact decoders, written from the IEEE-754 binary16 / binary32 layouts and
 * from bfloat16 = the upper half of a binary32; int8 and int32 are two's
 * complement integers (int8 operands with an int32 bias: "CANN pyasc
 * MatmulLeakyRelu 融合算子实战", section 补充说明).  n elements, src packed. */
double orc_f16_to_f64(uint16_t h);
double orc_bf16_to_f64(uint16_t h);
double orc_f32_to_f64(uint32_t u);
int orc_decode(int dtype, const void *src, int64_t n, double *dst);

/* Residual epilogue: y[i] = act(z[i] + r[i]) for a pre-activation z taken
 * from the GEMM / conv functions with act = NONE (the contraction plus bias)
 * and a residual r of the output's shape: the "matmul + add + bias" fusion
 * of the math class in the ops-nn article (section
 * ops-nn的融合算子分类与适用场景, residual networks). */
int orc_residual_act(const double *z, const double *r, double *y, int64_t n, int act,
                     double alpha);

/* Activation applied to one pre-activation value z (in double). */
double orc_act(int act, double z, double alpha);
void orc_act_array(int act, double alpha, const double *z, double *y, int64_t n);

/* C[M,N] = act(A[M,K] . B[K,N] + bias[N]); all row-major, bias may be NULL.
 * [MLR] 概述 (the MatmulLeakyRelu formula) and 样例规格 (bias is a [1,N]
 * row); [FMR] "fused_matmul_relu底层到底做了什么" (the host loop form). */
int orc_gemm_bias_act(const double *A, const double *B, const double *bias,
                      double *C, int64_t M, int64_t N, int64_t K,
                      int act, double alpha);

/* Only the listed output elements C[ii[t], jj[t]], t < n, same definition. */
int orc_gemm_bias_act_elems(const double *A, const double *B, const double *bias,
                            int64_t M, int64_t N, int64_t K,
                            const int64_t *ii, const int64_t *jj, int64_t n,
                            int act, double alpha, double *out);

/* Bias folded into the contraction as one extra reduction index:
 * A' = [A | 1] (K+1 columns), B' = [B ; bias] (K+1 rows), no separate add.
 * [FCT] "双 Kernel 是怎么分工的" (weight gains a bias column, input an
 * all-ones row). */
int orc_gemm_bias_fold(const double *A, const double *B, const double *bias,
                       double *C, int64_t M, int64_t N, int64_t K,
                       int act, double alpha);

/* Output size of one spatial axis of conv2d with zero padding:
 * floor((in + pad_lo + pad_hi - dil*(k-1) - 1) / stride) + 1, or <= 0. */
int64_t orc_conv_out_dim(int64_t in, int64_t k, int64_t stride,
                         int64_t pad_lo, int64_t pad_hi, int64_t dil);

/* y[N,Co,Ho,Wo] = act(conv2d(x[N,C,H,W], w[Co,C,kh,kw]) + bias[Co]),
 * cross-correlation, zero padding, groups = 1.  strides = {sh, sw},
 * pads = {top, bottom, left, right}, dils = {dh, dw}.  [FCT] "这个算子到底
 * 在算什么"; [PYA] 3.1 (output-size formula). */
int orc_conv2d_bias_act(const double *x, const double *w, const double *bias,
                        double *y, int64_t N, int64_t C, int64_t H, int64_t W,
                        int64_t Co, int64_t kh, int64_t kw,
                        const int64_t strides[2], const int64_t pads[4],
                        const int64_t dils[2], int act, double alpha);

/* Only the listed flat output indices of y (NCHW), same definition. */
int orc_conv2d_bias_act_elems(const double *x, const double *w, const double *bias,
                              int64_t N, int64_t C, int64_t H, int64_t W,
                              int64_t Co, int64_t kh, int64_t kw,
                              const int64_t strides[2], const int64_t pads[4],
                              const int64_t dils[2], const int64_t *idx, int64_t n,
                              int act, double alpha, double *out);

/* The same conv reached through an explicit im2col matrix
 * cols[(c,r,s)][(n,oh,ow)] and the GEMM above ([FCT] "双 Kernel 是怎么
 * 分工的": weight = A operand co x k, input features = B operand k x
 * spatial).  If fold_bias, bias enters as the extra reduction index. */
int orc_conv2d_im2col(const double *x, const double *w, const double *bias,
                      double *y, int64_t N, int64_t C, int64_t H, int64_t W,
                      int64_t Co, int64_t kh, int64_t kw,
                      const int64_t strides[2], const int64_t pads[4],
                      const int64_t dils[2], int act, double alpha, int fold_bias);

/* Number of OpenMP threads the oracle uses (1 when built without OpenMP). */
int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
