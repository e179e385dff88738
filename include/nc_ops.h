/*
 * nc_ops.h -- single-kernel entry points of libncgpt.so, for testing and
 * measuring the kernels the step is built from in isolation.  Same error
 * conventions as nc.h; all pointers are device pointers owned by the caller;
 * work is enqueued on `stream` (a hipStream_t, NULL = default stream).
 */
#ifndef NC_OPS_H_
#define NC_OPS_H_

#include "nc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Operand layouts for nc_op_gemm */
enum { NC_K_CONTIGUOUS = 0, NC_MN_CONTIGUOUS = 1 };
/* Epilogues for nc_op_gemm (acc = alpha * A B^T in fp32) */
enum {
  NC_EPI_STORE = 0,       /* C = acc, activation dtype */
  NC_EPI_STORE_F32 = 1,   /* C = acc, fp32 */
  NC_EPI_ACC_F32 = 2,     /* C += acc, fp32 (residual add, gradient accumulation) */
  NC_EPI_RELU2 = 3,       /* C = max(acc, 0)^2 (ReLU^2 MLP, apidog.com
                             "1. Model GPT (nanochat/gpt.py)") */
  NC_EPI_RELU2_BWD = 4,   /* C = 2 sqrt(max(aux_in, 0)) * acc with aux_in = g = max(h, 0)^2:
                             the derivative of ReLU^2, 2 max(h, 0) dg, from the stored
                             activation (sqrt(g) = max(h, 0)), so h itself is never kept */
  NC_EPI_POLY = 5,        /* C = p0 * aux_in + p1 * acc (Newton-Schulz steps
                             B = b A + c A A and X = a X + B X, apidog.com
                             "2. Pengoptimal Muon (nanochat/optim.py)") */
  NC_EPI_DUAL = 6         /* C (fp32) = p0 * aux_in (fp32, may be NULL) + p1 * acc and
                             aux_out = C in the activation dtype: the same steps with
                             an fp32 iterate and its matrix-core copy */
};

/* Batched GEMM: for each batch index z < batch,
 *   acc[m, n] = alpha * sum_k A_z(m, k) * B_z(n, k),  0 <= m < M, 0 <= n < N,
 * with A_z(m,k) = A[z*sA + m*lda + k] (a_layout = NC_K_CONTIGUOUS) or
 * A[z*sA + k*lda + m] (NC_MN_CONTIGUOUS), and B likewise with (n, k), ldb, sB.
 * The epilogue writes C_z[m*ldc + n] (batch stride sC); aux_in/aux_out use
 * C's layout.  dtype NC_BF16: A, B, activation-type C/aux are bf16 (MFMA
 * path); NC_FP32: fp32.  splits > 1 (bf16, epilogues STORE_F32 / ACC_F32
 * only) splits K over workgroups and reduces in a fixed order through
 * `workspace` (at least splits*batch*M*N*4 bytes).  Requirements: K, and M
 * or N where that operand is MN-contiguous, multiples of 8; 16-byte aligned
 * operands and leading dimensions (bf16 path). */
nc_status nc_op_gemm(int32_t dtype, const void* A, int64_t lda, int32_t a_layout, const void* B,
                     int64_t ldb, int32_t b_layout, void* C, int64_t ldc, int32_t M, int32_t N,
                     int32_t K, int32_t batch, int64_t sA, int64_t sB, int64_t sC,
                     int32_t epilogue, const void* aux_in, void* aux_out, float alpha, float p0,
                     float p1, int32_t splits, void* workspace, size_t workspace_bytes,
                     void* stream);

/* fp8 GEMM: acc[m, n] = alpha * sum_k A(m, k) B(n, k) with A [M, K] and B [N, K]
 * K-contiguous OCP fp8 e4m3 bytes (row strides lda, ldb in bytes), fp32
 * accumulation; the epilogue writes C (row stride ldc elements): NC_EPI_STORE
 * (bf16), NC_EPI_STORE_F32, NC_EPI_ACC_F32 (C += acc) or NC_EPI_RELU2 (bf16
 * max(acc, 0)^2), as for nc_op_gemm.  The pages' later runs train most linear layers in FP8
 * with one scale per tensor (apidog.com, "3. Manajemen Presisi
 * (nanochat/common.py)"); alpha carries the product of the two inverse scales.
 * Requirements: K % 128 == 0, lda and ldb multiples of 16, 16-byte aligned
 * operands (NC_ERR_UNSUPPORTED otherwise). */
nc_status nc_op_gemm_fp8(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                         int64_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue,
                         float alpha, void* stream);

/* Tensorwise fp8 quantisation of n values x (dtype NC_FP32 or NC_BF16):
 * amax_scale[0] = max |x|, amax_scale[1] = s = 448 / amax (1 if amax = 0), and
 * q[i] = e4m3(x[i] * s) rounded to nearest even and saturated at 448, so that
 * x ~ q / s.  amax_scale: 2 device floats; workspace: 1024 device floats. */
nc_status nc_op_fp8_quantize(int32_t dtype, const void* x, int64_t n, float* amax_scale,
                             void* q, float* workspace, void* stream);

/* Causal attention forward, head dim 128, scale 1/sqrt(128).  q, k, v:
 * token-major rows (row b*T + t, head h at columns h*128 .. h*128+127, row
 * stride ld_qkv elements); q has H heads, k and v n_kv_head heads (n_kv_head
 * divides H; query head h reads key/value head h / (H / n_kv_head)); o: the
 * layout of q with stride ld_o; lse: fp32 [B, H, T] natural-log log-sum-exp
 * of each query's scores.  window: -1 for
 * the plain causal mask (query t sees keys 0 .. t), w >= 0 for a sliding
 * window (keys max(0, t - w) .. t; apidog.com, "5. Penyatuan Flash
 * Attention"); below -1 is NC_ERR_INVALID_ARG.  bf16 path needs
 * T % 128 == 0. */
nc_status nc_op_attention_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                              int64_t ld_qkv, void* o, int64_t ld_o, float* lse, int32_t B,
                              int32_t T, int32_t H, int32_t n_kv_head, int32_t window,
                              void* stream);

/* Causal attention backward from o, lse of the forward and dO (layout of o).
 * D (fp32 [B, H, T]) is caller-provided scratch receiving rowsum(dO * o).
 * Writes dq, dk, dv (layout of q/k/v with row stride ld_d; dk and dv of a
 * key/value head sum over its query heads).  n_kv_head and window as for the
 * forward pass (the same values the forward pass used). */
nc_status nc_op_attention_bwd(int32_t dtype, const void* q, const void* k, const void* v,
                              int64_t ld_qkv, const void* o, const void* dO, int64_t ld_o,
                              const float* lse, float* D, void* dq, void* dk, void* dv,
                              int64_t ld_d, int32_t B, int32_t T, int32_t H, int32_t n_kv_head,
                              int32_t window, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NC_OPS_H_ */
