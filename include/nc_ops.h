/*
 * nc_ops.h -- single-kernel entry points of libncgpt.so, for testing and
 * measuring the kernels the step is built from in isolation.  Same error
 * conventions as nc.h; all pointers are device pointers owned by the caller;
 * work is enqueued on `stream` (a hipStream_t, NULL = default stream).
 *
 * Every operand pointer comes with the number of bytes the caller owns from
 * that address on (`<name>_bytes`).  Before anything is launched the library
 * computes the bytes the requested layout touches (rows, leading dimension,
 * batch stride, element size) and returns NC_ERR_INVALID_ARG if any operand
 * would reach past its extent, or if a leading dimension is narrower than
 * the rows it describes.
 */
#ifndef NC_OPS_H_
#define NC_OPS_H_

#include "nc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Operand layouts for nc_op_gemm */
enum { NC_K_CONTIGUOUS = 0, NC_MN_CONTIGUOUS = 1 };
/* fp8 formats (OCP 8-bit floating point): e4m3 for activations and weights,
 * e5m2 for gradients */
enum { NC_FP8_E4M3 = 0, NC_FP8_E5M2 = 1 };
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
nc_status nc_op_gemm(int32_t dtype, const void* A, size_t A_bytes, int64_t lda,
                     int32_t a_layout, const void* B, size_t B_bytes, int64_t ldb,
                     int32_t b_layout, void* C, size_t C_bytes, int64_t ldc, int32_t M,
                     int32_t N, int32_t K, int32_t batch, int64_t sA, int64_t sB, int64_t sC,
                     int32_t epilogue, const void* aux_in, size_t aux_in_bytes, void* aux_out,
                     size_t aux_out_bytes, float alpha, float p0, float p1, int32_t splits,
                     void* workspace, size_t workspace_bytes, void* stream);

/* nc_op_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same product, epilogues and arguments, but no workspace argument.  With
 * splits > 1 the split-K partial slabs go to a 16 MiB array the library
 * keeps in each GPU's memory for the life of the process, so
 * splits * batch * M * N * 4 must be at most 16 MiB (NC_ERR_INVALID_ARG
 * otherwise, before any launch); splits = 1 uses no scratch.  Every slab is
 * written before it is read, so no call depends on what an earlier one left.
 * Calls on one GPU share that array: calls that can overlap (on different
 * streams, or from different threads) race and must be serialised by the
 * caller.  No hipMalloc, hipFree or allocating library routine is called. */
nc_status nc_op_gemm_noalloc(int32_t dtype, const void* A, size_t A_bytes, int64_t lda,
                             int32_t a_layout, const void* B, size_t B_bytes, int64_t ldb,
                             int32_t b_layout, void* C, size_t C_bytes, int64_t ldc, int32_t M,
                             int32_t N, int32_t K, int32_t batch, int64_t sA, int64_t sB,
                             int64_t sC, int32_t epilogue, const void* aux_in,
                             size_t aux_in_bytes, void* aux_out, size_t aux_out_bytes,
                             float alpha, float p0, float p1, int32_t splits, void* stream);

/* fp8 GEMM: acc[m, n] = alpha * sum_k A(m, k) B(n, k) with A [M, K] and B [N, K]
 * K-contiguous OCP fp8 bytes (row strides lda, ldb in bytes), A in e4m3
 * (a_format NC_FP8_E4M3) or e5m2 (NC_FP8_E5M2), B in e4m3, fp32 accumulation;
 * the epilogue writes C (row stride ldc elements): NC_EPI_STORE (bf16),
 * NC_EPI_STORE_F32, NC_EPI_ACC_F32 (C += acc), NC_EPI_RELU2 (bf16
 * max(acc, 0)^2) or NC_EPI_RELU2_BWD (bf16 2 sqrt(aux_in) acc, aux_in bf16
 * [M, N] with stride ldc), as for nc_op_gemm.  The pages' later runs train most
 * linear layers in FP8 with one scale per tensor (apidog.com, "3. Manajemen
 * Presisi (nanochat/common.py)"); alpha carries the product of the two inverse
 * scales.  splits > 1 splits K over that many workgroups per output tile (fp32
 * epilogues only), the partials going to workspace (splits * M * N * 4 bytes)
 * and summed in a fixed order; splits 1 needs no workspace.
 * Requirements: K % 128 == 0, lda and ldb multiples of 16, 16-byte aligned
 * operands (NC_ERR_UNSUPPORTED otherwise). */
nc_status nc_op_gemm_fp8(int32_t a_format, const void* A, size_t A_bytes, int64_t lda,
                         const void* B, size_t B_bytes, int64_t ldb, void* C, size_t C_bytes,
                         int64_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue,
                         const void* aux_in, size_t aux_in_bytes, float alpha, int32_t splits,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Tensorwise fp8 quantisation of x [rows, cols] (row stride cols; dtype
 * NC_FP32 or NC_BF16) to format NC_FP8_E4M3 (largest finite 448) or
 * NC_FP8_E5M2 (57344): amax_scale[0] = max |x|, amax_scale[1] = s = largest /
 * amax (1 if amax = 0), and each code = fp8(x * s) rounded to nearest even and
 * saturated at the largest finite value, so that x ~ code / s.  Codes go to q
 * in x's layout [rows, cols] and/or to qt transposed [cols, rows] (either may
 * be null, not both; qt needs NC_BF16, rows and cols multiples of 64, 16-byte
 * aligned x and qt; q then 8-byte aligned).  A NaN in x makes amax and s NaN
 * and every code 0x7F (NaN in both formats).  amax_scale: 2 device floats;
 * workspace: 1024 device floats of scratch. */
nc_status nc_op_fp8_quantize(int32_t dtype, int32_t format, const void* x, size_t x_bytes,
                             int64_t rows, int64_t cols, float* amax_scale,
                             size_t amax_scale_bytes, void* q, size_t q_bytes, void* qt,
                             size_t qt_bytes, float* workspace, size_t workspace_bytes,
                             void* stream);

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
nc_status nc_op_attention_fwd(int32_t dtype, const void* q, size_t q_bytes, const void* k,
                              size_t k_bytes, const void* v, size_t v_bytes, int64_t ld_qkv,
                              void* o, size_t o_bytes, int64_t ld_o, float* lse,
                              size_t lse_bytes, int32_t B, int32_t T, int32_t H,
                              int32_t n_kv_head, int32_t window, void* stream);

/* Causal attention backward from o, lse of the forward and dO (layout of o).
 * D is caller-provided fp32 scratch receiving rowsum(dO * o) in its first
 * [B, H, T] (NC_BF16: [2, B, H, T], the second half receiving -lse log2(e)).
 * Writes dq, dk, dv (layout of q/k/v with row stride ld_d; dk and dv of a
 * key/value head sum over its query heads).  n_kv_head and window as for the
 * forward pass (the same values the forward pass used). */
nc_status nc_op_attention_bwd(int32_t dtype, const void* q, size_t q_bytes, const void* k,
                              size_t k_bytes, const void* v, size_t v_bytes, int64_t ld_qkv,
                              const void* o, size_t o_bytes, const void* dO, size_t dO_bytes,
                              int64_t ld_o, const float* lse, size_t lse_bytes, float* D,
                              size_t D_bytes, void* dq, size_t dq_bytes, void* dk,
                              size_t dk_bytes, void* dv, size_t dv_bytes, int64_t ld_d,
                              int32_t B, int32_t T, int32_t H, int32_t n_kv_head,
                              int32_t window, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NC_OPS_H_ */
