// GEMM launch interface: C[M,N] (epilogue) = A[M,K] * B[N,K]^T, fp32 accumulate.
//
// Operand layouts (both logical views are "row = output index, col = k"):
//   A: kKCont -> element (m,k) at A[m*lda + k];  kMNCont -> at A[k*lda + m]
//   B: kKCont -> element (n,k) at B[n*ldb + k];  kMNCont -> at B[k*ldb + n]
// This covers the forward products (both K-contiguous), the input gradients
// (B = weight read as its transpose, N-contiguous) and the weight gradients
// (both operands token-major, i.e. MN-contiguous).
#pragma once
#include "common.h"

enum NcLayout { kKCont = 0, kMNCont = 1 };

enum NcEpi {
  kEpiStore = 0,      // C = alpha*acc (C of the activation type)
  kEpiStoreF32 = 1,   // C(f32) = alpha*acc
  kEpiAccF32 = 2,     // C(f32) += alpha*acc
  kEpiRelu2 = 3,      // C = max(acc,0)^2           (the MLP activation g)
  kEpiRelu2Bwd = 4,   // C = 2*sqrt(max(aux_in,0))*acc   (aux_in = stored g: sqrt(g) = max(h,0))
  kEpiPoly = 5,       // C = p0*aux_in + p1*acc    (Newton-Schulz: b*A + c*A*A, a*X + B*X)
  kEpiDual = 6,       // C(f32) = p0*aux_in(f32, optional) + p1*acc; aux_out = C in the
                      // activation type (fp32 iterate + its matrix-core copy)
  kEpiQkNorm = 7,     // the QKV product (bf16, one batch, no split, K % 64 == 0, N % 128 ==
                      // 0): C = alpha*acc, and each of the first qk_heads 128-column heads
                      // of a row is RMS-normalised and rotated (rope, rqk below)
};

struct GemmParams {
  const void* A; const void* B; void* C;
  const void* aux_in; void* aux_out;
  int64_t lda, ldb, ldc;             // leading dimensions (elements)
  int64_t sA, sB, sC;                // batch strides (elements); aux uses sC/ldc
  int M, N, K, batch;
  int a_layout, b_layout, epi;
  float alpha, p0, p1;
  int splits;                        // split-K count (>1: C must be f32, workspace used)
  int vec_epi;                       // set by the launcher: C/aux 16-byte aligned, ldc and sC % 8 == 0
  float* workspace; size_t workspace_bytes;
  // fp8 only: per-tensor scales {amax, s} of A and B (device); acc is divided by
  // s_A * s_B before the epilogue.  Null: no device scales.
  const float* scale_a; const float* scale_b;
  int fmt_a;                         // fp8 only: A's format, 0 = e4m3, 1 = e5m2 (B is e4m3)
  // optional, ReLU^2 and ReLU^2-backward epilogues of the fp8 kernel (one
  // batch, no split): per workgroup the largest |C| as stored (bf16), one float
  // per output tile, for C's fp8 scale without another pass over C
  float* amax_part;
  // kEpiQkNorm only: row m is position m % rope_T of its sequence; head j < qk_heads
  // of the row (columns 128 j .. 128 j + 127) becomes R_t (x r) with
  // r = (mean(x^2) + qk_eps)^-1/2, and rqk[m * qk_heads + j] = r.  rope: cos | sin
  // tables [rope_T][64]; R_t pairs dims i and i + 64.
  const float* rope; float* rqk;
  int rope_T, qk_heads;
  float qk_eps;
};

// dtype: 0 = fp32 operands (VALU kernel), 1 = bf16 operands (MFMA kernel)
hipError_t nc_launch_gemm(int dtype, const GemmParams& p, hipStream_t stream);
// fp8 operands (bytes; A e4m3 or e5m2 by fmt_a, B e4m3), both K-contiguous:
// K % 128 == 0, lda, ldb (and batch strides) % 16 == 0, 16-byte aligned; epilogues
// as for bf16; split-K (splits > 1) with an fp32 output and the workspace
hipError_t nc_launch_gemm_f8(const GemmParams& p, hipStream_t stream);
// splits a weight-gradient GEMM would use for M x N with reduction K (bf16 path)
int nc_gemm_pick_splits(int M, int N, int K);
size_t nc_gemm_workspace_bytes(int M, int N, int splits);
