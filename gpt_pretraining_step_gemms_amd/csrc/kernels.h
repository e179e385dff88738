// Internal launchers of the memory-bound kernels and of attention.
// dtype 0 = fp32 activations, 1 = bf16 activations (fp32 residual, grads,
// masters and softmax statistics in both).
#pragma once
#include "common.h"

// ---- embedding
// token ids outside [0, vocab) are clamped (no out-of-bounds access)
hipError_t nc_embed_fwd(const int32_t* tok, const float* E, float* x, int n_tok, int d, int V,
                        hipStream_t st);
// scratch: see nc_embed_bwd_scratch_bytes
size_t nc_embed_bwd_scratch_bytes(int n_tok, int vocab, int d);
hipError_t nc_embed_bwd(const int32_t* tok, const float* dx, float* dE, int n_tok, int vocab,
                        int d, void* scratch, hipStream_t st);

// ---- RMSNorm (rows of length d; eps)
hipError_t nc_rmsnorm_fwd(int dtype, const float* x, void* y, float* r, int rows, int d,
                          float eps, hipStream_t st);
// dx (+)= r*(dy - y*mean(dy*y)); also writes dxT = dx in the activation type.
hipError_t nc_rmsnorm_bwd(int dtype, const float* dy, const void* y, const float* r, float* dx,
                          void* dxT, int rows, int d, int accumulate, hipStream_t st);

// ---- QK RMSNorm + rotary (qkv token-major [n_tok, (H + 2 Hkv)*128]: H q heads, Hkv k
// heads, Hkv v heads; in place on the q and k heads; rqk [n_tok, H + Hkv])
hipError_t nc_qk_norm_rope_fwd(int dtype, void* qkv, float* rqk, const float* cos_sin,
                               int n_tok, int T, int H, int Hkv, float eps, hipStream_t st);
hipError_t nc_qk_norm_rope_bwd(int dtype, void* dqkv, const void* qkv, const float* rqk,
                               const float* cos_sin, int n_tok, int T, int H, int Hkv,
                               hipStream_t st);

// ---- attention on token-major q/k/v (row stride ld_qkv), head dim 128; query t
// sees keys max(0, t - window) .. t (window < 0: keys 0 .. t); H query heads,
// Hkv key/value heads (H % Hkv == 0), query head h reads key/value head h / (H / Hkv)
hipError_t nc_attn_fwd(int dtype, const void* q, const void* k, const void* v, int64_t ld_qkv,
                       void* o, int64_t ld_o, float* lse, int B, int T, int H, int Hkv,
                       int window, hipStream_t st);
// D[b,h,t] = sum_d dO*O
hipError_t nc_attn_bwd_pre(int dtype, const void* o, const void* dO, int64_t ld_o, float* D,
                           int B, int T, int H, hipStream_t st);
hipError_t nc_attn_bwd(int dtype, const void* q, const void* k, const void* v, int64_t ld_qkv,
                       const void* dO, int64_t ld_o, const float* lse, const float* D,
                       void* dq, void* dk, void* dv, int64_t ld_dqkv, int B, int T, int H,
                       int Hkv, int window, hipStream_t st);

// ---- fp8 e4m3 with one scale per tensor: amax_scale[0] = max |x|, amax_scale[1] =
// 448 / amax (1 if amax = 0), q[i] = e4m3(x[i] * scale) (round to nearest even,
// saturating); partial: 1024 floats of scratch
hipError_t nc_fp8_quantize(int dtype, const void* x, int64_t n, float* partial,
                           float* amax_scale, uint8_t* q, hipStream_t st);

// ---- softmax cross-entropy over rows of fp32 logits
// dz = scale*(softmax(z) - onehot(y)) in the activation type; loss_rows[i] = lse - z[y]
hipError_t nc_cross_entropy(int dtype, const float* z, const int32_t* tgt, void* dz,
                            float* loss_rows, int rows, int V, float scale, hipStream_t st);
// out[0] = scale * sum(vals[0..n))   (fixed-order, single workgroup)
hipError_t nc_sum_scaled(const float* vals, int n, float scale, float* out, hipStream_t st);

// ---- elementwise utilities
hipError_t nc_fill_f32(float* p, float v, size_t n, hipStream_t st);
hipError_t nc_convert_f32(int dtype, const float* src, void* dst, size_t n, hipStream_t st);
hipError_t nc_init_normal(float* p, size_t n, uint64_t seed, uint64_t offset, float std,
                          hipStream_t st);
// flag[0] |= 1 if any element of p[0..n) is not finite
hipError_t nc_check_finite(const float* p, size_t n, int32_t* flag, hipStream_t st);

// ---- optimizers
// AdamW over p[0..n): elements [0, n_first) use lr0, the rest lr1.  If shadow
// is non-null, shadow[i - shadow_from] = bf16(p[i]) for i >= shadow_from.
hipError_t nc_adamw(float* p, const float* g, float* m, float* v, size_t n, size_t n_first,
                    float lr0, float lr1, float b1, float b2, float eps, float wd, float bc1,
                    float bc2, void* shadow, size_t shadow_from, hipStream_t st);
// M = mu*M + G over n elements (U = G + mu*M written to U if nesterov, else U = M)
hipError_t nc_momentum(float* M, const float* G, size_t n, float mu, hipStream_t st);
hipError_t nc_nesterov(const float* M, const float* G, float* U, size_t n, float mu,
                       hipStream_t st);

// Matrices of a batch: the i-th starts at element (i / per) * layer + (i % per) * inner
// of its base pointer (block matrices of one kind interleave with the others).
struct MatBatch {
  int per;
  int64_t inner, layer;
  NC_HD int64_t off(int i) const { return (int64_t)(i / per) * layer + (int64_t)(i % per) * inner; }
};

// Batched Frobenius norms of count matrices of `elems` elements each.
// partial must hold count * 256 floats.
hipError_t nc_frob_norms(const float* src, MatBatch mb, int64_t elems, int count,
                         float* partial, float* norms, hipStream_t st);
// X[i] = src[i] / (norms[i] + eps) with src[i] [R, C] fp32, written as fp32 (X32) and
// in the activation type (Xh); both contiguous (stride x_stride), [R, C] or, when
// transpose != 0, [C, R].
hipError_t nc_ns_prepare(int dtype, const float* src, MatBatch mb, int R, int C, int count,
                         const float* norms, float eps, int transpose, float* X32, void* Xh,
                         int64_t x_stride, hipStream_t st);
// W[i] = W[i]*(1 - lr*wd) - lr*X[i] (fp32 X read transposed when transpose != 0),
// with row r of X[i] multiplied by mat_scale[i] * row_mul[i*R + r] when row_mul != null;
// shadow[i] (same addressing as W) = bf16(W[i]) when shadow != null.
hipError_t nc_ns_apply(float* W, MatBatch mb, int R, int C, int count, const float* X,
                       int64_t x_stride, int transpose, float lr, float wd, const float* row_mul,
                       const float* mat_scale, void* shadow, hipStream_t st);
// NorMuon: per row r of W_i [R, C] (X_i as for nc_ns_apply) updates the second
// moment v2[i*R + r] with the row's mean X^2 and writes inv[i*R + r] = v2c^-1/2
// (v2c = max(v2, 1e-10)) and scale[i] = sqrt(sum vm) / max(sqrt(sum vm / v2c), 1e-10);
// vm and q are [count*R] scratch.  nc_ns_apply(row_mul = inv, mat_scale = scale)
// then applies the normalised update.
hipError_t nc_normuon_stats(const float* X, int64_t x_stride, int R, int C, int transpose,
                            int count, float* v2, float beta2, float* vm, float* q, float* inv,
                            float* scale, hipStream_t st);
