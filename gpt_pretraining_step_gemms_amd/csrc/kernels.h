// Internal launchers of the memory-bound kernels and of attention.
// dtype 0 = fp32 activations, 1 = bf16 activations (fp32 residual, grads,
// masters and softmax statistics in both).
#pragma once
#include "common.h"

// ---- embedding
// A token id outside [0, vocab) makes its row of x NaN and sets bit 0 of *flag
// (a device int); the backward sorts such ids as clamped (no out-of-bounds
// access), on rows that are NaN already.
hipError_t nc_embed_fwd(const int32_t* tok, const float* E, float* x, int n_tok, int d, int V,
                        int32_t* flag, hipStream_t st);
// scratch: see nc_embed_bwd_scratch_bytes
size_t nc_embed_bwd_scratch_bytes(int n_tok, int vocab, int d);
hipError_t nc_embed_bwd(const int32_t* tok, const float* dx, float* dE, int n_tok, int vocab,
                        int d, void* scratch, hipStream_t st);
// The same in two parts: the stable sort of token positions by id (kept in
// scratch), then dE[v, :width] += sum of rows[n, :width] over the positions
// of id v (rows of `width` <= d floats), as often as needed for one sort.
hipError_t nc_embed_sort(const int32_t* tok, int n_tok, int vocab, void* scratch,
                         hipStream_t st);
hipError_t nc_embed_segsum(const int32_t* tok, const float* rows, float* dE, int n_tok,
                           int vocab, int width, void* scratch, hipStream_t st);

// ---- the further model mechanisms (extras.hip); scalars are device pointers
// x = E[tok] + lam_s sigmoid(E[tok][:24] . Ws) E[previous tok] (0 at a row
// start); x0 (optional) = x; sig[n] = the sigmoid.  Out-of-range ids as nc_embed_fwd.
hipError_t nc_embed_smear_fwd(const int32_t* tok, const float* E, const float* Ws,
                              const float* lam_s, float* x, float* x0, float* sig, int n_tok,
                              int T, int d, int V, int32_t* flag, hipStream_t st);
// Per row: u = a x + sign_b b xo (a = *lam_a or 1, b = *lam_b or 0); xsave (optional)
// = x before the mix; write_back: x = u; y = u r, r = (mean(u^2) + eps)^-1/2.
hipError_t nc_rmsnorm_mix_fwd(int dtype, float* x, const float* xo, float* xsave,
                              const float* lam_a, const float* lam_b, float sign_b,
                              int write_back, void* y, float* r, int rows, int d, float eps,
                              hipStream_t st);
// RMSNorm backward at the mixed stream u = lam_r x_prev + lam_0 x0 (din), then
// per-row din . xprev and din . x0 (part_r, part_0, optional), dx0 += lam_0 din
// (optional), dx = dxT = lam_r din + gb (lam_r null: 1; gb optional).
hipError_t nc_rmsnorm_mix_bwd(int dtype, const float* dy, const void* y, const float* r,
                              float* dx, void* dxT, const float* xprev, const float* x0,
                              float* dx0, const float* lam_r, const float* lam_0, const float* gb,
                              float* part_r, float* part_0, int rows, int d, int accumulate,
                              hipStream_t st);
// Backward of x - lam_b xb: part[row] = -dx . xb, gb = -lam_b dx.
hipError_t nc_backout_bwd(const float* dx, const float* xb, const float* lam_b, float* gb,
                          float* part, int rows, int d, hipStream_t st);
// Smear backward with dX = dx + dx0 (dx0 optional): gs[n] = gamma sig, dz[n] =
// gamma lam_s sig (1 - sig) with gamma = dX[n] . E[previous tok]; dxe = the
// gradient at the looked-up embedding rows.
hipError_t nc_smear_bwd(const int32_t* tok, const float* E, const float* dx, const float* dx0,
                        const float* sig, const float* lam_s, const float* Ws, float* gs,
                        float* dz, float* dxe, int n_tok, int T, int d, int V, hipStream_t st);
// v[n, h] += 3 sigmoid(a[n, :C] . Wg[h]) VE[tok[n], h] per key/value head h (C % 8 == 0,
// C <= 64); sig [n_tok, Hkv] = the sigmoids.
hipError_t nc_ve_mix_fwd(int dtype, const int32_t* tok, const float* VE, const float* Wg,
                         const void* a, int64_t lda, void* v, int64_t ldv, float* sig, int n_tok,
                         int Hkv, int C, int V, hipStream_t st);
// rows[n, h] = 3 sig dv[n, h] (fp32 [n_tok, Hkv*128]); dz[n, h] = (dv . VE[tok, h]) 3 sig (1 - sig).
hipError_t nc_ve_bwd(int dtype, const int32_t* tok, const float* VE, const void* dv,
                     int64_t lddv, const float* sig, float* rows, float* dz, int n_tok, int Hkv,
                     int V, hipStream_t st);
// da[n, j] += sum_h dz[n, h] Wg[h, j], j < C.
hipError_t nc_ve_gate_da(const float* dz, const float* Wg, float* da, int64_t ldda, int n_tok,
                         int Hkv, int C, hipStream_t st);
// out[h, j] += sum_n A[n, h] B(n, j), h < H, j < C; B(n, j) = B[n ldb + j] or, with tok,
// B[tok[n] ldb + j] (an embedding row).  part: nc_outer_scratch_floats(H, C) floats.
constexpr int kOuterParts = 256;
size_t nc_outer_scratch_floats(int H, int C);
hipError_t nc_outer_accumulate(int dtype, const float* A, int H, const void* B, int64_t ldb,
                               const int32_t* tok, int V, int C, int n_tok, float* part,
                               float* out, hipStream_t st);
// out[0] += sum of vals[0..n), fixed order.
hipError_t nc_sum_into(const float* vals, int n, float* out, hipStream_t st);

// ---- RMSNorm (rows of length d; eps)
// amax_part (optional): per block of 4 rows, the largest |y| as stored (|dxT| in
// the backward), ceil(rows / 4) floats, for an fp8 scale of the output.
hipError_t nc_rmsnorm_fwd(int dtype, const float* x, void* y, float* r, int rows, int d,
                          float eps, hipStream_t st, float* amax_part = nullptr);
// dx (+)= r*(dy - y*mean(dy*y)); also writes dxT = dx in the activation type.
// dy: the gradient at the norm's output, fp32, or bf16 with dy_bf16 (bf16 only)
hipError_t nc_rmsnorm_bwd(int dtype, const void* dy, int dy_bf16, const void* y, const float* r,
                          float* dx, void* dxT, int rows, int d, int accumulate, hipStream_t st,
                          float* amax_part = nullptr);

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
// qk_normed: q and k rows are RMS-normalised (|q.k| <= 128), so the bf16
// kernel may use a fixed softmax offset instead of a running max
hipError_t nc_attn_fwd(int dtype, const void* q, const void* k, const void* v, int64_t ld_qkv,
                       void* o, int64_t ld_o, float* lse, int B, int T, int H, int Hkv,
                       int window, hipStream_t st, float* amax_part = nullptr, int qk_normed = 0);
// D[b,h,t] = sum_d dO*O
hipError_t nc_attn_bwd_pre(int dtype, const void* o, const void* dO, int64_t ld_o, float* D,
                           int B, int T, int H, hipStream_t st);
// Writes D = rowsum(dO*O) ([B, H, T]; bf16: followed by -lse log2(e), [B, H, T]) and
// dq, dk, dv.  With rqk and cos_sin
// (bf16 only) the QK-norm + rotary backward is applied to dq and dk on their
// way out (rqk [B*T, H + Hkv] reciprocal RMS of the forward's q/k heads,
// cos_sin the rotary table [2][T][64]): the gradients are then those at the
// un-normalised q and k.
hipError_t nc_attn_bwd(int dtype, const void* q, const void* k, const void* v, int64_t ld_qkv,
                       const void* o, const void* dO, int64_t ld_o, const float* lse, float* D,
                       void* dq, void* dk, void* dv, int64_t ld_dqkv, int B, int T, int H,
                       int Hkv, int window, const float* rqk, const float* cos_sin,
                       hipStream_t st, float* amax_part = nullptr);
// bf16 path, amax_part (optional): per workgroup the largest |stored output| (o in
// the forward; dq then dk/dv in the backward), nc_attn_amax_parts(...) floats, for
// the output's fp8 scale without another pass over it.
int nc_attn_amax_parts(int B, int T, int H, int Hkv, int window, int backward);

// ---- fp8 with one scale per tensor, x [rows, cols] (row stride cols): fmt 0 = e4m3
// (fmax 448), 1 = e5m2 (fmax 57344); amax_scale[0] = max |x|, amax_scale[1] = fmax /
// amax (1 if amax = 0); codes fp8(x * scale) (round to nearest even, saturating) in
// x's layout into q and/or transposed [cols, rows] into qt (qt needs bf16 x, rows and
// cols multiples of 64, 16-byte aligned x and qt, 8-byte aligned q; q alone may be
// any shape); partial: 1024 floats of scratch
hipError_t nc_fp8_quantize(int dtype, int fmt, const void* x, int64_t rows, int64_t cols,
                           float* partial, float* amax_scale, uint8_t* q, uint8_t* qt,
                           hipStream_t st);
// The same with the amax already reduced to n_parts per-block maxima of |x| by
// x's producer (amax_parts): no pass over x for the scale.
hipError_t nc_fp8_quantize_parts(int fmt, const void* x, int64_t rows, int64_t cols,
                                 const float* amax_parts, int n_parts, float* amax_scale,
                                 uint8_t* q, uint8_t* qt, hipStream_t st);

// ---- softmax cross-entropy over rows of fp32 logits
// dz = scale*(softmax(z) - onehot(y)) in the activation type; loss_rows[i] = lse - z[y].
// A target outside [0, V) gives a NaN loss row and dz row and sets bit 1 of *flag.
hipError_t nc_cross_entropy(int dtype, const float* z, const int32_t* tgt, void* dz,
                            float* loss_rows, int rows, int V, float scale, int32_t* flag,
                            hipStream_t st);
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
