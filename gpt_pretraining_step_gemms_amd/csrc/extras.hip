// Kernels of the pages' further model mechanisms (apidog.com, "Cara Melatih
// ChatGPT Sendiri dengan Budget 50 Dolar", "1. Model GPT (nanochat/gpt.py)":
// the value-embedding listing and the listing of three efficiency tricks):
//  * smear: x_t = e_t + lam_s sigmoid(e_t[:24] . Ws) e_{t-1} after the
//    embedding lookup (e_{-1} = 0 at the start of a row);
//  * residual scaling at the start of every layer, x <- lam_r x + lam_0 x0,
//    fused with the layer's first RMSNorm; the same fused kernel forms the
//    backout x - lam_b xb before the final norm;
//  * value embeddings: v += 3 sigmoid(a[:, :C] Wg^T) VE[tok] per key/value head;
//  * the backward of each, with deterministic reductions (per-row or
//    per-block partial sums folded in a fixed order) for the gradients of
//    the scalars and gates.
// Scalars are read from device memory (the fp32 master parameters), so no
// host synchronisation is needed.
#include "kernels.h"

namespace {

NC_DEV float sigmoidf(float z) { return 1.f / (1.f + __expf(-z)); }

NC_DEV void load4(const float* p, float (&o)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
NC_DEV void store4(float* p, const float (&o)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
}
NC_DEV void load4(const bf16* p, float (&o)[4]) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  o[0] = (float)v[0]; o[1] = (float)v[1]; o[2] = (float)v[2]; o[3] = (float)v[3];
}
NC_DEV void store4(bf16* p, const float (&o)[4]) {
  bf16x4 v;
  v[0] = (bf16)o[0]; v[1] = (bf16)o[1]; v[2] = (bf16)o[2]; v[3] = (bf16)o[3];
  *reinterpret_cast<bf16x4*>(p) = v;
}

constexpr int kMaxV4 = 8;    // float4 per lane: d <= 2048

// ---------------------------------------------------------------- smear
// One wave per token n (position t of its row): x[n] = E[tok] + g E[tok of
// n - 1] with g = lam_s sigmoid(E[tok][:24] . Ws) (t > 0), x0 = x if wanted,
// sig[n] = sigmoid(...).  Out-of-range ids: NaN row, flag bit 0.
__global__ void embed_smear_fwd_kernel(const int32_t* __restrict__ tok,
                                       const float* __restrict__ E,
                                       const float* __restrict__ Ws,
                                       const float* __restrict__ lam_s, float* __restrict__ x,
                                       float* __restrict__ x0, float* __restrict__ sig,
                                       int n_tok, int T, int d, int V,
                                       int32_t* __restrict__ flag) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= n_tok) return;
  const int lane = threadIdx.x & 63;
  const int t = n % T;
  const int id = tok[n], idp = t > 0 ? tok[n - 1] : 0;
  float* xr = x + (int64_t)n * d;
  float* x0r = x0 ? x0 + (int64_t)n * d : nullptr;
  if (id < 0 || id >= V || idp < 0 || idp >= V) {
    if (lane == 0) atomicOr(flag, 1);
    for (int i = lane * 4; i < d; i += 256) {
      const float nan4[4] = {NAN, NAN, NAN, NAN};
      store4(xr + i, nan4);
      if (x0r) store4(x0r + i, nan4);
    }
    if (lane == 0) sig[n] = NAN;
    return;
  }
  const float* er = E + (int64_t)id * d;
  const float* ep = E + (int64_t)idp * d;
  float z = 0.f;
  if (lane < 6) {                                   // channels 0..23
    float a[4], w[4];
    load4(er + lane * 4, a);
    load4(Ws + lane * 4, w);
    z = a[0] * w[0] + a[1] * w[1] + a[2] * w[2] + a[3] * w[3];
  }
  z = wave_sum(z);
  const float s = sigmoidf(z);
  const float g = t > 0 ? lam_s[0] * s : 0.f;
  for (int i = lane * 4; i < d; i += 256) {
    float a[4], b[4];
    load4(er + i, a);
    load4(ep + i, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += g * b[e];
    store4(xr + i, a);
    if (x0r) store4(x0r + i, a);
  }
  if (lane == 0) sig[n] = s;
}

// --------------------------------------------------- mixed RMSNorm forward
// One wave per row: u = ca x + cb xo with ca = *lam_a (1 if null) and
// cb = sign_b * *lam_b (0 if null); optional save of the row before the mix
// (xsave = x); write_back: x = u; y = u r, r = (mean(u^2) + eps)^-1/2.
template <typename T>
__global__ void rmsnorm_mix_fwd_kernel(float* __restrict__ x, const float* __restrict__ xo,
                                       float* __restrict__ xsave,
                                       const float* __restrict__ lam_a,
                                       const float* __restrict__ lam_b, float sign_b,
                                       int write_back, T* __restrict__ y,
                                       float* __restrict__ r, int rows, int d, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float ca = lam_a ? lam_a[0] : 1.f;
  const float cb = lam_b ? sign_b * lam_b[0] : 0.f;
  const int64_t off = (int64_t)row * d;
  float v[kMaxV4][4];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxV4; ++k) {
    const int i = (lane + k * 64) * 4;
    if (i < d) {
      float o[4];
      load4(x + off + i, v[k]);
      if (xsave) store4(xsave + off + i, v[k]);
      if (lam_b) {
        load4(xo + off + i, o);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[k][e] = ca * v[k][e] + cb * o[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[k][e] *= ca;
      }
      if (write_back) store4(x + off + i, v[k]);
      ss += v[k][0] * v[k][0] + v[k][1] * v[k][1] + v[k][2] * v[k][2] + v[k][3] * v[k][3];
    }
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / d + eps);
  if (lane == 0) r[row] = rs;
#pragma unroll
  for (int k = 0; k < kMaxV4; ++k) {
    const int i = (lane + k * 64) * 4;
    if (i < d) {
      float o[4] = {v[k][0] * rs, v[k][1] * rs, v[k][2] * rs, v[k][3] * rs};
      store4(y + off + i, o);
    }
  }
}

// --------------------------------------------------- mixed RMSNorm backward
// One wave per row.  din = (accumulate ? dx : 0) + r (dy - y mean(dy y)), the
// gradient at the mixed stream u = lam_r x_prev + lam_0 x0; then
//   part_r[row] = din . xprev, part_0[row] = din . x0   (if part_r),
//   dx0 += lam_0 din                                    (if dx0),
//   dx = dxT = lam_r din + gb                           (gb optional).
template <typename T>
__global__ void rmsnorm_mix_bwd_kernel(const float* __restrict__ dy, const T* __restrict__ y,
                                       const float* __restrict__ r, float* __restrict__ dx,
                                       T* __restrict__ dxT, const float* __restrict__ xprev,
                                       const float* __restrict__ x0, float* __restrict__ dx0,
                                       const float* __restrict__ lam_r,
                                       const float* __restrict__ lam_0,
                                       const float* __restrict__ gb, float* __restrict__ part_r,
                                       float* __restrict__ part_0, int rows, int d,
                                       int accumulate) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t off = (int64_t)row * d;
  float g[kMaxV4][4], yy[kMaxV4][4];
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxV4; ++k) {
    const int i = (lane + k * 64) * 4;
    if (i < d) {
      load4(dy + off + i, g[k]);
      load4(y + off + i, yy[k]);
      dot += g[k][0] * yy[k][0] + g[k][1] * yy[k][1] + g[k][2] * yy[k][2] + g[k][3] * yy[k][3];
    }
  }
  const float mean = wave_sum(dot) / d;
  const float rs = r[row];
  const float cr = lam_r ? lam_r[0] : 1.f, c0 = lam_0 ? lam_0[0] : 0.f;
  float pr = 0.f, p0 = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxV4; ++k) {
    const int i = (lane + k * 64) * 4;
    if (i < d) {
      float din[4];
      if (accumulate) load4(dx + off + i, din);
      else din[0] = din[1] = din[2] = din[3] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) din[e] += rs * (g[k][e] - yy[k][e] * mean);
      if (part_r) {
        float a[4], b[4];
        load4(xprev + off + i, a);
        load4(x0 + off + i, b);
#pragma unroll
        for (int e = 0; e < 4; ++e) { pr += din[e] * a[e]; p0 += din[e] * b[e]; }
      }
      if (dx0) {
        float a[4];
        load4(dx0 + off + i, a);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] += c0 * din[e];
        store4(dx0 + off + i, a);
      }
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = cr * din[e];
      if (gb) {
        float a[4];
        load4(gb + off + i, a);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] += a[e];
      }
      store4(dx + off + i, o);
      store4(dxT + off + i, o);
    }
  }
  if (part_r) {
    pr = wave_sum(pr);
    p0 = wave_sum(p0);
    if (lane == 0) { part_r[row] = pr; part_0[row] = p0; }
  }
}

// ------------------------------------------------------- backout backward
// One wave per row of dx (the gradient at x - lam_b xb): part[row] = -dx . xb
// and gb = -lam_b dx (added to the gradient where xb was taken).
__global__ void backout_bwd_kernel(const float* __restrict__ dx, const float* __restrict__ xb,
                                   const float* __restrict__ lam_b, float* __restrict__ gb,
                                   float* __restrict__ part, int rows, int d) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t off = (int64_t)row * d;
  const float cb = -lam_b[0];
  float p = 0.f;
  for (int i = lane * 4; i < d; i += 256) {
    float a[4], b[4], o[4];
    load4(dx + off + i, a);
    load4(xb + off + i, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) { p -= a[e] * b[e]; o[e] = cb * a[e]; }
    store4(gb + off + i, o);
  }
  p = wave_sum(p);
  if (lane == 0) part[row] = p;
}

// ------------------------------------------------------- smear backward
// dX = dx + dx0 (the gradient at x0) is read on the fly.
// (a) per token n, position t: gamma = dX[n] . e_{t-1} (0 at t = 0);
//     gs[n] = gamma sigmoid_n (for d lam_s), dz[n] = gamma lam_s s (1 - s).
__global__ void smear_bwd_a_kernel(const int32_t* __restrict__ tok, const float* __restrict__ E,
                                   const float* __restrict__ dx, const float* __restrict__ dx0,
                                   const float* __restrict__ sig, const float* __restrict__ lam_s,
                                   float* __restrict__ gs, float* __restrict__ dz, int n_tok,
                                   int T, int d, int V) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= n_tok) return;
  const int lane = threadIdx.x & 63;
  const int t = n % T;
  float gamma = 0.f;
  if (t > 0) {
    const float* ep = E + (int64_t)clamp_id(tok[n - 1], V) * d;
    const int64_t off = (int64_t)n * d;
    for (int i = lane * 4; i < d; i += 256) {
      float a[4], b[4], c[4];
      load4(dx + off + i, a);
      load4(ep + i, c);
      if (dx0) {
        load4(dx0 + off + i, b);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] += b[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) gamma += a[e] * c[e];
    }
    gamma = wave_sum(gamma);
  }
  if (lane == 0) {
    const float s = sig[n];
    gs[n] = gamma * s;
    dz[n] = gamma * lam_s[0] * s * (1.f - s);
  }
}

// (b) per token n: dxe[n] = dX[n] + lam_s sig[n+1] dX[n+1] (if n+1 is in the
//     row) + dz[n] Ws on channels 0..23.
__global__ void smear_bwd_b_kernel(const float* __restrict__ dx, const float* __restrict__ dx0,
                                   const float* __restrict__ sig, const float* __restrict__ lam_s,
                                   const float* __restrict__ dz, const float* __restrict__ Ws,
                                   float* __restrict__ dxe, int n_tok, int T, int d) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= n_tok) return;
  const int lane = threadIdx.x & 63;
  const int t = n % T;
  const bool next = t + 1 < T;
  const float gn = next ? lam_s[0] * sig[n + 1] : 0.f;
  const float zn = dz[n];
  const int64_t off = (int64_t)n * d;
  for (int i = lane * 4; i < d; i += 256) {
    float a[4], b[4];
    load4(dx + off + i, a);
    if (dx0) {
      load4(dx0 + off + i, b);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += b[e];
    }
    if (next) {
      load4(dx + off + d + i, b);
      float c[4] = {0.f, 0.f, 0.f, 0.f};
      if (dx0) load4(dx0 + off + d + i, c);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += gn * (b[e] + c[e]);
    }
    if (i < 24) {
      float w[4];
      load4(Ws + i, w);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += zn * w[e];
    }
    store4(dxe + off + i, a);
  }
}

// ------------------------------------------------- value embedding mix
// 8 lanes per (token n, key/value head h); lane u of the group owns dims
// 16u .. 16u+15 of the head.  gate = 3 sigmoid(a[n, :C] . Wg[h, :C]) (C a
// multiple of 8, at most 64: lane u reads channels u*C/8 ..), then
// v[n, h] += gate * VE[tok[n], h]; sig[n*Hkv + h] = sigmoid(...).
template <typename T>
__global__ __launch_bounds__(256) void ve_mix_fwd_kernel(
    const int32_t* __restrict__ tok, const float* __restrict__ VE, const float* __restrict__ Wg,
    const T* __restrict__ a, int64_t lda, T* __restrict__ v, int64_t ldv,
    float* __restrict__ sig, int n_tok, int Hkv, int C, int V) {
  const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
  if (item >= (int64_t)n_tok * Hkv) return;
  const int u = threadIdx.x & 7;
  const int n = (int)(item / Hkv), h = (int)(item % Hkv);
  const int per = C / 8;
  float z = 0.f;
  for (int j = u * per; j < (u + 1) * per; ++j) z += to_f(a[(int64_t)n * lda + j]) * Wg[h * C + j];
  z += __shfl_xor(z, 1, 64);
  z += __shfl_xor(z, 2, 64);
  z += __shfl_xor(z, 4, 64);
  const float s = sigmoidf(z), g = 3.f * s;
  const int dk = Hkv * 128;
  const float* ve = VE + (int64_t)clamp_id(tok[n], V) * dk + h * 128 + 16 * u;
  T* vp = v + (int64_t)n * ldv + h * 128 + 16 * u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float e4[4], v4[4];
    load4(ve + 4 * q, e4);
    load4(vp + 4 * q, v4);
#pragma unroll
    for (int e = 0; e < 4; ++e) v4[e] += g * e4[e];
    store4(vp + 4 * q, v4);
  }
  if (u == 0) sig[item] = s;
}

// Backward of the mix, same lane layout: from dv (the gradient at the mixed
// v): rows[n, h*128 + i] = 3 s dv (the value-embedding gradient rows, to be
// summed per token id) and dz[n*Hkv + h] = (dv . VE[tok, h]) 3 s (1 - s).
template <typename T>
__global__ __launch_bounds__(256) void ve_bwd_kernel(
    const int32_t* __restrict__ tok, const float* __restrict__ VE, const T* __restrict__ dv,
    int64_t lddv, const float* __restrict__ sig, float* __restrict__ rows,
    float* __restrict__ dz, int n_tok, int Hkv, int V) {
  const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
  if (item >= (int64_t)n_tok * Hkv) return;
  const int u = threadIdx.x & 7;
  const int n = (int)(item / Hkv), h = (int)(item % Hkv);
  const int dk = Hkv * 128;
  const float s = sig[item], g = 3.f * s;
  const float* ve = VE + (int64_t)clamp_id(tok[n], V) * dk + h * 128 + 16 * u;
  const T* dp = dv + (int64_t)n * lddv + h * 128 + 16 * u;
  float* rp = rows + (int64_t)n * dk + h * 128 + 16 * u;
  float dot = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float e4[4], d4[4], o[4];
    load4(ve + 4 * q, e4);
    load4(dp + 4 * q, d4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { dot += d4[e] * e4[e]; o[e] = g * d4[e]; }
    store4(rp + 4 * q, o);
  }
  dot += __shfl_xor(dot, 1, 64);
  dot += __shfl_xor(dot, 2, 64);
  dot += __shfl_xor(dot, 4, 64);
  if (u == 0) dz[item] = dot * 3.f * s * (1.f - s);
}

// da[n, j] += sum_h dz[n, h] Wg[h, j] for j < C (the gate's input gradient):
// one thread per (n, j).
__global__ void ve_gate_da_kernel(const float* __restrict__ dz, const float* __restrict__ Wg,
                                  float* __restrict__ da, int64_t ldda, int n_tok, int Hkv,
                                  int C) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)n_tok * C) return;
  const int n = (int)(i / C), j = (int)(i % C);
  float s = 0.f;
  for (int h = 0; h < Hkv; ++h) s += dz[(int64_t)n * Hkv + h] * Wg[h * C + j];
  da[(int64_t)n * ldda + j] += s;
}

// out[h, j] += sum_n A[n, h] B(n, j) for h < H, j < C, with B(n, j) =
// B[n * ldb + j], or E[tok[n] * ldb + j] when tok is given.  Block b sums
// rows n = b, b + G, ... into part[b][H*C]; then a fixed-order fold.
template <typename T>
__global__ __launch_bounds__(256) void outer_partial_kernel(
    const float* __restrict__ A, int H, const T* __restrict__ B, int64_t ldb,
    const int32_t* __restrict__ tok, int V, int C, int n_tok, float* __restrict__ part) {
  const int HC = H * C;
  for (int o = threadIdx.x; o < HC; o += 256) {
    const int h = o / C, j = o % C;
    float s = 0.f;
    for (int n = blockIdx.x; n < n_tok; n += gridDim.x) {
      const int64_t row = tok ? (int64_t)clamp_id(tok[n], V) : n;
      s += A[(int64_t)n * H + h] * to_f(B[row * ldb + j]);
    }
    part[(int64_t)blockIdx.x * HC + o] = s;
  }
}

__global__ void fold_partials_kernel(const float* __restrict__ part, int parts, int width,
                                     float* __restrict__ out) {
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= width) return;
  float s = 0.f;
  for (int b = 0; b < parts; ++b) s += part[(int64_t)b * width + o];
  out[o] += s;
}

// out[0] += sum of vals[0..n) (one workgroup, fixed order)
__global__ __launch_bounds__(1024) void sum_into_kernel(const float* __restrict__ vals, int n,
                                                        float* __restrict__ out) {
  __shared__ float red[16];
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) s += vals[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) out[0] += s;
}

}  // namespace

// =============================================================== launchers
hipError_t nc_embed_smear_fwd(const int32_t* tok, const float* E, const float* Ws,
                              const float* lam_s, float* x, float* x0, float* sig, int n_tok,
                              int T, int d, int V, int32_t* flag, hipStream_t st) {
  embed_smear_fwd_kernel<<<ceil_div(n_tok, 4), 256, 0, st>>>(tok, E, Ws, lam_s, x, x0, sig,
                                                             n_tok, T, d, V, flag);
  return hipGetLastError();
}

hipError_t nc_rmsnorm_mix_fwd(int dtype, float* x, const float* xo, float* xsave,
                              const float* lam_a, const float* lam_b, float sign_b,
                              int write_back, void* y, float* r, int rows, int d, float eps,
                              hipStream_t st) {
  const int g = ceil_div(rows, 4);
  if (dtype)
    rmsnorm_mix_fwd_kernel<bf16><<<g, 256, 0, st>>>(x, xo, xsave, lam_a, lam_b, sign_b,
                                                    write_back, (bf16*)y, r, rows, d, eps);
  else
    rmsnorm_mix_fwd_kernel<float><<<g, 256, 0, st>>>(x, xo, xsave, lam_a, lam_b, sign_b,
                                                     write_back, (float*)y, r, rows, d, eps);
  return hipGetLastError();
}

hipError_t nc_rmsnorm_mix_bwd(int dtype, const float* dy, const void* y, const float* r,
                              float* dx, void* dxT, const float* xprev, const float* x0,
                              float* dx0, const float* lam_r, const float* lam_0, const float* gb,
                              float* part_r, float* part_0, int rows, int d, int accumulate,
                              hipStream_t st) {
  const int g = ceil_div(rows, 4);
  if (dtype)
    rmsnorm_mix_bwd_kernel<bf16><<<g, 256, 0, st>>>(dy, (const bf16*)y, r, dx, (bf16*)dxT,
                                                    xprev, x0, dx0, lam_r, lam_0, gb, part_r,
                                                    part_0, rows, d, accumulate);
  else
    rmsnorm_mix_bwd_kernel<float><<<g, 256, 0, st>>>(dy, (const float*)y, r, dx, (float*)dxT,
                                                     xprev, x0, dx0, lam_r, lam_0, gb, part_r,
                                                     part_0, rows, d, accumulate);
  return hipGetLastError();
}

hipError_t nc_backout_bwd(const float* dx, const float* xb, const float* lam_b, float* gb,
                          float* part, int rows, int d, hipStream_t st) {
  backout_bwd_kernel<<<ceil_div(rows, 4), 256, 0, st>>>(dx, xb, lam_b, gb, part, rows, d);
  return hipGetLastError();
}

hipError_t nc_smear_bwd(const int32_t* tok, const float* E, const float* dx, const float* dx0,
                        const float* sig, const float* lam_s, const float* Ws, float* gs,
                        float* dz, float* dxe, int n_tok, int T, int d, int V, hipStream_t st) {
  smear_bwd_a_kernel<<<ceil_div(n_tok, 4), 256, 0, st>>>(tok, E, dx, dx0, sig, lam_s, gs, dz,
                                                         n_tok, T, d, V);
  smear_bwd_b_kernel<<<ceil_div(n_tok, 4), 256, 0, st>>>(dx, dx0, sig, lam_s, dz, Ws, dxe,
                                                         n_tok, T, d);
  return hipGetLastError();
}

hipError_t nc_ve_mix_fwd(int dtype, const int32_t* tok, const float* VE, const float* Wg,
                         const void* a, int64_t lda, void* v, int64_t ldv, float* sig, int n_tok,
                         int Hkv, int C, int V, hipStream_t st) {
  const int blocks = (int)ceil_div64((int64_t)n_tok * Hkv * 8, 256);
  if (dtype)
    ve_mix_fwd_kernel<bf16><<<blocks, 256, 0, st>>>(tok, VE, Wg, (const bf16*)a, lda, (bf16*)v,
                                                    ldv, sig, n_tok, Hkv, C, V);
  else
    ve_mix_fwd_kernel<float><<<blocks, 256, 0, st>>>(tok, VE, Wg, (const float*)a, lda,
                                                     (float*)v, ldv, sig, n_tok, Hkv, C, V);
  return hipGetLastError();
}

hipError_t nc_ve_bwd(int dtype, const int32_t* tok, const float* VE, const void* dv,
                     int64_t lddv, const float* sig, float* rows, float* dz, int n_tok, int Hkv,
                     int V, hipStream_t st) {
  const int blocks = (int)ceil_div64((int64_t)n_tok * Hkv * 8, 256);
  if (dtype)
    ve_bwd_kernel<bf16><<<blocks, 256, 0, st>>>(tok, VE, (const bf16*)dv, lddv, sig, rows, dz,
                                                n_tok, Hkv, V);
  else
    ve_bwd_kernel<float><<<blocks, 256, 0, st>>>(tok, VE, (const float*)dv, lddv, sig, rows, dz,
                                                 n_tok, Hkv, V);
  return hipGetLastError();
}

hipError_t nc_ve_gate_da(const float* dz, const float* Wg, float* da, int64_t ldda, int n_tok,
                         int Hkv, int C, hipStream_t st) {
  ve_gate_da_kernel<<<(int)ceil_div64((int64_t)n_tok * C, 256), 256, 0, st>>>(dz, Wg, da, ldda,
                                                                             n_tok, Hkv, C);
  return hipGetLastError();
}

size_t nc_outer_scratch_floats(int H, int C) { return (size_t)kOuterParts * H * C; }

hipError_t nc_outer_accumulate(int dtype, const float* A, int H, const void* B, int64_t ldb,
                               const int32_t* tok, int V, int C, int n_tok, float* part,
                               float* out, hipStream_t st) {
  if (dtype)
    outer_partial_kernel<bf16><<<kOuterParts, 256, 0, st>>>(A, H, (const bf16*)B, ldb, tok, V,
                                                            C, n_tok, part);
  else
    outer_partial_kernel<float><<<kOuterParts, 256, 0, st>>>(A, H, (const float*)B, ldb, tok, V,
                                                             C, n_tok, part);
  fold_partials_kernel<<<ceil_div(H * C, 256), 256, 0, st>>>(part, kOuterParts, H * C, out);
  return hipGetLastError();
}

hipError_t nc_sum_into(const float* vals, int n, float* out, hipStream_t st) {
  sum_into_kernel<<<1, 1024, 0, st>>>(vals, n, out);
  return hipGetLastError();
}
