// Shared device/host helpers for the gfx950 kernels of the GPT step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define NC_DEV __device__ __forceinline__
#define NC_HD __host__ __device__ __forceinline__

static constexpr int kWave = 64;

NC_HD int clamp_id(int v, int V) { return v < 0 ? 0 : (v >= V ? V - 1 : v); }
NC_HD int ceil_div(int a, int b) { return (a + b - 1) / b; }
NC_HD int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// float <-> storage type conversions (bf16 rounding is round-to-nearest-even)
template <typename T> NC_DEV T to_t(float v);
template <> NC_DEV float to_t<float>(float v) { return v; }
template <> NC_DEV bf16 to_t<bf16>(float v) { return static_cast<bf16>(v); }
NC_DEV float to_f(float v) { return v; }
NC_DEV float to_f(bf16 v) { return static_cast<float>(v); }

// ---------------------------------------------------------------- reductions
NC_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
NC_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Block-wide sum; every thread gets the result.  `red` must hold blockDim/64 floats.
NC_DEV float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}
NC_DEV float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = -INFINITY;
  for (int i = 0; i < nw; ++i) s = fmaxf(s, red[i]);
  return s;
}

// The maximum that keeps a NaN (fmaxf drops it): a NaN anywhere in a tensor
// makes its fp8 amax and scale NaN, and with them every code (0x7F).
NC_DEV float max_nan(float a, float b) { return (a > b || a != a) ? a : b; }
NC_DEV float block_max_nan(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max_nan(v, __shfl_xor(v, o, kWave));
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s = max_nan(s, red[i]);
  return s;
}
// |x| rounded to bf16 as a float: round-to-nearest is monotonic, so the largest
// |bf16(x_i)| of a set equals bf16(max |x_i|), and a producer can keep the max
// of its fp32 values and round once
NC_DEV float bf16_abs(float x) { return fabsf(static_cast<float>(static_cast<bf16>(x))); }

// ------------------------------------------------------ 8x8 16-bit transpose
// in[j] holds 8 consecutive 16-bit values of row j (4 dwords); out[i] receives
// column i, i.e. element i of every row, as 8 consecutive 16-bit values.
NC_DEV void transpose8x8_b16(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // low half from row 2q, high half from row 2q+1, both element i
      out[i][q] = __builtin_amdgcn_perm(in[2 * q + 1][i >> 1], in[2 * q][i >> 1], sel);
    }
  }
}
