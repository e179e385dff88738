// GEMMs of the GPT step on gfx950.
//
// bf16 path: LDS-tiled MFMA kernel (v_mfma_f32_32x32x16_bf16), fp32 accumulate.
//   * block tile BM x BN x 64, waves arranged WM x WN, each wave owns a
//     (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles;
//   * global -> registers -> LDS, double-buffered LDS, one barrier per k-tile;
//   * every LDS tile is stored K-contiguous (row = output index, 64 k per row,
//     16-byte chunks XOR-swizzled by row) so the MFMA fragment reads are the
//     same for every operand layout; MN-contiguous operands are transposed in
//     registers (8x8 16-bit blocks) on their way into LDS;
//   * split-K over blockIdx.z for the weight-gradient products (reduction over
//     all tokens), reduced deterministically by a second kernel;
//   * tile order grouped for L2 reuse and remapped so that neighbouring tiles
//     land on the same XCD (the dispatcher deals workgroups round-robin over
//     the 8 XCDs).
// fp32 path (tiny configuration): a plain LDS-tiled VALU kernel with the same
// operand layouts and epilogues.
#include "gemm.h"

namespace {

constexpr int BK = 64;

NC_DEV int swz(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }

// ------------------------------------------------------------------ epilogue
template <typename T>
NC_DEV void epilogue_store(const GemmParams& p, int b, int m, int n, float v) {
  const int64_t off = (int64_t)b * p.sC + (int64_t)m * p.ldc + n;
  switch (p.epi) {
    case kEpiStore:
      static_cast<T*>(p.C)[off] = to_t<T>(p.alpha * v);
      break;
    case kEpiStoreF32:
      static_cast<float*>(p.C)[off] = p.alpha * v;
      break;
    case kEpiAccF32:
      static_cast<float*>(p.C)[off] += p.alpha * v;
      break;
    case kEpiRelu2: {
      const T h = to_t<T>(v);
      static_cast<T*>(p.C)[off] = h;
      const float r = fmaxf(v, 0.f);
      static_cast<T*>(p.aux_out)[off] = to_t<T>(r * r);
      break;
    }
    case kEpiRelu2Bwd: {
      const float h = to_f(static_cast<const T*>(p.aux_in)[off]);
      static_cast<T*>(p.C)[off] = to_t<T>(2.f * fmaxf(h, 0.f) * v);
      break;
    }
    case kEpiDual: {
      const float a = p.aux_in ? static_cast<const float*>(p.aux_in)[off] : 0.f;
      const float r = p.p0 * a + p.p1 * v;
      static_cast<float*>(p.C)[off] = r;
      static_cast<T*>(p.aux_out)[off] = to_t<T>(r);
      break;
    }
    case kEpiPoly: {
      const float a = to_f(static_cast<const T*>(p.aux_in)[off]);
      static_cast<T*>(p.C)[off] = to_t<T>(p.p0 * a + p.p1 * v);
      break;
    }
    default: break;
  }
}

// --------------------------------------------------------------- tile loads
// Loads a ROWS x 64 (row, k) tile of one operand into registers and stores it
// into LDS K-contiguous.  ROWS is BM (operand A) or BN (operand B).
template <int ROWS, int NT, int LAYOUT>
struct TileLoader {
  static constexpr bool KC = (LAYOUT == kKCont);
  // K-contiguous: ROWS*8 chunks of 16 B; MN-contiguous: ROWS blocks of 8x8.
  static constexpr int NCH = KC ? (ROWS * 8 + NT - 1) / NT : (ROWS + NT - 1) / NT;
  static constexpr int NREG = KC ? NCH : NCH * 8;
  u32x4 r[NREG];

  NC_DEV void load(const bf16* __restrict__ base, int64_t ld, int row0, int rows_lim,
                   int k0, int k_lim) {
    const int tid = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int id = tid + i * NT;
        const int rr = id >> 3, c = id & 7;
        const int row = row0 + rr, k = k0 + c * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (id < ROWS * 8 && row < rows_lim && k < k_lim)
          v = *reinterpret_cast<const u32x4*>(base + (int64_t)row * ld + k);
        r[i] = v;
      }
    } else {
      constexpr int RB = ROWS / 8;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int id = tid + i * NT;
        const int rb = id % RB, kb = id / RB;
        const int row = row0 + rb * 8;
        const bool ok = id < ROWS && row < rows_lim;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = k0 + kb * 8 + j;
          u32x4 v = {0u, 0u, 0u, 0u};
          if (ok && k < k_lim) v = *reinterpret_cast<const u32x4*>(base + (int64_t)k * ld + row);
          r[i * 8 + j] = v;
        }
      }
    }
  }

  NC_DEV void store(bf16* lds) const {
    const int tid = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int id = tid + i * NT;
        if (id < ROWS * 8) {
          const int rr = id >> 3, c = id & 7;
          *reinterpret_cast<u32x4*>(lds + rr * BK + swz(rr, c) * 8) = r[i];
        }
      }
    } else {
      constexpr int RB = ROWS / 8;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int id = tid + i * NT;
        if (id < ROWS) {
          const int rb = id % RB, kb = id / RB;
          u32x4 t[8];
          transpose8x8_b16(&r[i * 8], t);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int rr = rb * 8 + j;
            *reinterpret_cast<u32x4*>(lds + rr * BK + swz(rr, kb) * 8) = t[j];
          }
        }
      }
    }
  }
};

// Maps the linear workgroup id to an (m-tile, n-tile) pair: XCD-aware remap,
// then groups of GM m-tiles sweep the n-tiles together (operand reuse in L2).
NC_DEV void tile_coords(int pid, int n_pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int XCD = 8;
  if ((n_pid % XCD) == 0) pid = (pid % XCD) * (n_pid / XCD) + pid / XCD;
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int g = pid / per_group;
  const int first_m = g * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_g = pid % per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

// ------------------------------------------------------------- MFMA kernel
template <int BM, int BN, int WM, int WN, int AL, int BL>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (BM + BN) * BK];

  const int tiles_m = ceil_div(p.M, BM), tiles_n = ceil_div(p.N, BN);
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int z = blockIdx.z;
  const int b = z / p.splits, split = z % p.splits;
  const int kt_total = ceil_div(p.K, BK);
  const int kt_per = ceil_div(kt_total, p.splits);
  const int kt0 = split * kt_per;
  const int kt1 = min(kt_total, kt0 + kt_per);

  const bf16* __restrict__ A = static_cast<const bf16*>(p.A) + (int64_t)b * p.sA;
  const bf16* __restrict__ B = static_cast<const bf16*>(p.B) + (int64_t)b * p.sB;
  const int m0 = tm * BM, n0 = tn * BN;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  TileLoader<BM, NT, AL> la;
  TileLoader<BN, NT, BL> lb;
  constexpr int STAGE = (BM + BN) * BK;

  if (kt0 < kt1) {
    la.load(A, p.lda, m0, p.M, kt0 * BK, p.K);
    lb.load(B, p.ldb, n0, p.N, kt0 * BK, p.K);
    la.store(smem);
    lb.store(smem + BM * BK);
  }
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) {
      la.load(A, p.lda, m0, p.M, (kt + 1) * BK, p.K);
      lb.load(B, p.ldb, n0, p.N, (kt + 1) * BK, p.K);
    }
    const bf16* as = smem + cur * STAGE;
    const bf16* bs = as + BM * BK;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = s * 2 + half;
      bf16x8 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WTM + i * 32 + l32;
        fa[i] = *reinterpret_cast<const bf16x8*>(as + r * BK + swz(r, c) * 8);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WTN + j * 32 + l32;
        fb[j] = *reinterpret_cast<const bf16x8*>(bs + r * BK + swz(r, c) * 8);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.store(smem + (cur ^ 1) * STAGE);
      lb.store(smem + (cur ^ 1) * STAGE + BM * BK);
    }
    __syncthreads();
  }

  // epilogue: 32x32 tile, lane holds column l32, rows 8*(e/4) + 4*half + e%4
  if (p.splits > 1) {
    float* W = p.workspace + ((int64_t)split * p.batch + b) * (int64_t)p.M * p.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm * WTM + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          const int n = n0 + wn * WTN + j * 32 + l32;
          if (m < p.M && n < p.N) W[(int64_t)m * p.N + n] = p.alpha * acc[i][j][e];
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * WTM + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
        const int n = n0 + wn * WTN + j * 32 + l32;
        if (m < p.M && n < p.N) epilogue_store<bf16>(p, b, m, n, acc[i][j][e]);
      }
}

// split-K reduction: C (+)= sum_s W[s] in fixed order (deterministic)
__global__ void splitk_reduce_kernel(GemmParams p) {
  const int64_t MN = (int64_t)p.M * p.N;
  const int64_t total = MN * p.batch;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int k = 0; k < p.splits; ++k) s += p.workspace[(int64_t)k * total + i];
    const int64_t b = i / MN, r = i % MN;
    const int m = (int)(r / p.N), n = (int)(r % p.N);
    float* C = static_cast<float*>(p.C) + b * p.sC + (int64_t)m * p.ldc + n;
    if (p.epi == kEpiAccF32) *C += s; else *C = s;
  }
}

// ------------------------------------------------------------- fp32 kernel
// 64x64 tile, k-step 16, 256 threads each computing 4x4 outputs.
template <int AL, int BL>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  constexpr int T = 64, KS = 16;
  __shared__ float As[KS][T + 4];
  __shared__ float Bs[KS][T + 4];
  const int tiles_n = ceil_div(p.N, T);
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int b = blockIdx.z;
  const float* A = static_cast<const float*>(p.A) + (int64_t)b * p.sA;
  const float* B = static_cast<const float*>(p.B) + (int64_t)b * p.sB;
  const int m0 = tm * T, n0 = tn * T;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += KS) {
    for (int e = threadIdx.x; e < T * KS; e += 256) {
      int r, k;
      if (AL == kKCont) { r = e / KS; k = e % KS; } else { k = e / T; r = e % T; }
      const int gm = m0 + r, gk = k0 + k;
      As[k][r] = (gm < p.M && gk < p.K)
                     ? A[AL == kKCont ? (int64_t)gm * p.lda + gk : (int64_t)gk * p.lda + gm]
                     : 0.f;
      if (BL == kKCont) { r = e / KS; k = e % KS; } else { k = e / T; r = e % T; }
      const int gn = n0 + r;
      const int gk2 = k0 + k;
      Bs[k][r] = (gn < p.N && gk2 < p.K)
                     ? B[BL == kKCont ? (int64_t)gn * p.ldb + gk2 : (int64_t)gk2 * p.ldb + gn]
                     : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < p.M && n < p.N) epilogue_store<float>(p, b, m, n, acc[i][j]);
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_bf16_cfg(const GemmParams& p, hipStream_t st) {
  const int tiles = ceil_div(p.M, BM) * ceil_div(p.N, BN);
  dim3 grid(tiles, 1, p.batch * p.splits);
  dim3 block(WM * WN * 64);
  const int code = p.a_layout * 2 + p.b_layout;
  switch (code) {
    case 0: gemm_bf16_kernel<BM, BN, WM, WN, kKCont, kKCont><<<grid, block, 0, st>>>(p); break;
    case 1: gemm_bf16_kernel<BM, BN, WM, WN, kKCont, kMNCont><<<grid, block, 0, st>>>(p); break;
    case 2: gemm_bf16_kernel<BM, BN, WM, WN, kMNCont, kKCont><<<grid, block, 0, st>>>(p); break;
    default: gemm_bf16_kernel<BM, BN, WM, WN, kMNCont, kMNCont><<<grid, block, 0, st>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace

int nc_gemm_pick_splits(int M, int N, int K) {
  const int tiles = ceil_div(M, 256) * ceil_div(N, 256);
  int s = 1;
  const int kt = ceil_div(K, BK);
  while (tiles * s < 1024 && s * 2 <= kt / 8) s *= 2;
  return s;
}

size_t nc_gemm_workspace_bytes(int M, int N, int splits) {
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

hipError_t nc_launch_gemm(int dtype, const GemmParams& p_in, hipStream_t st) {
  GemmParams p = p_in;
  if (p.M <= 0 || p.N <= 0 || p.batch <= 0) return hipSuccess;
  if (p.splits < 1) p.splits = 1;
  if (dtype == 0) {
    p.splits = 1;
    dim3 grid(ceil_div(p.M, 64) * ceil_div(p.N, 64), 1, p.batch);
    const int code = p.a_layout * 2 + p.b_layout;
    switch (code) {
      case 0: gemm_f32_kernel<kKCont, kKCont><<<grid, 256, 0, st>>>(p); break;
      case 1: gemm_f32_kernel<kKCont, kMNCont><<<grid, 256, 0, st>>>(p); break;
      case 2: gemm_f32_kernel<kMNCont, kKCont><<<grid, 256, 0, st>>>(p); break;
      default: gemm_f32_kernel<kMNCont, kMNCont><<<grid, 256, 0, st>>>(p); break;
    }
    return hipGetLastError();
  }
  if (p.K <= 0) return hipErrorInvalidValue;
  hipError_t e = launch_bf16_cfg<256, 256, 2, 2>(p, st);
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t total = (int64_t)p.M * p.N * p.batch;
  const int blocks = (int)std::min<int64_t>(ceil_div64(total, 256), 65536);
  splitk_reduce_kernel<<<blocks, 256, 0, st>>>(p);
  return hipGetLastError();
}
