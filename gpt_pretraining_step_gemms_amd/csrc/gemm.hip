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

#include <type_traits>

namespace {

constexpr int BK = 64;

NC_DEV int swz(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }

// ------------------------------------------------------------------ epilogue
// One output element at offset `off` of C (and of aux_in / aux_out); every
// epilogue takes acc = alpha * v.  The ReLU^2 epilogues return |the value
// before rounding| (for the output's amax), the others 0.
template <typename T, int EPI>
NC_DEV float epi_one(const GemmParams& p, int64_t off, float v) {
  if constexpr (EPI == kEpiStore) {
    static_cast<T*>(p.C)[off] = to_t<T>(p.alpha * v);
  } else if constexpr (EPI == kEpiStoreF32) {
    static_cast<float*>(p.C)[off] = p.alpha * v;
  } else if constexpr (EPI == kEpiAccF32) {
    static_cast<float*>(p.C)[off] += p.alpha * v;
  } else if constexpr (EPI == kEpiRelu2) {
    const float r = fmaxf(p.alpha * v, 0.f);
    static_cast<T*>(p.C)[off] = to_t<T>(r * r);
    return r * r;
  } else if constexpr (EPI == kEpiRelu2Bwd) {
    // v_sqrt_f32 (1 ulp) rather than the correctly rounded library sequence
    const float g = to_f(static_cast<const T*>(p.aux_in)[off]);
    const float r = 2.f * __builtin_amdgcn_sqrtf(fmaxf(g, 0.f)) * (p.alpha * v);
    static_cast<T*>(p.C)[off] = to_t<T>(r);
    return fabsf(r);
  } else if constexpr (EPI == kEpiPoly) {
    const float a = to_f(static_cast<const T*>(p.aux_in)[off]);
    static_cast<T*>(p.C)[off] = to_t<T>(p.p0 * a + p.p1 * (p.alpha * v));
  } else {  // kEpiDual
    const float a = p.aux_in ? static_cast<const float*>(p.aux_in)[off] : 0.f;
    const float r = p.p0 * a + p.p1 * (p.alpha * v);
    static_cast<float*>(p.C)[off] = r;
    static_cast<T*>(p.aux_out)[off] = to_t<T>(r);
  }
  return 0.f;
}

// largest |r[e]| of 8 values, NaN kept
NC_DEV float amax8(const float (&r)[8]) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = max_nan(m, fabsf(r[e]));
  return m;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// st8 writes GEMM outputs with non-temporal stores: the outputs (hundreds of
// MB per product) are not re-read from L2, and streaming them measured 2.5-3 %
// faster on the store-heavy products and 6.5 % on the ReLU^2 backward.
NC_DEV void ld8(const bf16* q, float (&x)[8]) {
  const bf16x8 h = *reinterpret_cast<const bf16x8*>(q);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(h[e]);
}
NC_DEV void st8(bf16* q, const float (&x)[8]) {
  bf16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = static_cast<bf16>(x[e]);
  __builtin_nontemporal_store(h, reinterpret_cast<bf16x8*>(q));
}
NC_DEV void ld8(const float* q, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(q), b = *reinterpret_cast<const f32x4*>(q + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[e + 4] = b[e]; }
}
NC_DEV void st8(float* q, const float (&x)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) { a[e] = x[e]; b[e] = x[e + 4]; }
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(q));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(q + 4));
}

// Eight consecutive outputs of one row at offset `off` of C (and aux), with
// 16-byte accesses: the same arithmetic as epi_one (bf16 activations).
template <int EPI>
NC_DEV float epi_vec8(const GemmParams& p, int64_t off, const float (&v)[8]) {
  float r[8], a[8];
  if constexpr (EPI == kEpiStore) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = p.alpha * v[e];
    st8(static_cast<bf16*>(p.C) + off, r);
  } else if constexpr (EPI == kEpiStoreF32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = p.alpha * v[e];
    st8(static_cast<float*>(p.C) + off, r);
  } else if constexpr (EPI == kEpiAccF32) {
    ld8(static_cast<const float*>(p.C) + off, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = a[e] + p.alpha * v[e];
    st8(static_cast<float*>(p.C) + off, r);
  } else if constexpr (EPI == kEpiRelu2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = fmaxf(p.alpha * v[e], 0.f);
      r[e] = t * t;
    }
    st8(static_cast<bf16*>(p.C) + off, r);
    return amax8(r);
  } else if constexpr (EPI == kEpiRelu2Bwd) {
    ld8(static_cast<const bf16*>(p.aux_in) + off, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = 2.f * __builtin_amdgcn_sqrtf(fmaxf(a[e], 0.f)) * (p.alpha * v[e]);
    st8(static_cast<bf16*>(p.C) + off, r);
    return amax8(r);
  } else if constexpr (EPI == kEpiPoly) {
    ld8(static_cast<const bf16*>(p.aux_in) + off, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = p.p0 * a[e] + p.p1 * (p.alpha * v[e]);
    st8(static_cast<bf16*>(p.C) + off, r);
  } else {  // kEpiDual
    if (p.aux_in) {
      ld8(static_cast<const float*>(p.aux_in) + off, a);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = p.p0 * a[e] + p.p1 * (p.alpha * v[e]);
    st8(static_cast<float*>(p.C) + off, r);
    st8(static_cast<bf16*>(p.aux_out) + off, r);
  }
  return 0.f;
}

// The epilogue in two phases, so that a wave can issue the loads of several
// row groups before any of its stores: a load issued after a store would wait
// for that store (the wait counter is shared), which serialised one load
// latency per 8 outputs.  EpiIn<EPI> is what an epilogue reads back for 8
// consecutive outputs (raw, converted only when applied): nothing, 8 bf16 of
// aux_in, or 8 fp32 of C or aux_in.
template <int EPI>
constexpr int epi_reads() {
  return EPI == kEpiAccF32 || EPI == kEpiDual ? 2 : (EPI == kEpiRelu2Bwd || EPI == kEpiPoly ? 1 : 0);
}
template <int EPI>
struct EpiIn {
  f32x4 f[epi_reads<EPI>() == 2 ? 2 : 1];
  bf16x8 h;
};
// (single-use streams: non-temporal loads, 1-3 % faster on the reading epilogues)
template <int EPI>
NC_DEV void epi_load8(const GemmParams& p, int64_t off, EpiIn<EPI>& in) {
  auto ld4 = [](const float* q) { return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(q)); };
  if constexpr (EPI == kEpiAccF32) {
    in.f[0] = ld4(static_cast<const float*>(p.C) + off);
    in.f[1] = ld4(static_cast<const float*>(p.C) + off + 4);
  } else if constexpr (EPI == kEpiDual) {
    if (p.aux_in) {
      in.f[0] = ld4(static_cast<const float*>(p.aux_in) + off);
      in.f[1] = ld4(static_cast<const float*>(p.aux_in) + off + 4);
    } else {
      in.f[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      in.f[1] = in.f[0];
    }
  } else if constexpr (EPI == kEpiRelu2Bwd || EPI == kEpiPoly) {
    in.h = __builtin_nontemporal_load(
        reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p.aux_in) + off));
  }
}
// Same arithmetic as epi_one / epi_vec8, on values read by epi_load8.
template <int EPI>
NC_DEV float epi_apply8(const GemmParams& p, int64_t off, const float (&v)[8],
                        const EpiIn<EPI>& in) {
  float a[8], r[8];
  if constexpr (epi_reads<EPI>() == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { a[e] = in.f[0][e]; a[e + 4] = in.f[1][e]; }
  } else if constexpr (epi_reads<EPI>() == 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = static_cast<float>(in.h[e]);
  }
  if constexpr (EPI == kEpiAccF32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = a[e] + p.alpha * v[e];
    st8(static_cast<float*>(p.C) + off, r);
  } else if constexpr (EPI == kEpiRelu2Bwd) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = 2.f * __builtin_amdgcn_sqrtf(fmaxf(a[e], 0.f)) * (p.alpha * v[e]);
    st8(static_cast<bf16*>(p.C) + off, r);
    return amax8(r);
  } else if constexpr (EPI == kEpiPoly) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = p.p0 * a[e] + p.p1 * (p.alpha * v[e]);
    st8(static_cast<bf16*>(p.C) + off, r);
  } else if constexpr (EPI == kEpiDual) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = p.p0 * a[e] + p.p1 * (p.alpha * v[e]);
    st8(static_cast<float*>(p.C) + off, r);
    st8(static_cast<bf16*>(p.aux_out) + off, r);
  } else {
    return epi_vec8<EPI>(p, off, v);               // stores only
  }
  return 0.f;
}

// Calls f.template operator()<EPI>() with the epilogue chosen at run time, so
// that each element loop is compiled for one epilogue.
template <typename F>
NC_DEV void with_epilogue(int epi, F&& f) {
  switch (epi) {
    case kEpiStore: f.template operator()<kEpiStore>(); break;
    case kEpiStoreF32: f.template operator()<kEpiStoreF32>(); break;
    case kEpiAccF32: f.template operator()<kEpiAccF32>(); break;
    case kEpiRelu2: f.template operator()<kEpiRelu2>(); break;
    case kEpiRelu2Bwd: f.template operator()<kEpiRelu2Bwd>(); break;
    case kEpiPoly: f.template operator()<kEpiPoly>(); break;
    default: f.template operator()<kEpiDual>(); break;
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
  const int64_t cb = (int64_t)b * p.sC;
  with_epilogue(p.epi, [&]<int EPI>() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm * WTM + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          const int n = n0 + wn * WTN + j * 32 + l32;
          if (m < p.M && n < p.N) epi_one<bf16, EPI>(p, cb + (int64_t)m * p.ldc + n, acc[i][j][e]);
        }
  });
}

// split-K reduction, one block per output row, four columns per thread:
// C (+)= sum_s W[s] in fixed order (deterministic; same sums as below).
// Needs N, ldc and sC multiples of 4 and a 16-byte aligned C.
__global__ __launch_bounds__(256) void splitk_reduce_rows_kernel(GemmParams p) {
  const int row = blockIdx.x;                      // b * M + m
  const int b = row / p.M, m = row - b * p.M;
  const int64_t total = (int64_t)p.M * p.N * p.batch;
  const float* w = p.workspace + (int64_t)row * p.N;
  float* c = static_cast<float*>(p.C) + b * p.sC + (int64_t)m * p.ldc;
  // (the slabs are read once: non-temporal loads, unrolled so that several
  // are in flight; the sum keeps the fixed split order)
  for (int n = threadIdx.x * 4; n < p.N; n += blockDim.x * 4) {
    f32x4 acc = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(w + n));
#pragma unroll 4
    for (int k = 1; k < p.splits; ++k)
      acc += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(w + k * total + n));
    f32x4* out = reinterpret_cast<f32x4*>(c + n);
    if (p.epi == kEpiAccF32) *out = *out + acc; else *out = acc;
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
  const int64_t cb = (int64_t)b * p.sC;
  with_epilogue(p.epi, [&]<int EPI>() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
        if (m < p.M && n < p.N) epi_one<float, EPI>(p, cb + (int64_t)m * p.ldc + n, acc[i][j]);
      }
  });
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

// ======================================== direct-to-LDS pipelined MFMA kernel
// Operand tiles travel global -> LDS with buffer_load ... lds (each lane moves
// 16 bytes; a wave's 64 lanes fill 1 KB of LDS contiguously), with no staging
// registers, through a ring of k-steps: 4 stages of 256x32 + 256x32 bf16
// tiles, or 2 stages of 256x64 + 256x64, or (both operands K-contiguous) the
// half-stage ring of five 256x64 operand tiles.  LDS keeps each operand in its
// global layout:
//   K-contiguous  [256 rows][32 or 64 k], 16-byte chunk c of row r stored at
//                 c ^ ((r >> 2) & 3) (depth 32) or c ^ ((r >> 1) & 7) (depth
//                 64)                             -> read with ds_read_b128;
//   MN-contiguous [32 or 64 k][256 rows], chunk c of k-row kr stored at
//                 c ^ mn_swz(kr), mn_swz(kr) = 4 (kr & 3) ^ 2 ((kr >> 3) & 1)
//                 -> read with ds_read_b64_tr_b16, which hands each lane of a
//                 16-lane group one column of a 4 x 16 block, i.e. 4 consecutive
//                 k of one output row: the MFMA operand layout.  (The k-row bit
//                 3 term keeps the 16 x 16 x 32 reads, whose lanes 16-31 read
//                 the k-rows 8 below lanes 0-15, off the same 64 banks.)
// Both swizzles make the fragment reads bank-conflict free; the swizzle is
// applied by choosing which global chunk each lane fetches.  Needs K % 32 == 0;
// rows beyond M or N lie past the operand's buffer range, read as zeros and
// only feed outputs that are discarded.
// Each wave owns a 128 x 64 output tile (4 x 2 tiles of 32 x 32 x 16 MFMAs or
// 8 x 4 tiles of 16 x 16 x 32 MFMAs): WM x WN waves make a (128 WM) x (64 WN)
// block tile; the launcher uses 2 x 4 waves (256 x 256 tiles, 128 or 160 KB of
// LDS, one block per CU).
template <int WM_, int WN_, int ST_, int PK_ = 32, int MI_ = 32, int WTN_ = 64>
struct Pipe {
  static constexpr int BM = 128 * WM_, BN = WTN_ * WN_, PK = PK_, STAGES = ST_;
  // MFMA shape: 32 (v_mfma_f32_32x32x16_bf16) or 16 (v_mfma_f32_16x16x32_bf16)
  static constexpr int MI = MI_, KSUB = MI_ == 32 ? 16 : 32;
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int kBlocksPerCU = (BM + BN) * PK * 2 * ST_ <= 80 * 1024 ? 2 : 1;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / MI, TN = WTN / MI;
  static constexpr int TILE_A = BM * PK, TILE_B = BN * PK, STAGE = TILE_A + TILE_B;
  static constexpr int LOADS_A = TILE_A * 2 / 1024 / (NT / 64);
  static constexpr int LOADS_B = TILE_B * 2 / 1024 / (NT / 64);
  static constexpr int LOADS = LOADS_A + LOADS_B;   // global_load_lds per wave per stage
  // STAGES == 5 is the half-stage ring: five buffers, each holding one
  // operand tile (A or B) of one k-step, so one and a half tiles load ahead.
  static constexpr bool HALF = ST_ == 5;
  static constexpr int BUF = HALF ? TILE_A : STAGE;  // bf16 elements per LDS buffer
  static_assert(!HALF || TILE_A == TILE_B, "the half-stage ring needs square block tiles");
};

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#define NC_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

typedef int i32x4 __attribute__((ext_vector_type(4)));

// An operand for the direct-to-LDS loads: a raw buffer resource over the
// operand's bytes (gfx9 layout: stride 0, dword 3 = 0x00020000), so that a load
// past the end reads zeros instead of touching memory, plus each lane's byte
// offset inside a 1-KB block for the two block parities (the LDS swizzle
// alternates between even and odd blocks).
struct Opnd {
  i32x4 rsrc;
  unsigned lane_off[4];                          // by block bit 0 (and bit 2, MN-contiguous)
  unsigned ld2;                                  // leading dimension in bytes
};

// Byte extent of a bf16 operand slice: rows of ld elements, the last one
// holding `last` elements.
__host__ __device__ inline int64_t operand_extent(int64_t rows, int64_t ld, int64_t last) {
  return rows <= 0 ? 0 : ((rows - 1) * ld + last) * 2;
}

// ROWS x PK tile layouts (see the kernel comment): K-contiguous blocks cover
// 16 (PK 32) or 8 (PK 64) rows of one k-step; MN-contiguous blocks cover 2
// k-rows of 256 columns.
template <int ROWS, int LAYOUT, int PK>
NC_DEV Opnd make_opnd(const bf16* base, int64_t ld, int64_t bytes, int lane) {
  static_assert(LAYOUT == kKCont || ROWS == 256, "MN-contiguous tiles are 256 wide");
  Opnd o;
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  o.rsrc[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  o.rsrc[1] = __builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xffffu));
  o.rsrc[2] = __builtin_amdgcn_readfirstlane((int)(unsigned)bytes);
  o.rsrc[3] = 0x00020000;
  o.ld2 = (unsigned)ld * 2u;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int par = v & 1, b2 = v >> 1;            // bits 0 and 2 of the block index
    unsigned r, c;
    if constexpr (LAYOUT == kKCont && PK == 32) {  // row r = 16 blk + lane / 4
      r = lane >> 2;
      c = (lane & 3) ^ ((lane >> 4) & 3);          // (r >> 2) & 3 of the tile row
    } else if constexpr (LAYOUT == kKCont) {       // row r = 8 blk + lane / 8
      r = lane >> 3;
      c = (lane & 7) ^ (4 * par + (r >> 1));       // (r >> 1) & 7 of the tile row
    } else {                                       // k-row kr = 2 blk + lane / 32
      r = lane >> 5;
      c = (lane & 31) ^ (4 * ((2 * par + r) & 3)) ^ (2 * b2);   // mn_swz(kr)
    }
    o.lane_off[v] = r * o.ld2 + c * 16u;
  }
  return o;
}

// buffer_load_dwordx4 ... lds: lane l's 16 bytes at byte offset voff of the
// operand land at LDS address lds + 16 l (lds is wave-uniform, passed in M0).
// Issued as inline assembly: the instruction has no register result, and the
// kernel tracks its completion itself (s_waitcnt vmcnt + s_barrier), which
// keeps the compiler from draining every load in flight before each LDS read.
// M0 is restored.
NC_DEV void dma16(const i32x4& rsrc, unsigned voff, const bf16* lds) {
  const unsigned a = (unsigned)(size_t)NC_LDS(const void, lds);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(a))
      : "memory");
}

// Load number i (0 <= i < NI) of this wave's NI 1-KB loads of the ROWS x PK
// operand tile at (row0, k0).  The block's wave-uniform offset is computed in
// scalar registers; rows (or columns) past the operand read as zeros and only
// feed outputs that are discarded.
template <int ROWS, int LAYOUT, int NI, int PK>
NC_DEV void issue_one(const Opnd& o, int row0, int k0, bf16* tile, int wave, int i) {
  const int blk = wave * NI + i;                 // 1-KB block of the tile
  unsigned u;
  if constexpr (LAYOUT == kKCont)
    u = (unsigned)(row0 + blk * (PK == 32 ? 16 : 8)) * o.ld2 + (unsigned)k0 * 2u;
  else
    u = (unsigned)(k0 + blk * 2) * o.ld2 + (unsigned)row0 * 2u;
  u = __builtin_amdgcn_readfirstlane(u);
  // explicit selects (a runtime array index would move lane_off to scratch)
  unsigned lo = (blk & 1) ? o.lane_off[1] : o.lane_off[0];
  if constexpr (LAYOUT != kKCont) {
    const unsigned hi = (blk & 1) ? o.lane_off[3] : o.lane_off[2];
    lo = ((blk >> 2) & 1) ? hi : lo;
  }
  dma16(o.rsrc, lo + u, tile + blk * 512);
}

// This wave's NI 1-KB loads of a ROWS x PK operand tile.
template <int ROWS, int LAYOUT, int NI, int PK>
NC_DEV void issue_tile(const Opnd& o, int row0, int k0, bf16* tile, int wave) {
#pragma unroll
  for (int i = 0; i < NI; ++i) issue_one<ROWS, LAYOUT, NI, PK>(o, row0, k0, tile, wave, i);
}

// MFMA operand fragment from a tile: 8 consecutive k of one output row, for
// k-substep s.  32 x 32 x 16: row o0 + lane % 32, k 8 (lane / 32) of the
// substep's 16; 16 x 16 x 32: row o0 + lane % 16, k 8 (lane / 16) of its 32.
template <int ROWS, int LAYOUT, int PK, int MI>
NC_DEV bf16x8 frag(const bf16* tile, int o0, int s, int lane) {
  if constexpr (LAYOUT == kKCont) {
    const int r = o0 + (MI == 32 ? (lane & 31) : (lane & 15));
    const int c = MI == 32 ? s * 2 + (lane >> 5) : s * 4 + (lane >> 4);
    const int sw = PK == 32 ? (r >> 2) & 3 : (r >> 1) & 7;
    return *reinterpret_cast<const bf16x8*>(tile + r * PK + ((c ^ sw) << 3));
  } else {
    // each 16-lane group reads a 4 (k) x 16 (rows) block twice (k and k + 4);
    // ds_read_b64_tr_b16 hands lane t of the group row t's 4 consecutive k
    const int g = lane >> 4, t = lane & 15;
    const int k = MI == 32 ? s * 16 + 8 * (g >> 1) + (t >> 2) : s * 32 + 8 * g + (t >> 2);
    const int o = o0 + (MI == 32 ? 16 * (g & 1) : 0) + 4 * (t & 3);
    const int sw = (4 * (k & 3)) ^ (2 * ((k >> 3) & 1));   // mn_swz(k), same for k + 4
    const bf16* p0 = tile + k * ROWS + (((o >> 3) ^ sw) << 3) + (o & 7);
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(NC_LDS(bf16x4_t, p0));
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(NC_LDS(bf16x4_t, p0 + 4 * ROWS));
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  }
}

template <int N>
NC_DEV void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One v_mfma_f32_16x16x128_f8f6f4: a lane's 32 operand bytes are the two
// 16-byte fragments the bf16 path reads for the two 32-deep substeps of a
// 64-element (128-byte) k-step.  Both operands take the same byte positions, so
// each of the step's 128 k is summed exactly once.  FA is A's format (0: e4m3,
// 1: e5m2, the instruction's format codes); B is e4m3.
template <int FA>
NC_DEV f32x4 mfma_f8(bf16x8 a0, bf16x8 a1, bf16x8 b0, bf16x8 b1, f32x4 c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x4 x0 = __builtin_bit_cast(i32x4, a0), x1 = __builtin_bit_cast(i32x4, a1);
  const i32x4 y0 = __builtin_bit_cast(i32x4, b0), y1 = __builtin_bit_cast(i32x4, b1);
  const i32x8 a = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  const i32x8 b = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, 0, 0, 0, 0, 0);
}

// F8: operands are fp8 bytes (A in format FA_, B e4m3), handled by the loads
// as pairs (the launcher halves K and the leading dimensions), K-contiguous,
// half-stage ring with 16 x 16 MFMAs only.
template <int AL, int BL, int WM_, int WN_, int ST_, int PK_, int MI_, bool F8 = false,
          int WTN_ = 64, int FA_ = 0>
__global__ __launch_bounds__(WM_ * WN_ * 64, (Pipe<WM_, WN_, ST_, PK_, MI_, WTN_>::kBlocksPerCU))
void gemm_bf16_pipe_kernel(GemmParams p) {
  using C = Pipe<WM_, WN_, ST_, PK_, MI_, WTN_>;
  constexpr int MI = C::MI;
  static_assert(!F8 || (MI == 16 && PK_ == 64 && ST_ == 5 && AL == kKCont && BL == kKCont),
                "fp8: K-contiguous operands in the 64-deep half-stage ring");
  using AccT = std::conditional_t<MI == 32, f32x16, f32x4>;
  constexpr int ACC_N = MI == 32 ? 16 : 4;
  constexpr int BM = C::BM, BN = C::BN, PK = C::PK, STAGES = C::STAGES, WN = C::WN;
  constexpr int WTM = C::WTM, WTN = C::WTN, TM = C::TM, TN = C::TN;
  constexpr int TILE_A = C::TILE_A, STAGE = C::STAGE;
  constexpr int LOADS_A = C::LOADS_A, LOADS_B = C::LOADS_B, LOADS = C::LOADS;
  constexpr int BUF = C::BUF;
  constexpr bool HALF = C::HALF;
  __shared__ __attribute__((aligned(1024))) bf16 st0[BUF];
  __shared__ __attribute__((aligned(1024))) bf16 st1[BUF];
  __shared__ __attribute__((aligned(1024))) bf16 st2[BUF];
  __shared__ __attribute__((aligned(1024))) bf16 st3[BUF];
  __shared__ __attribute__((aligned(1024))) bf16 st4[HALF ? BUF : 1];

  const int tiles_m = ceil_div(p.M, BM), tiles_n = ceil_div(p.N, BN);
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int z = blockIdx.z;
  const int b = z / p.splits, split = z % p.splits;
  const int kt_total = p.K / PK;
  const int kt_per = ceil_div(kt_total, p.splits);
  const int kt0 = split * kt_per;
  const int nk = max(0, min(kt_total, kt0 + kt_per) - kt0);

  const bf16* __restrict__ A = static_cast<const bf16*>(p.A) + (int64_t)b * p.sA;
  const bf16* __restrict__ B = static_cast<const bf16*>(p.B) + (int64_t)b * p.sB;
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;
  const Opnd oa = make_opnd<BM, AL, PK>(
      A, p.lda, AL == kKCont ? operand_extent(p.M, p.lda, p.K) : operand_extent(p.K, p.lda, p.M),
      lane);
  const Opnd ob = make_opnd<BN, BL, PK>(
      B, p.ldb, BL == kKCont ? operand_extent(p.N, p.ldb, p.K) : operand_extent(p.K, p.ldb, p.N),
      lane);

  AccT acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < ACC_N; ++e) acc[i][j][e] = 0.f;

  // Each stage is its own LDS object and the loop is unrolled over the 4
  // stages, so the compiler can tell that the loads in flight (other stages)
  // do not alias the stage being read and emits no drain before its reads.
  auto sbuf = [&]<int S>() -> bf16* {
    if constexpr (S == 0) return st0;
    else if constexpr (S == 1) return st1;
    else if constexpr (S == 2) return st2;
    else if constexpr (S == 3) return st3;
    else return st4;
  };
  auto issue = [&](int kt, bf16* st) {
    issue_tile<BM, AL, LOADS_A, PK>(oa, m0, kt * PK, st, wave);
    issue_tile<BN, BL, LOADS_B, PK>(ob, n0, kt * PK, st + TILE_A, wave);
  };
  bf16x8 frA[C::TM], frB[2][C::TN];                  // fragments of the mid-step schedule
  auto step = [&]<int S>(int i) {
    if constexpr (HALF) {
      // loads go out as B of tile i + 1, then A of tile i + 2: tile i has
      // landed once at most the A loads of tile i + 1 remain
      if (i + 1 < nk) wait_vmcnt<LOADS_A>();
      else wait_vmcnt<0>();
    } else {
      // tile i has landed once at most the loads of the (up to two) younger tiles remain
      const int younger = min(nk - 1 - i, STAGES - 2);
      if (younger >= 2) wait_vmcnt<2 * LOADS>();
      else if (younger == 1) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
    }
    // Plain barrier: every wave has waited for its own loads of tile i above,
    // and has consumed its fragment reads of tile i-1 (whose stage the next
    // issue overwrites).  A fenced __syncthreads would also drain the younger
    // prefetches.
    asm volatile("s_barrier" ::: "memory");
    // The loads of tile i + STAGES - 1 are spread between this step's MFMAs
    // (one after every MPL of them, pinned with scheduling barriers): a wave
    // issues in order, so loads issued back to back would hold back the
    // fragment reads and MFMAs behind them, while an MFMA in the matrix pipe
    // covers the issue of the load after it.
    // half ring: A of tile t in buffer 2t mod 5, B in 2t + 1 mod 5; this step
    // loads B of tile i + 1 into the buffer A of tile i - 1 held and A of
    // tile i + 2 into that of B of tile i - 1, both read before the barrier
    const bool more = HALF ? i + 1 < nk : i + STAGES - 1 < nk;
    const bool more_a2 = i + 2 < nk;
    const int ktn = kt0 + i + (HALF ? 1 : STAGES - 1);
    bf16* nxt = HALF ? nullptr : sbuf.template operator()<(S + STAGES - 1) % STAGES>();
    bf16* nxt_b = HALF ? sbuf.template operator()<(2 * S + 3) % 5>() : nxt + TILE_A;
    bf16* nxt_a2 = HALF ? sbuf.template operator()<(2 * S + 4) % 5>() : nullptr;
    const bf16* as = HALF ? sbuf.template operator()<(2 * S) % 5>() : sbuf.template operator()<S>();
    const bf16* bs = HALF ? sbuf.template operator()<(2 * S + 1) % 5>() : as + TILE_A;
    // With two stages the next tile is waited for at the start of the next
    // step, so its loads go early (one per MFMA of the first substep); with
    // more stages they are spread over the whole step.
    constexpr int NSUB = PK / C::KSUB, NM = TM * TN;
    constexpr int SPAN = (STAGES == 2 || HALF) ? NM : NSUB * NM;   // MFMAs the loads are spread over
    constexpr int MPL = SPAN / LOADS;                    // MFMAs per load (rounded down)
    static_assert(MPL >= 1, "at most one load per MFMA");
    // Fragments of substep s + 1 are read one at a time between the MFMAs of
    // substep s (two register sets), so only the first substep after the
    // barrier waits for LDS.  Measured faster for every layout but A
    // K-contiguous with B MN-contiguous, which reads each substep's
    // fragments at its start; both MN-contiguous with 16 x 16 x 32 MFMAs
    // has no registers for the second set.
    constexpr bool PREF = !(AL == kKCont && BL == kMNCont) &&
                          !(AL == kMNCont && BL == kMNCont && MI == 16);
    constexpr int NR = TM + TN;                        // fragment reads per substep
    static_assert(NR <= NM, "one read per MFMA slot");
    bf16x8 fr[2][NR];
    auto read_one = [&](int s, int r, bf16x8& dst) {
      if (r < TM) dst = frag<BM, AL, PK, MI>(as, wm * WTM + r * MI, s, lane);
      else dst = frag<BN, BL, PK, MI>(bs, wn * WTN + (r - TM) * MI, s, lane);
    };
    // next tiles' loads, one at MFMA index u of the step
    auto load_at = [&](int u) {
      if constexpr (HALF) {
        const int l = u / MPL;
        if (u < SPAN && u % MPL == 0 && l < LOADS && (l < LOADS_B ? more : more_a2)) {
          __builtin_amdgcn_sched_barrier(0);
          if (l < LOADS_B)
            issue_one<BN, BL, LOADS_B, PK>(ob, n0, ktn * PK, nxt_b, wave, l);
          else
            issue_one<BM, AL, LOADS_A, PK>(oa, m0, (ktn + 1) * PK, nxt_a2, wave, l - LOADS_B);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else if (u < SPAN && u % MPL == 0 && u / MPL < LOADS && more) {
        const int l = u / MPL;                       // load index
        __builtin_amdgcn_sched_barrier(0);
        if (l < LOADS_A)
          issue_one<BM, AL, LOADS_A, PK>(oa, m0, ktn * PK, nxt, wave, l);
        else
          issue_one<BN, BL, LOADS_B, PK>(ob, n0, ktn * PK, nxt_b, wave, l - LOADS_A);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (F8) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        read_one(0, r, fr[0][r]);
        read_one(1, r, fr[1][r]);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        const int ii = t / TN, j = t % TN;
        acc[ii][j] = mfma_f8<FA_>(fr[0][ii], fr[1][ii], fr[0][TM + j], fr[1][TM + j], acc[ii][j]);
        load_at(t);
      }
      __builtin_amdgcn_s_setprio(0);
      return;
    }
    if constexpr (PREF) {
#pragma unroll
      for (int r = 0; r < NR; ++r) read_one(0, r, fr[0][r]);
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      bf16x8 (&cur)[NR] = fr[PREF ? s & 1 : 0];
      bf16x8 (&nxf)[NR] = fr[(s + 1) & 1];
      if constexpr (!PREF) {
#pragma unroll
        for (int r = 0; r < NR; ++r) read_one(s, r, cur[r]);
      }
      // Raised wave priority over the substep's MFMAs: 1.5-2 % faster with A
      // K-contiguous (forward and input-gradient products), 1.7 % slower for the
      // weight gradients, where it stays off.
      if constexpr (AL == kKCont) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        const int ii = t / TN, j = t % TN;
        if constexpr (MI == 32)
          acc[ii][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[ii], cur[TM + j], acc[ii][j], 0, 0, 0);
        else
          acc[ii][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur[ii], cur[TM + j], acc[ii][j], 0, 0, 0);
        if constexpr (PREF) __builtin_amdgcn_sched_barrier(0);
        if (PREF && s + 1 < NSUB && t < NR) {
          read_one(s + 1, t, nxf[t]);
          __builtin_amdgcn_sched_barrier(0);
        }
        load_at(s * NM + t);                           // MFMA index within the step
      }
      if constexpr (AL == kKCont) __builtin_amdgcn_s_setprio(0);
    }
  };
  // Mid-step barrier (half-stage ring, 16 x 16 x 32 MFMAs): the wait and
  // barrier for tile i + 1 sit between the two substeps of tile i, once this
  // wave's fragment reads of tile i are complete.  The fragments of tile
  // i + 1's first substep are then read, and the loads that reuse tile i's
  // buffers issued, under the MFMAs of tile i's second substep, so no
  // substep starts with a burst of LDS reads in front of an idle matrix pipe
  // (with the barrier at the start of a step, all eight waves read their
  // first fragments at once and wait for them).
  // Registers: an A fragment is used by the TN MFMAs of one row of the wave
  // tile, so the next substep's A fragment is read into the same registers
  // right after that row's last MFMA; only the B fragments, used by every
  // row, have two sets.
  // Ring: A(t) in buffer 2t mod 5, B(t) in 2t + 1 mod 5; after the barrier of
  // step i, B(i + 2) goes into A(i)'s buffer and A(i + 3) into B(i)'s.
  // Same-box A/B against the barrier at the start of each step: forward
  // products 2-5 % faster, input gradients 1-3 %; the weight gradients (both
  // operands read transposed) need more registers for the second B set and
  // spill (13-18 % slower), so they keep the start-of-step barrier.
  constexpr bool MIDBAR = HALF && !F8 && MI == 16 &&
                          (C::NT == 256 || !(AL == kMNCont && BL == kMNCont));
  if constexpr (MIDBAR) {
    auto step_mb = [&]<int S>(int i) {
      constexpr int NSUB = PK / C::KSUB, NM = TM * TN;
      static_assert(NSUB == 2, "two substeps per k-step");
      static_assert(TN <= TN * TM && LOADS <= NM / 4, "reads and loads fit between MFMAs");
      const bf16* as = sbuf.template operator()<(2 * S) % 5>();
      const bf16* bs = sbuf.template operator()<(2 * S + 1) % 5>();
      const bf16* as1 = sbuf.template operator()<(2 * S + 2) % 5>();
      const bf16* bs1 = sbuf.template operator()<(2 * S + 3) % 5>();
      bf16* nxt_b = sbuf.template operator()<(2 * S) % 5>();
      bf16* nxt_a = sbuf.template operator()<(2 * S + 1) % 5>();
      // one substep: MFMAs on (frA, frB[cur]); reads of the next substep's
      // fragments (tile ta/tb, substep sub) into frA and frB[cur ^ 1]
      auto substep = [&](int cur, const bf16* ta, const bf16* tb, int sub, auto&& after_mfma) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < NM; ++t) {
          const int ii = t / TN, j = t % TN;
          acc[ii][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frA[ii], frB[cur][j], acc[ii][j],
                                                                0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (t < TN) {
            frB[cur ^ 1][t] = frag<BN, BL, PK, MI>(tb, wn * WTN + t * MI, sub, lane);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (j == TN - 1) {                         // row ii's last MFMA of this substep
            frA[ii] = frag<BM, AL, PK, MI>(ta, wm * WTM + ii * MI, sub, lane);
            __builtin_amdgcn_sched_barrier(0);
          }
          after_mfma(t);
        }
        __builtin_amdgcn_s_setprio(0);
      };
      substep(0, as, bs, 1, [](int) {});
      // substep 1's fragments complete on every path (the compiler then
      // places no wait for them among the reads issued after the barrier)
#pragma unroll
      for (int r = 0; r < TM; ++r) asm volatile("" : "+v"(frA[r]));
#pragma unroll
      for (int r = 0; r < TN; ++r) asm volatile("" : "+v"(frB[1][r]));
      if (i + 1 < nk) {
        // tile i + 1 has landed once at most the A loads of tile i + 2 remain
        if (i + 2 < nk) wait_vmcnt<LOADS_A>();
        else wait_vmcnt<0>();
        asm volatile("s_barrier" ::: "memory");
      }
      const bool more_b = i + 2 < nk, more_a = i + 3 < nk;
      const int kb = (kt0 + i + 2) * PK, ka = (kt0 + i + 3) * PK;
      // (after the last step the reads below fetch an idle buffer, unused)
      substep(1, as1, bs1, 0, [&](int t) {
        if (t % 4 == 1 && t / 4 < LOADS) {
          const int l = t / 4;
          if (l < LOADS_B ? more_b : more_a) {
            if (l < LOADS_B)
              issue_one<BN, BL, LOADS_B, PK>(ob, n0, kb, nxt_b, wave, l);
            else
              issue_one<BM, AL, LOADS_A, PK>(oa, m0, ka, nxt_a, wave, l - LOADS_B);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      });
    };
    if (nk > 0) {
      issue_tile<BM, AL, LOADS_A, PK>(oa, m0, kt0 * PK, st0, wave);
      issue_tile<BN, BL, LOADS_B, PK>(ob, n0, kt0 * PK, st1, wave);
      if (nk > 1) {
        issue_tile<BM, AL, LOADS_A, PK>(oa, m0, (kt0 + 1) * PK, st2, wave);
        wait_vmcnt<LOADS_A>();
      } else {
        wait_vmcnt<0>();
      }
      asm volatile("s_barrier" ::: "memory");
      if (nk > 1) issue_tile<BN, BL, LOADS_B, PK>(ob, n0, (kt0 + 1) * PK, st3, wave);
      if (nk > 2) issue_tile<BM, AL, LOADS_A, PK>(oa, m0, (kt0 + 2) * PK, st4, wave);
#pragma unroll
      for (int r = 0; r < TM; ++r) frA[r] = frag<BM, AL, PK, MI>(st0, wm * WTM + r * MI, 0, lane);
#pragma unroll
      for (int r = 0; r < TN; ++r) frB[0][r] = frag<BN, BL, PK, MI>(st1, wn * WTN + r * MI, 0, lane);
    }
    for (int i = 0; i < nk; i += 5) {
      step_mb.template operator()<0>(i);
      if (i + 1 < nk) step_mb.template operator()<1>(i + 1);
      if (i + 2 < nk) step_mb.template operator()<2>(i + 2);
      if (i + 3 < nk) step_mb.template operator()<3>(i + 3);
      if (i + 4 < nk) step_mb.template operator()<4>(i + 4);
    }
  } else if constexpr (HALF) {
    if (nk > 0) {
      issue_tile<BM, AL, LOADS_A, PK>(oa, m0, kt0 * PK, st0, wave);
      issue_tile<BN, BL, LOADS_B, PK>(ob, n0, kt0 * PK, st1, wave);
    }
    if (nk > 1) issue_tile<BM, AL, LOADS_A, PK>(oa, m0, (kt0 + 1) * PK, st2, wave);
  } else {
    if (nk > 0) issue(kt0, st0);
    if constexpr (STAGES >= 3)
      if (nk > 1) issue(kt0 + 1, st1);
    if constexpr (STAGES == 4)
      if (nk > 2) issue(kt0 + 2, st2);
  }
  if constexpr (!MIDBAR)
  for (int i = 0; i < nk; i += STAGES) {
    step.template operator()<0>(i);
    if (i + 1 < nk) step.template operator()<1>(i + 1);
    if constexpr (STAGES >= 3)
      if (i + 2 < nk) step.template operator()<2>(i + 2);
    if constexpr (STAGES >= 4)
      if (i + 3 < nk) step.template operator()<3>(i + 3);
    if constexpr (STAGES == 5)
      if (i + 4 < nk) step.template operator()<4>(i + 4);
  }

  // ---- epilogue, staged through the (now idle) stage buffers: each wave
  // writes a 32 x 64 block of its fp32 accumulators into its own padded LDS
  // region, then every lane takes 8 consecutive columns of one row, so that
  // C, the auxiliary tensors and the split-K workspace are accessed with
  // 16-byte, row-contiguous loads and stores.
  static_assert(WTN % 64 == 0, "the epilogue maps 8 lanes to 64 columns of a wave tile");
  constexpr int NH = WTN / 64, TNH = TN / NH;          // 64-column halves of the wave tile
  if constexpr (F8) {
    if (p.scale_a) {                                   // tensorwise scales kept on the device
      const float inv = 1.f / (p.scale_a[1] * p.scale_b[1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < ACC_N; ++e) acc[i][j][e] *= inv;
    }
  }
  // padded row (floats): conflict-free staging writes for either MFMA layout
  constexpr int EP_LD = MI == 32 ? 72 : 68;
  constexpr int EP_FLOATS = 32 * EP_LD;
  constexpr int EP_PER = BUF * 2 / (EP_FLOATS * 4);    // wave regions per stage buffer
  constexpr int EP_BUFS = STAGES < 3 ? STAGES : 3;
  static_assert(C::NT / 64 <= EP_BUFS * EP_PER, "staging must fit in the stage buffers");
  asm volatile("s_barrier" ::: "memory");            // every wave is done with the ring
  const int sidx = wave / EP_PER;
  bf16* sbase;
  if constexpr (EP_BUFS >= 3) sbase = sidx == 0 ? st0 : (sidx == 1 ? st1 : st2);
  else sbase = sidx == 0 ? st0 : st1;
  float* stg = reinterpret_cast<float*>(sbase) + (wave % EP_PER) * EP_FLOATS;
  const bool split_out = p.splits > 1;
  float amx = 0.f;                                 // largest |output| of this lane (amax_part)
  float* W = split_out ? p.workspace + ((int64_t)split * p.batch + b) * (int64_t)p.M * p.N
                       : nullptr;
  const int64_t cb = (int64_t)b * p.sC;
  const int64_t ld_out = split_out ? p.N : p.ldc;
  const bool vec = split_out ? (p.N % 8 == 0) : p.vec_epi;
  const int rsub = lane >> 3, q = lane & 7;
  auto run = [&]<int EPI>() {
    // row blocks whose loads (previous C or aux_in, if the epilogue reads
    // any) are issued together, ahead of their stores: 8 (bf16) or 16 (fp32)
    // VGPRs per lane and row block
    constexpr int NIB = WTM / 32, GI = epi_reads<EPI>() == 2 ? 2 : NIB;
#pragma unroll
    for (int hc = 0; hc < NH; ++hc)
#pragma unroll
    for (int i0 = 0; i0 < NIB; i0 += GI) {
      EpiIn<EPI> in[GI][4];
      if constexpr (epi_reads<EPI>() > 0) {
#pragma unroll
        for (int ii = 0; ii < GI; ++ii)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int m = m0 + wm * WTM + (i0 + ii) * 32 + rsub + 8 * t;
            const int n = n0 + wn * WTN + hc * 64 + 8 * q;
            if (m < p.M && vec && n + 8 <= p.N)
              epi_load8<EPI>(p, cb + (int64_t)m * ld_out + n, in[ii][t]);
          }
      }
#pragma unroll
      for (int ii = 0; ii < GI; ++ii) {
        const int i = i0 + ii;                           // 32-row block of the wave tile
        // 32 x 32 tile: lane c + 32 h holds column c, rows 8 (e / 4) + 4 h + e % 4;
        // 16 x 16 tile: lane c + 16 g holds column c, rows 4 g + e
        if constexpr (MI == 32) {
#pragma unroll
          for (int j = 0; j < TNH; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              stg[((e >> 2) * 8 + half * 4 + (e & 3)) * EP_LD + j * 32 + l32] =
                  acc[i][hc * TNH + j][e];
        } else {
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int j = 0; j < TNH; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                stg[(i2 * 16 + 4 * (lane >> 4) + e) * EP_LD + j * 16 + (lane & 15)] =
                    acc[2 * i + i2][hc * TNH + j][e];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = rsub + 8 * t;
          float v[8];
          ld8(stg + row * EP_LD + 8 * q, v);
          const int m = m0 + wm * WTM + i * 32 + row;
          const int n = n0 + wn * WTN + hc * 64 + 8 * q;
          if (m >= p.M || n >= p.N) continue;
          if (split_out) {
            float* w = W + (int64_t)m * ld_out + n;
            if (vec && n + 8 <= p.N) {
              float r[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) r[e] = p.alpha * v[e];
              st8(w, r);
            } else {
              for (int e = 0; e < 8 && n + e < p.N; ++e) w[e] = p.alpha * v[e];
            }
          } else {
            const int64_t off = cb + (int64_t)m * ld_out + n;
            // (the output amax is kept by the fp8 instantiations only, so that
            // the bf16 kernels stay as they were)
            if (vec && n + 8 <= p.N) {
              const float m8 = epi_apply8<EPI>(p, off, v, in[ii][t]);
              if constexpr (F8) amx = max_nan(amx, m8);
            } else {
              for (int e = 0; e < 8 && n + e < p.N; ++e) {
                const float m1 = epi_one<bf16, EPI>(p, off + e, v[e]);
                if constexpr (F8) amx = max_nan(amx, m1);
              }
            }
          }
        }
      }
    }
  };
  // QK-norm + rotary epilogue of the QKV product.  A head's 128 columns are
  // the tiles of waves wn and wn ^ 1 (wn even: dims 0-63); the two read each
  // other's staged block, so each lane holds 8 dims of its row and their
  // rotary partners 64 apart: 8 lanes per row sum the squares, then the lane
  // normalises, rotates and stores its 8 outputs.  Two barriers per 32-row
  // block (the partner's block is staged; it has been read before the next
  // block overwrites it).
  auto run_qk = [&]() {
    constexpr int NIB = WTM / 32;
    const int pw = wave ^ 1;
    const int psidx = pw / EP_PER;
    bf16* pbase;
    if constexpr (EP_BUFS >= 3) pbase = psidx == 0 ? st0 : (psidx == 1 ? st1 : st2);
    else pbase = psidx == 0 ? st0 : st1;
    const float* pstg = reinterpret_cast<const float*>(pbase) + (pw % EP_PER) * EP_FLOATS;
    const int ncol = n0 + wn * WTN;
    const int head = ncol >> 7;
    const bool normed = head < p.qk_heads, lo = (wn & 1) == 0;
    bf16* Cb = static_cast<bf16*>(p.C) + cb;
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            stg[(i2 * 16 + 4 * (lane >> 4) + e) * EP_LD + j * 16 + (lane & 15)] = acc[2 * i + i2][j][e];
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = rsub + 8 * t;
        float v[8], w[8], o[8];
        ld8(stg + row * EP_LD + 8 * q, v);
        ld8(pstg + row * EP_LD + 8 * q, w);
        const int m = m0 + wm * WTM + i * 32 + row;
        const int n = ncol + 8 * q;
        if (normed) {
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] *= p.alpha;
            w[e] *= p.alpha;
            ss += v[e] * v[e] + w[e] * w[e];
          }
          ss += __shfl_xor(ss, 1, kWave);
          ss += __shfl_xor(ss, 2, kWave);
          ss += __shfl_xor(ss, 4, kWave);
          const float rs = 1.0f / sqrtf(ss / 128.f + p.qk_eps);
          const int tp = m % p.rope_T;
          float c[8], sn[8];
          ld8(p.rope + tp * 64 + 8 * q, c);
          ld8(p.rope + p.rope_T * 64 + tp * 64 + 8 * q, sn);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float y1 = (lo ? v[e] : w[e]) * rs, y2 = (lo ? w[e] : v[e]) * rs;
            o[e] = lo ? y1 * c[e] - y2 * sn[e] : y1 * sn[e] + y2 * c[e];
          }
          if (lo && q == 0 && m < p.M) p.rqk[(int64_t)m * p.qk_heads + head] = rs;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = p.alpha * v[e];
        }
        if (m < p.M && n < p.N) st8(Cb + (int64_t)m * p.ldc + n, o);
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };
  if (split_out) run.template operator()<kEpiStoreF32>();
  else if constexpr (AL == kKCont && BL == kKCont && !F8 && MI == 16 && WTN == 64 && WN % 2 == 0) {
    if (p.epi == kEpiQkNorm) run_qk();
    else with_epilogue(p.epi, run);
  } else {
    with_epilogue(p.epi, run);
  }
  if (F8 && p.amax_part) {
    // the staging buffers are free once every wave has passed the first
    // barrier inside block_max_nan
    amx = block_max_nan(amx, reinterpret_cast<float*>(st0));
    if (threadIdx.x == 0) p.amax_part[blockIdx.x] = bf16_abs(amx);
  }
}

// The pipelined kernel applies when K is a multiple of 32, every operand start
// and leading dimension is 16-byte aligned, and M (N) is a multiple of 8 where
// A (B) is MN-contiguous.
bool pipe_ok(const GemmParams& p) {
  auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (p.K % 32 || p.lda % 8 || p.ldb % 8 || !al16(p.A) || !al16(p.B)) return false;
  if (p.batch > 1 && (p.sA % 8 || p.sB % 8)) return false;
  if (p.a_layout == kMNCont && p.M % 8) return false;
  if (p.b_layout == kMNCont && p.N % 8) return false;
  // operand offsets are 32-bit (buffer addressing)
  const int64_t ea = p.a_layout == kKCont ? operand_extent(p.M, p.lda, p.K)
                                          : operand_extent(p.K, p.lda, p.M);
  const int64_t eb = p.b_layout == kKCont ? operand_extent(p.N, p.ldb, p.K)
                                          : operand_extent(p.K, p.ldb, p.N);
  if (ea >= (int64_t(1) << 32) || eb >= (int64_t(1) << 32)) return false;
  return true;
}

template <int AL, int BL, int WM, int WN, int ST, int PK, int MI, bool F8 = false, int WTN = 64,
          int FA = 0>
hipError_t launch_pipe_cfg(const GemmParams& p, hipStream_t st) {
  using C = Pipe<WM, WN, ST, PK, MI, WTN>;
  const int tiles = ceil_div(p.M, C::BM) * ceil_div(p.N, C::BN);
  dim3 grid(tiles, 1, p.batch * p.splits);
  gemm_bf16_pipe_kernel<AL, BL, WM, WN, ST, PK, MI, F8, WTN, FA><<<grid, C::NT, 0, st>>>(p);
  return hipGetLastError();
}

// 256 x 256 block tiles (8 waves of 128 x 64), one block per CU.
//  * Both operands K-contiguous (forward products, Newton-Schulz Gram and
//    polynomial steps): k-depth 64 per step (one barrier per 64 k, whole
//    128-byte rows per load), 3-7 % faster than depth 32 with 4 stages; the
//    half-stage ring, which keeps the A loads of the tile after next in
//    flight across the barrier, another 1.5-2.5 %; v_mfma_f32_16x16x32_bf16,
//    which moves fewer accumulator bytes per FLOP than the 32 x 32 x 16 form
//    and so draws less power at the same rate, another 3 %.
//  * A K-contiguous, B MN-contiguous (input gradients): the same half-stage
//    ring with 16 x 16 x 32 MFMAs, 6-9 % faster than depth 32 with 4 stages.
//  * Both MN-contiguous (weight gradients): the half-stage ring with
//    16 x 16 x 32 MFMAs and no fragment prefetch (which would spill), 1-2 %
//    faster than depth 32 with 4 stages and 32 x 32 x 16 MFMAs; depth 32 with
//    16 x 16 x 32 (no room for prefetch either) measured 3.5 % slower.
// 256 x 128 tiles at two blocks per CU, 5 stages of depth 32 and 4 waves of
// 128 x 128 (which spills) were all slower.
hipError_t launch_pipe(const GemmParams& p, hipStream_t st) {
  switch (p.a_layout * 2 + p.b_layout) {
    case 0:
      if (p.K % 64 == 0) return launch_pipe_cfg<kKCont, kKCont, 2, 4, 5, 64, 16>(p, st);
      return launch_pipe_cfg<kKCont, kKCont, 2, 4, 4, 32, 32>(p, st);
    case 1:
      if (p.K % 64 == 0) return launch_pipe_cfg<kKCont, kMNCont, 2, 4, 5, 64, 16>(p, st);
      return launch_pipe_cfg<kKCont, kMNCont, 2, 4, 4, 32, 32>(p, st);
    case 2: return launch_pipe_cfg<kMNCont, kKCont, 2, 4, 4, 32, 32>(p, st);
    default:
      if (p.K % 64 == 0) return launch_pipe_cfg<kMNCont, kMNCont, 2, 4, 5, 64, 16>(p, st);
      return launch_pipe_cfg<kMNCont, kMNCont, 2, 4, 4, 32, 32>(p, st);
  }
}

}  // namespace

// Split count for a K-heavy product (the weight gradients), from a simple cost
// model of the 256 x 256 kernel on a 256-CU device (one block per CU): blocks
// run in waves of 256, each 32-deep k-step takes about 1.1 us, and the split
// partials cost (2 splits + 2) M N fp32 values of memory traffic at 5 TB/s.
// A larger split count is taken only when it is at least 2 % faster.
int nc_gemm_pick_splits(int M, int N, int K) {
  constexpr int kCUs = 256;
  const int64_t tiles = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
  const int kt = ceil_div(K, 32);                     // 32-deep steps (the 1.1 us unit)
  double best = 0.0;
  int best_s = 1;
  for (int s = 1; s <= 64 && (s == 1 || s <= kt / 8); ++s) {
    const int64_t waves = (tiles * s + kCUs - 1) / kCUs;
    const double t = (double)waves * ceil_div(kt, s) * 1.1e-6 +
                     (s > 1 ? (2.0 * s + 2.0) * M * N * 4.0 / 5e12 : 0.0);
    if (s == 1 || t < 0.98 * best) {
      best = t;
      best_s = s;
    }
  }
  return best_s;
}

size_t nc_gemm_workspace_bytes(int M, int N, int splits) {
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

// C (+)= the split-K slabs in fixed order
static hipError_t splitk_reduce(const GemmParams& p, hipStream_t st) {
  const int64_t total = (int64_t)p.M * p.N * p.batch;
  const bool rows_ok = p.N % 4 == 0 && p.ldc % 4 == 0 && (p.batch == 1 || p.sC % 4 == 0) &&
                       (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 &&
                       (int64_t)p.M * p.batch <= 0x7fffffff;
  if (rows_ok) {
    splitk_reduce_rows_kernel<<<p.M * p.batch, 256, 0, st>>>(p);
  } else {
    const int blocks = (int)std::min<int64_t>(ceil_div64(total, 256), 65536);
    splitk_reduce_kernel<<<blocks, 256, 0, st>>>(p);
  }
  return hipGetLastError();
}

hipError_t nc_launch_gemm_f8(const GemmParams& p_in, hipStream_t st) {
  GemmParams p = p_in;
  if (p.M <= 0 || p.N <= 0 || p.batch <= 0) return hipSuccess;
  auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (p.a_layout != kKCont || p.b_layout != kKCont || p.K <= 0 || p.K % 128 || p.lda % 16 ||
      p.ldb % 16 || (p.batch > 1 && (p.sA % 16 || p.sB % 16)) || !al16(p.A) || !al16(p.B) ||
      (p.fmt_a != 0 && p.fmt_a != 1) || p.epi == kEpiQkNorm)
    return hipErrorInvalidValue;
  if (p.splits < 1) p.splits = 1;
  if (p.amax_part && (p.batch != 1 || p.splits != 1)) return hipErrorInvalidValue;
  if (p.splits > 1 && ((p.epi != kEpiStoreF32 && p.epi != kEpiAccF32) || !p.workspace ||
                       p.workspace_bytes < nc_gemm_workspace_bytes(p.M, p.N, p.splits) * p.batch))
    return hipErrorInvalidValue;
  p.vec_epi = p.ldc % 8 == 0 && (p.batch == 1 || p.sC % 8 == 0) && al16(p.C) &&
              al16(p.aux_in) && al16(p.aux_out);
  // the loads move byte pairs: K, leading dimensions and batch strides in pairs
  p.K /= 2;
  p.lda /= 2;
  p.ldb /= 2;
  p.sA /= 2;
  p.sB /= 2;
  if (!pipe_ok(p)) return hipErrorInvalidValue;
  const hipError_t e = p.fmt_a ? launch_pipe_cfg<kKCont, kKCont, 2, 4, 5, 64, 16, true, 64, 1>(p, st)
                               : launch_pipe_cfg<kKCont, kKCont, 2, 4, 5, 64, 16, true, 64, 0>(p, st);
  if (e != hipSuccess || p.splits == 1) return e;
  return splitk_reduce(p, st);
}

hipError_t nc_launch_gemm(int dtype, const GemmParams& p_in, hipStream_t st) {
  GemmParams p = p_in;
  if (p.M <= 0 || p.N <= 0 || p.batch <= 0) return hipSuccess;
  if (p.splits < 1) p.splits = 1;
  if (dtype == 0) {
    if (p.amax_part || p.epi == kEpiQkNorm) return hipErrorInvalidValue;
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
  {
    auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    p.vec_epi = p.ldc % 8 == 0 && (p.batch == 1 || p.sC % 8 == 0) && al16(p.C) &&
                al16(p.aux_in) && al16(p.aux_out);
  }
  const bool use_pipe = pipe_ok(p);
  if (p.amax_part) return hipErrorInvalidValue;    // kept by the fp8 kernels only
  // the QK-norm epilogue: in the 64-deep K-contiguous configuration only
  if (p.epi == kEpiQkNorm &&
      (!use_pipe || p.a_layout != kKCont || p.b_layout != kKCont || p.K % 64 || p.N % 128 ||
       p.splits != 1 || p.batch != 1 || !p.vec_epi || !p.rope || !p.rqk || p.rope_T < 1 ||
       p.qk_heads < 0 || p.qk_heads * 128 > p.N))
    return hipErrorInvalidValue;
  hipError_t e = use_pipe ? launch_pipe(p, st) : launch_bf16_cfg<256, 256, 2, 4>(p, st);
  if (e != hipSuccess || p.splits == 1) return e;
  return splitk_reduce(p, st);
}
