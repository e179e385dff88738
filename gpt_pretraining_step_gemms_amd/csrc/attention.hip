// Causal self-attention (head dim 128) on gfx950, forward and backward.
//
// q, k, v, o and their gradients stay token-major ([token, head*128], row
// stride ld) as the QKV and output-projection GEMMs produce and consume them;
// the log-sum-exp and D = rowsum(dO*O) are [B, H, T] fp32.
//
// bf16 path (flash attention with v_mfma_f32_32x32x16_bf16):
//  * forward: a workgroup owns 128 queries of one (b, h) (4 waves x 32), walks
//    the 64-key tiles up to the diagonal with K and V^T staged in LDS (double
//    buffered).  It computes S^T = K Q^T so that every lane owns one query
//    column: the online-softmax max/sum are lane-local plus one exchange with
//    the lane 32 apart, and the rescale of O^T = V^T P^T is a per-lane scalar.
//    P^T feeds the second MFMA straight from the accumulators (the reduction
//    index is permuted identically on both operands).
//  * backward: two deterministic kernels, no atomics.  dK/dV: a workgroup owns
//    128 keys and walks the query tiles from the diagonal down, recomputing
//    P = exp(S - lse) and dS = P (dP - D).  dQ: a workgroup owns 128 queries
//    and walks the key tiles up to the diagonal.
//  * Tiles reach LDS in their token-major layout by direct loads; the operands
//    needed transposed (V^T, Q^T, dO^T, K^T) are read with ds_read_b64_tr_b16,
//    which transposes 16-bit values in the LDS read.
// fp32 path (tiny configuration): one wave per query (or key) row, plain
// loops over the causal range.
//
// Grouped-query attention: H query heads share Hkv key/value heads in groups
// of G = H / Hkv consecutive heads (query head h reads key/value head h / G).
// The forward and dQ kernels run per query head; a dK/dV workgroup owns keys of
// one key/value head and walks the query tiles of its G query heads in turn.
//
// Sliding window: with a window w, query t sees keys t - w .. t (the causal
// mask plus a left edge).  Every kernel takes it as `win`, with win = T for
// the plain causal mask; tiles wholly outside the band are never loaded and
// only the tiles the band's edges cross are masked element by element.
#include "kernels.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// accumulator registers hf*8 .. hf*8+7 of a 32x32 tile, as an MFMA operand
NC_DEV bf16x8 pack_half(const float* v, int hf) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)v[hf * 8 + e];
  return r;
}

// 2^x with the hardware instruction alone (v_exp_f32): softmax weights below
// 2^-126 flush to zero, which the library exp2f's denormal range handling
// (a compare, two selects and a v_ldexp per call) would otherwise preserve.
NC_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Make the compiler wait for a register loaded from global memory here, once.
// Without it, the first use inside the main loop carries s_waitcnt vmcnt(n)
// in every iteration (the count cannot tell the preheader's loads from the
// loop's), and those waits also drain the next tile's prefetch in flight.
NC_DEV void settle(bf16x8& x) { asm volatile("" : "+v"(x)); }
NC_DEV void settle(float& x) { asm volatile("" : "+v"(x)); }

NC_DEV f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ================================================================ forward
// K and V tiles reach LDS by direct loads (global_load_lds, 16 B per lane, 1 KB
// per wave instruction), double-buffered, in their token-major layout:
//   K tile [64 keys][128] -> S^T fragments (rows = keys) read with ds_read_b128;
//   V tile [64 keys][128] -> O^T = V^T P^T fragments (rows = head dims, 8 keys per lane) read with
//        ds_read_b64_tr_b16, each 16-lane group taking a 4-key x 16-dim block.
// Two workgroups fit on a CU (64 KB of LDS each, <= 256 registers per wave),
// so one workgroup's softmax overlaps the other's matrix products.
NC_DEV void fa_dma16(const void* g, const bf16* lds) {
  const unsigned a = (unsigned)(size_t)(__attribute__((address_space(3))) const void*)lds;
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(__builtin_amdgcn_readfirstlane(a))
      : "memory");
}

template <int N>
NC_DEV void fa_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
NC_DEV void fa_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Swizzle of 16-byte chunks in a [rows][128] bf16 tile: chunk c of row r is
// stored at c ^ fa_swz(r).  Eight consecutive rows read at one chunk
// (ds_read_b128) and four consecutive rows read at two neighbouring chunks
// (ds_read_b64_tr_b16) both hit 8 distinct bank groups.
NC_DEV int fa_swz(int r) { return (2 * (r & 3)) | ((r >> 2) & 1); }

// this wave's share (4 x 1 KB) of a 64-row x 128 token-major tile into LDS
NC_DEV void fa_issue_rows(const bf16* src, int64_t ld, int row0, bf16* tile, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = wave * 4 + i;                 // 16 blocks of 4 rows
    const int r = blk * 4 + (lane >> 4);
    const int c = (lane & 15) ^ fa_swz(r);
    fa_dma16(src + (int64_t)(row0 + r) * ld + c * 8, tile + blk * 512);
  }
}

// 64 consecutive floats (4 bytes per lane) into LDS; one wave
NC_DEV void fa_dma4(const float* g, const float* lds) {
  const unsigned a = (unsigned)(size_t)(__attribute__((address_space(3))) const void*)lds;
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(__builtin_amdgcn_readfirstlane(a))
      : "memory");
}

typedef __bf16 fa_bf16x4 __attribute__((ext_vector_type(4)));
NC_DEV bf16x8 fa_frag_k(const bf16* tile, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + r * 128 + ((c ^ fa_swz(r)) << 3));
}
// 8 values of head dim `col_base + lane%16` (within a 16-wide column block) at
// key rows row_base + {0..3} and row_base + 8 + {0..3}, from a [key][128] tile
// stored with the fa_swz swizzle (rows r and r + 8 share it)
NC_DEV bf16x8 fa_frag_vt(const bf16* tile, int row_base, int col_base, int lane) {
  const int t = lane & 15;
  const int r = row_base + (t >> 2);
  const int col = col_base + 4 * (t & 3);
  const bf16* p0 = tile + r * 128 + (((col >> 3) ^ fa_swz(r)) << 3) + (col & 7);
  const bf16* p1 = p0 + 8 * 128;                 // row + 8: same swizzle
  const fa_bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) fa_bf16x4*)p0);
  const fa_bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) fa_bf16x4*)p1);
  bf16x8 v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// one 128-query block qb of head bh; st0 / st1: K | V stages of 2 x 64 x 128
NC_DEV void attn_fwd_block(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    int64_t ld, bf16* __restrict__ o, int64_t ldo, float* __restrict__ lse, int T, int H,
    int G, int win, float scale_log2, int qb, int bh, bf16* st0, bf16* st1) {
  constexpr int KT = 64 * 128;                    // one 64 x 128 tile
  const int b = bh / H, h = bh % H;
  const int64_t base = (int64_t)b * T * ld + h * 128;
  const int64_t kvbase = (int64_t)b * T * ld + (h / G) * 128;
  const bf16* qg = q + base;
  const bf16* kg = k + kvbase;
  const bf16* vg = v + kvbase;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int q0w = qb * 128 + wave * 32;
  const int myq = q0w + l32;

  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = *reinterpret_cast<const bf16x8*>(qg + (int64_t)myq * ld + s * 16 + half * 8);
#pragma unroll
  for (int s = 0; s < 8; ++s) settle(qf[s]);

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m = -INFINITY, l = 0.f;

  // key tiles from the block's first window start to the diagonal
  const int n_kv = 2 * qb + 2;
  const int kv_lo = max(0, qb * 128 - win) / 64;
  auto issue = [&](int kv, bf16* st) {
    fa_issue_rows(kg, ld, kv * 64, st, wave, lane);
    fa_issue_rows(vg, ld, kv * 64, st + KT, wave, lane);
  };
  auto step = [&](int kv, const bf16* ks, bf16* next) {
    fa_wait_vmcnt<0>();         // this wave's loads of tile kv have landed
    fa_barrier();               // ... and every wave's; tile kv-1 is no longer read
    if (kv + 1 < n_kv) issue(kv + 1, next);
    if (kv * 64 > q0w + 31) return;               // keys all after this wave's queries
    if (kv * 64 + 63 < q0w - win) return;         // keys all before this wave's windows
    const bf16* vs = ks + KT;
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        sacc[kb] = mfma(fa_frag_k(ks, kb * 32 + l32, s * 2 + half), qf[s], sacc[kb]);
    }
    // Online softmax in the log2 domain.  The running max m of a query only
    // moves when the tile's max exceeds it by more than 8: the weights
    // 2^(x - m) then stay below 2^8, and O and l are rescaled only on the
    // (rare, after the first tiles) moves, skipped when no lane moves.
    // Masks: keys after the query (tiles reaching the diagonal) and keys
    // before its window (tiles crossing the window's left edge).  A lane can
    // then see no key at all in a tile; its running max stays -inf and the
    // weights below use a finite stand-in so that they come out 0, not NaN.
    const bool need_mask = kv * 64 + 63 > q0w || kv * 64 < q0w + 31 - win;
    float mt = -INFINITY;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kv * 64 + kb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          if (key > myq || key < myq - win) sacc[kb][e] = -INFINITY;
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kb][e]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * scale_log2;
    const bool move = mt > m + 8.f;
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float alpha = move ? fast_exp2(m - mt) : 1.f;
      if (move) m = mt;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
    float sv[2][16];
    float ls = 0.f;
    const float mf = fmaxf(m, -3.0e38f);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = fast_exp2(fmaf(sacc[kb][e], scale_log2, -mf));
        sv[kb][e] = pv;
        ls += pv;
      }
    l += ls;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 pf = pack_half(sv[j >> 1], j & 1);
      const int row_base = (j >> 1) * 32 + (j & 1) * 16 + half * 4;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        oacc[db] = mfma(fa_frag_vt(vs, row_base, db * 32 + 16 * ((lane >> 4) & 1), lane), pf,
                        oacc[db]);
    }
  };

  issue(kv_lo, st0);
  for (int kv = kv_lo; kv < n_kv; kv += 2) {
    step(kv, st0, st1);
    if (kv + 1 < n_kv) step(kv + 1, st1, st0);
  }

  const float lt_sum = l + __shfl_xor(l, 32, 64);
  const float inv = 1.f / lt_sum;
  if (half == 0) lse[((int64_t)b * H + h) * T + myq] = (m + log2f(lt_sum)) * kLn2;

  // stage O (this wave's 32 x 128) through LDS with padded rows, then 16-B stores
  constexpr int OSTR = 136;
  __syncthreads();
  bf16* os = (wave < 2 ? st0 : st1) + (wave & 1) * 32 * OSTR;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (bf16)(oacc[db][g * 4 + i] * inv);
      *reinterpret_cast<bf16x4*>(os + l32 * OSTR + db * 32 + g * 8 + half * 4) = w;
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = lane + 64 * i, r = idx >> 4, c = idx & 15;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(os + r * OSTR + c * 8);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(os + r * OSTR + c * 8 + 4);
    u32x4 val = {lo[0], lo[1], hi[0], hi[1]};
    *reinterpret_cast<u32x4*>(o + ((int64_t)b * T + q0w + r) * ldo + h * 128 + c * 8) = val;
  }
}


// ============================================================ dK / dV
// A workgroup owns 128 keys (4 waves x 32; K and V rows of each wave's keys
// stay in registers as the B operands) and walks the 64-query tiles from the
// diagonal down.  Q, dO and the tile's log-sum-exp and D reach LDS by direct
// loads, double-buffered; Q^T and dO^T fragments come from transpose reads.
constexpr int kDkvStage = 2 * 64 * 128 + 256;     // Q | dO | lse[64] D[64] (fp32)

// one 128-key block kblk of key/value head bhk; st0 / st1: stages of kDkvStage
// elements.  kGrouped: G > 1 query heads per key/value head, walked in turn (a
// separate instantiation keeps the plain path's registers as they were).
template <bool kGrouped>
NC_DEV void attn_bwd_dkv_block(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    int64_t ld, const bf16* __restrict__ dO, int64_t ldo, const float* __restrict__ lse,
    const float* __restrict__ Dv, bf16* __restrict__ dk, bf16* __restrict__ dv, int64_t ldd,
    int T, int H, int G, int win, float scale_log2, float scale, int kblk, int bhk, bf16* st0,
    bf16* st1) {
  constexpr int KT = 64 * 128;
  const int Hkv = kGrouped ? H / G : H;
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int64_t kvbase = (int64_t)b * T * ld + hk * 128;
  // the query head being walked: hk itself, or each head of the group in turn
  const int h0 = kGrouped ? hk * G : hk;
  int64_t base = (int64_t)b * T * ld + h0 * 128;
  int64_t obase = (int64_t)b * T * ldo + h0 * 128;
  const float* lse_bh = lse + ((int64_t)b * H + h0) * T;
  const float* D_bh = Dv + ((int64_t)b * H + h0) * T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int k0w = kblk * 128 + wave * 32;
  const int mykey = k0w + l32;

  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    kf[s] = *reinterpret_cast<const bf16x8*>(k + kvbase + (int64_t)mykey * ld + s * 16 + half * 8);
    vf[s] = *reinterpret_cast<const bf16x8*>(v + kvbase + (int64_t)mykey * ld + s * 16 + half * 8);
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    settle(kf[s]);
    settle(vf[s]);
  }
  f32x16 dkacc[4], dvacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dkacc[i][e] = 0.f; dvacc[i][e] = 0.f; }

  // query tiles from the diagonal to the last query whose window holds a key of the block
  const int qt0 = kblk * 2, nqt = min(T / 64, (kblk * 128 + 127 + win) / 64 + 1);
  auto issue = [&](int qt, bf16* st) {
    fa_issue_rows(q + base, ld, qt * 64, st, wave, lane);
    fa_issue_rows(dO + obase, ldo, qt * 64, st + KT, wave, lane);
    if (wave == 0) {
      float* stats = reinterpret_cast<float*>(st + 2 * KT);
      fa_dma4(lse_bh + qt * 64 + lane, stats);
      fa_dma4(D_bh + qt * 64 + lane, stats + 64);
    }
  };
  auto step = [&](int qt, const bf16* cur, bf16* next) {
    fa_wait_vmcnt<0>();
    fa_barrier();
    if (qt + 1 < nqt) issue(qt + 1, next);
    if (qt * 64 + 63 < k0w) return;               // queries all before this wave's keys
    if (qt * 64 > k0w + 31 + win) return;         // queries all past these keys' windows
    const bf16* Qs = cur;
    const bf16* dOs = cur + KT;
    const float* lse_s = reinterpret_cast<const float*>(cur + 2 * KT);
    const float* D_s = lse_s + 64;
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) { sacc[qb][e] = 0.f; pacc[qb][e] = 0.f; }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        sacc[qb] = mfma(fa_frag_k(Qs, qb * 32 + l32, s * 2 + half), kf[s], sacc[qb]);
        pacc[qb] = mfma(fa_frag_k(dOs, qb * 32 + l32, s * 2 + half), vf[s], pacc[qb]);
      }
    }
    // masks (only tiles crossing an edge of the band): queries before the
    // key, and queries whose window ends before it
    if (qt * 64 < k0w + 31 || qt * 64 + 63 > k0w + win) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qq = qt * 64 + qb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          if (qq < mykey || qq > mykey + win) sacc[qb][e] = -INFINITY;
        }
    }
    float p[2][16], ds[2][16];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ql = qb * 32 + g * 8 + half * 4;
        const float4 l4 = *reinterpret_cast<const float4*>(lse_s + ql);
        const float4 d4 = *reinterpret_cast<const float4*>(D_s + ql);
        const float la[4] = {l4.x, l4.y, l4.z, l4.w};
        const float da[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = g * 4 + i;
          const float pv = fast_exp2(fmaf(sacc[qb][e], scale_log2, -la[i] * kLog2e));
          p[qb][e] = pv;
          ds[qb][e] = pv * (pacc[qb][e] - da[i]);
        }
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 pa = pack_half(p[j >> 1], j & 1);
      const bf16x8 dsa = pack_half(ds[j >> 1], j & 1);
      const int row_base = (j >> 1) * 32 + (j & 1) * 16 + half * 4;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int cb = db * 32 + 16 * ((lane >> 4) & 1);
        dvacc[db] = mfma(pa, fa_frag_vt(dOs, row_base, cb, lane), dvacc[db]);
        dkacc[db] = mfma(dsa, fa_frag_vt(Qs, row_base, cb, lane), dkacc[db]);
      }
    }
  };

  auto walk = [&]() {
    issue(qt0, st0);
    for (int qt = qt0; qt < nqt; qt += 2) {
      step(qt, st0, st1);
      if (qt + 1 < nqt) step(qt + 1, st1, st0);
    }
  };
  if constexpr (kGrouped) {
    for (int g = 0; g < G; ++g) {
      if (g) {
        const int h = h0 + g;
        base = (int64_t)b * T * ld + h * 128;
        obase = (int64_t)b * T * ldo + h * 128;
        lse_bh = lse + ((int64_t)b * H + h) * T;
        D_bh = Dv + ((int64_t)b * H + h) * T;
        __syncthreads();                           // the previous head's last tile is read
      }
      walk();
    }
  } else {
    walk();
  }

  // C[key][d]: lane holds column d = db*32 + l32, rows key = 8*(e/4) + 4*half + e%4
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = k0w + (e >> 2) * 8 + half * 4 + (e & 3);
      const int64_t off = ((int64_t)b * T + key) * ldd + hk * 128 + db * 32 + l32;
      dk[off] = (bf16)(dkacc[db][e] * scale);
      dv[off] = (bf16)dvacc[db][e];
    }
}

// ================================================================== dQ
// A workgroup owns 128 queries (4 waves x 32) and walks the 64-key tiles up
// to the diagonal, like the forward pass: S^T = K Q^T and dP^T = V dO^T with
// one query per lane, then dQ += dS K with K^T fragments from transpose reads.
// one 128-query block qb of head bh; st0 / st1: K | V stages of 2 x 64 x 128
NC_DEV void attn_bwd_dq_block(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    int64_t ld, const bf16* __restrict__ dO, int64_t ldo, const float* __restrict__ lse,
    const float* __restrict__ Dv, bf16* __restrict__ dq, int64_t ldd, int T, int H, int G,
    int win, float scale_log2, float scale, int qb, int bh, bf16* st0, bf16* st1) {
  constexpr int KT = 64 * 128;
  const int b = bh / H, h = bh % H;
  const int64_t base = (int64_t)b * T * ld + h * 128;
  const int64_t obase = (int64_t)b * T * ldo + h * 128;
  const int64_t kvbase = (int64_t)b * T * ld + (h / G) * 128;
  const bf16* kg = k + kvbase;
  const bf16* vg = v + kvbase;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int q0w = qb * 128 + wave * 32;
  const int myq = q0w + l32;

  bf16x8 qf[8], df[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qf[s] = *reinterpret_cast<const bf16x8*>(q + base + (int64_t)myq * ld + s * 16 + half * 8);
    df[s] = *reinterpret_cast<const bf16x8*>(dO + obase + (int64_t)myq * ldo + s * 16 + half * 8);
  }
  float lse2 = lse[((int64_t)b * H + h) * T + myq] * kLog2e;
  float Dq = Dv[((int64_t)b * H + h) * T + myq];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    settle(qf[s]);
    settle(df[s]);
  }
  settle(lse2);
  settle(Dq);
  f32x16 dqacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqacc[i][e] = 0.f;

  const int n_kv = 2 * qb + 2;
  const int kv_lo = max(0, qb * 128 - win) / 64;
  auto issue = [&](int kv, bf16* st) {
    fa_issue_rows(kg, ld, kv * 64, st, wave, lane);
    fa_issue_rows(vg, ld, kv * 64, st + KT, wave, lane);
  };
  auto step = [&](int kv, const bf16* cur, bf16* next) {
    fa_wait_vmcnt<0>();
    fa_barrier();
    if (kv + 1 < n_kv) issue(kv + 1, next);
    if (kv * 64 > q0w + 31) return;
    if (kv * 64 + 63 < q0w - win) return;
    const bf16* Ks = cur;
    const bf16* Vs = cur + KT;
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) { sacc[kb][e] = 0.f; pacc[kb][e] = 0.f; }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        sacc[kb] = mfma(fa_frag_k(Ks, kb * 32 + l32, s * 2 + half), qf[s], sacc[kb]);
        pacc[kb] = mfma(fa_frag_k(Vs, kb * 32 + l32, s * 2 + half), df[s], pacc[kb]);
      }
    }
    // masks (only tiles crossing an edge of the band): keys after the query
    // and keys before its window
    if (kv * 64 + 63 > q0w || kv * 64 < q0w + 31 - win) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kv * 64 + kb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          if (key > myq || key < myq - win) sacc[kb][e] = -INFINITY;
        }
    }
    float ds[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = fast_exp2(fmaf(sacc[kb][e], scale_log2, -lse2));
        ds[kb][e] = pv * (pacc[kb][e] - Dq);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 a = pack_half(ds[j >> 1], j & 1);
      const int row_base = (j >> 1) * 32 + (j & 1) * 16 + half * 4;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        dqacc[db] = mfma(a, fa_frag_vt(Ks, row_base, db * 32 + 16 * ((lane >> 4) & 1), lane),
                         dqacc[db]);
    }
  };

  issue(kv_lo, st0);
  for (int kv = kv_lo; kv < n_kv; kv += 2) {
    step(kv, st0, st1);
    if (kv + 1 < n_kv) step(kv + 1, st1, st0);
  }

#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int qq = q0w + (e >> 2) * 8 + half * 4 + (e & 3);
      dq[((int64_t)b * T + qq) * ldd + h * 128 + db * 32 + l32] = (bf16)(dqacc[db][e] * scale);
    }
}

// Workgroup -> (b*H + h, 128-row blocks).
//  * Workgroups are dealt to the 8 XCDs round robin.  When the (b, h) count is
//    a multiple of 8, all workgroups of one (b, h) go to the same XCD, one
//    after the other, so that the K/V (or Q/dO) tiles they all walk are shared
//    in that XCD's L2 and every XCD gets the same mix of long and short jobs.
//  * Plain causal mask (paired): the work of a 128-row block grows linearly
//    with its index, so a workgroup takes block i and its mirror nb-1-i (the
//    middle block alone when nb is odd): equal work per workgroup.
//  * Sliding window: the work levels off once the window is full, so a
//    workgroup takes one block, the longest ones first (high_first: the
//    block index at which work is largest is the highest one).
struct BlockJob { int bh, first, second; };
NC_DEV BlockJob block_job(int nb, bool paired, bool high_first) {
  const int per = paired ? (nb + 1) / 2 : nb;     // workgroups per (b, h)
  const int nbh = gridDim.x / per, b = blockIdx.x;
  int j;
  BlockJob jb;
  if (nbh % 8 == 0) {
    const int x = b % 8, r = b / 8;
    jb.bh = x + 8 * (r / per);
    j = r % per;
  } else {
    jb.bh = b / per;
    j = b % per;
  }
  if (paired) {
    jb.first = nb - 1 - j;
    jb.second = j == nb - 1 - j ? -1 : j;
  } else {
    jb.first = high_first ? nb - 1 - j : j;
    jb.second = -1;
  }
  return jb;
}

// workgroups per (b, h) for the bf16 kernels
inline int attn_jobs_per_head(int T, int win) { return win >= T ? (T / 128 + 1) / 2 : T / 128; }

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    int64_t ld, bf16* __restrict__ o, int64_t ldo, float* __restrict__ lse, int T, int H,
    int G, int win, float scale_log2) {
  __shared__ __attribute__((aligned(1024))) bf16 st0[2 * 64 * 128];   // K | V of even tiles
  __shared__ __attribute__((aligned(1024))) bf16 st1[2 * 64 * 128];   // K | V of odd tiles
  const BlockJob jb = block_job(T / 128, win >= T, true);
  attn_fwd_block(q, k, v, ld, o, ldo, lse, T, H, G, win, scale_log2, jb.first, jb.bh, st0, st1);
  if (jb.second < 0) return;
  __syncthreads();                                 // the first block's O staging is read
  attn_fwd_block(q, k, v, ld, o, ldo, lse, T, H, G, win, scale_log2, jb.second, jb.bh, st0,
                 st1);
}

template <bool kGrouped>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    int64_t ld, const bf16* __restrict__ dO, int64_t ldo, const float* __restrict__ lse,
    const float* __restrict__ Dv, bf16* __restrict__ dk, bf16* __restrict__ dv, int64_t ldd,
    int T, int H, int G, int win, float scale_log2, float scale) {
  __shared__ __attribute__((aligned(1024))) bf16 st0[kDkvStage];
  __shared__ __attribute__((aligned(1024))) bf16 st1[kDkvStage];
  // key block kblk walks up to T/64 - 2 kblk query tiles: the low blocks are the long ones
  const BlockJob jb = block_job(T / 128, win >= T, false);
  if (jb.second >= 0) {
    attn_bwd_dkv_block<kGrouped>(q, k, v, ld, dO, ldo, lse, Dv, dk, dv, ldd, T, H, G, win,
                                 scale_log2, scale, jb.second, jb.bh, st0, st1);
    __syncthreads();
  }
  attn_bwd_dkv_block<kGrouped>(q, k, v, ld, dO, ldo, lse, Dv, dk, dv, ldd, T, H, G, win,
                               scale_log2, scale, jb.first, jb.bh, st0, st1);
}

__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    int64_t ld, const bf16* __restrict__ dO, int64_t ldo, const float* __restrict__ lse,
    const float* __restrict__ Dv, bf16* __restrict__ dq, int64_t ldd, int T, int H, int G,
    int win, float scale_log2, float scale) {
  __shared__ __attribute__((aligned(1024))) bf16 st0[2 * 64 * 128];   // K | V
  __shared__ __attribute__((aligned(1024))) bf16 st1[2 * 64 * 128];
  const BlockJob jb = block_job(T / 128, win >= T, true);
  attn_bwd_dq_block(q, k, v, ld, dO, ldo, lse, Dv, dq, ldd, T, H, G, win, scale_log2, scale,
                    jb.first, jb.bh, st0, st1);
  if (jb.second < 0) return;
  __syncthreads();
  attn_bwd_dq_block(q, k, v, ld, dO, ldo, lse, Dv, dq, ldd, T, H, G, win, scale_log2, scale,
                    jb.second, jb.bh, st0, st1);
}

// ========================================================== fp32 path
// one wave per (b, h, t) query row; lane owns head dims lane and lane + 64
__global__ void attn_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                    const float* __restrict__ v, int64_t ld,
                                    float* __restrict__ o, int64_t ldo, float* __restrict__ lse,
                                    int B, int T, int H, int G, int win, float scale) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= B * H * T) return;
  const int lane = threadIdx.x & 63;
  const int t = item % T, bh = item / T, b = bh / H, h = bh % H;
  const int64_t base = (int64_t)b * T * ld + h * 128;
  const int64_t kvb = (int64_t)b * T * ld + (h / G) * 128;
  const float q1 = q[base + (int64_t)t * ld + lane], q2 = q[base + (int64_t)t * ld + lane + 64];
  float m = -INFINITY, l = 0.f, o1 = 0.f, o2 = 0.f;
  for (int u = max(0, t - win); u <= t; ++u) {
    const int64_t ku = kvb + (int64_t)u * ld;
    const float s = wave_sum(q1 * k[ku + lane] + q2 * k[ku + lane + 64]) * scale;
    const float mn = fmaxf(m, s);
    const float a = expf(m - mn), p = expf(s - mn);
    l = l * a + p;
    o1 = o1 * a + p * v[ku + lane];
    o2 = o2 * a + p * v[ku + lane + 64];
    m = mn;
  }
  const int64_t oo = ((int64_t)b * T + t) * ldo + h * 128;
  o[oo + lane] = o1 / l;
  o[oo + lane + 64] = o2 / l;
  if (lane == 0) lse[((int64_t)b * H + h) * T + t] = m + logf(l);
}

__global__ void attn_bwd_dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                       const float* __restrict__ v, int64_t ld,
                                       const float* __restrict__ dO, int64_t ldo,
                                       const float* __restrict__ lse,
                                       const float* __restrict__ Dv, float* __restrict__ dq,
                                       int64_t ldd, int B, int T, int H, int G, int win,
                                       float scale) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= B * H * T) return;
  const int lane = threadIdx.x & 63;
  const int t = item % T, bh = item / T, b = bh / H, h = bh % H;
  const int64_t base = (int64_t)b * T * ld + h * 128;
  const int64_t kvb = (int64_t)b * T * ld + (h / G) * 128;
  const int64_t ob = ((int64_t)b * T + t) * ldo + h * 128;
  const float q1 = q[base + (int64_t)t * ld + lane], q2 = q[base + (int64_t)t * ld + lane + 64];
  const float g1 = dO[ob + lane], g2 = dO[ob + lane + 64];
  const float L = lse[(int64_t)bh * T + t], Dt = Dv[(int64_t)bh * T + t];
  float a1 = 0.f, a2 = 0.f;
  for (int u = max(0, t - win); u <= t; ++u) {
    const int64_t ku = kvb + (int64_t)u * ld;
    const float s = wave_sum(q1 * k[ku + lane] + q2 * k[ku + lane + 64]) * scale;
    const float p = expf(s - L);
    const float dp = wave_sum(g1 * v[ku + lane] + g2 * v[ku + lane + 64]);
    const float ds = p * (dp - Dt);
    a1 += ds * k[ku + lane];
    a2 += ds * k[ku + lane + 64];
  }
  const int64_t dd = ((int64_t)b * T + t) * ldd + h * 128;
  dq[dd + lane] = a1 * scale;
  dq[dd + lane + 64] = a2 * scale;
}

// one wave per (b, key/value head, u) key row, summing over the head's G query heads
__global__ void attn_bwd_dkv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                        const float* __restrict__ v, int64_t ld,
                                        const float* __restrict__ dO, int64_t ldo,
                                        const float* __restrict__ lse,
                                        const float* __restrict__ Dv, float* __restrict__ dk,
                                        float* __restrict__ dv, int64_t ldd, int B, int T, int H,
                                        int G, int win, float scale) {
  const int Hkv = H / G;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= B * Hkv * T) return;
  const int lane = threadIdx.x & 63;
  const int u = item % T, bhk = item / T, b = bhk / Hkv, hk = bhk % Hkv;
  const int64_t ku = (int64_t)b * T * ld + hk * 128 + (int64_t)u * ld;
  const float k1 = k[ku + lane], k2 = k[ku + lane + 64];
  const float v1 = v[ku + lane], v2 = v[ku + lane + 64];
  float ak1 = 0.f, ak2 = 0.f, av1 = 0.f, av2 = 0.f;
  const int t_end = min(T - 1, u + win);
  for (int g = 0; g < G; ++g) {
    const int h = hk * G + g;
    const int64_t bh = (int64_t)b * H + h;
    for (int t = u; t <= t_end; ++t) {
      const int64_t qt = (int64_t)b * T * ld + h * 128 + (int64_t)t * ld;
      const int64_t ot = ((int64_t)b * T + t) * ldo + h * 128;
      const float q1 = q[qt + lane], q2 = q[qt + lane + 64];
      const float g1 = dO[ot + lane], g2 = dO[ot + lane + 64];
      const float s = wave_sum(q1 * k1 + q2 * k2) * scale;
      const float p = expf(s - lse[bh * T + t]);
      const float dp = wave_sum(g1 * v1 + g2 * v2);
      const float ds = p * (dp - Dv[bh * T + t]);
      av1 += p * g1;
      av2 += p * g2;
      ak1 += ds * q1;
      ak2 += ds * q2;
    }
  }
  const int64_t dd = ((int64_t)b * T + u) * ldd + hk * 128;
  dk[dd + lane] = ak1 * scale;
  dk[dd + lane + 64] = ak2 * scale;
  dv[dd + lane] = av1;
  dv[dd + lane + 64] = av2;
}

}  // namespace

hipError_t nc_attn_fwd(int dtype, const void* q, const void* k, const void* v, int64_t ld,
                       void* o, int64_t ldo, float* lse, int B, int T, int H, int Hkv, int window,
                       hipStream_t st) {
  const float scale = 1.0f / sqrtf(128.f);
  const int win = window < 0 || window > T ? T : window;
  if (Hkv < 1 || H % Hkv) return hipErrorInvalidValue;
  const int G = H / Hkv;
  if (dtype) {
    if (T % 128) return hipErrorInvalidValue;
    attn_fwd_kernel<<<B * H * attn_jobs_per_head(T, win), 256, 0, st>>>(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, ld, (bf16*)o, ldo, lse, T, H, G, win,
        scale * kLog2e);
  } else {
    attn_fwd_f32_kernel<<<ceil_div(B * H * T, 4), 256, 0, st>>>(
        (const float*)q, (const float*)k, (const float*)v, ld, (float*)o, ldo, lse, B, T, H, G,
        win, scale);
  }
  return hipGetLastError();
}

hipError_t nc_attn_bwd(int dtype, const void* q, const void* k, const void* v, int64_t ld,
                       const void* dO, int64_t ldo, const float* lse, const float* D, void* dq,
                       void* dk, void* dv, int64_t ldd, int B, int T, int H, int Hkv, int window,
                       hipStream_t st) {
  const float scale = 1.0f / sqrtf(128.f);
  const int win = window < 0 || window > T ? T : window;
  if (Hkv < 1 || H % Hkv) return hipErrorInvalidValue;
  const int G = H / Hkv;
  if (dtype) {
    if (T % 128) return hipErrorInvalidValue;
    const int jobs = attn_jobs_per_head(T, win);
    auto dkv_kernel = G > 1 ? attn_bwd_dkv_kernel<true> : attn_bwd_dkv_kernel<false>;
    dkv_kernel<<<B * Hkv * jobs, 256, 0, st>>>(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, ld, (const bf16*)dO, ldo, lse, D,
        (bf16*)dk, (bf16*)dv, ldd, T, H, G, win, scale * kLog2e, scale);
    attn_bwd_dq_kernel<<<B * H * jobs, 256, 0, st>>>(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, ld, (const bf16*)dO, ldo, lse, D,
        (bf16*)dq, ldd, T, H, G, win, scale * kLog2e, scale);
  } else {
    attn_bwd_dq_f32_kernel<<<ceil_div(B * H * T, 4), 256, 0, st>>>(
        (const float*)q, (const float*)k, (const float*)v, ld, (const float*)dO, ldo, lse, D,
        (float*)dq, ldd, B, T, H, G, win, scale);
    attn_bwd_dkv_f32_kernel<<<ceil_div(B * Hkv * T, 4), 256, 0, st>>>(
        (const float*)q, (const float*)k, (const float*)v, ld, (const float*)dO, ldo, lse, D,
        (float*)dk, (float*)dv, ldd, B, T, H, G, win, scale);
  }
  return hipGetLastError();
}
