// Host runtime behind the C ABI (include/nc.h, include/nc_ops.h): arena
// planning, the parameter registry, and the launch sequences of one
// micro-batch forward/backward and of one optimizer step.
//
// Parameter arena (caller-owned, fp32 unless noted), element layout shared by
// masters, gradients and Muon momenta:
//   block region: layer l at l*S, S = 4 d^2 + 2 d F:
//     Wq [d,d] | Wk [d,d] | Wv [d,d] | Wo [d,d] | W1 [F,d] | W2 [d,F]
//   (Wq|Wk|Wv is one [3d, d] matrix for the QKV product), then E [V,d], Wh [V,d].
//   regions: masters | grads | Muon momenta (block region) | AdamW m (E|Wh) |
//   AdamW v (E|Wh) | bf16 copies (block region + Wh; bf16 models only) |
//   rotary table cos/sin [2][T][64].
// Activation arena: what the backward pass reads per layer (RMSNorm outputs
// and reciprocal RMS, q/k/v after QK-norm+rotary, QK-norm reciprocal RMS,
// attention output and log-sum-exp, the MLP activation g = max(h,0)^2; the
// pre-activation h is not kept, since max(h,0) = sqrt(g)), then scratch
// (residual stream x and its gradient, lm_head logits of one row chunk,
// split-K, embedding-sort and Newton-Schulz workspaces).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "nc.h"
#include "nc_ops.h"
#include "gemm.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Layout {
  size_t cur = 0;
  size_t take(size_t bytes) {
    const size_t o = cur;
    cur += align_up(bytes);
    return o;
  }
};

struct ParamInfo {
  std::string name;
  int rows, cols, group;
  size_t elem;        // element offset in the master/grad layout
  int64_t adam_elem;  // element offset in the AdamW regions, -1 for Muon
};

struct LayerAct { size_t a1, r1, qkv, rqk, o, lse, a2, r2, g; };

}  // namespace

struct nc_ctx {
  nc_model_config cfg;
  nc_optim_config ocfg;
  int dt;      // 0 fp32, 1 bf16
  size_t es;   // activation element size
  int L, d, H, F, V, T, maxB, Nmax, chunk;
  int Hkv, dk, W;   // key/value heads, their width Hkv*128, qkv row width d + 2 dk
  bool fp8 = false;  // forward block products in fp8 e4m3 (tensorwise scales)
  size_t q8a = 0, q8w = 0, q8s = 0, q8ws = 0;   // their codes, scales and amax scratch
  int64_t S, n_block, n_total;
  std::vector<ParamInfo> params;
  // parameter arena byte offsets
  size_t oP, oG, oM, oAm, oAv, oSh, oTab, oV2, param_bytes;
  // activation arena byte offsets
  std::vector<LayerAct> la;
  size_t xf, rf, x, dx, dxT, da, dqkv, dO, Dbuf, dh, z, dz, loss_rows, ws, ws_bytes, emb,
      nsU, frob, norms, nm_vm, nm_q, nm_inv, nm_scale, act_bytes;
  int64_t nm_rows = 0;   // NorMuon: rows of all block matrices (4L d + L F + L d)
  // Newton-Schulz buffers per group (0: square [d,d] (4L, or 2L with grouped
  // key/value heads), 1: 2L wide [d,F], 2: 2L [dk,d] with grouped key/value heads):
  // the fp32 iterate X (two, ping-pong), A = X X^T, B = b A + c A A, and a copy of
  // each in the activation type for the matrix cores.
  struct NsBufs { size_t x32[2], xh[2], a32, ah, b32, bh; } ns[3];
  int splits_qkv, splits_o, splits_1, splits_2, splits_head, splits_dxf;
  std::vector<int> windows;   // attention window per layer, -1 = plain causal
  char* pa = nullptr;
  char* aa = nullptr;
  hipStream_t st = nullptr;
  bool bound = false;
  bool dry_run = false;   // host-only validation of the launch sequence
  int64_t step = 0;
  std::string err;
  std::string range_error;
};

namespace {

nc_status fail(nc_ctx* c, nc_status s, const std::string& msg) {
  if (c) c->err = msg;
  return s;
}

nc_status hipcheck(nc_ctx* c, hipError_t e, const char* what) {
  if (e == hipSuccess) return NC_OK;
  return fail(c, NC_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// NC_TRY: a HIP call or non-GEMM launch (skipped in a dry run).
// NC_GEMM: a GEMM through gemm(), whose operand ranges are checked on the host
// (and which only checks, without launching, in a dry run).
#define NC_TRY(expr, what)                               \
  do {                                                   \
    if (!ctx->dry_run) {                                 \
      nc_status _s = hipcheck(ctx, (expr), what);        \
      if (_s != NC_OK) return _s;                        \
    }                                                    \
  } while (0)
#define NC_GEMM(expr, what)                              \
  do {                                                   \
    nc_status _s = hipcheck(ctx, (expr), what);          \
    if (_s != NC_OK) {                                   \
      if (ctx->range_error.size()) ctx->err += " (" + ctx->range_error + ")"; \
      return _s;                                         \
    }                                                    \
  } while (0)

nc_status validate(const nc_model_config* m, const nc_optim_config* o, std::string& why) {
  if (!m || !o) { why = "null config"; return NC_ERR_INVALID_ARG; }
  if (m->n_layer < 0 || m->d_model <= 0 || m->n_head <= 0 || m->d_ff <= 0 || m->vocab <= 0 ||
      m->seq_len <= 0 || m->max_micro_batch <= 0) {
    why = "non-positive dimension";
    return NC_ERR_INVALID_ARG;
  }
  if (m->dtype != NC_FP32 && m->dtype != NC_BF16) { why = "dtype"; return NC_ERR_INVALID_ARG; }
  if (m->fp8_forward != 0 && m->fp8_forward != 1) { why = "fp8_forward is 0 or 1"; return NC_ERR_INVALID_ARG; }
  if (m->fp8_forward && m->dtype != NC_BF16) {
    why = "fp8_forward needs the bf16 configuration";
    return NC_ERR_UNSUPPORTED;
  }
  if (m->n_kv_head < 0 || (m->n_kv_head > 0 && m->n_head % m->n_kv_head)) {
    why = "n_kv_head must divide n_head (0: n_head)";
    return NC_ERR_INVALID_ARG;
  }
  if (m->head_dim != 128 || m->d_model != m->n_head * 128) {
    why = "head_dim must be 128 and d_model = n_head * 128";
    return NC_ERR_UNSUPPORTED;
  }
  if (m->d_model > 2048 || m->d_ff % 64 || m->vocab % 64 || m->vocab > 32768) {
    why = "d_model <= 2048, d_ff and vocab multiples of 64, vocab <= 32768 required";
    return NC_ERR_UNSUPPORTED;
  }
  if (m->dtype == NC_BF16 && m->seq_len % 128) {
    why = "bf16 attention needs seq_len % 128 == 0";
    return NC_ERR_UNSUPPORTED;
  }
  if (!(m->norm_eps >= 0.f) || !(m->rope_base > 0.f)) { why = "eps/base"; return NC_ERR_INVALID_ARG; }
  if (o->ns_steps < 0 || o->ns_steps > 8) { why = "ns_steps in [0, 8]"; return NC_ERR_INVALID_ARG; }
  if (o->normuon != 0 && o->normuon != 1) { why = "normuon is 0 or 1"; return NC_ERR_INVALID_ARG; }
  if (o->normuon && !(o->normuon_beta2 >= 0.f && o->normuon_beta2 < 1.f)) {
    why = "normuon_beta2 in [0, 1)";
    return NC_ERR_INVALID_ARG;
  }
  const int64_t n_tok = (int64_t)m->max_micro_batch * m->seq_len;
  if (n_tok > (int64_t)1 << 30) { why = "micro-batch too large"; return NC_ERR_UNSUPPORTED; }
  return NC_OK;
}

void plan(nc_ctx* c) {
  const int L = c->L, d = c->d, F = c->F, V = c->V, T = c->T, H = c->H;
  const int dk = c->dk, Hkv = c->Hkv, W = c->W;
  const size_t es = c->es;
  // per layer: Wq [d,d] | Wk [dk,d] | Wv [dk,d] | Wo [d,d] | W1 [F,d] | W2 [d,F]
  c->S = 2LL * d * d + 2LL * dk * d + 2LL * d * F;
  c->n_block = c->S * L;
  c->n_total = c->n_block + 2LL * V * d;
  // registry
  c->params.clear();
  c->params.push_back({"E", V, d, NC_GROUP_ADAMW, (size_t)c->n_block, 0});
  const char* names[6] = {"Wq", "Wk", "Wv", "Wo", "W1", "W2"};
  for (int l = 0; l < L; ++l) {
    size_t base = (size_t)l * c->S;
    const int64_t dd = (int64_t)d * d, kd = (int64_t)dk * d;
    const int64_t offs[6] = {0, dd, dd + kd, dd + 2 * kd, 2 * dd + 2 * kd,
                             2 * dd + 2 * kd + (int64_t)F * d};
    const int rows[6] = {d, dk, dk, d, F, d}, cols[6] = {d, d, d, d, d, F};
    for (int j = 0; j < 6; ++j)
      c->params.push_back({std::to_string(l) + "." + names[j], rows[j], cols[j], NC_GROUP_MUON,
                           base + (size_t)offs[j], -1});
  }
  c->params.push_back({"Wh", V, d, NC_GROUP_ADAMW, (size_t)(c->n_block + (int64_t)V * d),
                       (int64_t)V * d});

  Layout p;
  c->oP = p.take(c->n_total * 4);
  c->oG = p.take(c->n_total * 4);
  c->oM = p.take(c->n_block * 4);
  c->oAm = p.take(2ULL * V * d * 4);
  c->oAv = p.take(2ULL * V * d * 4);
  c->oSh = c->dt ? p.take((c->n_block + (size_t)V * d) * 2) : 0;
  c->oTab = p.take(2ULL * T * 64 * 4);
  c->nm_rows = c->ocfg.normuon ? (int64_t)L * (3LL * d + 2LL * dk + F) : 0;
  c->oV2 = c->nm_rows ? p.take((size_t)c->nm_rows * 4) : 0;
  c->param_bytes = p.cur;

  const size_t N = (size_t)c->Nmax;
  c->chunk = (int)std::min<size_t>(N, 8192);
  Layout a;
  c->la.resize(L);
  for (int l = 0; l < L; ++l) {
    LayerAct& x = c->la[l];
    x.a1 = a.take(N * d * es);
    x.r1 = a.take(N * 4);
    x.qkv = a.take(N * W * es);
    x.rqk = a.take(N * (H + Hkv) * 4);
    x.o = a.take(N * d * es);
    x.lse = a.take(N * H * 4);
    x.a2 = a.take(N * d * es);
    x.r2 = a.take(N * 4);
    x.g = a.take(N * F * es);
  }
  c->xf = a.take(N * d * es);
  c->rf = a.take(N * 4);
  c->x = a.take(N * d * 4);
  c->dx = a.take(N * d * 4);
  c->dxT = a.take(N * d * es);
  c->da = a.take(N * d * 4);
  c->dqkv = a.take(N * W * es);
  c->dO = a.take(N * d * es);
  c->Dbuf = a.take(N * H * 4);
  c->dh = a.take(N * F * es);
  c->z = a.take((size_t)c->chunk * V * 4);
  c->dz = a.take((size_t)c->chunk * V * es);
  c->loss_rows = a.take(N * 4);
  // split-K for the weight-gradient products (bf16 MFMA path)
  auto sp = [&](int M, int Nn, int K) { return c->dt ? nc_gemm_pick_splits(M, Nn, K) : 1; };
  c->splits_qkv = sp(W, d, (int)N);
  c->splits_o = sp(d, d, (int)N);
  c->splits_1 = sp(F, d, (int)N);
  c->splits_2 = sp(d, F, (int)N);
  c->splits_head = sp(V, d, c->chunk);
  c->splits_dxf = sp(c->chunk, d, V);   // few output tiles, K = vocabulary
  size_t ws = 0;
  ws = std::max(ws, nc_gemm_workspace_bytes(W, d, c->splits_qkv));
  ws = std::max(ws, nc_gemm_workspace_bytes(d, d, c->splits_o));
  ws = std::max(ws, nc_gemm_workspace_bytes(F, d, c->splits_1));
  ws = std::max(ws, nc_gemm_workspace_bytes(d, F, c->splits_2));
  ws = std::max(ws, nc_gemm_workspace_bytes(V, d, c->splits_head));
  ws = std::max(ws, nc_gemm_workspace_bytes(c->chunk, d, c->splits_dxf));
  c->ws_bytes = ws;
  c->ws = a.take(std::max<size_t>(ws, 256));
  c->emb = a.take(nc_embed_bwd_scratch_bytes((int)N, V, d));
  // Newton-Schulz groups (see NsBufs)
  const bool gqa = dk != d;
  const int ns_cnt[3] = {(gqa ? 2 : 4) * L, 2 * L, gqa ? 2 * L : 0};
  const int ns_r[3] = {d, d, dk}, ns_c[3] = {d, F, d};
  for (int g = 0; g < 3; ++g) {
    auto& b = c->ns[g];
    b = {};
    if (!ns_cnt[g]) continue;
    const size_t cnt = ns_cnt[g], xe = cnt * ns_r[g] * ns_c[g], ae = cnt * ns_r[g] * ns_r[g];
    for (int k = 0; k < 2; ++k) {
      b.x32[k] = a.take(xe * 4);
      b.xh[k] = a.take(xe * es);
    }
    b.a32 = a.take(ae * 4);
    b.ah = a.take(ae * es);
    b.b32 = a.take(ae * 4);
    b.bh = a.take(ae * es);
  }
  c->nsU = c->ocfg.muon_nesterov ? a.take((size_t)c->n_block * 4) : 0;
  c->frob = a.take((size_t)6 * std::max(L, 1) * 256 * 4);
  c->norms = a.take((size_t)6 * std::max(L, 1) * 4);
  if (c->nm_rows) {
    c->nm_vm = a.take((size_t)c->nm_rows * 4);
    c->nm_q = a.take((size_t)c->nm_rows * 4);
    c->nm_inv = a.take((size_t)c->nm_rows * 4);
    c->nm_scale = a.take((size_t)6 * L * 4);
  }
  if (c->fp8) {
    // codes of the largest activation operand [N, max(d, F)] and weight operand
    c->q8a = a.take(N * (size_t)std::max(d, F));
    c->q8w = a.take((size_t)std::max(W, F) * std::max(d, F));
    c->q8s = a.take(4 * sizeof(float));
    c->q8ws = a.take(1024 * sizeof(float));
  }
  c->act_bytes = a.cur;
}

template <typename T = void>
T* P(nc_ctx* c, size_t off) { return reinterpret_cast<T*>(c->pa + off); }
template <typename T = void>
T* A(nc_ctx* c, size_t off) { return reinterpret_cast<T*>(c->aa + off); }

// Weight operand of a GEMM: the bf16 copy (bf16 models) or the fp32 master.
// `elem` is the master-layout offset of a block matrix (< n_block); the bf16
// region mirrors the block region and then holds Wh (E has no bf16 copy).
const void* wptr(nc_ctx* c, size_t elem) {
  if (c->dt) return c->pa + c->oSh + elem * 2;
  return c->pa + c->oP + elem * 4;
}
const void* wptr_head(nc_ctx* c) {
  if (c->dt) return c->pa + c->oSh + (size_t)c->n_block * 2;
  return c->pa + c->oP + ((size_t)c->n_block + (size_t)c->V * c->d) * 4;
}

// True if [p, p + bytes) lies inside the parameter or the activation arena.
bool in_arena(const nc_ctx* c, const void* p, size_t bytes) {
  const char* q = static_cast<const char*>(p);
  auto inside = [&](const char* base, size_t size) {
    return q >= base && q + bytes <= base + size;
  };
  return inside(c->pa, c->param_bytes) || inside(c->aa, c->act_bytes);
}

// Host check of every operand extent of a GEMM against the arenas.
bool operands_in_arenas(nc_ctx* c, const GemmParams& g) {
  const size_t es = c->es;
  const bool c_f32 = g.epi == kEpiStoreF32 || g.epi == kEpiAccF32 || g.epi == kEpiDual;
  auto extent = [](int64_t rows, int64_t cols, int64_t ld, int64_t bstride, int batch) {
    // elements spanned by a [rows, cols] row-major view with leading dim ld
    return (int64_t)(batch - 1) * bstride + (rows - 1) * ld + cols;
  };
  const int64_t ea = g.a_layout == kKCont ? extent(g.M, g.K, g.lda, g.sA, g.batch)
                                          : extent(g.K, g.M, g.lda, g.sA, g.batch);
  const int64_t eb = g.b_layout == kKCont ? extent(g.N, g.K, g.ldb, g.sB, g.batch)
                                          : extent(g.K, g.N, g.ldb, g.sB, g.batch);
  const int64_t ec = extent(g.M, g.N, g.ldc, g.sC, g.batch);
  std::string bad;
  if (!in_arena(c, g.A, ea * es)) bad = "A";
  else if (!in_arena(c, g.B, eb * es)) bad = "B";
  else if (!in_arena(c, g.C, ec * (c_f32 ? 4 : es))) bad = "C";
  else if (g.aux_in && !in_arena(c, g.aux_in, ec * (g.epi == kEpiDual ? 4 : es))) bad = "aux_in";
  else if (g.aux_out && !in_arena(c, g.aux_out, ec * es)) bad = "aux_out";
  else if (g.splits > 1 && (size_t)g.splits * g.batch * g.M * g.N * 4 > g.workspace_bytes)
    bad = "split-K workspace";
  if (bad.empty()) return true;
  c->range_error = "GEMM operand " + bad + " outside its arena (M=" + std::to_string(g.M) +
                   " N=" + std::to_string(g.N) + " K=" + std::to_string(g.K) + ")";
  return false;
}

hipError_t gemm(nc_ctx* c, const void* A_, int64_t lda, int al, const void* B_, int64_t ldb,
                int bl, void* C_, int64_t ldc, int M, int N, int K, int epi,
                const void* aux_in = nullptr, void* aux_out = nullptr, int splits = 1,
                int batch = 1, int64_t sA = 0, int64_t sB = 0, int64_t sC = 0, float p0 = 0.f,
                float p1 = 0.f) {
  GemmParams g{};
  g.A = A_; g.B = B_; g.C = C_; g.aux_in = aux_in; g.aux_out = aux_out;
  g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.sA = sA; g.sB = sB; g.sC = sC;
  g.M = M; g.N = N; g.K = K; g.batch = batch;
  g.a_layout = al; g.b_layout = bl; g.epi = epi;
  g.alpha = 1.f; g.p0 = p0; g.p1 = p1;
  g.splits = splits;
  g.workspace = reinterpret_cast<float*>(c->aa + c->ws);
  g.workspace_bytes = c->ws_bytes;
  if (!operands_in_arenas(c, g)) return hipErrorInvalidValue;
  if (c->dry_run) return hipSuccess;
  return nc_launch_gemm(c->dt, g, c->st);
}

// Forward block product in fp8: C (epilogue epi) = X W^T with X bf16 [N, K]
// and W the bf16 weight copy [Nout, K], both quantised to e4m3 with one scale
// per tensor (codes in q8a / q8w, scales {amax, s} in q8s[0..1] / q8s[2..3]);
// the kernel divides the sums by s_X s_W.
hipError_t gemm_fp8_fwd(nc_ctx* c, const void* X, int K, const void* Wt, int Nout, void* C,
                        int64_t ldc, int N, int epi) {
  float* sc = reinterpret_cast<float*>(c->aa + c->q8s);
  float* ws = reinterpret_cast<float*>(c->aa + c->q8ws);
  uint8_t* xa = reinterpret_cast<uint8_t*>(c->aa + c->q8a);
  uint8_t* wq = reinterpret_cast<uint8_t*>(c->aa + c->q8w);
  const bool c_f32 = epi == kEpiStoreF32 || epi == kEpiAccF32;
  const size_t nx = (size_t)N * K, nw = (size_t)Nout * K;
  // every extent inside its arena, also in a dry run
  if (!in_arena(c, X, nx * 2) || !in_arena(c, Wt, nw * 2) || !in_arena(c, xa, nx) ||
      !in_arena(c, wq, nw) || !in_arena(c, C, ((size_t)(N - 1) * ldc + Nout) * (c_f32 ? 4 : 2))) {
    c->range_error = "fp8 GEMM operand outside its arena (N=" + std::to_string(N) +
                     " Nout=" + std::to_string(Nout) + " K=" + std::to_string(K) + ")";
    return hipErrorInvalidValue;
  }
  if (c->dry_run) return hipSuccess;
  hipError_t e = nc_fp8_quantize(1, X, (int64_t)nx, ws, sc, xa, c->st);
  if (e != hipSuccess) return e;
  e = nc_fp8_quantize(1, Wt, (int64_t)nw, ws, sc + 2, wq, c->st);
  if (e != hipSuccess) return e;
  GemmParams g{};
  g.A = xa; g.B = wq; g.C = C;
  g.lda = K; g.ldb = K; g.ldc = ldc;
  g.M = N; g.N = Nout; g.K = K; g.batch = 1; g.splits = 1;
  g.a_layout = kKCont; g.b_layout = kKCont; g.epi = epi; g.alpha = 1.f;
  g.scale_a = sc; g.scale_b = sc + 2;
  return nc_launch_gemm_f8(g, c->st);
}

}  // namespace

// =================================================================== C ABI
extern "C" {

const char* nc_status_str(nc_status s) {
  switch (s) {
    case NC_OK: return "ok";
    case NC_ERR_INVALID_ARG: return "invalid argument";
    case NC_ERR_UNSUPPORTED: return "unsupported";
    case NC_ERR_OUT_OF_MEMORY: return "arena too small";
    case NC_ERR_HIP: return "HIP error";
    case NC_ERR_STATE: return "bad call order";
    case NC_ERR_NONFINITE: return "non-finite value";
  }
  return "unknown status";
}

const char* nc_last_error(const nc_ctx* ctx) { return ctx ? ctx->err.c_str() : ""; }

static nc_ctx* make_ctx(const nc_model_config* cfg, const nc_optim_config* ocfg) {
  nc_ctx* c = new nc_ctx();
  c->cfg = *cfg;
  c->ocfg = *ocfg;
  c->dt = cfg->dtype == NC_BF16 ? 1 : 0;
  c->es = c->dt ? 2 : 4;
  c->L = cfg->n_layer; c->d = cfg->d_model; c->H = cfg->n_head; c->F = cfg->d_ff;
  c->Hkv = cfg->n_kv_head > 0 ? cfg->n_kv_head : cfg->n_head;
  c->fp8 = cfg->fp8_forward != 0;
  c->dk = c->Hkv * 128;
  c->W = c->d + 2 * c->dk;
  c->V = cfg->vocab; c->T = cfg->seq_len; c->maxB = cfg->max_micro_batch;
  c->Nmax = c->maxB * c->T;
  c->windows.assign(c->L, -1);
  plan(c);
  return c;
}

nc_status nc_plan(const nc_model_config* cfg, const nc_optim_config* ocfg,
                  size_t* param_arena_bytes, size_t* act_arena_bytes) {
  try {
    std::string why;
    nc_status s = validate(cfg, ocfg, why);
    if (s != NC_OK) return s;
    nc_ctx* c = make_ctx(cfg, ocfg);
    if (param_arena_bytes) *param_arena_bytes = c->param_bytes;
    if (act_arena_bytes) *act_arena_bytes = c->act_bytes;
    delete c;
    return NC_OK;
  } catch (...) {
    return NC_ERR_INVALID_ARG;
  }
}

nc_status nc_create(const nc_model_config* cfg, const nc_optim_config* ocfg, nc_ctx** out) {
  if (!out) return NC_ERR_INVALID_ARG;
  *out = nullptr;
  try {
    std::string why;
    nc_status s = validate(cfg, ocfg, why);
    if (s != NC_OK) return s;
    *out = make_ctx(cfg, ocfg);
    return NC_OK;
  } catch (...) {
    return NC_ERR_INVALID_ARG;
  }
}

void nc_destroy(nc_ctx* ctx) { delete ctx; }

nc_status nc_bind(nc_ctx* ctx, void* d_param_arena, size_t param_bytes, void* d_act_arena,
                  size_t act_bytes, void* hip_stream) {
  if (!ctx || !d_param_arena || !d_act_arena) return fail(ctx, NC_ERR_INVALID_ARG, "null arena");
  if ((reinterpret_cast<uintptr_t>(d_param_arena) | reinterpret_cast<uintptr_t>(d_act_arena)) %
      kAlign)
    return fail(ctx, NC_ERR_INVALID_ARG, "arenas must be 256-byte aligned");
  if (param_bytes < ctx->param_bytes || act_bytes < ctx->act_bytes)
    return fail(ctx, NC_ERR_OUT_OF_MEMORY,
                "arena too small: need " + std::to_string(ctx->param_bytes) + " + " +
                    std::to_string(ctx->act_bytes) + " bytes");
  ctx->pa = static_cast<char*>(d_param_arena);
  ctx->aa = static_cast<char*>(d_act_arena);
  ctx->st = static_cast<hipStream_t>(hip_stream);
  // rotary table: angle(t, i) = t * base^(-2i/128), computed in double
  const int T = ctx->T;
  std::vector<float> tab(2 * (size_t)T * 64);
  for (int t = 0; t < T; ++t)
    for (int i = 0; i < 64; ++i) {
      const double ang = (double)t * std::pow((double)ctx->cfg.rope_base, -2.0 * i / 128.0);
      tab[(size_t)t * 64 + i] = (float)std::cos(ang);
      tab[(size_t)T * 64 + (size_t)t * 64 + i] = (float)std::sin(ang);
    }
  NC_TRY(hipMemcpyAsync(ctx->pa + ctx->oTab, tab.data(), tab.size() * 4, hipMemcpyHostToDevice,
                        ctx->st), "upload rotary table");
  // gradients and optimizer state start at zero, step count at 0
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oG), 0.f, ctx->n_total, ctx->st), "zero grads");
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oM), 0.f, ctx->n_block, ctx->st), "zero momentum");
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oAm), 0.f, 2ULL * ctx->V * ctx->d, ctx->st), "zero m");
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oAv), 0.f, 2ULL * ctx->V * ctx->d, ctx->st), "zero v");
  if (ctx->nm_rows)
    NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oV2), 0.f, ctx->nm_rows, ctx->st), "zero normuon v2");
  ctx->step = 0;
  NC_TRY(hipStreamSynchronize(ctx->st), "bind sync");
  ctx->bound = true;
  return NC_OK;
}

static nc_status refresh_shadows(nc_ctx* ctx) {
  if (!ctx->dt) return NC_OK;
  NC_TRY(nc_convert_f32(1, P<float>(ctx, ctx->oP), ctx->pa + ctx->oSh, ctx->n_block, ctx->st),
         "shadow blocks");
  NC_TRY(nc_convert_f32(1, P<float>(ctx, ctx->oP) + ctx->n_block + (size_t)ctx->V * ctx->d,
                        ctx->pa + ctx->oSh + ctx->n_block * 2, (size_t)ctx->V * ctx->d, ctx->st),
         "shadow head");
  return NC_OK;
}

nc_status nc_init_params(nc_ctx* ctx, uint64_t seed, float std) {
  if (!ctx) return NC_ERR_INVALID_ARG;
  if (!ctx->bound) return fail(ctx, NC_ERR_STATE, "bind first");
  if (!(std >= 0.f)) return fail(ctx, NC_ERR_INVALID_ARG, "std");
  NC_TRY(nc_init_normal(P<float>(ctx, ctx->oP), ctx->n_total, seed, 0, std, ctx->st), "init");
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oM), 0.f, ctx->n_block, ctx->st), "zero momentum");
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oAm), 0.f, 2ULL * ctx->V * ctx->d, ctx->st), "zero m");
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oAv), 0.f, 2ULL * ctx->V * ctx->d, ctx->st), "zero v");
  if (ctx->nm_rows)
    NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oV2), 0.f, ctx->nm_rows, ctx->st), "zero normuon v2");
  ctx->step = 0;
  return refresh_shadows(ctx);
}

nc_status nc_set_attention_windows(nc_ctx* ctx, const int32_t* windows) {
  if (!ctx) return NC_ERR_INVALID_ARG;
  if (!windows) {
    ctx->windows.assign(ctx->L, -1);
    return NC_OK;
  }
  for (int l = 0; l < ctx->L; ++l)
    if (windows[l] < -1)
      return fail(ctx, NC_ERR_INVALID_ARG, "window of layer " + std::to_string(l) + " below -1");
  for (int l = 0; l < ctx->L; ++l) ctx->windows[l] = windows[l] >= ctx->T ? -1 : windows[l];
  return NC_OK;
}

nc_status nc_zero_grads(nc_ctx* ctx) {
  if (!ctx) return NC_ERR_INVALID_ARG;
  if (!ctx->bound) return fail(ctx, NC_ERR_STATE, "bind first");
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oG), 0.f, ctx->n_total, ctx->st), "zero grads");
  return NC_OK;
}

nc_status nc_fwd_bwd(nc_ctx* ctx, const int32_t* tok, const int32_t* tgt, int32_t B,
                     float grad_scale, float* d_loss) {
  if (!ctx) return NC_ERR_INVALID_ARG;
  if (!ctx->bound) return fail(ctx, NC_ERR_STATE, "bind first");
  if (!tok || !tgt || !d_loss) return fail(ctx, NC_ERR_INVALID_ARG, "null pointer");
  if (B < 1 || B > ctx->maxB) return fail(ctx, NC_ERR_INVALID_ARG, "B out of [1, max_micro_batch]");
  if (!std::isfinite(grad_scale)) return fail(ctx, NC_ERR_INVALID_ARG, "grad_scale");
  const int dt = ctx->dt, L = ctx->L, d = ctx->d, H = ctx->H, F = ctx->F, V = ctx->V,
            T = ctx->T;
  const int N = B * T;
  const int Hkv = ctx->Hkv, dk = ctx->dk, Wd = ctx->W;
  // offsets of Wo and W1 inside a layer's block (Wq | Wk | Wv | Wo | W1 | W2)
  const size_t oWo = (size_t)d * d + 2ULL * dk * d, oW1 = oWo + (size_t)d * d;
  const float eps = ctx->cfg.norm_eps;
  hipStream_t st = ctx->st;
  const size_t es = ctx->es;
  float* x = A<float>(ctx, ctx->x);
  float* dx = A<float>(ctx, ctx->dx);
  float* da = A<float>(ctx, ctx->da);
  void* dxT = A(ctx, ctx->dxT);
  const float* tab = P<float>(ctx, ctx->oTab);
  float* G = P<float>(ctx, ctx->oG);
  char* aa = ctx->aa;

  // ---------------------------------------------------------------- forward
  NC_TRY(nc_embed_fwd(tok, P<float>(ctx, ctx->oP) + ctx->n_block, x, N, d, V, st), "embed");
  for (int l = 0; l < L; ++l) {
    const LayerAct& la = ctx->la[l];
    const size_t wb = (size_t)l * ctx->S;
    char* qkv = aa + la.qkv;
    NC_TRY(nc_rmsnorm_fwd(dt, x, aa + la.a1, A<float>(ctx, la.r1), N, d, eps, st), "norm1");
    NC_GEMM(ctx->fp8 ? gemm_fp8_fwd(ctx, aa + la.a1, d, wptr(ctx, wb), Wd, qkv, Wd, N, kEpiStore)
                     : gemm(ctx, aa + la.a1, d, kKCont, wptr(ctx, wb), d, kKCont, qkv, Wd, N, Wd,
                            d, kEpiStore), "qkv");
    NC_TRY(nc_qk_norm_rope_fwd(dt, qkv, A<float>(ctx, la.rqk), tab, N, T, H, Hkv, eps, st),
           "qknorm");
    NC_TRY(nc_attn_fwd(dt, qkv, qkv + d * es, qkv + (d + dk) * es, Wd, aa + la.o, d,
                       A<float>(ctx, la.lse), B, T, H, Hkv, ctx->windows[l], st), "attn fwd");
    NC_GEMM(ctx->fp8 ? gemm_fp8_fwd(ctx, aa + la.o, d, wptr(ctx, wb + oWo), d, x, d, N, kEpiAccF32)
                     : gemm(ctx, aa + la.o, d, kKCont, wptr(ctx, wb + oWo), d, kKCont, x, d, N, d,
                            d, kEpiAccF32), "out proj");
    NC_TRY(nc_rmsnorm_fwd(dt, x, aa + la.a2, A<float>(ctx, la.r2), N, d, eps, st), "norm2");
    NC_GEMM(ctx->fp8 ? gemm_fp8_fwd(ctx, aa + la.a2, d, wptr(ctx, wb + oW1), F, aa + la.g, F, N,
                                    kEpiRelu2)
                     : gemm(ctx, aa + la.a2, d, kKCont, wptr(ctx, wb + oW1), d, kKCont, aa + la.g,
                            F, N, F, d, kEpiRelu2), "mlp up");
    NC_GEMM(ctx->fp8 ? gemm_fp8_fwd(ctx, aa + la.g, F, wptr(ctx, wb + oW1 + (size_t)F * d), d, x,
                                    d, N, kEpiAccF32)
                     : gemm(ctx, aa + la.g, F, kKCont, wptr(ctx, wb + oW1 + (size_t)F * d), F,
                            kKCont, x, d, N, d, F, kEpiAccF32), "mlp down");
  }
  NC_TRY(nc_rmsnorm_fwd(dt, x, aa + ctx->xf, A<float>(ctx, ctx->rf), N, d, eps, st), "normf");

  // ------------------------------------------- lm_head + cross-entropy, chunked
  const size_t wh = (size_t)(ctx->n_block + (int64_t)V * d);
  const float ce_scale = grad_scale / (float)N;
  for (int c0 = 0; c0 < N; c0 += ctx->chunk) {
    const int nc = std::min(ctx->chunk, N - c0);
    const char* xfc = aa + ctx->xf + (size_t)c0 * d * es;
    NC_GEMM(gemm(ctx, xfc, d, kKCont, wptr_head(ctx), d, kKCont, aa + ctx->z, V, nc, V, d,
                kEpiStoreF32), "logits");
    NC_TRY(nc_cross_entropy(dt, A<float>(ctx, ctx->z), tgt + c0, aa + ctx->dz,
                            A<float>(ctx, ctx->loss_rows) + c0, nc, V, ce_scale, st), "ce");
    NC_GEMM(gemm(ctx, aa + ctx->dz, V, kKCont, wptr_head(ctx), d, kMNCont, da + (size_t)c0 * d, d,
                nc, d, V, kEpiStoreF32, nullptr, nullptr, ctx->splits_dxf), "dxf");
    NC_GEMM(gemm(ctx, aa + ctx->dz, V, kMNCont, xfc, d, kMNCont, G + wh, d, V, d, nc, kEpiAccF32,
                nullptr, nullptr, ctx->splits_head), "dWh");
  }
  NC_TRY(nc_sum_scaled(A<float>(ctx, ctx->loss_rows), N, 1.f / (float)N, d_loss, st), "loss");
  NC_TRY(nc_rmsnorm_bwd(dt, da, aa + ctx->xf, A<float>(ctx, ctx->rf), dx, dxT, N, d, 0, st),
         "normf bwd");

  // --------------------------------------------------------------- backward
  for (int l = L - 1; l >= 0; --l) {
    const LayerAct& la = ctx->la[l];
    const size_t wb = (size_t)l * ctx->S;
    const size_t w1 = wb + oW1, w2 = w1 + (size_t)F * d;
    char* qkv = aa + la.qkv;
    char* dqkv = aa + ctx->dqkv;
    // MLP
    NC_GEMM(gemm(ctx, dxT, d, kKCont, wptr(ctx, w2), F, kMNCont, aa + ctx->dh, F, N, F, d,
                kEpiRelu2Bwd, aa + la.g), "dh");
    NC_GEMM(gemm(ctx, dxT, d, kMNCont, aa + la.g, F, kMNCont, G + w2, F, d, F, N, kEpiAccF32,
                nullptr, nullptr, ctx->splits_2), "dW2");
    NC_GEMM(gemm(ctx, aa + ctx->dh, F, kMNCont, aa + la.a2, d, kMNCont, G + w1, d, F, d, N,
                kEpiAccF32, nullptr, nullptr, ctx->splits_1), "dW1");
    NC_GEMM(gemm(ctx, aa + ctx->dh, F, kKCont, wptr(ctx, w1), d, kMNCont, da, d, N, d, F,
                kEpiStoreF32), "da2");
    NC_TRY(nc_rmsnorm_bwd(dt, da, aa + la.a2, A<float>(ctx, la.r2), dx, dxT, N, d, 1, st),
           "norm2 bwd");
    // attention
    NC_GEMM(gemm(ctx, dxT, d, kKCont, wptr(ctx, wb + oWo), d, kMNCont, aa + ctx->dO, d,
                N, d, d, kEpiStore), "dO");
    NC_GEMM(gemm(ctx, dxT, d, kMNCont, aa + la.o, d, kMNCont, G + wb + oWo, d, d, d, N,
                kEpiAccF32, nullptr, nullptr, ctx->splits_o), "dWo");
    NC_TRY(nc_attn_bwd_pre(dt, aa + la.o, aa + ctx->dO, d, A<float>(ctx, ctx->Dbuf), B, T, H, st),
           "attn D");
    NC_TRY(nc_attn_bwd(dt, qkv, qkv + d * es, qkv + (d + dk) * es, Wd, aa + ctx->dO, d,
                       A<float>(ctx, la.lse), A<float>(ctx, ctx->Dbuf), dqkv, dqkv + d * es,
                       dqkv + (d + dk) * es, Wd, B, T, H, Hkv, ctx->windows[l], st), "attn bwd");
    NC_TRY(nc_qk_norm_rope_bwd(dt, dqkv, qkv, A<float>(ctx, la.rqk), tab, N, T, H, Hkv, st),
           "qknorm bwd");
    NC_GEMM(gemm(ctx, dqkv, Wd, kMNCont, aa + la.a1, d, kMNCont, G + wb, d, Wd, d, N,
                kEpiAccF32, nullptr, nullptr, ctx->splits_qkv), "dWqkv");
    NC_GEMM(gemm(ctx, dqkv, Wd, kKCont, wptr(ctx, wb), d, kMNCont, da, d, N, d, Wd,
                kEpiStoreF32), "da1");
    NC_TRY(nc_rmsnorm_bwd(dt, da, aa + la.a1, A<float>(ctx, la.r1), dx, dxT, N, d, 1, st),
           "norm1 bwd");
  }
  NC_TRY(nc_embed_bwd(tok, dx, G + ctx->n_block, N, V, d, aa + ctx->emb, st), "embed bwd");
  return NC_OK;
}

// Newton-Schulz on `count` matrices X [R, C] (R <= C) of group g, starting from
// the prepared buffers x32[0]/xh[0].  Every iterate is kept in fp32; only the
// matrix-core inputs are rounded.  *result = byte offset of the final fp32 X.
static nc_status newton_schulz(nc_ctx* ctx, int g, int count, int R, int C, size_t* result) {
  const nc_optim_config& o = ctx->ocfg;
  char* aa = ctx->aa;
  const auto& b = ctx->ns[g];
  int cur = 0;
  const int64_t sx = (int64_t)R * C, sa = (int64_t)R * R;
  for (int it = 0; it < o.ns_steps; ++it) {
    const float ca = o.ns_coeffs[it][0], cb = o.ns_coeffs[it][1], cc = o.ns_coeffs[it][2];
    // A = X X^T
    NC_GEMM(gemm(ctx, aa + b.xh[cur], C, kKCont, aa + b.xh[cur], C, kKCont, aa + b.a32, R, R, R,
                 C, kEpiDual, nullptr, aa + b.ah, 1, count, sx, sx, sa, 0.f, 1.f), "ns gram");
    // B = b A + c A A   (A symmetric: A A = A A^T)
    NC_GEMM(gemm(ctx, aa + b.ah, R, kKCont, aa + b.ah, R, kKCont, aa + b.b32, R, R, R, R,
                 kEpiDual, aa + b.a32, aa + b.bh, 1, count, sa, sa, sa, cb, cc), "ns poly");
    // X' = a X + B X
    NC_GEMM(gemm(ctx, aa + b.bh, R, kKCont, aa + b.xh[cur], C, kMNCont, aa + b.x32[cur ^ 1], C,
                 R, C, R, kEpiDual, aa + b.x32[cur], aa + b.xh[cur ^ 1], 1, count, sa, sx, sx,
                 ca, 1.f), "ns update");
    cur ^= 1;
  }
  *result = b.x32[cur];
  return NC_OK;
}

nc_status nc_optimizer_step(nc_ctx* ctx, float lr_mult) {
  if (!ctx) return NC_ERR_INVALID_ARG;
  if (!ctx->bound) return fail(ctx, NC_ERR_STATE, "bind first");
  if (!std::isfinite(lr_mult)) return fail(ctx, NC_ERR_INVALID_ARG, "lr_mult");
  const nc_optim_config& o = ctx->ocfg;
  const int dt = ctx->dt, L = ctx->L, d = ctx->d, F = ctx->F, V = ctx->V;
  hipStream_t st = ctx->st;
  ctx->step += 1;
  const double t = (double)ctx->step;
  const float bc1 = (float)(1.0 - std::pow((double)o.adam_beta1, t));
  const float bc2 = (float)(1.0 - std::pow((double)o.adam_beta2, t));
  float* Pm = P<float>(ctx, ctx->oP);
  float* G = P<float>(ctx, ctx->oG);
  const size_t Vd = (size_t)V * d;
  // AdamW: E | Wh contiguous after the block region
  NC_TRY(nc_adamw(Pm + ctx->n_block, G + ctx->n_block, P<float>(ctx, ctx->oAm),
                  P<float>(ctx, ctx->oAv), 2 * Vd, Vd, o.adam_lr_embed * lr_mult,
                  o.adam_lr_head * lr_mult, o.adam_beta1, o.adam_beta2, o.adam_eps, o.adam_wd,
                  bc1, bc2, dt ? (void*)(ctx->pa + ctx->oSh + ctx->n_block * 2) : nullptr, Vd, st),
         "adamw");
  if (L == 0) return NC_OK;
  // Muon
  float* Mom = P<float>(ctx, ctx->oM);
  NC_TRY(nc_momentum(Mom, G, ctx->n_block, o.muon_momentum, st), "momentum");
  const float* U = Mom;
  if (o.muon_nesterov) {
    NC_TRY(nc_nesterov(Mom, G, A<float>(ctx, ctx->nsU), ctx->n_block, o.muon_momentum, st),
           "nesterov");
    U = A<float>(ctx, ctx->nsU);
  }
  float* norms = A<float>(ctx, ctx->norms);
  float* frob = A<float>(ctx, ctx->frob);
  char* aa = ctx->aa;
  const int dk = ctx->dk;
  const int64_t dd = (int64_t)d * d, dF = (int64_t)d * F, kd = (int64_t)dk * d;
  const size_t oWo = (size_t)(dd + 2 * kd), o1 = oWo + (size_t)dd, o2 = o1 + (size_t)dF;
  // Matrix groups, each orthogonalised as one batch on its short side.  Their
  // Frobenius norms, NorMuon rows and scales follow each other in this order.
  struct Grp {
    size_t woff;   // block-region offset of the group's first matrix
    MatBatch mb;   // offsets of its matrices from there
    int R, C;      // W shape [R, C]
    int count;
    int tr;        // 1: orthogonalised as [C, R] (W1)
    int ns;        // Newton-Schulz buffer group
    size_t xoff;   // offset of the group's iterates in that buffer group
  };
  const MatBatch one{1, 0, ctx->S};
  Grp grps[4];
  int ng = 0;
  if (dk == d) {
    grps[ng++] = {0, MatBatch{4, dd, ctx->S}, d, d, 4 * L, 0, 0, 0};            // Wq Wk Wv Wo
  } else {
    grps[ng++] = {0, MatBatch{2, (int64_t)oWo, ctx->S}, d, d, 2 * L, 0, 0, 0};  // Wq Wo
    grps[ng++] = {(size_t)dd, MatBatch{2, kd, ctx->S}, dk, d, 2 * L, 0, 2, 0};  // Wk Wv
  }
  grps[ng++] = {o1, one, F, d, L, 1, 1, 0};                                     // W1
  grps[ng++] = {o2, one, d, F, L, 0, 1, (size_t)L * dF};                        // W2
  int nidx = 0;
  for (int i = 0; i < ng; ++i) {
    const Grp& g = grps[i];
    const int64_t el = (int64_t)g.R * g.C;
    const auto& b = ctx->ns[g.ns];
    NC_TRY(nc_frob_norms(U + g.woff, g.mb, el, g.count, frob + (size_t)nidx * 256, norms + nidx,
                         st), "norms");
    NC_TRY(nc_ns_prepare(dt, U + g.woff, g.mb, g.R, g.C, g.count, norms + nidx, o.ns_eps, g.tr,
                         A<float>(ctx, b.x32[0]) + g.xoff, aa + b.xh[0] + g.xoff * ctx->es, el,
                         st), "ns prepare");
    nidx += g.count;
  }
  // Newton-Schulz per buffer group: 0 square, 1 W1^T | W2 [d, F], 2 Wk | Wv [dk, d]
  size_t xres[3] = {0, 0, 0};
  nc_status s = newton_schulz(ctx, 0, grps[0].count, d, d, &xres[0]);
  if (s != NC_OK) return s;
  s = newton_schulz(ctx, 1, 2 * L, d, F, &xres[1]);
  if (s != NC_OK) return s;
  if (dk != d) {
    s = newton_schulz(ctx, 2, 2 * L, dk, d, &xres[2]);
    if (s != NC_OK) return s;
  }
  const float lr = o.muon_lr * lr_mult;
  char* sh = dt ? ctx->pa + ctx->oSh : nullptr;
  // NorMuon (optional): per-row statistics of each orthogonalised update, in the
  // orientation of W (W1's update is held transposed)
  int64_t roff = 0;
  nidx = 0;
  for (int i = 0; i < ng; ++i) {
    const Grp& g = grps[i];
    const int64_t el = (int64_t)g.R * g.C;
    const float* X = A<float>(ctx, xres[g.ns]) + g.xoff;
    const float* rm = nullptr;
    const float* ms = nullptr;
    if (ctx->nm_rows) {
      float* inv = A<float>(ctx, ctx->nm_inv) + roff;
      float* scl = A<float>(ctx, ctx->nm_scale) + nidx;
      NC_TRY(nc_normuon_stats(X, el, g.R, g.C, g.tr, g.count, P<float>(ctx, ctx->oV2) + roff,
                              o.normuon_beta2, A<float>(ctx, ctx->nm_vm) + roff,
                              A<float>(ctx, ctx->nm_q) + roff, inv, scl, st), "normuon");
      rm = inv;
      ms = scl;
    }
    NC_TRY(nc_ns_apply(Pm + g.woff, g.mb, g.R, g.C, g.count, X, el, g.tr, lr, o.muon_wd, rm, ms,
                       sh ? sh + g.woff * 2 : nullptr, st), "ns apply");
    roff += (int64_t)g.count * g.R;
    nidx += g.count;
  }
  return NC_OK;
}

nc_status nc_validate_launches(nc_ctx* ctx, int32_t B) {
  if (!ctx) return NC_ERR_INVALID_ARG;
  if (B < 1 || B > ctx->maxB) return fail(ctx, NC_ERR_INVALID_ARG, "B out of [1, max_micro_batch]");
  nc_ctx probe = *ctx;   // same plan, fake arena bases, nothing launched
  probe.pa = reinterpret_cast<char*>(uintptr_t(1) << 40);
  probe.aa = reinterpret_cast<char*>(uintptr_t(1) << 44);
  probe.bound = true;
  probe.dry_run = true;
  probe.err.clear();
  probe.range_error.clear();
  const int32_t* fake_tok = reinterpret_cast<const int32_t*>(probe.aa);
  float* fake_loss = reinterpret_cast<float*>(probe.aa);
  nc_status s = nc_fwd_bwd(&probe, fake_tok, fake_tok, B, 1.f, fake_loss);
  if (s == NC_OK) s = nc_optimizer_step(&probe, 1.f);
  ctx->err = probe.err;
  return s;
}

nc_status nc_param_count(const nc_ctx* ctx, int32_t* n) {
  if (!ctx || !n) return NC_ERR_INVALID_ARG;
  *n = (int32_t)ctx->params.size();
  return NC_OK;
}

nc_status nc_param_desc(const nc_ctx* ctx, int32_t i, nc_param_info* out) {
  if (!ctx || !out || i < 0 || i >= (int32_t)ctx->params.size()) return NC_ERR_INVALID_ARG;
  const ParamInfo& p = ctx->params[i];
  std::memset(out, 0, sizeof(*out));
  std::snprintf(out->name, sizeof(out->name), "%s", p.name.c_str());
  out->rows = p.rows;
  out->cols = p.cols;
  out->group = p.group;
  out->param_offset = (int64_t)(ctx->oP + p.elem * 4);
  out->grad_offset = (int64_t)(ctx->oG + p.elem * 4);
  if (p.group == NC_GROUP_MUON) {
    out->state0_offset = (int64_t)(ctx->oM + p.elem * 4);
    out->state1_offset = -1;
  } else {
    out->state0_offset = (int64_t)(ctx->oAm + p.adam_elem * 4);
    out->state1_offset = (int64_t)(ctx->oAv + p.adam_elem * 4);
  }
  return NC_OK;
}

nc_status nc_set_param(nc_ctx* ctx, int32_t i, const float* src, int32_t src_on_device) {
  if (!ctx || !src || i < 0 || i >= (int32_t)ctx->params.size()) return NC_ERR_INVALID_ARG;
  if (!ctx->bound) return fail(ctx, NC_ERR_STATE, "bind first");
  const ParamInfo& p = ctx->params[i];
  const size_t n = (size_t)p.rows * p.cols;
  float* dst = P<float>(ctx, ctx->oP) + p.elem;
  NC_TRY(hipMemcpyAsync(dst, src, n * 4,
                        src_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, ctx->st),
         "set param");
  if (ctx->dt && p.name != "E") {
    // bf16 copy: block region mirrors the master layout, then Wh
    const size_t sh_elem = p.name == "Wh" ? (size_t)ctx->n_block : p.elem;
    NC_TRY(nc_convert_f32(1, dst, ctx->pa + ctx->oSh + sh_elem * 2, n, ctx->st), "set shadow");
  }
  NC_TRY(hipStreamSynchronize(ctx->st), "set param sync");
  return NC_OK;
}

nc_status nc_get_tensor(nc_ctx* ctx, int32_t i, int32_t which, float* dst, int32_t dst_on_device) {
  if (!ctx || !dst || i < 0 || i >= (int32_t)ctx->params.size()) return NC_ERR_INVALID_ARG;
  if (!ctx->bound) return fail(ctx, NC_ERR_STATE, "bind first");
  nc_param_info d;
  nc_param_desc(ctx, i, &d);
  int64_t off;
  switch (which) {
    case NC_PARAM: off = d.param_offset; break;
    case NC_GRAD: off = d.grad_offset; break;
    case NC_MOMENTUM: off = d.group == NC_GROUP_MUON ? d.state0_offset : -1; break;
    case NC_ADAM_M: off = d.group == NC_GROUP_ADAMW ? d.state0_offset : -1; break;
    case NC_ADAM_V: off = d.group == NC_GROUP_ADAMW ? d.state1_offset : -1; break;
    default: off = -1;
  }
  if (off < 0) return fail(ctx, NC_ERR_INVALID_ARG, "parameter has no such tensor");
  const size_t n = (size_t)d.rows * d.cols;
  NC_TRY(hipMemcpyAsync(dst, ctx->pa + off, n * 4,
                        dst_on_device ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost, ctx->st),
         "get tensor");
  NC_TRY(hipStreamSynchronize(ctx->st), "get sync");
  return NC_OK;
}

nc_status nc_check_finite(nc_ctx* ctx, int32_t* host_flag) {
  if (!ctx || !host_flag) return NC_ERR_INVALID_ARG;
  if (!ctx->bound) return fail(ctx, NC_ERR_STATE, "bind first");
  // flag lives in the first 4 bytes of the norms scratch
  int32_t* flag = A<int32_t>(ctx, ctx->norms);
  NC_TRY(nc_fill_f32(reinterpret_cast<float*>(flag), 0.f, 1, ctx->st), "flag clear");
  NC_TRY(nc_check_finite(P<float>(ctx, ctx->oP), (size_t)ctx->n_total, flag, ctx->st), "finite p");
  NC_TRY(nc_check_finite(P<float>(ctx, ctx->oG), (size_t)ctx->n_total, flag, ctx->st), "finite g");
  int32_t h = 0;
  NC_TRY(hipMemcpyAsync(&h, flag, 4, hipMemcpyDeviceToHost, ctx->st), "flag copy");
  NC_TRY(hipStreamSynchronize(ctx->st), "finite sync");
  *host_flag = h ? 1 : 0;
  return h ? NC_ERR_NONFINITE : NC_OK;
}

nc_status nc_flops(const nc_ctx* ctx, int32_t B, double* fb, double* opt) {
  if (!ctx || B < 0) return NC_ERR_INVALID_ARG;
  const double L = ctx->L, d = ctx->d, F = ctx->F, V = ctx->V, T = ctx->T;
  const double N = (double)B * T;
  // attention: 12 d FLOP per (query, visible key) pair over forward and
  // backward; a plain causal layer is counted at T/2 keys per query, a
  // windowed one at its exact mean number of visible keys
  double keys = 0;
  for (int l = 0; l < ctx->L; ++l) {
    const int w = ctx->windows[l];
    if (w < 0) {
      keys += T / 2;
    } else {
      double sum = 0;
      for (int t = 0; t < ctx->T; ++t) sum += std::min(t, w) + 1;
      keys += sum / T;
    }
  }
  const double dk = ctx->dk;
  if (fb) *fb = 6.0 * N * (L * (2 * d * d + 2 * dk * d + 2 * d * F) + V * d) + 12.0 * N * d * keys;
  if (opt) {
    const double steps = ctx->ocfg.ns_steps;
    // 4 m^2 n + 2 m^3 per iteration for an m x n matrix, m <= n
    const double dk = ctx->dk;
    const double sq = 4.0 * d * d * d + 2.0 * d * d * d;     // m = n = d
    const double kv = 4.0 * dk * dk * d + 2.0 * dk * dk * dk; // m = dk, n = d
    const double rect = 4.0 * d * d * F + 2.0 * d * d * d;   // m = d, n = F
    *opt = steps * L * (2 * sq + 2 * kv + 2 * rect);
  }
  return NC_OK;
}

// ----------------------------------------------------------- single ops
nc_status nc_op_gemm(int32_t dtype, const void* A_, int64_t lda, int32_t al, const void* B_,
                     int64_t ldb, int32_t bl, void* C_, int64_t ldc, int32_t M, int32_t N,
                     int32_t K, int32_t batch, int64_t sA, int64_t sB, int64_t sC,
                     int32_t epi, const void* aux_in, void* aux_out, float alpha, float p0,
                     float p1, int32_t splits, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!A_ || !B_ || !C_ || M < 0 || N < 0 || K < 1 || batch < 1) return NC_ERR_INVALID_ARG;
  if ((dtype != NC_FP32 && dtype != NC_BF16) || al < 0 || al > 1 || bl < 0 || bl > 1 ||
      epi < 0 || epi > kEpiDual)
    return NC_ERR_INVALID_ARG;
  if ((epi == kEpiDual && !aux_out) ||
      ((epi == kEpiRelu2Bwd || epi == kEpiPoly) && !aux_in))
    return NC_ERR_INVALID_ARG;
  if (dtype == NC_BF16) {
    if (K % 8 || (al == kMNCont && M % 8) || (bl == kMNCont && N % 8)) return NC_ERR_UNSUPPORTED;
    if (lda % 8 || ldb % 8) return NC_ERR_UNSUPPORTED;
  }
  if (splits < 1) splits = 1;
  if (splits > 1) {
    if (dtype != NC_BF16 || (epi != kEpiStoreF32 && epi != kEpiAccF32)) return NC_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < (size_t)splits * batch * M * N * 4)
      return NC_ERR_INVALID_ARG;
  }
  GemmParams g{};
  g.A = A_; g.B = B_; g.C = C_; g.aux_in = aux_in; g.aux_out = aux_out;
  g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.sA = sA; g.sB = sB; g.sC = sC;
  g.M = M; g.N = N; g.K = K; g.batch = batch; g.a_layout = al; g.b_layout = bl; g.epi = epi;
  g.alpha = alpha; g.p0 = p0; g.p1 = p1; g.splits = splits;
  g.workspace = static_cast<float*>(workspace); g.workspace_bytes = workspace_bytes;
  return nc_launch_gemm(dtype, g, static_cast<hipStream_t>(stream)) == hipSuccess ? NC_OK
                                                                                 : NC_ERR_HIP;
}

nc_status nc_op_gemm_fp8(const void* A_, int64_t lda, const void* B_, int64_t ldb, void* C_,
                         int64_t ldc, int32_t M, int32_t N, int32_t K, int32_t epi, float alpha,
                         void* stream) {
  if (!A_ || !B_ || !C_ || M < 0 || N < 0 || K < 1) return NC_ERR_INVALID_ARG;
  if (epi != kEpiStore && epi != kEpiStoreF32 && epi != kEpiAccF32 && epi != kEpiRelu2)
    return NC_ERR_INVALID_ARG;
  if (lda < K || ldb < K || ldc < N) return NC_ERR_INVALID_ARG;
  if (K % 128 || lda % 16 || ldb % 16) return NC_ERR_UNSUPPORTED;
  GemmParams g{};
  g.A = A_; g.B = B_; g.C = C_;
  g.lda = lda; g.ldb = ldb; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K; g.batch = 1; g.splits = 1;
  g.a_layout = kKCont; g.b_layout = kKCont; g.epi = epi;
  g.alpha = alpha;
  const hipError_t e = nc_launch_gemm_f8(g, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return NC_ERR_UNSUPPORTED;
  return e == hipSuccess ? NC_OK : NC_ERR_HIP;
}

nc_status nc_op_fp8_quantize(int32_t dtype, const void* x, int64_t n, float* amax_scale,
                             void* q, float* workspace, void* stream) {
  if (!x || !amax_scale || !q || !workspace || n < 1) return NC_ERR_INVALID_ARG;
  if (dtype != NC_FP32 && dtype != NC_BF16) return NC_ERR_INVALID_ARG;
  return nc_fp8_quantize(dtype == NC_BF16, x, n, workspace, amax_scale,
                         static_cast<uint8_t*>(q), static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? NC_OK
             : NC_ERR_HIP;
}

nc_status nc_op_attention_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                              int64_t ld_qkv, void* o, int64_t ld_o, float* lse, int32_t B,
                              int32_t T, int32_t H, int32_t n_kv_head, int32_t window,
                              void* stream) {
  if (!q || !k || !v || !o || !lse || B < 1 || T < 1 || H < 1 || window < -1 ||
      n_kv_head < 1 || H % n_kv_head)
    return NC_ERR_INVALID_ARG;
  if (dtype == NC_BF16 && (T % 128 || ld_qkv % 8 || ld_o % 8)) return NC_ERR_UNSUPPORTED;
  return nc_attn_fwd(dtype == NC_BF16, q, k, v, ld_qkv, o, ld_o, lse, B, T, H, n_kv_head, window,
                     static_cast<hipStream_t>(stream)) == hipSuccess ? NC_OK : NC_ERR_HIP;
}

nc_status nc_op_attention_bwd(int32_t dtype, const void* q, const void* k, const void* v,
                              int64_t ld_qkv, const void* o, const void* dO, int64_t ld_o,
                              const float* lse, float* D, void* dq, void* dk, void* dv,
                              int64_t ld_d, int32_t B, int32_t T, int32_t H, int32_t n_kv_head,
                              int32_t window, void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !D || !dq || !dk || !dv || B < 1 || T < 1 || H < 1 ||
      window < -1 || n_kv_head < 1 || H % n_kv_head)
    return NC_ERR_INVALID_ARG;
  if (dtype == NC_BF16 && (T % 128 || ld_qkv % 8 || ld_o % 8 || ld_d % 8)) return NC_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = dtype == NC_BF16;
  if (nc_attn_bwd_pre(dt, o, dO, ld_o, D, B, T, H, st) != hipSuccess) return NC_ERR_HIP;
  return nc_attn_bwd(dt, q, k, v, ld_qkv, dO, ld_o, lse, D, dq, dk, dv, ld_d, B, T, H, n_kv_head,
                     window, st) ==
                 hipSuccess
             ? NC_OK
             : NC_ERR_HIP;
}

}  // extern "C"
