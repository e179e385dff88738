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
#include <mutex>
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
  bool fp8b = false; // and their backward products (gradients e5m2)
  // further mechanisms (nc_model_config.features)
  bool ve_on = false, resid_on = false, smear_on = false, backout_on = false;
  int Cg = 32;                 // value-embedding gate channels
  std::vector<int> ve_layers;  // layers with a value embedding, ascending
  std::vector<int> ve_slot;    // layer -> index in ve_layers, or -1
  int Lb = 0;                  // backout layer: xb is the stream entering it
  // element offsets (master / gradient layout) of the feature parameters
  size_t e_wg = 0, e_ws = 0, e_ve = 0, e_rl = 0, e_x0l = 0, e_sl = 0, e_bl = 0;
  int64_t n_vet = 0, n_sc = 0, n_adam = 0;   // VE table and scalar elements, AdamW region
  // activation arena: feature buffers
  size_t x0b = 0, xprev = 0, dx0b = 0, gbb = 0, xbb = 0, part_a = 0, part_b = 0, sig_s = 0,
         gs_s = 0, dz_s = 0, sig_ve = 0, dz_ve = 0, ve_rows = 0, outer_part = 0;
  size_t q8a = 0, q8s = 0, q8ws = 0;   // activation codes, a scale pair, amax scratch
  // fp8 backward: per layer the transposed codes of the four forward activations
  // (a1 [d, N] | o [d, N] | a2 [d, N] | g [F, N]) and their scales (8 floats);
  // the gradient's codes in its layout and transposed, and its scale
  size_t q8xt = 0, q8xt_layer = 0, q8xs = 0, q8dy = 0, q8dyt = 0, q8dys = 0;
  // the weights' e4m3 codes per layer (Wqkv | Wo | W1 | W2 in their layout,
  // then, with fp8 backward, transposed) and scales (8 floats per layer), made
  // once after each change of the weights and reused by every micro-batch
  size_t q8wc = 0, q8wc_layer = 0, q8wcs = 0;
  bool w8_ok = false;
  // per-block maxima of |a tensor|, written by its producer (RMSNorm, the
  // ReLU^2 epilogues) for the tensor's fp8 scale; q8part_n floats
  size_t q8part = 0, q8part_n = 0;
  int64_t S, n_block, n_total;
  std::vector<ParamInfo> params;
  // parameter arena byte offsets
  size_t oP, oG, oM, oAm, oAv, oSh, oTab, oV2, param_bytes;
  // activation arena byte offsets
  std::vector<LayerAct> la;
  size_t xf, rf, x, dx, dxT, da, dqkv, dO, Dbuf, dh, z, dz, loss_rows, ws, ws_bytes, emb,
      nsU, frob, norms, nm_vm, nm_q, nm_inv, nm_scale, flags, act_bytes;
  int64_t nm_rows = 0;   // NorMuon: rows of all block matrices (4L d + L F + L d)
  // Newton-Schulz buffers per group (0: square [d,d] (4L, or 2L with grouped
  // key/value heads), 1: 2L wide [d,F], 2: 2L [dk,d] with grouped key/value heads):
  // the fp32 iterate X (two, ping-pong), A = X X^T, B = b A + c A A, and a copy of
  // each in the activation type for the matrix cores.
  // Groups 3 and 4 (value-embedding gates, smear gate) are tiny and iterate in
  // fp32 with the VALU product (their xh buffers are their x32 buffers).
  struct NsBufs { size_t x32[2], xh[2], a32, ah, b32, bh; } ns[5];
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
  if (m->fp8_backward != 0 && m->fp8_backward != 1) {
    why = "fp8_backward is 0 or 1";
    return NC_ERR_INVALID_ARG;
  }
  if (m->fp8_backward && !m->fp8_forward) {
    why = "fp8_backward needs fp8_forward (it reuses the forward's activation codes)";
    return NC_ERR_UNSUPPORTED;
  }
  if (m->fp8_backward && m->seq_len % 128) {
    why = "fp8_backward needs seq_len % 128 == 0 (the weight gradients sum tokens in steps of 128)";
    return NC_ERR_UNSUPPORTED;
  }
  if (m->fp8_forward && m->d_ff % 128) {
    why = "fp8_forward needs d_ff % 128 == 0 (the fp8 products take K in steps of 128)";
    return NC_ERR_UNSUPPORTED;
  }
  if (m->features < 0 || m->features > 15) { why = "unknown feature bits"; return NC_ERR_INVALID_ARG; }
  if (m->ve_gate_channels < 0) { why = "ve_gate_channels"; return NC_ERR_INVALID_ARG; }
  {
    const int cg = m->ve_gate_channels ? m->ve_gate_channels : 32;
    if ((m->features & NC_FEAT_VALUE_EMBEDS) && (cg % 8 || cg > 64 || cg > m->d_model)) {
      why = "ve_gate_channels must be a multiple of 8, at most 64 and at most d_model";
      return NC_ERR_UNSUPPORTED;
    }
    if ((m->features & NC_FEAT_SMEAR) && m->d_model < 24) {
      why = "smear reads 24 embedding channels";
      return NC_ERR_UNSUPPORTED;
    }
    if ((m->features & NC_FEAT_BACKOUT) && m->n_layer < 1) {
      why = "backout needs at least one layer";
      return NC_ERR_UNSUPPORTED;
    }
    if ((m->features & (NC_FEAT_VALUE_EMBEDS | NC_FEAT_SMEAR)) && o && o->normuon) {
      why = "NorMuon is not combined with the gate parameters";
      return NC_ERR_UNSUPPORTED;
    }
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
  // Muon region: the layers' blocks, then the value-embedding gates
  // [n_ve][Hkv, Cg] and the smear gate [1, 24]; then E, Wh and the AdamW
  // extras: the value-embedding tables [n_ve][V, dk] and the scalars
  // (resid_lambdas [L], x0_lambdas [L], smear_lambda, backout_lambda), padded to 8.
  const int n_ve = (int)c->ve_layers.size();
  c->e_wg = (size_t)c->S * L;
  c->e_ws = c->e_wg + (size_t)n_ve * Hkv * c->Cg;
  c->n_block = (int64_t)c->e_ws + (c->smear_on ? 24 : 0);
  c->e_ve = (size_t)c->n_block + 2ULL * V * d;
  c->n_vet = (int64_t)n_ve * V * dk;
  c->e_rl = c->e_ve + (size_t)c->n_vet;
  c->e_x0l = c->e_rl + (c->resid_on ? L : 0);
  c->e_sl = c->e_x0l + (c->resid_on ? L : 0);
  c->e_bl = c->e_sl + (c->smear_on ? 1 : 0);
  c->n_sc = (int64_t)(c->e_bl + (c->backout_on ? 1 : 0) - c->e_rl);
  c->n_sc = (c->n_sc + 7) / 8 * 8;
  c->n_total = (int64_t)c->e_rl + c->n_sc;
  c->n_adam = 2LL * V * d + c->n_vet + c->n_sc;
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
  const int64_t ad0 = c->n_block;   // AdamW state offsets count from E
  for (int i = 0; i < n_ve; ++i) {
    const int l = c->ve_layers[i];
    c->params.push_back({"ve." + std::to_string(l), V, dk, NC_GROUP_ADAMW,
                         c->e_ve + (size_t)i * V * dk,
                         (int64_t)(c->e_ve + (size_t)i * V * dk) - ad0});
    c->params.push_back({std::to_string(l) + ".Wg", Hkv, c->Cg, NC_GROUP_MUON,
                         c->e_wg + (size_t)i * Hkv * c->Cg, -1});
  }
  if (c->resid_on) {
    c->params.push_back({"resid_lambdas", 1, L, NC_GROUP_ADAMW, c->e_rl, (int64_t)c->e_rl - ad0});
    c->params.push_back({"x0_lambdas", 1, L, NC_GROUP_ADAMW, c->e_x0l, (int64_t)c->e_x0l - ad0});
  }
  if (c->smear_on) {
    c->params.push_back({"smear_gate", 1, 24, NC_GROUP_MUON, c->e_ws, -1});
    c->params.push_back({"smear_lambda", 1, 1, NC_GROUP_ADAMW, c->e_sl, (int64_t)c->e_sl - ad0});
  }
  if (c->backout_on)
    c->params.push_back({"backout_lambda", 1, 1, NC_GROUP_ADAMW, c->e_bl, (int64_t)c->e_bl - ad0});

  Layout p;
  c->oP = p.take(c->n_total * 4);
  c->oG = p.take(c->n_total * 4);
  c->oM = p.take(c->n_block * 4);
  c->oAm = p.take((size_t)c->n_adam * 4);
  c->oAv = p.take((size_t)c->n_adam * 4);
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
  c->Dbuf = a.take(2 * N * H * 4);     // D, and -lse log2(e) for the bf16 dK/dV kernel
  c->dh = a.take(N * F * es);
  c->z = a.take((size_t)c->chunk * V * 4);
  c->dz = a.take((size_t)c->chunk * V * es);
  c->loss_rows = a.take(N * 4);
  c->flags = a.take(256);   // [0]: bits of out-of-range ids seen (1 token, 2 target)
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
  const size_t n_mats = (size_t)6 * std::max(L, 1) + n_ve + 1;   // Muon matrices
  c->frob = a.take(n_mats * 256 * 4);
  c->norms = a.take(n_mats * 4);
  // Newton-Schulz buffers of the gate groups (fp32 only)
  {
    const int cnt[2] = {n_ve, c->smear_on ? 1 : 0};
    const int R[2] = {std::min(Hkv, c->Cg), 1}, Cc[2] = {std::max(Hkv, c->Cg), 24};
    for (int g = 0; g < 2; ++g) {
      auto& b = c->ns[3 + g];
      b = {};
      if (!cnt[g]) continue;
      const size_t xe = (size_t)cnt[g] * R[g] * Cc[g], ae = (size_t)cnt[g] * R[g] * R[g];
      for (int k = 0; k < 2; ++k) {
        b.x32[k] = a.take(xe * 4);
        b.xh[k] = b.x32[k];
      }
      b.a32 = b.ah = a.take(ae * 4);
      b.b32 = b.bh = a.take(ae * 4);
    }
  }
  // feature buffers
  if (c->resid_on) {
    c->x0b = a.take(N * d * 4);
    c->xprev = a.take((size_t)L * N * d * 4);      // each layer's stream before its mix
    c->dx0b = a.take(N * d * 4);
  }
  if (c->backout_on) {
    c->gbb = a.take(N * d * 4);
    if (!c->resid_on) c->xbb = a.take(N * d * 4);
  }
  if (c->resid_on || c->backout_on) {
    c->part_a = a.take(N * 4);
    c->part_b = a.take(N * 4);
  }
  if (c->smear_on) {
    c->sig_s = a.take(N * 4);
    c->gs_s = a.take(N * 4);
    c->dz_s = a.take(N * 4);
  }
  if (n_ve) {
    c->sig_ve = a.take((size_t)n_ve * N * Hkv * 4);
    c->dz_ve = a.take(N * Hkv * 4);
    c->ve_rows = a.take(N * (size_t)dk * 4);
  }
  if (n_ve || c->smear_on)
    c->outer_part = a.take(nc_outer_scratch_floats(std::max(Hkv, 1), std::max(c->Cg, 24)) * 4);
  if (c->nm_rows) {
    c->nm_vm = a.take((size_t)c->nm_rows * 4);
    c->nm_q = a.take((size_t)c->nm_rows * 4);
    c->nm_inv = a.take((size_t)c->nm_rows * 4);
    c->nm_scale = a.take((size_t)6 * L * 4);
  }
  if (c->fp8) {
    // codes of the largest activation operand [N, max(d, F)]
    c->q8a = a.take(N * (size_t)std::max(d, F));
    c->q8s = a.take(4 * sizeof(float));
    c->q8ws = a.take(1024 * sizeof(float));
  }
  if (c->fp8) {
    // (RMSNorm: a block per 4 rows; GEMM: a tile per 256 x 256; attention: at most
    // a workgroup per 128 rows of each query and key/value head)
    c->q8part_n = std::max<size_t>({(size_t)ceil_div64(N, 4),
                                    (size_t)ceil_div64(N, 256) * ceil_div(std::max(F, W), 256),
                                    (size_t)ceil_div64(N, 128) * (H + Hkv)});
    c->q8part = a.take(c->q8part_n * sizeof(float));
    const size_t wn = (size_t)W * d + (size_t)d * d + 2 * (size_t)F * d;
    c->q8wc_layer = (c->fp8b ? 2 : 1) * wn;
    c->q8wc = a.take((size_t)L * c->q8wc_layer);
    c->q8wcs = a.take((size_t)L * 8 * sizeof(float));
  }
  if (c->fp8b) {
    c->q8xt_layer = N * (size_t)(3 * d + F);
    c->q8xt = a.take((size_t)L * c->q8xt_layer);
    c->q8xs = a.take((size_t)L * 8 * sizeof(float));
    const size_t wmax = (size_t)std::max(W, F);
    c->q8dy = a.take(N * wmax);
    c->q8dyt = a.take(N * wmax);
    c->q8dys = a.take(2 * sizeof(float));
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
bool operands_in_arenas(nc_ctx* c, const GemmParams& g, size_t es) {
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
                float p1 = 0.f, int dtype = -1) {
  const int dt = dtype < 0 ? c->dt : dtype;   // fp32 products of a bf16 model: dtype 0
  GemmParams g{};
  g.A = A_; g.B = B_; g.C = C_; g.aux_in = aux_in; g.aux_out = aux_out;
  g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.sA = sA; g.sB = sB; g.sC = sC;
  g.M = M; g.N = N; g.K = K; g.batch = batch;
  g.a_layout = al; g.b_layout = bl; g.epi = epi;
  g.alpha = 1.f; g.p0 = p0; g.p1 = p1;
  g.splits = splits;
  g.workspace = reinterpret_cast<float*>(c->aa + c->ws);
  g.workspace_bytes = c->ws_bytes;
  if (!operands_in_arenas(c, g, dt ? 2 : 4)) return hipErrorInvalidValue;
  if (c->dry_run) return hipSuccess;
  return nc_launch_gemm(dt, g, c->st);
}

// The QKV product (bf16) with the QK-norm + rotary forward in its epilogue:
// the first nh heads of each row (the query and key heads) come out
// RMS-normalised and rotated, and rqk gets their 1 / rms.
hipError_t gemm_qk_norm(nc_ctx* c, const void* A_, const void* W, void* C_, int M, int Wd, int K,
                        float* rqk, const float* tab, int T, int nh, float eps) {
  GemmParams g{};
  g.A = A_; g.B = W; g.C = C_;
  g.lda = K; g.ldb = K; g.ldc = Wd;
  g.M = M; g.N = Wd; g.K = K; g.batch = 1;
  g.a_layout = kKCont; g.b_layout = kKCont; g.epi = kEpiQkNorm;
  g.alpha = 1.f; g.splits = 1;
  g.rope = tab; g.rqk = rqk; g.rope_T = T; g.qk_heads = nh; g.qk_eps = eps;
  if (!operands_in_arenas(c, g, 2)) return hipErrorInvalidValue;
  if (!in_arena(c, tab, (size_t)2 * T * 64 * 4) || !in_arena(c, rqk, (size_t)M * nh * 4)) {
    c->range_error = "QK-norm table or rms output outside its arena";
    return hipErrorInvalidValue;
  }
  if (c->dry_run) return hipSuccess;
  return nc_launch_gemm(1, g, c->st);
}

// fp8 block products: one e4m3 scale per tensor (the pair {amax, s}); the
// kernel divides the sums by the two operands' s.
// The weight codes of layer l, product j (0 Wqkv [W, d], 1 Wo [d, d], 2 W1 [F, d],
// 3 W2 [d, F]): in the weight's layout (transposed = false) or transposed, and
// the scale pair.
struct WCodes { uint8_t* q; float* s; };
WCodes wcodes(nc_ctx* c, int l, int j, bool transposed) {
  const size_t d = c->d, F = c->F, W = c->W;
  const size_t off[4] = {0, W * d, W * d + d * d, W * d + d * d + F * d};
  const size_t half = W * d + d * d + 2 * F * d;
  uint8_t* base = reinterpret_cast<uint8_t*>(c->aa + c->q8wc) + (size_t)l * c->q8wc_layer;
  return {base + (transposed ? half : 0) + off[j],
          reinterpret_cast<float*>(c->aa + c->q8wcs) + (size_t)l * 8 + 2 * j};
}

// element offsets of Wo and W1 inside a layer's block (Wq | Wk | Wv | Wo | W1 | W2)
size_t oWo_of(const nc_ctx* c) { return (size_t)c->d * c->d + 2ULL * c->dk * c->d; }
size_t oW1_of(const nc_ctx* c) { return oWo_of(c) + (size_t)c->d * c->d; }

// The e4m3 codes of every layer's four weights (bf16 copies), in their layout
// and, with fp8 backward, transposed: once after each change of the weights.
hipError_t quantize_weights(nc_ctx* c) {
  const int d = c->d, F = c->F, W = c->W;
  const int rows[4] = {W, d, F, d}, cols[4] = {d, d, d, F};
  const size_t off[4] = {0, oWo_of(c), oW1_of(c), oW1_of(c) + (size_t)F * d};
  for (int l = 0; l < c->L; ++l)
    for (int j = 0; j < 4; ++j) {
      const WCodes q = wcodes(c, l, j, false), qt = wcodes(c, l, j, true);
      const void* w = wptr(c, (size_t)l * c->S + off[j]);
      const size_t n = (size_t)rows[j] * cols[j];
      if (!in_arena(c, w, n * 2) || !in_arena(c, q.q, n) || !in_arena(c, q.s, 8) ||
          (c->fp8b && !in_arena(c, qt.q, n))) {
        c->range_error = "fp8 weight codes outside the arena (layer " + std::to_string(l) + ")";
        return hipErrorInvalidValue;
      }
      if (c->dry_run) continue;
      const hipError_t e = nc_fp8_quantize(1, 0, w, rows[j], cols[j],
                                           reinterpret_cast<float*>(c->aa + c->q8ws), q.s, q.q,
                                           c->fp8b ? qt.q : nullptr, c->st);
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

// Forward block product in fp8: C (epilogue epi) = X W^T with X bf16 [N, K]
// quantised here (codes in q8a, and transposed into xt when given; scale pair
// in xscale or q8s[0..1]) and the weight's codes wq [Nout, K] with scale ws.
// x_parts (n_parts floats): per-block maxima of |X| from X's producer, used
// instead of a pass over X; c_parts: C's own per-tile maxima (ReLU^2 epilogue).
hipError_t gemm_fp8_fwd(nc_ctx* c, const void* X, int K, WCodes w, int Nout, void* C,
                        int64_t ldc, int N, int epi, uint8_t* xt = nullptr,
                        float* xscale = nullptr, const float* x_parts = nullptr,
                        int n_parts = 0, float* c_parts = nullptr) {
  float* sc = reinterpret_cast<float*>(c->aa + c->q8s);
  float* ws = reinterpret_cast<float*>(c->aa + c->q8ws);
  uint8_t* xa = reinterpret_cast<uint8_t*>(c->aa + c->q8a);
  const bool c_f32 = epi == kEpiStoreF32 || epi == kEpiAccF32;
  const size_t nx = (size_t)N * K, nw = (size_t)Nout * K;
  if (K % 128) {
    c->range_error = "fp8 GEMM needs K % 128 == 0 (K=" + std::to_string(K) + ")";
    return hipErrorInvalidValue;
  }
  // every extent inside its arena, also in a dry run
  if (!in_arena(c, X, nx * 2) || !in_arena(c, w.q, nw) || !in_arena(c, xa, nx) ||
      !in_arena(c, C, ((size_t)(N - 1) * ldc + Nout) * (c_f32 ? 4 : 2)) ||
      (xt && !in_arena(c, xt, nx)) || (xscale && !in_arena(c, xscale, 2 * sizeof(float))) ||
      (x_parts && !in_arena(c, x_parts, (size_t)n_parts * 4)) ||
      (c_parts && !in_arena(c, c_parts, (size_t)ceil_div(N, 256) * ceil_div(Nout, 256) * 4))) {
    c->range_error = "fp8 GEMM operand outside its arena (N=" + std::to_string(N) +
                     " Nout=" + std::to_string(Nout) + " K=" + std::to_string(K) + ")";
    return hipErrorInvalidValue;
  }
  if (c->dry_run) return hipSuccess;
  float* xs = xscale ? xscale : sc;
  const hipError_t e = x_parts ? nc_fp8_quantize_parts(0, X, N, K, x_parts, n_parts, xs, xa, xt,
                                                       c->st)
                               : nc_fp8_quantize(1, 0, X, N, K, ws, xs, xa, xt, c->st);
  if (e != hipSuccess) return e;
  GemmParams g{};
  g.A = xa; g.B = w.q; g.C = C;
  g.amax_part = c_parts;
  g.lda = K; g.ldb = K; g.ldc = ldc;
  g.M = N; g.N = Nout; g.K = K; g.batch = 1; g.splits = 1;
  g.a_layout = kKCont; g.b_layout = kKCont; g.epi = epi; g.alpha = 1.f;
  g.scale_a = xs; g.scale_b = w.s;
  return nc_launch_gemm_f8(g, c->st);
}

// Backward of an fp8 block product y = x W^T.  fp8_grad_codes: the bf16
// gradient dY [N, w] to e5m2 codes in its layout (q8dy) and transposed
// (q8dyt), scale in q8dys.
// parts (n_parts floats): per-block maxima of |dY| from dY's producer.
hipError_t fp8_grad_codes(nc_ctx* c, const void* dY, int N, int w, const float* parts = nullptr,
                          int n_parts = 0) {
  uint8_t* q = reinterpret_cast<uint8_t*>(c->aa + c->q8dy);
  uint8_t* qt = reinterpret_cast<uint8_t*>(c->aa + c->q8dyt);
  float* ds = reinterpret_cast<float*>(c->aa + c->q8dys);
  const size_t n = (size_t)N * w;
  if (!in_arena(c, dY, n * 2) || !in_arena(c, q, n) || !in_arena(c, qt, n) ||
      (parts && !in_arena(c, parts, (size_t)n_parts * 4))) {
    c->range_error = "fp8 gradient codes outside the arena (N=" + std::to_string(N) +
                     " w=" + std::to_string(w) + ")";
    return hipErrorInvalidValue;
  }
  if (c->dry_run) return hipSuccess;
  if (parts) return nc_fp8_quantize_parts(1, dY, N, w, parts, n_parts, ds, q, qt, c->st);
  return nc_fp8_quantize(1, 1, dY, N, w, reinterpret_cast<float*>(c->aa + c->q8ws), ds, q, qt,
                         c->st);
}

// dX (epilogue epi, aux g for the ReLU^2 backward) = dY W from the gradient's
// codes [N, out] and the transposed codes wt [in, out] of the weight W [out, in].
hipError_t gemm_fp8_dx(nc_ctx* c, WCodes wt, int out, int in, void* C, int64_t ldc, int N,
                       int epi, const void* aux = nullptr, float* c_parts = nullptr) {
  const uint8_t* dyq = reinterpret_cast<const uint8_t*>(c->aa + c->q8dy);
  const bool c_f32 = epi == kEpiStoreF32 || epi == kEpiAccF32;
  const size_t nw = (size_t)out * in, cext = ((size_t)(N - 1) * ldc + in) * (c_f32 ? 4 : 2);
  if (!in_arena(c, wt.q, nw) || !in_arena(c, dyq, (size_t)N * out) || !in_arena(c, C, cext) ||
      (aux && !in_arena(c, aux, cext)) ||
      (c_parts && !in_arena(c, c_parts, (size_t)ceil_div(N, 256) * ceil_div(in, 256) * 4))) {
    c->range_error = "fp8 input-gradient operand outside its arena (N=" + std::to_string(N) +
                     " out=" + std::to_string(out) + " in=" + std::to_string(in) + ")";
    return hipErrorInvalidValue;
  }
  if (c->dry_run) return hipSuccess;
  GemmParams g{};
  g.A = dyq; g.B = wt.q; g.C = C; g.aux_in = aux;
  g.amax_part = c_parts;
  g.lda = out; g.ldb = out; g.ldc = ldc;
  g.M = N; g.N = in; g.K = out; g.batch = 1; g.splits = 1;
  g.a_layout = kKCont; g.b_layout = kKCont; g.epi = epi; g.alpha = 1.f;
  g.scale_a = reinterpret_cast<const float*>(c->aa + c->q8dys); g.scale_b = wt.s;
  g.fmt_a = 1;
  return nc_launch_gemm_f8(g, c->st);
}

// dW [out, in] += dY^T X from the transposed gradient codes [out, N] and the
// forward's transposed activation codes xt [in, N] (scale xs), split over K = N.
hipError_t gemm_fp8_dw(nc_ctx* c, const uint8_t* xt, const float* xs, int out, int in, float* G,
                       int N, int splits) {
  const uint8_t* dyt = reinterpret_cast<const uint8_t*>(c->aa + c->q8dyt);
  if (splits > 1 && nc_gemm_workspace_bytes(out, in, splits) > c->ws_bytes) splits = 1;
  if (!in_arena(c, xt, (size_t)in * N) || !in_arena(c, xs, 2 * sizeof(float)) ||
      !in_arena(c, dyt, (size_t)out * N) || !in_arena(c, G, (size_t)out * in * 4)) {
    c->range_error = "fp8 weight-gradient operand outside its arena (N=" + std::to_string(N) +
                     " out=" + std::to_string(out) + " in=" + std::to_string(in) + ")";
    return hipErrorInvalidValue;
  }
  if (c->dry_run) return hipSuccess;
  GemmParams g{};
  g.A = dyt; g.B = xt; g.C = G;
  g.lda = N; g.ldb = N; g.ldc = in;
  g.M = out; g.N = in; g.K = N; g.batch = 1; g.splits = splits;
  g.a_layout = kKCont; g.b_layout = kKCont; g.epi = kEpiAccF32; g.alpha = 1.f;
  g.scale_a = reinterpret_cast<const float*>(c->aa + c->q8dys); g.scale_b = xs;
  g.fmt_a = 1;
  g.workspace = reinterpret_cast<float*>(c->aa + c->ws);
  g.workspace_bytes = c->ws_bytes;
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
  c->fp8b = c->fp8 && cfg->fp8_backward != 0;
  c->dk = c->Hkv * 128;
  c->W = c->d + 2 * c->dk;
  c->V = cfg->vocab; c->T = cfg->seq_len; c->maxB = cfg->max_micro_batch;
  c->Nmax = c->maxB * c->T;
  c->windows.assign(c->L, -1);
  c->ve_on = cfg->features & NC_FEAT_VALUE_EMBEDS;
  c->resid_on = cfg->features & NC_FEAT_RESID_LAMBDAS;
  c->smear_on = cfg->features & NC_FEAT_SMEAR;
  c->backout_on = cfg->features & NC_FEAT_BACKOUT;
  c->Cg = cfg->ve_gate_channels ? cfg->ve_gate_channels : 32;
  c->ve_slot.assign(c->L, -1);
  if (c->ve_on)
    for (int l = 0; l < c->L; ++l)
      if ((c->L - 1 - l) % 2 == 0) {
        c->ve_slot[l] = (int)c->ve_layers.size();
        c->ve_layers.push_back(l);
      }
  c->Lb = c->L / 2;
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
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oAm), 0.f, ctx->n_adam, ctx->st), "zero m");
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oAv), 0.f, ctx->n_adam, ctx->st), "zero v");
  if (ctx->nm_rows)
    NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oV2), 0.f, ctx->nm_rows, ctx->st), "zero normuon v2");
  NC_TRY(nc_fill_f32(A<float>(ctx, ctx->flags), 0.f, 1, ctx->st), "clear input flags");
  ctx->step = 0;
  NC_TRY(hipStreamSynchronize(ctx->st), "bind sync");
  ctx->w8_ok = false;
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
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oAm), 0.f, ctx->n_adam, ctx->st), "zero m");
  NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oAv), 0.f, ctx->n_adam, ctx->st), "zero v");
  if (ctx->nm_rows)
    NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oV2), 0.f, ctx->nm_rows, ctx->st), "zero normuon v2");
  // scalars at the values that leave the plain model unchanged: resid 1, x0,
  // smear and backout 0 (and the padding after them 0)
  if (ctx->n_sc) {
    NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oP) + ctx->e_rl, 0.f, ctx->n_sc, ctx->st), "scalars");
    if (ctx->resid_on)
      NC_TRY(nc_fill_f32(P<float>(ctx, ctx->oP) + ctx->e_rl, 1.f, ctx->L, ctx->st), "resid");
  }
  ctx->step = 0;
  ctx->w8_ok = false;
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
  const size_t oWo = oWo_of(ctx), oW1 = oW1_of(ctx);
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
  int32_t* flags = A<int32_t>(ctx, ctx->flags);
  if (ctx->fp8 && !ctx->w8_ok) {   // weight codes for this and the following micro-batches
    NC_GEMM(quantize_weights(ctx), "weight codes");
    if (!ctx->dry_run) ctx->w8_ok = true;
  }
  const float* Pm = P<float>(ctx, ctx->oP);
  const float* E = Pm + ctx->n_block;
  float* x0b = ctx->resid_on ? A<float>(ctx, ctx->x0b) : nullptr;
  const size_t Nd = (size_t)N * d;
  auto xprev_of = [&](int l) { return A<float>(ctx, ctx->xprev) + (size_t)l * Nd; };
  // the stream entering layer Lb (backout's xb)
  float* xb = !ctx->backout_on ? nullptr
              : ctx->resid_on  ? xprev_of(ctx->Lb)
                               : A<float>(ctx, ctx->xbb);
  if (ctx->smear_on) {
    NC_TRY(nc_embed_smear_fwd(tok, E, Pm + ctx->e_ws, Pm + ctx->e_sl, x, x0b,
                              A<float>(ctx, ctx->sig_s), N, T, d, V, flags, st), "embed smear");
  } else {
    NC_TRY(nc_embed_fwd(tok, E, x, N, d, V, flags, st), "embed");
    if (x0b) NC_TRY(hipMemcpyAsync(x0b, x, Nd * 4, hipMemcpyDeviceToDevice, st), "x0");
  }
  // fp8: the producers of a1, a2 (RMSNorm) and g (the ReLU^2 epilogue) leave
  // per-block maxima of their output for its scale
  float* parts = ctx->fp8 ? A<float>(ctx, ctx->q8part) : nullptr;
  // fp8 backward: the forward quantiser also writes the transposed codes of
  // each layer's four activations (a1, o, a2, g) and keeps their scales
  auto xt_of = [&](int l, int which) -> uint8_t* {
    if (!ctx->fp8b) return nullptr;
    return A<uint8_t>(ctx, ctx->q8xt) + (size_t)l * ctx->q8xt_layer + (size_t)which * d * N;
  };
  auto xs_of = [&](int l, int which) -> float* {
    if (!ctx->fp8b) return nullptr;
    return A<float>(ctx, ctx->q8xs) + (size_t)l * 8 + 2 * which;
  };
  for (int l = 0; l < L; ++l) {
    const LayerAct& la = ctx->la[l];
    const size_t wb = (size_t)l * ctx->S;
    char* qkv = aa + la.qkv;
    const bool mixed = ctx->resid_on || (ctx->backout_on && l == ctx->Lb);
    if (mixed) {
      // x <- resid_l x + x0_l x0 (saving the stream before the mix), then norm1
      NC_TRY(nc_rmsnorm_mix_fwd(dt, x, x0b, ctx->resid_on ? xprev_of(l) : xb,
                                ctx->resid_on ? Pm + ctx->e_rl + l : nullptr,
                                ctx->resid_on ? Pm + ctx->e_x0l + l : nullptr, 1.f,
                                ctx->resid_on, aa + la.a1, A<float>(ctx, la.r1), N, d, eps, st),
             "mix norm1");
    } else {
      NC_TRY(nc_rmsnorm_fwd(dt, x, aa + la.a1, A<float>(ctx, la.r1), N, d, eps, st, parts),
             "norm1");
    }
    NC_GEMM(ctx->fp8 ? gemm_fp8_fwd(ctx, aa + la.a1, d, wcodes(ctx, l, 0, false), Wd, qkv, Wd, N,
                                    kEpiStore, xt_of(l, 0), xs_of(l, 0),
                                    mixed ? nullptr : parts, ceil_div(N, 4))
                     : dt ? gemm_qk_norm(ctx, aa + la.a1, wptr(ctx, wb), qkv, N, Wd, d,
                                         A<float>(ctx, la.rqk), tab, T, H + Hkv, eps)
                     : gemm(ctx, aa + la.a1, d, kKCont, wptr(ctx, wb), d, kKCont, qkv, Wd, N, Wd,
                            d, kEpiStore), "qkv");
    if (ctx->ve_slot[l] >= 0) {
      const int i = ctx->ve_slot[l];
      NC_TRY(nc_ve_mix_fwd(dt, tok, Pm + ctx->e_ve + (size_t)i * V * dk,
                           Pm + ctx->e_wg + (size_t)i * Hkv * ctx->Cg, aa + la.a1, d,
                           qkv + (d + dk) * es, Wd, A<float>(ctx, ctx->sig_ve) + (size_t)i * N * Hkv,
                           N, Hkv, ctx->Cg, V, st), "value embedding");
    }
    if (ctx->fp8 || !dt)   // bf16: formed in the QKV product's epilogue
      NC_TRY(nc_qk_norm_rope_fwd(dt, qkv, A<float>(ctx, la.rqk), tab, N, T, H, Hkv, eps, st),
             "qknorm");
    NC_TRY(nc_attn_fwd(dt, qkv, qkv + d * es, qkv + (d + dk) * es, Wd, aa + la.o, d,
                       A<float>(ctx, la.lse), B, T, H, Hkv, ctx->windows[l], st, parts, 1),
           "attn fwd");
    NC_GEMM(ctx->fp8 ? gemm_fp8_fwd(ctx, aa + la.o, d, wcodes(ctx, l, 1, false), d, x, d, N, kEpiAccF32,
                                    xt_of(l, 1), xs_of(l, 1), parts,
                                    nc_attn_amax_parts(B, T, H, Hkv, ctx->windows[l], 0))
                     : gemm(ctx, aa + la.o, d, kKCont, wptr(ctx, wb + oWo), d, kKCont, x, d, N, d,
                            d, kEpiAccF32), "out proj");
    NC_TRY(nc_rmsnorm_fwd(dt, x, aa + la.a2, A<float>(ctx, la.r2), N, d, eps, st, parts), "norm2");
    NC_GEMM(ctx->fp8 ? gemm_fp8_fwd(ctx, aa + la.a2, d, wcodes(ctx, l, 2, false), F, aa + la.g, F, N,
                                    kEpiRelu2, xt_of(l, 2), xs_of(l, 2), parts, ceil_div(N, 4),
                                    parts)
                     : gemm(ctx, aa + la.a2, d, kKCont, wptr(ctx, wb + oW1), d, kKCont, aa + la.g,
                            F, N, F, d, kEpiRelu2), "mlp up");
    NC_GEMM(ctx->fp8 ? gemm_fp8_fwd(ctx, aa + la.g, F, wcodes(ctx, l, 3, false), d, x,
                                    d, N, kEpiAccF32, xt_of(l, 3), xs_of(l, 3), parts,
                                    ceil_div(N, 256) * ceil_div(F, 256))
                     : gemm(ctx, aa + la.g, F, kKCont, wptr(ctx, wb + oW1 + (size_t)F * d), F,
                            kKCont, x, d, N, d, F, kEpiAccF32), "mlp down");
  }
  if (ctx->backout_on)        // xf = N(x - backout xb)
    NC_TRY(nc_rmsnorm_mix_fwd(dt, x, xb, nullptr, nullptr, Pm + ctx->e_bl, -1.f, 0, aa + ctx->xf,
                              A<float>(ctx, ctx->rf), N, d, eps, st), "backout normf");
  else
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
                            A<float>(ctx, ctx->loss_rows) + c0, nc, V, ce_scale, flags, st),
           "ce");
    NC_GEMM(gemm(ctx, aa + ctx->dz, V, kKCont, wptr_head(ctx), d, kMNCont, da + (size_t)c0 * d, d,
                nc, d, V, kEpiStoreF32, nullptr, nullptr, ctx->splits_dxf), "dxf");
    NC_GEMM(gemm(ctx, aa + ctx->dz, V, kMNCont, xfc, d, kMNCont, G + wh, d, V, d, nc, kEpiAccF32,
                nullptr, nullptr, ctx->splits_head), "dWh");
  }
  NC_TRY(nc_sum_scaled(A<float>(ctx, ctx->loss_rows), N, 1.f / (float)N, d_loss, st), "loss");
  // fp8 backward: dxT's per-block maxima come from the RMSNorm backward that
  // wrote it (the mixed-stream backward leaves none: dxT_parts false)
  float* bparts = ctx->fp8b ? parts : nullptr;
  const int nb_rows = ceil_div(N, 4), nb_ff = ceil_div(N, 256) * ceil_div(F, 256);
  NC_TRY(nc_rmsnorm_bwd(dt, da, 0, aa + ctx->xf, A<float>(ctx, ctx->rf), dx, dxT, N, d, 0, st,
                        bparts), "normf bwd");
  bool dxT_parts = bparts != nullptr;
  float* part_a = (ctx->resid_on || ctx->backout_on) ? A<float>(ctx, ctx->part_a) : nullptr;
  float* part_b = (ctx->resid_on || ctx->backout_on) ? A<float>(ctx, ctx->part_b) : nullptr;
  float* gb = ctx->backout_on ? A<float>(ctx, ctx->gbb) : nullptr;
  float* dx0b = ctx->resid_on ? A<float>(ctx, ctx->dx0b) : nullptr;
  void* emb_scratch = aa + ctx->emb;
  if (ctx->backout_on) {      // d backout = -dx . xb; gb = -backout dx joins at layer Lb
    NC_TRY(nc_backout_bwd(dx, xb, Pm + ctx->e_bl, gb, part_a, N, d, st), "backout bwd");
    NC_TRY(nc_sum_into(part_a, N, G + ctx->e_bl, st), "backout grad");
  }
  if (dx0b) NC_TRY(nc_fill_f32(dx0b, 0.f, Nd, st), "zero dx0");
  if (ctx->ve_on) NC_TRY(nc_embed_sort(tok, N, V, emb_scratch, st), "token sort");

  // The gradient at a block norm's output (da, from the da1 / da2 products)
  // is stored in bf16 when nothing else adds into it (no value-embedding gate,
  // no mixed-stream norm): half the bytes for the product's epilogue and the
  // norm backward.  The final norm's comes from the split-K lm_head product
  // and stays fp32.
  const bool da16 = dt && !ctx->ve_on && !ctx->resid_on && !ctx->backout_on;
  const int epi_da = da16 ? kEpiStore : kEpiStoreF32;

  // --------------------------------------------------------------- backward
  for (int l = L - 1; l >= 0; --l) {
    const LayerAct& la = ctx->la[l];
    const size_t wb = (size_t)l * ctx->S;
    const size_t w1 = wb + oW1, w2 = w1 + (size_t)F * d;
    char* qkv = aa + la.qkv;
    char* dqkv = aa + ctx->dqkv;
    // MLP
    if (ctx->fp8b) {   // the eight products in fp8: dY e5m2, X and W e4m3
      NC_GEMM(fp8_grad_codes(ctx, dxT, N, d, dxT_parts ? bparts : nullptr, nb_rows), "dx codes");
      NC_GEMM(gemm_fp8_dx(ctx, wcodes(ctx, l, 3, true), d, F, aa + ctx->dh, F, N, kEpiRelu2Bwd,
                          aa + la.g, bparts),
              "dh");
      NC_GEMM(gemm_fp8_dw(ctx, xt_of(l, 3), xs_of(l, 3), d, F, G + w2, N, ctx->splits_2), "dW2");
      NC_GEMM(fp8_grad_codes(ctx, aa + ctx->dh, N, F, bparts, nb_ff), "dh codes");
      NC_GEMM(gemm_fp8_dw(ctx, xt_of(l, 2), xs_of(l, 2), F, d, G + w1, N, ctx->splits_1), "dW1");
      NC_GEMM(gemm_fp8_dx(ctx, wcodes(ctx, l, 2, true), F, d, da, d, N, epi_da), "da2");
    } else {
      NC_GEMM(gemm(ctx, dxT, d, kKCont, wptr(ctx, w2), F, kMNCont, aa + ctx->dh, F, N, F, d,
                  kEpiRelu2Bwd, aa + la.g), "dh");
      NC_GEMM(gemm(ctx, dxT, d, kMNCont, aa + la.g, F, kMNCont, G + w2, F, d, F, N, kEpiAccF32,
                  nullptr, nullptr, ctx->splits_2), "dW2");
      NC_GEMM(gemm(ctx, aa + ctx->dh, F, kMNCont, aa + la.a2, d, kMNCont, G + w1, d, F, d, N,
                  kEpiAccF32, nullptr, nullptr, ctx->splits_1), "dW1");
      NC_GEMM(gemm(ctx, aa + ctx->dh, F, kKCont, wptr(ctx, w1), d, kMNCont, da, d, N, d, F,
                  epi_da), "da2");
    }
    NC_TRY(nc_rmsnorm_bwd(dt, da, da16, aa + la.a2, A<float>(ctx, la.r2), dx, dxT, N, d, 1, st,
                          bparts),
           "norm2 bwd");
    // attention
    if (ctx->fp8b) {
      NC_GEMM(fp8_grad_codes(ctx, dxT, N, d, bparts, nb_rows), "dx codes");
      NC_GEMM(gemm_fp8_dx(ctx, wcodes(ctx, l, 1, true), d, d, aa + ctx->dO, d, N, kEpiStore), "dO");
      NC_GEMM(gemm_fp8_dw(ctx, xt_of(l, 1), xs_of(l, 1), d, d, G + wb + oWo, N, ctx->splits_o),
              "dWo");
    } else {
      NC_GEMM(gemm(ctx, dxT, d, kKCont, wptr(ctx, wb + oWo), d, kMNCont, aa + ctx->dO, d,
                  N, d, d, kEpiStore), "dO");
      NC_GEMM(gemm(ctx, dxT, d, kMNCont, aa + la.o, d, kMNCont, G + wb + oWo, d, d, d, N,
                  kEpiAccF32, nullptr, nullptr, ctx->splits_o), "dWo");
    }
    // bf16: D and the QK-norm + rotary backward are formed inside the attention
    // backward kernels; fp32: separate kernels
    NC_TRY(nc_attn_bwd(dt, qkv, qkv + d * es, qkv + (d + dk) * es, Wd, aa + la.o, aa + ctx->dO, d,
                       A<float>(ctx, la.lse), A<float>(ctx, ctx->Dbuf), dqkv, dqkv + d * es,
                       dqkv + (d + dk) * es, Wd, B, T, H, Hkv, ctx->windows[l],
                       dt ? A<float>(ctx, la.rqk) : nullptr, dt ? tab : nullptr, st, bparts),
           "attn bwd");
    if (!dt)
      NC_TRY(nc_qk_norm_rope_bwd(dt, dqkv, qkv, A<float>(ctx, la.rqk), tab, N, T, H, Hkv, st),
             "qknorm bwd");
    const int vs = ctx->ve_slot[l];
    if (vs >= 0) {   // value embedding: table rows, gate matrix, gate input
      const float* VEl = Pm + ctx->e_ve + (size_t)vs * V * dk;
      float* dz = A<float>(ctx, ctx->dz_ve);
      float* rows = A<float>(ctx, ctx->ve_rows);
      NC_TRY(nc_ve_bwd(dt, tok, VEl, dqkv + (d + dk) * es, Wd,
                       A<float>(ctx, ctx->sig_ve) + (size_t)vs * N * Hkv, rows, dz, N, Hkv, V, st),
             "value embedding bwd");
      NC_TRY(nc_embed_segsum(tok, rows, G + ctx->e_ve + (size_t)vs * V * dk, N, V, dk,
                             emb_scratch, st), "value embedding rows");
      NC_TRY(nc_outer_accumulate(dt, dz, Hkv, aa + la.a1, d, nullptr, V, ctx->Cg, N,
                                 A<float>(ctx, ctx->outer_part),
                                 G + ctx->e_wg + (size_t)vs * Hkv * ctx->Cg, st), "gate grad");
    }
    if (ctx->fp8b) {
      NC_GEMM(fp8_grad_codes(ctx, dqkv, N, Wd, bparts,
                             nc_attn_amax_parts(B, T, H, Hkv, ctx->windows[l], 1)),
              "dqkv codes");
      NC_GEMM(gemm_fp8_dw(ctx, xt_of(l, 0), xs_of(l, 0), Wd, d, G + wb, N, ctx->splits_qkv),
              "dWqkv");
      NC_GEMM(gemm_fp8_dx(ctx, wcodes(ctx, l, 0, true), Wd, d, da, d, N, epi_da), "da1");
    } else {
      NC_GEMM(gemm(ctx, dqkv, Wd, kMNCont, aa + la.a1, d, kMNCont, G + wb, d, Wd, d, N,
                  kEpiAccF32, nullptr, nullptr, ctx->splits_qkv), "dWqkv");
      NC_GEMM(gemm(ctx, dqkv, Wd, kKCont, wptr(ctx, wb), d, kMNCont, da, d, N, d, Wd,
                  epi_da), "da1");
    }
    if (vs >= 0)
      NC_TRY(nc_ve_gate_da(A<float>(ctx, ctx->dz_ve), Pm + ctx->e_wg + (size_t)vs * Hkv * ctx->Cg,
                           da, d, N, Hkv, ctx->Cg, st), "gate input grad");
    if (ctx->resid_on || (ctx->backout_on && l == ctx->Lb)) {
      NC_TRY(nc_rmsnorm_mix_bwd(dt, da, aa + la.a1, A<float>(ctx, la.r1), dx, dxT,
                                ctx->resid_on ? xprev_of(l) : nullptr, x0b, dx0b,
                                ctx->resid_on ? Pm + ctx->e_rl + l : nullptr,
                                ctx->resid_on ? Pm + ctx->e_x0l + l : nullptr,
                                ctx->backout_on && l == ctx->Lb ? gb : nullptr,
                                ctx->resid_on ? part_a : nullptr, ctx->resid_on ? part_b : nullptr,
                                N, d, 1, st), "mix norm1 bwd");
      if (ctx->resid_on) {
        NC_TRY(nc_sum_into(part_a, N, G + ctx->e_rl + l, st), "resid grad");
        NC_TRY(nc_sum_into(part_b, N, G + ctx->e_x0l + l, st), "x0 grad");
      }
      dxT_parts = false;
    } else {
      NC_TRY(nc_rmsnorm_bwd(dt, da, da16, aa + la.a1, A<float>(ctx, la.r1), dx, dxT, N, d, 1, st,
                            bparts), "norm1 bwd");
      dxT_parts = bparts != nullptr;
    }
  }
  // the gradient at the embedding output: dx (+ dx0b, the x0 paths)
  float* dEm = G + ctx->n_block;
  const float* rows = dx;
  if (ctx->smear_on) {        // through the smear mix to the looked-up rows (into da)
    NC_TRY(nc_smear_bwd(tok, E, dx, dx0b, A<float>(ctx, ctx->sig_s), Pm + ctx->e_sl,
                        Pm + ctx->e_ws, A<float>(ctx, ctx->gs_s), A<float>(ctx, ctx->dz_s), da,
                        N, T, d, V, st), "smear bwd");
    NC_TRY(nc_sum_into(A<float>(ctx, ctx->gs_s), N, G + ctx->e_sl, st), "smear lambda grad");
    NC_TRY(nc_outer_accumulate(0, A<float>(ctx, ctx->dz_s), 1, E, d, tok, V, 24, N,
                               A<float>(ctx, ctx->outer_part), G + ctx->e_ws, st), "smear gate grad");
    rows = da;
  }
  if (!ctx->ve_on) NC_TRY(nc_embed_sort(tok, N, V, emb_scratch, st), "token sort");
  NC_TRY(nc_embed_segsum(tok, rows, dEm, N, V, d, emb_scratch, st), "embed bwd");
  if (dx0b && !ctx->smear_on)
    NC_TRY(nc_embed_segsum(tok, dx0b, dEm, N, V, d, emb_scratch, st), "embed bwd (x0)");
  return NC_OK;
}

// Newton-Schulz on `count` matrices X [R, C] (R <= C) of group g, starting from
// the prepared buffers x32[0]/xh[0].  Every iterate is kept in fp32; only the
// matrix-core inputs are rounded.  *result = byte offset of the final fp32 X.
static nc_status newton_schulz(nc_ctx* ctx, int g, int count, int R, int C, size_t* result,
                               int dtype = -1) {
  const nc_optim_config& o = ctx->ocfg;
  char* aa = ctx->aa;
  const auto& b = ctx->ns[g];
  int cur = 0;
  const int64_t sx = (int64_t)R * C, sa = (int64_t)R * R;
  for (int it = 0; it < o.ns_steps; ++it) {
    const float ca = o.ns_coeffs[it][0], cb = o.ns_coeffs[it][1], cc = o.ns_coeffs[it][2];
    // A = X X^T
    NC_GEMM(gemm(ctx, aa + b.xh[cur], C, kKCont, aa + b.xh[cur], C, kKCont, aa + b.a32, R, R, R,
                 C, kEpiDual, nullptr, aa + b.ah, 1, count, sx, sx, sa, 0.f, 1.f, dtype),
            "ns gram");
    // B = b A + c A A   (A symmetric: A A = A A^T)
    NC_GEMM(gemm(ctx, aa + b.ah, R, kKCont, aa + b.ah, R, kKCont, aa + b.b32, R, R, R, R,
                 kEpiDual, aa + b.a32, aa + b.bh, 1, count, sa, sa, sa, cb, cc, dtype),
            "ns poly");
    // X' = a X + B X
    NC_GEMM(gemm(ctx, aa + b.bh, R, kKCont, aa + b.xh[cur], C, kMNCont, aa + b.x32[cur ^ 1], C,
                 R, C, R, kEpiDual, aa + b.x32[cur], aa + b.xh[cur ^ 1], 1, count, sa, sx, sx,
                 ca, 1.f, dtype), "ns update");
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
  ctx->w8_ok = false;        // the weights change: their fp8 codes are made again
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
  // value-embedding tables and scalars: AdamW state continues after E | Wh
  if (ctx->n_vet)
    NC_TRY(nc_adamw(Pm + ctx->e_ve, G + ctx->e_ve, P<float>(ctx, ctx->oAm) + 2 * Vd,
                    P<float>(ctx, ctx->oAv) + 2 * Vd, ctx->n_vet, ctx->n_vet,
                    o.adam_lr_embed * lr_mult, o.adam_lr_embed * lr_mult, o.adam_beta1,
                    o.adam_beta2, o.adam_eps, o.adam_wd, bc1, bc2, nullptr, 0, st), "adamw ve");
  if (ctx->n_sc)
    NC_TRY(nc_adamw(Pm + ctx->e_rl, G + ctx->e_rl, P<float>(ctx, ctx->oAm) + 2 * Vd + ctx->n_vet,
                    P<float>(ctx, ctx->oAv) + 2 * Vd + ctx->n_vet, ctx->n_sc, ctx->n_sc,
                    o.adam_lr_scalar * lr_mult, o.adam_lr_scalar * lr_mult, o.adam_beta1,
                    o.adam_beta2, o.adam_eps, o.adam_wd, bc1, bc2, nullptr, 0, st),
           "adamw scalars");
  if (ctx->n_block == 0) return NC_OK;
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
  Grp grps[6];
  int ng = 0;
  if (dk == d) {
    grps[ng++] = {0, MatBatch{4, dd, ctx->S}, d, d, 4 * L, 0, 0, 0};            // Wq Wk Wv Wo
  } else {
    grps[ng++] = {0, MatBatch{2, (int64_t)oWo, ctx->S}, d, d, 2 * L, 0, 0, 0};  // Wq Wo
    grps[ng++] = {(size_t)dd, MatBatch{2, kd, ctx->S}, dk, d, 2 * L, 0, 2, 0};  // Wk Wv
  }
  if (L) {
    grps[ng++] = {o1, one, F, d, L, 1, 1, 0};                                   // W1
    grps[ng++] = {o2, one, d, F, L, 0, 1, (size_t)L * dF};                      // W2
  } else {
    ng = 0;
  }
  const int ng_block = ng;
  // gates (fp32 Newton-Schulz groups 3 and 4), oriented on their short side
  const int n_ve = (int)ctx->ve_layers.size(), Hkv = ctx->Hkv, Cg = ctx->Cg;
  if (n_ve)
    grps[ng++] = {ctx->e_wg, MatBatch{1, 0, (int64_t)Hkv * Cg}, Hkv, Cg, n_ve, Hkv > Cg ? 1 : 0,
                  3, 0};
  if (ctx->smear_on) grps[ng++] = {ctx->e_ws, one, 1, 24, 1, 0, 4, 0};
  int nidx = 0;
  for (int i = 0; i < ng; ++i) {
    const Grp& g = grps[i];
    const int64_t el = (int64_t)g.R * g.C;
    const auto& b = ctx->ns[g.ns];
    NC_TRY(nc_frob_norms(U + g.woff, g.mb, el, g.count, frob + (size_t)nidx * 256, norms + nidx,
                         st), "norms");
    const int gdt = g.ns >= 3 ? 0 : dt;           // gate groups iterate in fp32
    NC_TRY(nc_ns_prepare(gdt, U + g.woff, g.mb, g.R, g.C, g.count, norms + nidx, o.ns_eps, g.tr,
                         A<float>(ctx, b.x32[0]) + g.xoff,
                         aa + b.xh[0] + g.xoff * (gdt ? ctx->es : 4), el, st), "ns prepare");
    nidx += g.count;
  }
  // Newton-Schulz per buffer group: 0 square, 1 W1^T | W2 [d, F], 2 Wk | Wv [dk, d],
  // 3 value-embedding gates, 4 smear gate
  size_t xres[5] = {0, 0, 0, 0, 0};
  nc_status s = NC_OK;
  if (L) {
    s = newton_schulz(ctx, 0, grps[0].count, d, d, &xres[0]);
    if (s != NC_OK) return s;
    s = newton_schulz(ctx, 1, 2 * L, d, F, &xres[1]);
    if (s != NC_OK) return s;
    if (dk != d) {
      s = newton_schulz(ctx, 2, 2 * L, dk, d, &xres[2]);
      if (s != NC_OK) return s;
    }
  }
  if (n_ve) {
    s = newton_schulz(ctx, 3, n_ve, std::min(Hkv, Cg), std::max(Hkv, Cg), &xres[3], 0);
    if (s != NC_OK) return s;
  }
  if (ctx->smear_on) {
    s = newton_schulz(ctx, 4, 1, 1, 24, &xres[4], 0);
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
                       sh && i < ng_block ? sh + g.woff * 2 : nullptr, st), "ns apply");
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
  ctx->w8_ok = false;
  NC_TRY(hipMemcpyAsync(dst, src, n * 4,
                        src_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, ctx->st),
         "set param");
  if (ctx->dt && ((int64_t)p.elem < ctx->n_block || p.name == "Wh")) {
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

nc_status nc_check_inputs(nc_ctx* ctx, int32_t* host_flags) {
  if (!ctx || !host_flags) return NC_ERR_INVALID_ARG;
  if (!ctx->bound) return fail(ctx, NC_ERR_STATE, "bind first");
  int32_t* flag = A<int32_t>(ctx, ctx->flags);
  int32_t h = 0;
  NC_TRY(hipMemcpyAsync(&h, flag, 4, hipMemcpyDeviceToHost, ctx->st), "flag copy");
  NC_TRY(nc_fill_f32(reinterpret_cast<float*>(flag), 0.f, 1, ctx->st), "flag clear");
  NC_TRY(hipStreamSynchronize(ctx->st), "inputs sync");
  *host_flags = h & 3;
  if (!h) return NC_OK;
  return fail(ctx, NC_ERR_INVALID_ARG,
              std::string("out-of-range ") + ((h & 1) ? "token" : "") + ((h & 3) == 3 ? " and " : "") +
                  ((h & 2) ? "target" : "") + " id(s) since the last check");
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
// True if `batch` row-major [rows, cols] slices with leading dimension ld and
// batch stride bs, of es-byte elements, fit in `have` bytes from their base,
// and ld is at least cols.  Empty operands always fit.
static bool span_ok(size_t have, int64_t rows, int64_t cols, int64_t ld, int64_t bs, int64_t batch,
                    size_t es) {
  if (rows <= 0 || cols <= 0 || batch <= 0) return true;
  if (ld < cols || bs < 0) return false;
  const unsigned __int128 elems = (unsigned __int128)(batch - 1) * (uint64_t)bs +
                                  (unsigned __int128)(rows - 1) * (uint64_t)ld + (uint64_t)cols;
  return elems * es <= (unsigned __int128)have;
}

nc_status nc_op_gemm(int32_t dtype, const void* A_, size_t A_bytes, int64_t lda, int32_t al,
                     const void* B_, size_t B_bytes, int64_t ldb, int32_t bl, void* C_,
                     size_t C_bytes, int64_t ldc, int32_t M, int32_t N, int32_t K, int32_t batch,
                     int64_t sA, int64_t sB, int64_t sC, int32_t epi, const void* aux_in,
                     size_t aux_in_bytes, void* aux_out, size_t aux_out_bytes, float alpha,
                     float p0, float p1, int32_t splits, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!A_ || !B_ || !C_ || M < 0 || N < 0 || K < 1 || batch < 1) return NC_ERR_INVALID_ARG;
  if ((dtype != NC_FP32 && dtype != NC_BF16) || al < 0 || al > 1 || bl < 0 || bl > 1 ||
      epi < 0 || epi > kEpiDual)
    return NC_ERR_INVALID_ARG;
  if ((epi == kEpiDual && !aux_out) ||
      ((epi == kEpiRelu2Bwd || epi == kEpiPoly) && !aux_in))
    return NC_ERR_INVALID_ARG;
  if (splits < 1) splits = 1;
  // operand extents
  const size_t es = dtype == NC_BF16 ? 2 : 4;
  const bool c_f32 = splits > 1 || epi == kEpiStoreF32 || epi == kEpiAccF32 || epi == kEpiDual;
  const bool a_ok = al == kKCont ? span_ok(A_bytes, M, K, lda, sA, batch, es)
                                 : span_ok(A_bytes, K, M, lda, sA, batch, es);
  const bool b_ok = bl == kKCont ? span_ok(B_bytes, N, K, ldb, sB, batch, es)
                                 : span_ok(B_bytes, K, N, ldb, sB, batch, es);
  const bool c_ok = span_ok(C_bytes, M, N, ldc, sC, batch, c_f32 ? 4 : es);
  const bool aux_reads = epi == kEpiRelu2Bwd || epi == kEpiPoly || (epi == kEpiDual && aux_in);
  const bool ai_ok = !aux_reads || span_ok(aux_in_bytes, M, N, ldc, sC, batch,
                                           epi == kEpiDual ? 4 : es);
  const bool ao_ok = epi != kEpiDual || span_ok(aux_out_bytes, M, N, ldc, sC, batch, es);
  if (!a_ok || !b_ok || !c_ok || !ai_ok || !ao_ok) return NC_ERR_INVALID_ARG;
  if (dtype == NC_BF16) {
    if (K % 8 || (al == kMNCont && M % 8) || (bl == kMNCont && N % 8)) return NC_ERR_UNSUPPORTED;
    if (lda % 8 || ldb % 8) return NC_ERR_UNSUPPORTED;
  }
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

// ------------------------------------------- GEMM without a caller workspace
// The split-K partial slabs of nc_op_gemm_noalloc live in this file-scope
// device array (one copy per GPU, held until the process ends).  Host code
// never passes the array's name to a kernel: it looks up each device's
// address once with hipGetSymbolAddress and passes that.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

// Address of `scratch` on `dev`, looked up on the first call for that device
// (with that device current, then the caller's device restored).
static hipError_t scratch_on_device(int dev, float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* ptr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    ptr[dev] = static_cast<float*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

nc_status nc_op_gemm_noalloc(int32_t dtype, const void* A_, size_t A_bytes, int64_t lda,
                             int32_t al, const void* B_, size_t B_bytes, int64_t ldb, int32_t bl,
                             void* C_, size_t C_bytes, int64_t ldc, int32_t M, int32_t N, int32_t K,
                             int32_t batch, int64_t sA, int64_t sB, int64_t sC, int32_t epi,
                             const void* aux_in, size_t aux_in_bytes, void* aux_out,
                             size_t aux_out_bytes, float alpha, float p0, float p1,
                             int32_t splits, void* stream) {
  if (splits < 1) splits = 1;
  float* ws = nullptr;
  size_t ws_bytes = 0;
  if (splits > 1) {
    if (M < 0 || N < 0 || batch < 1) return NC_ERR_INVALID_ARG;
    const unsigned __int128 need = (unsigned __int128)splits * (uint64_t)batch * (uint64_t)M *
                                   (uint64_t)N * sizeof(float);
    if (need > kNoAllocScratchBytes) return NC_ERR_INVALID_ARG;   // splits*batch*M*N*4 > 16 MiB
    int dev = 0;
    const hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                                : hipGetDevice(&dev);
    if (e != hipSuccess || scratch_on_device(dev, &ws) != hipSuccess) return NC_ERR_HIP;
    ws_bytes = kNoAllocScratchBytes;
  }
  return nc_op_gemm(dtype, A_, A_bytes, lda, al, B_, B_bytes, ldb, bl, C_, C_bytes, ldc, M, N, K,
                    batch, sA, sB, sC, epi, aux_in, aux_in_bytes, aux_out, aux_out_bytes, alpha,
                    p0, p1, splits, ws, ws_bytes, stream);
}

nc_status nc_op_gemm_fp8(int32_t a_format, const void* A_, size_t A_bytes, int64_t lda,
                         const void* B_, size_t B_bytes, int64_t ldb, void* C_, size_t C_bytes,
                         int64_t ldc, int32_t M, int32_t N, int32_t K, int32_t epi,
                         const void* aux_in, size_t aux_in_bytes, float alpha, int32_t splits,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!A_ || !B_ || !C_ || M < 0 || N < 0 || K < 1 || splits < 1) return NC_ERR_INVALID_ARG;
  if (a_format != NC_FP8_E4M3 && a_format != NC_FP8_E5M2) return NC_ERR_INVALID_ARG;
  if (epi != kEpiStore && epi != kEpiStoreF32 && epi != kEpiAccF32 && epi != kEpiRelu2 &&
      epi != kEpiRelu2Bwd)
    return NC_ERR_INVALID_ARG;
  if (lda < K || ldb < K || ldc < N) return NC_ERR_INVALID_ARG;
  const bool f32_out = epi == kEpiStoreF32 || epi == kEpiAccF32;
  if (splits > 1 && !f32_out) return NC_ERR_INVALID_ARG;
  const size_t ce = f32_out ? 4 : 2;
  if (!span_ok(A_bytes, M, K, lda, 0, 1, 1) || !span_ok(B_bytes, N, K, ldb, 0, 1, 1) ||
      !span_ok(C_bytes, M, N, ldc, 0, 1, ce))
    return NC_ERR_INVALID_ARG;
  if (epi == kEpiRelu2Bwd && (!aux_in || !span_ok(aux_in_bytes, M, N, ldc, 0, 1, 2)))
    return NC_ERR_INVALID_ARG;
  if (splits > 1 && (!workspace || workspace_bytes < nc_gemm_workspace_bytes(M, N, splits)))
    return NC_ERR_INVALID_ARG;
  if (K % 128 || lda % 16 || ldb % 16) return NC_ERR_UNSUPPORTED;
  GemmParams g{};
  g.A = A_; g.B = B_; g.C = C_; g.aux_in = aux_in;
  g.lda = lda; g.ldb = ldb; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K; g.batch = 1; g.splits = splits;
  g.a_layout = kKCont; g.b_layout = kKCont; g.epi = epi;
  g.alpha = alpha;
  g.fmt_a = a_format;
  g.workspace = static_cast<float*>(workspace);
  g.workspace_bytes = workspace_bytes;
  const hipError_t e = nc_launch_gemm_f8(g, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return NC_ERR_UNSUPPORTED;
  return e == hipSuccess ? NC_OK : NC_ERR_HIP;
}

nc_status nc_op_fp8_quantize(int32_t dtype, int32_t format, const void* x, size_t x_bytes,
                             int64_t rows, int64_t cols, float* amax_scale,
                             size_t amax_scale_bytes, void* q, size_t q_bytes, void* qt,
                             size_t qt_bytes, float* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!x || !amax_scale || (!q && !qt) || !workspace || rows < 1 || cols < 1)
    return NC_ERR_INVALID_ARG;
  if (dtype != NC_FP32 && dtype != NC_BF16) return NC_ERR_INVALID_ARG;
  if (format != NC_FP8_E4M3 && format != NC_FP8_E5M2) return NC_ERR_INVALID_ARG;
  if (rows > INT64_MAX / cols) return NC_ERR_INVALID_ARG;
  const uint64_t n = (uint64_t)rows * (uint64_t)cols;
  const size_t es = dtype == NC_BF16 ? 2 : 4;
  if (n > x_bytes / es || (q && n > q_bytes) || (qt && n > qt_bytes) ||
      amax_scale_bytes < 2 * sizeof(float) || workspace_bytes < 1024 * sizeof(float))
    return NC_ERR_INVALID_ARG;
  auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  if (qt && !(dtype == NC_BF16 && rows % 64 == 0 && cols % 64 == 0 && al(x, 16) && al(qt, 16) &&
              al(q, 8)))
    return NC_ERR_UNSUPPORTED;
  const hipError_t e = nc_fp8_quantize(dtype == NC_BF16, format, x, rows, cols, workspace,
                                       amax_scale, static_cast<uint8_t*>(q),
                                       static_cast<uint8_t*>(qt), static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return NC_ERR_UNSUPPORTED;
  return e == hipSuccess ? NC_OK : NC_ERR_HIP;
}

// Extents of the attention operands: q, o, dq have H heads, k, v, dk, dv
// n_kv_head heads, of 128 columns each, on B*T token rows; lse and D are
// [B, H, T] fp32.
static bool attn_rows_ok(size_t have, int64_t rows, int64_t heads, int64_t ld, size_t es) {
  return span_ok(have, rows, heads * 128, ld, 0, 1, es);
}

nc_status nc_op_attention_fwd(int32_t dtype, const void* q, size_t q_bytes, const void* k,
                              size_t k_bytes, const void* v, size_t v_bytes, int64_t ld_qkv,
                              void* o, size_t o_bytes, int64_t ld_o, float* lse, size_t lse_bytes,
                              int32_t B, int32_t T, int32_t H, int32_t n_kv_head, int32_t window,
                              void* stream) {
  if (!q || !k || !v || !o || !lse || B < 1 || T < 1 || H < 1 || window < -1 ||
      n_kv_head < 1 || H % n_kv_head || (dtype != NC_FP32 && dtype != NC_BF16))
    return NC_ERR_INVALID_ARG;
  const size_t es = dtype == NC_BF16 ? 2 : 4;
  const int64_t rows = (int64_t)B * T;
  if (!attn_rows_ok(q_bytes, rows, H, ld_qkv, es) || !attn_rows_ok(k_bytes, rows, n_kv_head, ld_qkv, es) ||
      !attn_rows_ok(v_bytes, rows, n_kv_head, ld_qkv, es) || !attn_rows_ok(o_bytes, rows, H, ld_o, es) ||
      !span_ok(lse_bytes, (int64_t)B * H, T, T, 0, 1, 4))
    return NC_ERR_INVALID_ARG;
  if (dtype == NC_BF16 && (T % 128 || ld_qkv % 8 || ld_o % 8)) return NC_ERR_UNSUPPORTED;
  return nc_attn_fwd(dtype == NC_BF16, q, k, v, ld_qkv, o, ld_o, lse, B, T, H, n_kv_head, window,
                     static_cast<hipStream_t>(stream)) == hipSuccess ? NC_OK : NC_ERR_HIP;
}

nc_status nc_op_attention_bwd(int32_t dtype, const void* q, size_t q_bytes, const void* k,
                              size_t k_bytes, const void* v, size_t v_bytes, int64_t ld_qkv,
                              const void* o, size_t o_bytes, const void* dO, size_t dO_bytes,
                              int64_t ld_o, const float* lse, size_t lse_bytes, float* D,
                              size_t D_bytes, void* dq, size_t dq_bytes, void* dk,
                              size_t dk_bytes, void* dv, size_t dv_bytes, int64_t ld_d, int32_t B,
                              int32_t T, int32_t H, int32_t n_kv_head, int32_t window,
                              void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !D || !dq || !dk || !dv || B < 1 || T < 1 || H < 1 ||
      window < -1 || n_kv_head < 1 || H % n_kv_head || (dtype != NC_FP32 && dtype != NC_BF16))
    return NC_ERR_INVALID_ARG;
  const size_t es = dtype == NC_BF16 ? 2 : 4;
  const int64_t rows = (int64_t)B * T, hk = n_kv_head;
  if (!attn_rows_ok(q_bytes, rows, H, ld_qkv, es) || !attn_rows_ok(k_bytes, rows, hk, ld_qkv, es) ||
      !attn_rows_ok(v_bytes, rows, hk, ld_qkv, es) || !attn_rows_ok(o_bytes, rows, H, ld_o, es) ||
      !attn_rows_ok(dO_bytes, rows, H, ld_o, es) || !attn_rows_ok(dq_bytes, rows, H, ld_d, es) ||
      !attn_rows_ok(dk_bytes, rows, hk, ld_d, es) || !attn_rows_ok(dv_bytes, rows, hk, ld_d, es) ||
      !span_ok(lse_bytes, (int64_t)B * H, T, T, 0, 1, 4) ||
      !span_ok(D_bytes, (int64_t)(dtype == NC_BF16 ? 2 : 1) * B * H, T, T, 0, 1, 4))
    return NC_ERR_INVALID_ARG;
  if (dtype == NC_BF16 && (T % 128 || ld_qkv % 8 || ld_o % 8 || ld_d % 8)) return NC_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = dtype == NC_BF16;
  return nc_attn_bwd(dt, q, k, v, ld_qkv, o, dO, ld_o, lse, D, dq, dk, dv, ld_d, B, T, H,
                     n_kv_head, window, nullptr, nullptr, st) == hipSuccess
             ? NC_OK
             : NC_ERR_HIP;
}

}  // extern "C"
