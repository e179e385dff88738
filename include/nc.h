/*
 * nc.h -- C ABI of libncgpt.so: one pretraining step of a depth-parameterised,
 * decoder-only GPT on one AMD MI355X (gfx950).
 *
 * The step (forward + backward of token embedding, RMSNorm, QK-normalised
 * rotary causal self-attention, ReLU^2 MLP and an untied lm_head with
 * next-token cross-entropy, then Muon for the 2-D block matrices and AdamW
 * for the embedding and lm_head) is the model and optimizer described on:
 *   apidog.com, "Cara Melatih ChatGPT Sendiri dengan Budget 50 Dolar",
 *     "1. Model GPT (nanochat/gpt.py)" (architecture feature list),
 *     "2. Pengoptimal Muon (nanochat/optim.py)" (Newton-Schulz loop),
 *     "3. Manajemen Presisi (nanochat/common.py)" (fp32 master weights, the
 *       compute dtype per device, bias-free linear layers);
 *   dev.to, "วิธีฝึก ChatGPT ส่วนตัว งบ 50 ดอลลาร์", "2. ตัวปรับปรุง Muon"
 *     (parameter groups: embeddings and lm_head -> AdamW, matrices -> Muon);
 *   vi.news.hada.io, "NanoChat - ChatGPT tốt nhất bạn có thể mua với 100 USD"
 *     (a single GPU replaces data parallelism by gradient accumulation).
 *
 * Conventions (all entry points):
 *  - Every function returns an nc_status; none throws or aborts.  Argument,
 *    shape and call-order errors are returned synchronously before anything
 *    is enqueued (NC_ERR_INVALID_ARG, NC_ERR_UNSUPPORTED, NC_ERR_STATE).
 *    A failed kernel launch or HIP call returns NC_ERR_HIP; the HIP message
 *    is then available from nc_last_error().
 *  - Device memory is owned by the caller: one parameter arena and one
 *    activation arena (sizes from nc_plan), the token/target arrays and the
 *    loss scalar.  The library never allocates device memory.
 *  - Work is enqueued asynchronously on the HIP stream given to nc_bind;
 *    functions documented as synchronous wait on that stream.
 *  - Matrices are row-major fp32 [rows, cols] in the [out, in] orientation
 *    of a linear layer.  One context per stream and per host thread.
 */
#ifndef NC_H_
#define NC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NC_OK = 0,
  NC_ERR_INVALID_ARG = 1,   /* null pointer, bad size, value out of range */
  NC_ERR_UNSUPPORTED = 2,   /* shape or option the library does not implement */
  NC_ERR_OUT_OF_MEMORY = 3, /* an arena is smaller than nc_plan requires */
  NC_ERR_HIP = 4,           /* a HIP call or kernel launch failed */
  NC_ERR_STATE = 5,         /* call order: e.g. fwd_bwd before bind */
  NC_ERR_NONFINITE = 6      /* nc_check_finite found a NaN or Inf */
} nc_status;

enum { NC_FP32 = 0, NC_BF16 = 1 };

/* Model shape.  head_dim must be 128 and d_model = n_head * 128.  n_kv_head
 * key/value heads (0 = n_head; it must divide n_head): grouped-query
 * attention as listed on apidog.com, "1. Model GPT (nanochat/gpt.py)" (no
 * ratio is printed there) -- Wk and Wv are [n_kv_head * 128, d_model] and
 * query head h reads key/value head h / (n_head / n_kv_head).  dtype
 * NC_FP32 computes everything in fp32; NC_BF16 feeds bf16 (round to nearest
 * even) to the matrix cores with fp32 accumulation and keeps fp32 master
 * weights, residual stream, softmax statistics and gradients.  The norm is a
 * parameter-free RMSNorm with epsilon norm_eps; rotary angles are
 * t * rope_base^(-2i/128) for position t of a row, pairing dims i and i+64. */
typedef struct {
  int32_t n_layer, d_model, n_head, head_dim, d_ff, vocab, seq_len;
  int32_t max_micro_batch; /* rows per nc_fwd_bwd call the arenas are planned for */
  int32_t dtype;           /* NC_FP32 | NC_BF16 */
  float rope_base, norm_eps;
  int32_t n_kv_head;
  int32_t fp8_forward;     /* 1: the four forward block products of every layer (QKV,
                              output projection, MLP up and down) run in fp8 e4m3 with
                              one scale per tensor -- the activation and the weight
                              copy are quantised on the device before each product
                              (apidog.com, "3. Manajemen Presisi (nanochat/common.py)":
                              later runs train most linear layers in FP8 with tensorwise
                              scaling); the backward products stay bf16 and take the
                              unquantised operands.  NC_BF16 only. */
  int32_t features;        /* bits of NC_FEAT_*: the further mechanisms of apidog.com,
                              "1. Model GPT (nanochat/gpt.py)" (value-embedding listing and
                              the three efficiency tricks); 0 = the plain model */
  int32_t ve_gate_channels;/* channels of the value-embedding gate input (0 = 32;
                              a multiple of 8, at most 64 and at most d_model) */
  int32_t fp8_backward;    /* 1: also the eight backward products of those four (the
                              input gradient dY W and the weight gradient dY^T X of each)
                              in fp8, the gradient dY in e5m2 (scale 57344 / amax) and X,
                              W in e4m3 with the forward's scales; the transposed codes
                              of X are written by the forward quantiser and kept per
                              layer.  Needs fp8_forward and seq_len % 128 == 0. */
} nc_model_config;

/* Feature bits of nc_model_config.features.
 * NC_FEAT_VALUE_EMBEDS: every other layer counted down from the last
 *   (l = L-1, L-3, ...) has a table "ve.<l>" [vocab, n_kv_head*128] and a gate
 *   "<l>.Wg" [n_kv_head, C]; v += 3 sigmoid(a[:, :C] Wg^T) ve.<l>[token] per
 *   key/value head, a being the layer's first RMSNorm output.
 * NC_FEAT_RESID_LAMBDAS: "resid_lambdas", "x0_lambdas" [1, n_layer]; layer i
 *   starts from resid_lambdas[i] x + x0_lambdas[i] x0 (x0: the embedding output).
 * NC_FEAT_SMEAR: "smear_gate" [1, 24], "smear_lambda" [1, 1]; the embedding
 *   output is e_t + smear_lambda sigmoid(e_t[:24] . smear_gate) e_{t-1}.
 * NC_FEAT_BACKOUT: "backout_lambda" [1, 1]; after the last layer
 *   x <- x - backout_lambda xb, xb being the stream entering layer n_layer/2.
 * Tables and scalars take AdamW (tables at adam_lr_embed, scalars at
 * adam_lr_scalar), the gates take Muon.  nc_init_params sets resid_lambdas to
 * 1 and the other scalars to 0 (the plain model plus value embeddings).
 * Not combined with normuon (NC_ERR_UNSUPPORTED). */
enum { NC_FEAT_VALUE_EMBEDS = 1, NC_FEAT_RESID_LAMBDAS = 2, NC_FEAT_SMEAR = 4,
       NC_FEAT_BACKOUT = 8 };

/* Optimizer settings.  Muon (per block matrix): M <- mu M + G;
 * X0 = U / (||U||_F + ns_eps) with U = M (or G + mu M if muon_nesterov);
 * for i < ns_steps: A = X X^T, B = b_i A + c_i A A, X = a_i X + B X (on the
 * short side); W <- W (1 - lr wd) - lr X.  AdamW (E, Wh): decoupled, bias
 * corrected, with the given betas, eps, weight decay and per-group LR.  The
 * coefficient table is data: any (a_i, b_i, c_i) rows may be given.
 * normuon = 1 adds NorMuon's per-neuron normalisation after Newton-Schulz
 * (apidog.com, "2. Pengoptimal Muon (nanochat/optim.py)", variance
 * reduction; the page's fragment is incomplete and is read as follows): per
 * output row r of W [out, in], vm_r = mean over the row of X^2 and a second
 * moment v2_r <- normuon_beta2 v2_r + (1 - normuon_beta2) vm_r (zero after
 * nc_bind / nc_init_params); row r of X is divided by sqrt(max(v2_r, 1e-10))
 * and the whole update rescaled by sqrt(sum vm) / max(sqrt(sum of the new
 * rows' mean squares), 1e-10), so W <- W (1 - lr wd) - lr X'.  normuon_beta2
 * in [0, 1); both fields are ignored when normuon = 0. */
typedef struct {
  float muon_lr, muon_momentum, muon_wd, ns_eps;
  int32_t ns_steps, muon_nesterov;
  float ns_coeffs[8][3];
  float adam_lr_embed, adam_lr_head, adam_beta1, adam_beta2, adam_eps, adam_wd;
  int32_t normuon;
  float normuon_beta2;
  float adam_lr_scalar;    /* AdamW learning rate of the scalar parameters (features) */
} nc_optim_config;

typedef struct nc_ctx nc_ctx;

/* Parameter groups */
enum { NC_GROUP_ADAMW = 0, NC_GROUP_MUON = 1 };
/* Tensors of a parameter for nc_get_tensor */
enum { NC_PARAM = 0, NC_GRAD = 1, NC_MOMENTUM = 2, NC_ADAM_M = 3, NC_ADAM_V = 4 };

typedef struct {
  char name[32];           /* "E", "<layer>.Wq|Wk|Wv|Wo|W1|W2", "Wh" (a layer's six
                              matrices are contiguous in this order), then the
                              feature parameters (see NC_FEAT_*) */
  int32_t rows, cols, group;
  int64_t param_offset;    /* byte offsets into the parameter arena (fp32) */
  int64_t grad_offset;
  int64_t state0_offset;   /* Muon momentum or AdamW first moment */
  int64_t state1_offset;   /* AdamW second moment, -1 for Muon */
} nc_param_info;

/* Host only.  Bytes of the two device arenas for this configuration
 * (either output pointer may be NULL). */
nc_status nc_plan(const nc_model_config* cfg, const nc_optim_config* ocfg,
                  size_t* param_arena_bytes, size_t* act_arena_bytes);

/* Host only.  Validates the configuration and creates a context (*out);
 * release it with nc_destroy. */
nc_status nc_create(const nc_model_config* cfg, const nc_optim_config* ocfg, nc_ctx** out);

/* Gives the context its device arenas (256-byte aligned, at least the
 * planned sizes; NC_ERR_OUT_OF_MEMORY otherwise) and the hipStream_t to
 * enqueue on (NULL = default stream).  Uploads the rotary tables, sets
 * gradients and optimizer state to zero and the step count to 0 (weights are
 * left as they are: set them with nc_init_params or nc_set_param);
 * synchronous.  May be called again to rebind. */
nc_status nc_bind(nc_ctx* ctx, void* d_param_arena, size_t param_bytes, void* d_act_arena,
                  size_t act_bytes, void* hip_stream);

/* Every parameter i.i.d. N(0, std^2) from a Philox4x32-10 counter stream
 * keyed by seed (deterministic per seed); optimizer state and step count
 * reset to zero. */
nc_status nc_init_params(nc_ctx* ctx, uint64_t seed, float std);

/* Host only.  Sliding-window attention per layer: windows[l] = w >= 0 lets
 * query t of layer l see keys max(0, t - w) .. t (w earlier positions and its
 * own), -1 keeps the plain causal mask; values >= seq_len equal -1.  The
 * pages name a configurable pattern of short and long windows ("SSSL") and
 * pass a window size to the attention call (apidog.com, "1. Model GPT
 * (nanochat/gpt.py)" and "5. Penyatuan Flash Attention"); they print no
 * size, so the sizes are the caller's.  windows: host array of n_layer
 * entries, or NULL to make every layer plain causal again (the state after
 * nc_create).  NC_ERR_INVALID_ARG (nothing changed) if an entry is below -1.
 * Applies to later nc_fwd_bwd calls and to nc_flops. */
nc_status nc_set_attention_windows(nc_ctx* ctx, const int32_t* windows);

/* Sets every gradient to zero (start of a step). */
nc_status nc_zero_grads(nc_ctx* ctx);

/* One micro-batch: forward and backward on B rows of seq_len tokens.
 * d_tokens, d_targets: device int32 [B, seq_len], ids in [0, vocab) (the
 * targets are the inputs shifted by one position; no ignore index).  The ids
 * are read on the device only: an id outside [0, vocab) is never used as an
 * index -- its embedding row, or its loss and logit-gradient row, becomes NaN
 * (so the loss and the gradients of the step are non-finite) and a device
 * flag records it for nc_check_inputs.
 * Adds grad_scale * d(mean cross-entropy over the B*seq_len positions)/dtheta
 * to every gradient (grad_scale = 1/K for K accumulated micro-batches) and
 * writes that mean cross-entropy (natural log, before grad_scale) to the
 * device float *d_loss.  1 <= B <= max_micro_batch. */
nc_status nc_fwd_bwd(nc_ctx* ctx, const int32_t* d_tokens, const int32_t* d_targets, int32_t B,
                     float grad_scale, float* d_loss);

/* One optimizer step from the accumulated gradients (AdamW for E and Wh,
 * Muon for every block matrix, each on its own), learning rates multiplied
 * by lr_mult.  Increments the step count used for AdamW bias correction.
 * Gradients are left as they are. */
nc_status nc_optimizer_step(nc_ctx* ctx, float lr_mult);

/* Host only, no device access: walks the launch sequence of nc_fwd_bwd on B
 * rows and of nc_optimizer_step against placeholder arena addresses and
 * checks that every matrix-product operand lies inside its arena (the same
 * check guards every real launch).  NC_OK, or NC_ERR_HIP with the first
 * violation in nc_last_error().  The context's state is not changed. */
nc_status nc_validate_launches(nc_ctx* ctx, int32_t B);

/* Parameter registry: count, then descriptors i = 0 .. count-1. */
nc_status nc_param_count(const nc_ctx* ctx, int32_t* n);
nc_status nc_param_desc(const nc_ctx* ctx, int32_t i, nc_param_info* out);

/* Copies rows*cols fp32 values into parameter i (src on host or device) and
 * refreshes its bf16 copy; synchronous. */
nc_status nc_set_param(nc_ctx* ctx, int32_t i, const float* src, int32_t src_on_device);

/* Copies a tensor of parameter i (which = NC_PARAM .. NC_ADAM_V) to dst
 * (host or device, rows*cols fp32); synchronous.  NC_ERR_INVALID_ARG if the
 * parameter has no such state. */
nc_status nc_get_tensor(nc_ctx* ctx, int32_t i, int32_t which, float* dst, int32_t dst_on_device);

/* Checks every parameter and gradient for NaN/Inf; synchronous.
 * *host_flag = 1 and NC_ERR_NONFINITE if one is found, else 0 and NC_OK. */
nc_status nc_check_finite(nc_ctx* ctx, int32_t* host_flag);

/* Synchronous.  *host_flags = the kinds of out-of-range ids nc_fwd_bwd has
 * seen since nc_bind or the previous call (bit 0: a token id, bit 1: a target
 * id), then clears the record; NC_ERR_INVALID_ARG if any, else NC_OK. */
nc_status nc_check_inputs(nc_ctx* ctx, int32_t* host_flags);

/* Model FLOPs of one nc_fwd_bwd on B rows (matrix products only; a plain
 * causal layer's attention counted at seq_len/2 keys per query, a windowed
 * layer's at its exact mean number of visible keys) and of one Newton-Schulz
 * pass. */
nc_status nc_flops(const nc_ctx* ctx, int32_t B, double* fwd_bwd_flops, double* optimizer_flops);

const char* nc_status_str(nc_status s);
/* Last error message of this context ("" if none); valid until the next call. */
const char* nc_last_error(const nc_ctx* ctx);
void nc_destroy(nc_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* NC_H_ */
