"""Forward pass, loss and hand-written backward of the GPT, in numpy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything is done with
whole-array numpy operations in float64; matrix products use ``@``.  There is
no blocking, fusion or reordering beyond the definition.

Model (decoder-only, pre-norm), per [APIDOG] "1. Model GPT (nanochat/gpt.py)":

    x   = E[tok]                                   (untied token embedding)
    for each layer:
        a   = N(x)
        q,k,v = a Wq^T, a Wk^T, a Wv^T              (bias-free, [APIDOG] "3.")
        q,k = R_t(N(q_h)), R_t(N(k_h)) per head      (QK normalisation, RoPE)
        o   = softmax(q k^T / sqrt(hd), causal) v
        x   = x + o Wo^T
        m   = N(x);  h = m W1^T;  g = max(h, 0)^2   (ReLU^2 MLP)
        x   = x + g W2^T
    z   = N(x) Wh^T                                 (untied lm_head)
    loss = mean over all B*T positions of lse(z) - z[target]

Readings where the pages are silent:

* N is the parameter-free RMSNorm u * (mean(u^2) + eps)^-1/2, eps = 1e-6; no
  norm on the embedding output; no logit soft-cap.
* QK normalisation is the same parameter-free RMSNorm over each head vector,
  applied before the rotation (the two commute: the rotation keeps the norm).
* RoPE pairs dimension i with i + hd/2 (half split), angle t * base^(-2i/hd)
  for position t = 0..T-1 of each row, y_i = x_i cos - x_{i+h} sin,
  y_{i+h} = x_i sin + x_{i+h} cos.
* Attention scale 1/sqrt(hd); causal mask keeps keys u <= t (diagonal kept);
  no document masking; one key/value head per query head unless
  cfg["n_kv_head"] says otherwise (below).
* Sliding-window layers ([APIDOG] "1. Model GPT (nanochat/gpt.py)" lists a
  configurable short/long window pattern such as "SSSL", and section
  "5. Penyatuan Flash Attention" passes a window size to the attention call
  next to causal=True): a layer with window w keeps keys t - w <= u <= t, the
  w earlier positions plus the query's own (the left extent of a
  flash-attention window with nothing on the right).  cfg["windows"] holds
  one entry per layer, None for the plain causal mask; without the key every
  layer is plain causal.  The pages print no window size.
* Grouped-query attention ([APIDOG] "1. Model GPT (nanochat/gpt.py)" lists
  fewer key/value heads than query heads, without a ratio): cfg["n_kv_head"]
  key/value heads (default n_head), Wk and Wv [n_kv_head * hd, d]; query
  head h reads key/value head h // (n_head / n_kv_head), so consecutive query
  heads share one, and a key/value head's gradient sums over its query heads.
* FP8 forward products ([APIDOG] "3. Manajemen Presisi (nanochat/common.py)":
  most linear layers in FP8 with tensorwise scaling): with cfg["fp8_forward"]
  the four block products of every layer (QKV -- its fused weight Wq|Wk|Wv
  taken as one tensor -- output projection, MLP up and down) use the e4m3
  values of the bf16 copies of their two operands (the fp8 path exists in
  the bf16 configuration, whose activations and weight copies are bf16), one
  scale per tensor (oracle.fp8), and the
  backward treats the rounding as the identity (gradients with the
  unrounded operands).  The lm_head is exact.
* FP8 backward products (cfg["fp8_backward"], the same passage: the
  reading takes the linear layers meant there to cover their backward products
  too): the input gradient dX = dY W and the weight gradient dW = dY^T X of
  each of the four block products use the e5m2 values of the bf16 gradient
  dY (one scale per tensor; the fused QKV gradient [dq | dk | dv] is one
  tensor) and the e4m3 values of the bf16 copies of X and W, the operands
  the forward products quantise.  Everything else in the backward (norms,
  attention, the ReLU^2 derivative, the lm_head) stays exact.
* Loss: natural log, mean over every position, no ignore index.

The rest of the pages' model ([APIDOG] "1. Model GPT (nanochat/gpt.py)",
the "Value Embeddings (ResFormer)" and efficiency-trick listings), each
switched on by a cfg flag; readings where the listings leave a step open:

* value embeddings (cfg["value_embeds"]): every second layer carries a
  learnable table VE_l [V, n_kv_head * hd] looked up by the input token ids,
  added to v through a per-(token, key/value head) gate
  g = 3 sigmoid(a[:, :C] Wg_l^T), Wg_l [n_kv_head, C] bias-free, where a is
  the attention block's (normalised) input.  Readings: the layers are every
  other one counted down from the last (l = L-1, L-3, ...); C = 32
  (cfg["ve_gate_channels"]); the mix happens before attention, v has no
  QK-norm or rotation.
* residual scaling (cfg["resid_lambdas"]): at the start of layer i the
  stream becomes resid_lambdas[i] x + x0_lambdas[i] x0, x0 being the
  embedding output (after smear).  Parameters [1, L] each.
* smear (cfg["smear"]): after the embedding, x_t = e_t + lam_s
  sigmoid(e_t[:24] Ws^T) e_{t-1}, e_t = E[tok_t] and e_{-1} = 0 (the
  previous token of the same row; Ws [1, 24] bias-free, lam_s [1, 1]).
* backout (cfg["backout"]): after the last layer x <- x - lam_b xb, where
  xb is the stream entering layer L // 2 (before its residual scaling);
  lam_b [1, 1] (the final stream itself when L // 2 == L).
"""

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------
def rmsnorm(u, eps):
    """Parameter-free RMSNorm over the last axis.  Returns (y, r) with
    r = (mean(u^2) + eps)^-1/2 and y = u * r."""
    u = np.asarray(u, F64)
    r = 1.0 / np.sqrt(np.mean(u * u, axis=-1) + eps)
    return u * r[..., None], r


def rmsnorm_backward(dy, y, r):
    """Gradient of y = u * r(u) with respect to u, given y and r:
    du = r * (dy - y * mean(dy * y))   (differentiating r = (mean(u^2)+eps)^-1/2)."""
    return r[..., None] * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def rope_tables(T, hd, base):
    """cos/sin tables [T, hd/2]: angle[t, i] = t * base^(-2i/hd)."""
    half = hd // 2
    inv_freq = base ** (-(2.0 * np.arange(half, dtype=F64)) / hd)
    ang = np.arange(T, dtype=F64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x, cos, sin):
    """Rotate pairs (i, i+hd/2) of x [..., T, hd] by the position angle."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


def rope_inverse(y, cos, sin):
    """Transpose (= inverse) of the rotation: rotate by the negative angle."""
    half = y.shape[-1] // 2
    y1, y2 = y[..., :half], y[..., half:]
    return np.concatenate([y1 * cos + y2 * sin, -y1 * sin + y2 * cos], axis=-1)


def _causal_mask(T, window=None):
    """True where key u is hidden from query t: u > t, or u < t - window."""
    t = np.arange(T)[:, None]
    u = np.arange(T)[None, :]
    hidden = u > t
    if window is not None:
        hidden |= u < t - window
    return hidden


def causal_attention(q, k, v, window=None):
    """o = softmax(q k^T / sqrt(hd) with keys u > t, and u < t - window when a
    window is given, removed) v.

    q, k, v: [..., T, hd].  Returns (o, P) with P the attention probabilities.
    """
    hd = q.shape[-1]
    T = q.shape[-2]
    s = (q @ np.swapaxes(k, -1, -2)) / np.sqrt(hd)
    s = np.where(_causal_mask(T, window), -np.inf, s)
    s = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / np.sum(p, axis=-1, keepdims=True)
    return p @ v, p


def causal_attention_backward(q, k, v, do, window=None):
    """(dq, dk, dv) of o = causal_attention(q, k, v, window) for an upstream gradient do:
    with P the probabilities, dv = P^T do, dP = do v^T,
    dS = P * (dP - rowsum(dP * P)) (softmax Jacobian), dq = dS k / sqrt(hd),
    dk = dS^T q / sqrt(hd)."""
    hd = q.shape[-1]
    _, p = causal_attention(q, k, v, window)
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
    dq = (ds @ k) / np.sqrt(hd)
    dk = (np.swapaxes(ds, -1, -2) @ q) / np.sqrt(hd)
    return dq, dk, dv


def _sum_outer(a, b):
    """sum over every leading (batch, position) index of a_n^T b_n:
    a [..., m], b [..., n] -> [m, n]."""
    return a.reshape(-1, a.shape[-1]).T @ b.reshape(-1, b.shape[-1])


def _layer_names(i):
    return [f"{i}.Wq", f"{i}.Wk", f"{i}.Wv", f"{i}.Wo", f"{i}.W1", f"{i}.W2"]


def n_kv_heads(cfg):
    return cfg.get("n_kv_head") or cfg["n_head"]


SMEAR_CHANNELS = 24


def ve_layers(cfg):
    """Layers carrying a value embedding: every other one down from the last."""
    if not cfg.get("value_embeds"):
        return []
    L = cfg["n_layer"]
    return [l for l in range(L) if (L - 1 - l) % 2 == 0]


def ve_gate_channels(cfg):
    return cfg.get("ve_gate_channels", 32)


def backout_layer(cfg):
    return cfg["n_layer"] // 2


def param_shapes(cfg):
    """Name -> shape of every parameter ([out, in] like a bias-free Linear)."""
    d, F, V = cfg["d_model"], cfg["d_ff"], cfg["vocab"]
    dk = n_kv_heads(cfg) * cfg["head_dim"]
    L = cfg["n_layer"]
    shapes = {"E": (V, d)}
    for i in range(L):
        for n, s in zip(_layer_names(i), [(d, d), (dk, d), (dk, d), (d, d), (F, d), (d, F)]):
            shapes[n] = s
    shapes["Wh"] = (V, d)
    for l in ve_layers(cfg):
        shapes[f"ve.{l}"] = (V, dk)
        shapes[f"{l}.Wg"] = (n_kv_heads(cfg), ve_gate_channels(cfg))
    if cfg.get("resid_lambdas"):
        shapes["resid_lambdas"] = (1, L)
        shapes["x0_lambdas"] = (1, L)
    if cfg.get("smear"):
        shapes["smear_gate"] = (1, SMEAR_CHANNELS)
        shapes["smear_lambda"] = (1, 1)
    if cfg.get("backout"):
        shapes["backout_lambda"] = (1, 1)
    return shapes


def identity_values(cfg):
    """Values of the scalar parameters at which residual scaling, smear and
    backout leave the plain model unchanged (resid 1, x0 0, smear 0,
    backout 0)."""
    out = {}
    L = cfg["n_layer"]
    if cfg.get("resid_lambdas"):
        out["resid_lambdas"] = np.ones((1, L))
        out["x0_lambdas"] = np.zeros((1, L))
    if cfg.get("smear"):
        out["smear_lambda"] = np.zeros((1, 1))
    if cfg.get("backout"):
        out["backout_lambda"] = np.zeros((1, 1))
    return out


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
def _fp8_linear(x, W):
    """x W^T with both operands replaced by the tensorwise e4m3 values of
    their bf16 copies (the codes are decided on the same bf16 values the
    kernels quantise)."""
    from . import fp8
    qx, _, sx = fp8.quantize_tensorwise(fp8.bf16_round(x.reshape(-1, x.shape[-1])))
    qw, _, sw = fp8.quantize_tensorwise(fp8.bf16_round(W))
    y = (fp8.e4m3_decode(qx) / sx) @ (fp8.e4m3_decode(qw) / sw).T
    return y.reshape(*x.shape[:-1], W.shape[0])


def _fp8_backward_pair(dY, X, W):
    """(dX, dW) of y = x W^T with dY in e5m2 and X, W in e4m3 (tensorwise
    scales, codes decided on the bf16 values): dX = dY W, dW = dY^T X."""
    from . import fp8
    out, inp = W.shape
    d = fp8.dequantized(fp8.bf16_round(dY.reshape(-1, out)), fp8.E5M2)
    x = fp8.dequantized(fp8.bf16_round(X.reshape(-1, inp)), fp8.E4M3)
    w = fp8.dequantized(fp8.bf16_round(W), fp8.E4M3)
    return (d @ w).reshape(*dY.shape[:-1], inp), d.T @ x


def _grad_pair(dY, X, W, cfg):
    """Input and weight gradients of y = x W^T."""
    if cfg.get("fp8_backward"):
        return _fp8_backward_pair(dY, X, W)
    return dY @ W, _sum_outer(dY, X)


def _linear(x, W, cfg):
    return _fp8_linear(x, W) if cfg.get("fp8_forward") else x @ W.T


def _split_heads(u, H):
    B, T, d = u.shape
    return u.reshape(B, T, H, d // H).transpose(0, 2, 1, 3)      # [B,H,T,hd]


def _merge_heads(u):
    B, H, T, hd = u.shape
    return u.transpose(0, 2, 1, 3).reshape(B, T, H * hd)


def layer_windows(cfg):
    """Attention window of every layer (None = plain causal)."""
    w = cfg.get("windows")
    if w is None:
        return [None] * cfg["n_layer"]
    assert len(w) == cfg["n_layer"]
    return list(w)


def _repeat_kv(u, group):
    """[B, Hkv, T, hd] -> [B, Hkv * group, T, hd]: query head h gets key/value
    head h // group."""
    return np.repeat(u, group, axis=1)


def _sum_groups(u, group):
    """[B, Hkv * group, T, hd] -> [B, Hkv, T, hd]: sum over each key/value
    head's query heads (the transpose of _repeat_kv)."""
    B, H, T, hd = u.shape
    return u.reshape(B, H // group, group, T, hd).sum(axis=2)


def forward(params, tokens, targets, cfg, keep_cache=True):
    """Loss of one micro-batch.  tokens, targets: int [B, T].

    Returns (loss, cache); the cache holds what the backward pass needs.
    """
    eps = cfg["norm_eps"]
    H = cfg["n_head"]
    Hkv = n_kv_heads(cfg)
    group = H // Hkv
    hd = cfg["head_dim"]
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    cos, sin = rope_tables(T, hd, cfg["rope_base"])
    P = {k: np.asarray(v, F64) for k, v in params.items()}

    L = cfg["n_layer"]
    xe = P["E"][tokens]                                 # [B,T,d]
    x = xe
    smear = None
    if cfg.get("smear"):
        prev = np.zeros_like(xe)
        prev[:, 1:] = xe[:, :-1]
        ss = _sigmoid(xe[..., :SMEAR_CHANNELS] @ P["smear_gate"].T)      # [B,T,1]
        gs = P["smear_lambda"][0, 0] * ss
        x = xe + gs * prev
        smear = dict(prev=prev, ss=ss, gs=gs)
    x0 = x
    resid = cfg.get("resid_lambdas")
    Lb = backout_layer(cfg) if cfg.get("backout") else None
    xb = None
    vls = set(ve_layers(cfg))
    Cg = ve_gate_channels(cfg)
    windows = layer_windows(cfg)
    layers = []
    for i in range(L):
        Wq, Wk, Wv, Wo, W1, W2 = (P[n] for n in _layer_names(i))
        x_prev = x
        if i == Lb:
            xb = x
        if resid:
            x = P["resid_lambdas"][0, i] * x + P["x0_lambdas"][0, i] * x0
        a, r1 = rmsnorm(x, eps)
        if cfg.get("fp8_forward"):             # the fused QKV weight is one tensor
            qkv = _fp8_linear(a, np.concatenate([Wq, Wk, Wv], axis=0))
            dq_, dk_ = Wq.shape[0], Wk.shape[0]
            q_, k_, v_ = qkv[..., :dq_], qkv[..., dq_:dq_ + dk_], qkv[..., dq_ + dk_:]
        else:
            q_, k_, v_ = a @ Wq.T, a @ Wk.T, a @ Wv.T
        ve_cache = None
        if i in vls:                                     # value embedding, gated per head
            ve = _split_heads(P[f"ve.{i}"][tokens], Hkv)                   # [B,Hkv,T,hd]
            sg = _sigmoid(a[..., :Cg] @ P[f"{i}.Wg"].T)                     # [B,T,Hkv]
            gg = 3.0 * sg.transpose(0, 2, 1)[..., None]                     # [B,Hkv,T,1]
            v_ = v_ + _merge_heads(gg * ve)
            ve_cache = dict(ve=ve, sg=sg)
        q = _split_heads(q_, H)
        k = _split_heads(k_, Hkv)
        v = _split_heads(v_, Hkv)
        qn, rq = rmsnorm(q, eps)
        kn, rk = rmsnorm(k, eps)
        qr = rope(qn, cos, sin)
        kr = rope(kn, cos, sin)
        o_h, _ = causal_attention(qr, _repeat_kv(kr, group), _repeat_kv(v, group), windows[i])
        o = _merge_heads(o_h)
        x = x + _linear(o, Wo, cfg)
        m, r2 = rmsnorm(x, eps)
        h = _linear(m, W1, cfg)
        g = np.maximum(h, 0.0) ** 2
        x = x + _linear(g, W2, cfg)
        if keep_cache:
            layers.append(dict(a=a, r1=r1, qn=qn, rq=rq, kn=kn, rk=rk,
                               qr=qr, kr=kr, v=v, o=o, m=m, r2=r2, h=h, g=g,
                               x_prev=x_prev, ve=ve_cache))
    if Lb is not None:
        if xb is None:                                   # L // 2 == L: the final stream
            xb = x
        x = x - P["backout_lambda"][0, 0] * xb
    xf, rf = rmsnorm(x, eps)
    z = xf @ P["Wh"].T                                  # [B,T,V]
    zmax = np.max(z, axis=-1, keepdims=True)
    lse = (zmax + np.log(np.sum(np.exp(z - zmax), axis=-1, keepdims=True)))[..., 0]
    tz = np.take_along_axis(z, np.asarray(targets)[..., None], axis=-1)[..., 0]
    loss = float(np.mean(lse - tz))
    cache = None
    if keep_cache:
        cache = dict(P=P, tokens=tokens, targets=np.asarray(targets), cos=cos, sin=sin,
                     layers=layers, xf=xf, rf=rf, z=z, lse=lse, xe=xe, x0=x0, xb=xb,
                     smear=smear)
    return loss, cache


def logits_of(params, tokens, cfg):
    """Logits z [B,T,V] of the forward pass (targets play no role)."""
    tokens = np.asarray(tokens)
    _, cache = forward(params, tokens, np.zeros_like(tokens), cfg)
    return cache["z"]


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def loss_and_grads(params, tokens, targets, cfg, grad_scale=1.0):
    """Loss and grad_scale * d(loss)/d(param) for every parameter (fp64)."""
    eps = cfg["norm_eps"]
    hd = cfg["head_dim"]
    loss, c = forward(params, tokens, targets, cfg)
    P = c["P"]
    B, T = c["tokens"].shape
    n_tok = B * T
    cos, sin = c["cos"], c["sin"]
    windows = layer_windows(cfg)
    group = cfg["n_head"] // n_kv_heads(cfg)
    grads = {}

    # cross-entropy: dz = (softmax(z) - onehot(y)) / (B*T)
    dz = np.exp(c["z"] - c["lse"][..., None])
    np.put_along_axis(dz, c["targets"][..., None],
                      np.take_along_axis(dz, c["targets"][..., None], axis=-1) - 1.0, axis=-1)
    dz *= grad_scale / n_tok
    grads["Wh"] = _sum_outer(dz, c["xf"])
    dxf = dz @ P["Wh"]
    dx = rmsnorm_backward(dxf, c["xf"], c["rf"])
    nL = cfg["n_layer"]
    Lb = backout_layer(cfg) if cfg.get("backout") else None
    dxb = None
    if Lb is not None:                      # x_final = x - lam_b xb
        grads["backout_lambda"] = np.array([[-np.sum(dx * c["xb"])]])
        dxb = -P["backout_lambda"][0, 0] * dx
        if Lb >= nL:
            dx = dx + dxb
    resid = cfg.get("resid_lambdas")
    if resid:
        grads["resid_lambdas"] = np.zeros((1, nL))
        grads["x0_lambdas"] = np.zeros((1, nL))
    dx0 = np.zeros_like(dx)
    Cg = ve_gate_channels(cfg)

    for i in reversed(range(nL)):
        L = c["layers"][i]
        nWq, nWk, nWv, nWo, nW1, nW2 = _layer_names(i)
        # MLP: x += max(h,0)^2 W2^T, h = m W1^T, m = N(x)
        dg, grads[nW2] = _grad_pair(dx, L["g"], P[nW2], cfg)
        dh = 2.0 * np.maximum(L["h"], 0.0) * dg
        dm, grads[nW1] = _grad_pair(dh, L["m"], P[nW1], cfg)
        dx = dx + rmsnorm_backward(dm, L["m"], L["r2"])
        # attention: x += o Wo^T
        do, grads[nWo] = _grad_pair(dx, L["o"], P[nWo], cfg)
        do = _split_heads(do, cfg["n_head"])
        dqr, dkr, dv = causal_attention_backward(L["qr"], _repeat_kv(L["kr"], group),
                                                 _repeat_kv(L["v"], group), do, windows[i])
        dkr, dv = _sum_groups(dkr, group), _sum_groups(dv, group)
        da_gate = None
        if L["ve"] is not None:             # v += 3 sigmoid(a[:, :Cg] Wg^T) ve, per head
            ve, sg = L["ve"]["ve"], L["ve"]["sg"]
            gg = 3.0 * sg.transpose(0, 2, 1)[..., None]                     # [B,Hkv,T,1]
            dve = _merge_heads(gg * dv)                                     # [B,T,dk]
            dVE = np.zeros_like(P[f"ve.{i}"])
            np.add.at(dVE, c["tokens"].reshape(-1), dve.reshape(n_tok, -1))
            grads[f"ve.{i}"] = dVE
            dgg = np.sum(dv * ve, axis=-1).transpose(0, 2, 1)               # [B,T,Hkv]
            dzg = dgg * 3.0 * sg * (1.0 - sg)
            grads[f"{i}.Wg"] = _sum_outer(dzg, L["a"][..., :Cg])
            da_gate = dzg @ P[f"{i}.Wg"]                                    # [B,T,Cg]
        dq = rmsnorm_backward(rope_inverse(dqr, cos, sin), L["qn"], L["rq"])
        dk = rmsnorm_backward(rope_inverse(dkr, cos, sin), L["kn"], L["rk"])
        dq, dk, dv = _merge_heads(dq), _merge_heads(dk), _merge_heads(dv)
        if cfg.get("fp8_backward"):         # the fused QKV product: one tensor each side
            d_model, dkv = dq.shape[-1], dk.shape[-1]
            da, dWqkv = _fp8_backward_pair(np.concatenate([dq, dk, dv], axis=-1), L["a"],
                                           np.concatenate([P[nWq], P[nWk], P[nWv]], axis=0))
            grads[nWq] = dWqkv[:d_model]
            grads[nWk] = dWqkv[d_model:d_model + dkv]
            grads[nWv] = dWqkv[d_model + dkv:]
        else:
            grads[nWq] = _sum_outer(dq, L["a"])
            grads[nWk] = _sum_outer(dk, L["a"])
            grads[nWv] = _sum_outer(dv, L["a"])
            da = dq @ P[nWq] + dk @ P[nWk] + dv @ P[nWv]
        if da_gate is not None:
            da[..., :Cg] += da_gate
        dx = dx + rmsnorm_backward(da, L["a"], L["r1"])
        if resid:                           # x_in = resid_i x_prev + x0_i x0
            grads["resid_lambdas"][0, i] = np.sum(dx * L["x_prev"])
            grads["x0_lambdas"][0, i] = np.sum(dx * c["x0"])
            dx0 += P["x0_lambdas"][0, i] * dx
            dx = P["resid_lambdas"][0, i] * dx
        if i == Lb:                         # xb is the stream entering this layer
            dx = dx + dxb

    dx = dx + dx0                           # gradient at x0 (the smeared embedding)
    if cfg.get("smear"):                    # x0_t = e_t + lam_s sigmoid(e_t[:24] Ws^T) e_{t-1}
        sm = c["smear"]
        gamma = np.sum(dx * sm["prev"], axis=-1, keepdims=True)            # [B,T,1]
        grads["smear_lambda"] = np.array([[np.sum(gamma * sm["ss"])]])
        dzs = gamma * P["smear_lambda"][0, 0] * sm["ss"] * (1.0 - sm["ss"])
        grads["smear_gate"] = _sum_outer(dzs, c["xe"][..., :SMEAR_CHANNELS])
        dxe = dx.copy()
        dxe[:, :-1] += sm["gs"][:, 1:] * dx[:, 1:]
        dxe[..., :SMEAR_CHANNELS] += dzs * P["smear_gate"]
        dx = dxe
    dE = np.zeros_like(P["E"])
    np.add.at(dE, c["tokens"].reshape(-1), dx.reshape(n_tok, -1))
    grads["E"] = dE
    return loss, grads
