"""AdamW and Muon updates, in numpy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Parameter groups follow [DEVTO] "2. ตัวปรับปรุง Muon" (table of optimizer per
parameter type): embeddings (the token embedding E and the value-embedding
tables ve.<l>) and the lm_head Wh take AdamW, and so do the scalar
parameters (resid_lambdas, x0_lambdas, smear_lambda, backout_lambda, at
adam_lr_scalar); every 2-D matrix -- Wq, Wk, Wv, Wo, W1, W2 of every layer
and the gates <l>.Wg and smear_gate, each one on its own -- takes Muon.

Readings where the pages are silent:

* AdamW is the textbook decoupled form (Loshchilov & Hutter) with bias
  correction; betas, eps, weight decay and learning rates are inputs
  (defaults used by the tests: (0.9, 0.95), 1e-8, 0).
* Muon momentum is the heavy-ball buffer M <- mu M + G (Nesterov optional),
  pre-normalised by its Frobenius norm before Newton-Schulz (the iteration
  needs a spectral norm <= 1; the pages do not show this step), update
  W <- W (1 - lr wd) - lr * X.
* NorMuon ([APIDOG] "2. Pengoptimal Muon (nanochat/optim.py)", the variance
  reduction paragraph and its fragment): the fragment computes per-neuron
  mean squares of the orthogonalised update, the norm they add up to, and a
  final rescale by that norm over a "new" norm, but the lines between them
  are missing.  Reading: a per-neuron second moment v2 (one value per output
  row of W [out, in], zero at the start, no bias correction) follows
  v2 <- beta2 v2 + (1 - beta2) mean_in(X^2); the update is X / sqrt(max(v2,
  1e-10)) row by row, rescaled so that sqrt(sum over rows of mean_in(.^2))
  equals the same quantity of X, times the Muon learning rate (the fragment's
  step size); the new norm is clamped at 1e-10 as printed.
* The Newton-Schulz coefficient table is data passed in; the pages print a
  partial Polar Express table.  Each iteration follows the loop printed in
  [APIDOG] "2. Pengoptimal Muon (nanochat/optim.py)": with X oriented tall,
  A = X^T X, B = b A + c A A, X = a X + X B.
"""

import numpy as np

F64 = np.float64


def adamw_step(p, g, m, v, t, lr, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.0):
    """One decoupled AdamW step at step number t (1-based).
    Returns new (p, m, v)."""
    p, g, m, v = (np.asarray(a, F64) for a in (p, g, m, v))
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    p = p * (1.0 - lr * wd) - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


def newton_schulz(M, coeffs, eps=1e-7):
    """Approximate orthogonalisation of M by the quintic Newton-Schulz loop.

    X0 = M / (||M||_F + eps); if X0 is wide it is transposed so that A = X^T X
    is the small Gram matrix, then for each (a, b, c) in ``coeffs``:
    A = X^T X; B = b A + c A A; X = a X + X B.  The result has M's shape.
    """
    X = np.asarray(M, F64)
    X = X / (np.linalg.norm(X) + eps)
    wide = X.shape[0] < X.shape[1]
    if wide:
        X = X.T
    for a, b, c in coeffs:
        A = X.T @ X
        Bm = b * A + c * (A @ A)
        X = a * X + X @ Bm
    return X.T if wide else X


def muon_step(W, G, M, lr, coeffs, momentum=0.95, eps=1e-7, wd=0.0,
              nesterov=False, shape_scale=False):
    """One Muon step for one matrix.  Returns new (W, M).

    shape_scale multiplies the update by sqrt(max(1, rows/cols)) (off by
    default; the pages give no scale factor)."""
    W, G, M = (np.asarray(a, F64) for a in (W, G, M))
    M = momentum * M + G
    U = G + momentum * M if nesterov else M
    X = newton_schulz(U, coeffs, eps)
    s = np.sqrt(max(1.0, W.shape[0] / W.shape[1])) if shape_scale else 1.0
    W = W * (1.0 - lr * wd) - lr * s * X
    return W, M


def normuon_update(X, v2, beta2, lr):
    """NorMuon's per-neuron normalisation of an orthogonalised update X
    [out, in] (the reading in the module docstring).  Returns (update, new v2);
    the update is subtracted from W."""
    X = np.asarray(X, F64)
    vm = np.mean(X * X, axis=1)                       # per output neuron
    v2 = beta2 * np.asarray(v2, F64) + (1.0 - beta2) * vm
    Y = X / np.sqrt(np.maximum(v2, 1e-10))[:, None]
    v_norm = np.sqrt(np.sum(vm))
    v_norm_new = np.sqrt(np.sum(np.mean(Y * Y, axis=1)))
    return Y * (lr * v_norm / max(v_norm_new, 1e-10)), v2


def muon_normuon_step(W, G, M, v2, lr, coeffs, beta2, momentum=0.95, eps=1e-7, wd=0.0,
                      nesterov=False):
    """One Muon step followed by NorMuon's normalisation.  Returns new
    (W, M, v2)."""
    W, G, M = (np.asarray(a, F64) for a in (W, G, M))
    M = momentum * M + G
    U = G + momentum * M if nesterov else M
    X = newton_schulz(U, coeffs, eps)
    upd, v2 = normuon_update(X, v2, beta2, lr)
    return W * (1.0 - lr * wd) - upd, M, v2


ADAMW_SCALARS = ("resid_lambdas", "x0_lambdas", "smear_lambda", "backout_lambda")


def train_step(params, grads, state, step, hp):
    """Apply one optimizer step to every parameter.

    params, grads: name -> array; state: name -> dict of buffers ("m", "v"
    for AdamW; "mom" for Muon), created on first use; step: 1-based step
    number; hp: dict with adam_lr_embed, adam_lr_head, adam_beta1,
    adam_beta2, adam_eps, adam_wd, muon_lr, muon_momentum, muon_wd, ns_eps,
    muon_nesterov, ns_coeffs, and optionally normuon (bool) and
    normuon_beta2 (Muon state then also holds "v2").  Returns (new params,
    new state).
    """
    new_p, new_s = {}, {}
    for name, W in params.items():
        G = grads[name]
        if name in ADAMW_SCALARS or name in ("E", "Wh") or name.startswith("ve."):
            st = state.get(name) or {"m": np.zeros_like(W, F64), "v": np.zeros_like(W, F64)}
            if name in ADAMW_SCALARS:
                lr = hp["adam_lr_scalar"]
            else:
                lr = hp["adam_lr_head"] if name == "Wh" else hp["adam_lr_embed"]
            p, m, v = adamw_step(W, G, st["m"], st["v"], step, lr, hp["adam_beta1"],
                                 hp["adam_beta2"], hp["adam_eps"], hp["adam_wd"])
            new_p[name], new_s[name] = p, {"m": m, "v": v}
        elif hp.get("normuon"):
            st = state.get(name) or {"mom": np.zeros_like(W, F64),
                                     "v2": np.zeros(W.shape[0], F64)}
            p, mom, v2 = muon_normuon_step(W, G, st["mom"], st["v2"], hp["muon_lr"],
                                           hp["ns_coeffs"], hp["normuon_beta2"],
                                           hp["muon_momentum"], hp["ns_eps"], hp["muon_wd"],
                                           bool(hp.get("muon_nesterov", False)))
            new_p[name], new_s[name] = p, {"mom": mom, "v2": v2}
        else:
            st = state.get(name) or {"mom": np.zeros_like(W, F64)}
            p, mom = muon_step(W, G, st["mom"], hp["muon_lr"], hp["ns_coeffs"],
                               hp["muon_momentum"], hp["ns_eps"], hp["muon_wd"],
                               bool(hp.get("muon_nesterov", False)))
            new_p[name], new_s[name] = p, {"mom": mom}
    return new_p, new_s
