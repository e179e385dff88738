"""Pins of the oracle's value embeddings, residual/x0 lambdas, smear and
backout (CPU only): central finite differences with every mechanism on,
identity values that must give the plain model exactly, and closed forms
(an all-equal token row, a zeroed layer, a single position, the receptive
field of smear)."""

import math

import numpy as np
import pytest

import oracle
from oracle.model import param_shapes, identity_values, ve_layers
from oracle.optim import train_step
from gpt_pretraining_step_gemms_amd import synthetic

FEATURES = ("value_embeds", "resid_lambdas", "smear", "backout")


def cfg_with(L=3, d=32, H=1, V=16, T=8, kv=0, **feats):
    c = dict(n_layer=L, d_model=d, n_head=H, head_dim=d // H, d_ff=4 * d, vocab=V, seq_len=T,
             rope_base=10000.0, norm_eps=1e-6, n_kv_head=kv or H)
    c.update(feats)
    return c


def make(cfg, B, seed=0, std=0.3):
    params = synthetic.normal_params(seed, param_shapes(cfg), std)
    params = {k: v.astype(np.float64) for k, v in params.items()}
    rng = np.random.default_rng(seed + 100)
    # scalars away from their identity values, so that every term is exercised
    if "resid_lambdas" in params:
        params["resid_lambdas"] = 1.0 + 0.3 * rng.standard_normal(params["resid_lambdas"].shape)
        params["x0_lambdas"] = 0.5 * rng.standard_normal(params["x0_lambdas"].shape)
    if "smear_lambda" in params:
        params["smear_lambda"][:] = 0.8
    if "backout_lambda" in params:
        params["backout_lambda"][:] = 0.4
    tok, tgt = synthetic.token_rows(seed + 1, B, cfg["seq_len"], cfg["vocab"], "uniform")
    return params, tok, tgt


def fd_check(cfg, B=2, seed=0, max_coords=30, std=0.3):
    params, tok, tgt = make(cfg, B, seed, std)
    _, g = oracle.loss_and_grads(params, tok, tgt, cfg)
    assert set(g) == set(params)
    h = 1e-5
    rng = np.random.default_rng(seed)
    for name, W in params.items():
        idx = list(np.ndindex(W.shape))
        if name == "E" or name.startswith("ve."):
            used = set(tok.reshape(-1).tolist())
            idx = [ij for ij in idx if ij[0] in used] + [ij for ij in idx if ij[0] not in used][:2]
        if len(idx) > max_coords:
            idx = [idx[i] for i in rng.choice(len(idx), max_coords, replace=False)]
        fd = np.zeros(len(idx))
        for j, ij in enumerate(idx):
            old = W[ij]
            W[ij] = old + h
            lp, _ = oracle.forward(params, tok, tgt, cfg, keep_cache=False)
            W[ij] = old - h
            lm, _ = oracle.forward(params, tok, tgt, cfg, keep_cache=False)
            W[ij] = old
            fd[j] = (lp - lm) / (2 * h)
        an = np.array([g[name][ij] for ij in idx])
        scale = max(np.max(np.abs(g[name])), 1e-30)
        assert np.max(np.abs(fd - an)) / scale <= 1e-6, (name, np.max(np.abs(fd - an)) / scale)


def test_fd_all_mechanisms_three_layers():
    fd_check(cfg_with(L=3, **{f: True for f in FEATURES}), seed=1)


def test_fd_all_mechanisms_grouped_heads_two_layers():
    # 2 query heads over 1 key/value head: the value-embedding gate is per kv head
    fd_check(cfg_with(L=2, d=64, H=2, kv=1, **{f: True for f in FEATURES}), seed=2)


@pytest.mark.parametrize("feat", FEATURES)
def test_fd_each_mechanism_alone(feat):
    fd_check(cfg_with(L=2, **{feat: True}), seed=3)


def test_fd_backout_at_the_final_stream():
    # one layer: L // 2 = 0, the stream entering layer 0 is x0
    fd_check(cfg_with(L=1, backout=True, resid_lambdas=True), seed=4)


def test_identity_values_give_the_plain_model_exactly():
    """resid 1, x0 0, smear 0, backout 0 and zero value-embedding tables: the
    loss and every shared gradient equal the plain model's; the gates then
    get exactly zero gradient."""
    base = cfg_with(L=3)
    full = cfg_with(L=3, **{f: True for f in FEATURES})
    params, tok, tgt = make(full, B=2, seed=5)
    params.update(identity_values(full))
    for l in ve_layers(full):
        params[f"ve.{l}"][:] = 0.0
    plain = {k: params[k] for k in param_shapes(base)}
    l0, g0 = oracle.loss_and_grads(plain, tok, tgt, base)
    l1, g1 = oracle.loss_and_grads(params, tok, tgt, full)
    assert abs(l0 - l1) <= 1e-12 * abs(l0)
    for k in g0:
        assert np.max(np.abs(g0[k] - g1[k])) <= 1e-12 * max(np.max(np.abs(g0[k])), 1e-300), k
    for l in ve_layers(full):
        assert not np.any(g1[f"{l}.Wg"])            # ve = 0: the gate has no effect
    assert not np.any(g1["smear_gate"])             # smear lambda 0


def test_x0_only_residual_reduces_to_the_last_layer_alone():
    """resid 0 and x0 1 at every layer: each layer reads x0, so only the last
    layer's output reaches the head -- the 1-layer model with its weights."""
    cfg = cfg_with(L=3, resid_lambdas=True)
    params, tok, tgt = make(cfg, B=2, seed=6)
    params["resid_lambdas"][:] = 0.0
    params["x0_lambdas"][:] = 1.0
    one = cfg_with(L=1)
    p1 = {"E": params["E"], "Wh": params["Wh"]}
    for n in ("Wq", "Wk", "Wv", "Wo", "W1", "W2"):
        p1[f"0.{n}"] = params[f"2.{n}"]
    l3, _ = oracle.forward(params, tok, tgt, cfg)
    l1, _ = oracle.forward(p1, tok, tgt, one)
    assert abs(l3 - l1) <= 1e-12 * abs(l1)


def test_backout_of_a_silent_last_layer_gives_zero_logits():
    """Two layers, backout 1, layer 1's output projections zero: the stream
    after layer 1 equals the one entering it, so x - xb = 0, every logit is
    0 and the loss is ln V."""
    cfg = cfg_with(L=2, V=16, backout=True)
    params, tok, tgt = make(cfg, B=2, seed=7)
    params["backout_lambda"][:] = 1.0
    params["1.Wo"][:] = 0.0
    params["1.W2"][:] = 0.0
    loss, _ = oracle.forward(params, tok, tgt, cfg)
    assert loss == pytest.approx(math.log(16), abs=1e-12)


def test_smear_has_no_effect_on_a_single_position():
    cfg = cfg_with(L=2, T=1, smear=True)
    base = cfg_with(L=2, T=1)
    params, tok, tgt = make(cfg, B=3, seed=8)
    l1, g1 = oracle.loss_and_grads(params, tok, tgt, cfg)
    l0, _ = oracle.loss_and_grads({k: params[k] for k in param_shapes(base)}, tok, tgt, base)
    assert abs(l1 - l0) <= 1e-12 * abs(l0)
    assert not np.any(g1["smear_gate"]) and not np.any(g1["smear_lambda"])


def test_smear_reaches_exactly_one_token_back_without_layers():
    """No layers: the logits of position t are a function of tokens t and t-1
    only (the bigram mix), not of t-2 or later tokens."""
    cfg = cfg_with(L=0, T=8, V=16, smear=True)
    params, tok, tgt = make(cfg, B=1, seed=9)
    z = oracle.logits_of(params, tok, cfg)
    t = 5
    for pos, changes in [(t - 1, True), (t - 2, False), (t + 1, False)]:
        tk = tok.copy()
        tk[0, pos] = (tk[0, pos] + 3) % 16
        z2 = oracle.logits_of(params, tk, cfg)
        assert (np.max(np.abs(z2[0, t] - z[0, t])) > 1e-6) == changes, pos


def test_value_embedding_of_an_all_equal_row_is_the_attention_output():
    """All tokens equal c, Wv = 0 and a zero gate matrix: every v is
    3 sigmoid(0) VE[c] = 1.5 VE[c], so every attention output row of the
    value-embedding layer is 1.5 VE[c] (the softmax weights sum to one)."""
    cfg = cfg_with(L=1, d=64, H=2, kv=2, value_embeds=True)
    params, _, _ = make(cfg, B=1, seed=10)
    c = 7
    tok = np.full((2, cfg["seq_len"]), c, np.int32)
    params["0.Wv"][:] = 0.0
    params["0.Wg"][:] = 0.0
    _, cache = oracle.forward(params, tok, tok, cfg)
    o = cache["layers"][0]["o"]                                  # [B, T, H * hd]
    np.testing.assert_allclose(o, np.broadcast_to(1.5 * params["ve.0"][c], o.shape),
                               rtol=0, atol=1e-13)


def test_causality_with_every_mechanism():
    cfg = cfg_with(L=3, T=8, **{f: True for f in FEATURES})
    params, tok, _ = make(cfg, B=1, seed=11)
    z = oracle.logits_of(params, tok, cfg)
    tk = tok.copy()
    tk[0, 5] = (tk[0, 5] + 1) % cfg["vocab"]
    z2 = oracle.logits_of(params, tk, cfg)
    assert np.array_equal(z[0, :5], z2[0, :5])


def test_optimizer_groups_of_the_new_parameters():
    """Scalars and value-embedding tables take AdamW (first step: -lr sign(G)
    up to eps), the gates take Muon (the update is -lr NS(G))."""
    cfg = cfg_with(L=2, **{f: True for f in FEATURES})
    params, tok, tgt = make(cfg, B=2, seed=12)
    _, g = oracle.loss_and_grads(params, tok, tgt, cfg)
    hp = dict(adam_lr_embed=3e-3, adam_lr_head=2e-3, adam_lr_scalar=5e-3, adam_beta1=0.9,
              adam_beta2=0.95, adam_eps=1e-8, adam_wd=0.0, muon_lr=0.02, muon_momentum=0.95,
              muon_wd=0.0, ns_eps=1e-7, ns_coeffs=[(15 / 8, -10 / 8, 3 / 8)] * 40)
    new, _ = train_step(params, g, {}, 1, hp)
    for n, lr in [("resid_lambdas", 5e-3), ("x0_lambdas", 5e-3), ("smear_lambda", 5e-3),
                  ("backout_lambda", 5e-3), ("ve.1", 3e-3)]:
        d = new[n] - params[n]
        big = np.abs(g[n]) > 1e-3                    # eps / |G| <= 1e-5
        np.testing.assert_allclose(d[big], -lr * np.sign(g[n][big]), rtol=1e-4)
    for n in ("1.Wg", "smear_gate"):
        d = (new[n] - params[n]) / -0.02
        s = np.linalg.svd(d, compute_uv=False)       # 40 textbook steps: the polar factor
        np.testing.assert_allclose(s, 1.0, atol=1e-8)
