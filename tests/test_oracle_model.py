"""Pins of the oracle's model, loss and backward (CPU only).

Each check is tied to something other than the oracle itself: closed forms,
invariants of the definition, textbook reductions and central finite
differences.  None of these needs a GPU.
"""

import math

import numpy as np
import pytest

import oracle
from oracle.model import param_shapes
from gpt_pretraining_step_gemms_amd import synthetic



def micro_cfg(L=1, d=16, H=1, V=16, T=8, F=None):
    return dict(n_layer=L, d_model=d, n_head=H, head_dim=d // H, d_ff=F or 4 * d,
                vocab=V, seq_len=T, rope_base=10000.0, norm_eps=1e-6)


def make(cfg, B, seed=0, std=0.02, dist="uniform"):
    params = synthetic.normal_params(seed, param_shapes(cfg), std)
    tok, tgt = synthetic.token_rows(seed + 1, B, cfg["seq_len"], cfg["vocab"], dist)
    return {k: v.astype(np.float64) for k, v in params.items()}, tok, tgt


# ----------------------------------------------------------------- loss pins
def test_zero_head_loss_is_ln_vocab_and_upstream_grads_vanish():
    cfg = micro_cfg(L=2, d=32, H=2, V=64)
    params, tok, tgt = make(cfg, B=2, std=0.3)
    params["Wh"][:] = 0.0
    loss, g = oracle.loss_and_grads(params, tok, tgt, cfg)
    assert loss == pytest.approx(math.log(64), abs=1e-14)
    for name, val in g.items():
        if name != "Wh":
            assert np.all(val == 0.0), name
    # all logits are 0, softmax is uniform: dWh[v] = (1/N) sum_n (1/V - [y_n = v]) xf_n
    _, cache = oracle.forward(params, tok, tgt, cfg)
    xf = cache["xf"].reshape(-1, 32)
    y = tgt.reshape(-1)
    onehot = np.zeros((y.size, 64))
    onehot[np.arange(y.size), y] = 1.0
    expect = (1.0 / 64 - onehot).T @ xf / y.size
    np.testing.assert_allclose(g["Wh"], expect, rtol=0, atol=1e-15)


def test_zero_head_loss_golden_vocab():
    # the pages' vocabulary size (tests/golden/zero_head_loss.txt)
    fields = dict(line.split("=", 1) for line in open(
        __file__.replace("test_oracle_model.py", "golden/zero_head_loss.txt")).read().split("\n")
        if "=" in line and not line.startswith("#"))
    V = int(fields["vocab"])
    cfg = micro_cfg(L=1, d=16, H=1, V=V, T=4)
    params, tok, tgt = make(cfg, B=1, std=0.5, dist="zipf")
    params["Wh"][:] = 0.0
    loss, _ = oracle.forward(params, tok, tgt, cfg, keep_cache=False)
    assert loss == pytest.approx(float(fields["loss"]), abs=1e-6)
    assert loss == pytest.approx(math.log(V), abs=1e-13)


@pytest.mark.parametrize("d,V", [(128, 512), (256, 4096)])
def test_random_init_loss_near_ln_vocab_plus_half_logit_variance(d, V):
    # xf has unit RMS, Wh ~ N(0, 0.02^2): z ~ N(0, 0.02^2 d) -> E[lse] ~ ln V + var/2
    cfg = micro_cfg(L=2, d=d, H=d // 64, V=V, T=32)
    params, tok, tgt = make(cfg, B=2, std=0.02)
    loss, _ = oracle.forward(params, tok, tgt, cfg, keep_cache=False)
    expect = math.log(V) + 0.02 ** 2 * d / 2
    assert abs(loss - expect) / expect < 0.01


def test_softmax_rows_sum_to_one_and_head_gradient_columns_sum_to_zero():
    cfg = micro_cfg(L=2, d=32, H=2, V=64, T=8)
    params, tok, tgt = make(cfg, B=2, std=0.3)
    _, cache = oracle.forward(params, tok, tgt, cfg)
    L0 = cache["layers"][0]
    _, p = oracle.causal_attention(L0["qr"], L0["kr"], L0["v"])
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-13)
    _, g = oracle.loss_and_grads(params, tok, tgt, cfg)
    # sum_v dz[n, v] = 0 for every position, hence sum_v dWh[v, :] = 0
    assert np.max(np.abs(g["Wh"].sum(0))) <= 1e-12 * max(1.0, np.max(np.abs(g["Wh"])))


def test_causality_future_token_does_not_change_earlier_logits():
    cfg = micro_cfg(L=2, d=32, H=2, V=64, T=12)
    params, tok, _ = make(cfg, B=2, std=0.3)
    z0 = oracle.logits_of(params, tok, cfg)
    t_star = 7
    tok2 = tok.copy()
    tok2[1, t_star] = (tok2[1, t_star] + 5) % 64
    z1 = oracle.logits_of(params, tok2, cfg)
    assert np.array_equal(z0[:, :t_star], z1[:, :t_star])
    assert np.array_equal(z0[0], z1[0])
    assert not np.allclose(z0[1, t_star:], z1[1, t_star:])


# ----------------------------------------------------------- building blocks
def test_rope_identity_at_zero_norm_preserving_and_shift_invariant():
    T, hd = 16, 32
    cos, sin = oracle.rope_tables(T + 5, hd, 10000.0)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((T, hd))
    y = oracle.rope(x, cos[:T], sin[:T])
    np.testing.assert_allclose(y[0], x[0], atol=0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(oracle.rope_inverse(y, cos[:T], sin[:T]), x, atol=1e-13)
    # scores depend only on the position difference
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    for t, u, c in [(5, 2, 3), (9, 9, 4), (3, 0, 5)]:
        s1 = oracle.rope(q, cos[t], sin[t]) @ oracle.rope(k, cos[u], sin[u])
        s2 = oracle.rope(q, cos[t + c], sin[t + c]) @ oracle.rope(k, cos[u + c], sin[u + c])
        assert s1 == pytest.approx(s2, abs=1e-12)
    # the half-split pairing: dim i rotates with dim i + hd/2 by t * base^(-2i/hd)
    e = np.zeros(hd)
    e[3] = 1.0
    r = oracle.rope(e, cos[2], sin[2])
    ang = 2 * 10000.0 ** (-6.0 / hd)
    assert r[3] == pytest.approx(math.cos(ang), abs=1e-14)
    assert r[3 + hd // 2] == pytest.approx(math.sin(ang), abs=1e-14)


def test_rmsnorm_scale_invariant_and_unit_rms():
    rng = np.random.default_rng(1)
    u = rng.standard_normal((5, 64)) * 3.0
    y, _ = oracle.rmsnorm(u, 0.0)
    y2, _ = oracle.rmsnorm(7.5 * u, 0.0)
    np.testing.assert_allclose(y, y2, atol=1e-13)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), 1.0, atol=1e-13)


def test_attention_single_key_and_equal_keys():
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((3, 1, 8)) for _ in range(3))
    o, _ = oracle.causal_attention(q, k, v)
    np.testing.assert_allclose(o, v, atol=1e-15)
    T = 9
    q = rng.standard_normal((T, 8))
    k = np.tile(rng.standard_normal((1, 8)), (T, 1))
    v = rng.standard_normal((T, 8))
    o, _ = oracle.causal_attention(q, k, v)
    expect = np.cumsum(v, 0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(o, expect, atol=1e-13)


# ---------------------------------------------------- sliding-window pins
def test_window_zero_attends_to_self_only():
    # one visible key: softmax weight 1, so o = v and the scores get no gradient
    rng = np.random.default_rng(11)
    q, k, v, do = (rng.standard_normal((2, 12, 8)) for _ in range(4))
    o, p = oracle.causal_attention(q, k, v, window=0)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_array_equal(p, np.broadcast_to(np.eye(12), p.shape))
    dq, dk, dv = oracle.causal_attention_backward(q, k, v, do, window=0)
    np.testing.assert_array_equal(dq, 0.0)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_array_equal(dv, do)


def test_window_covering_the_row_is_plain_causal():
    rng = np.random.default_rng(12)
    T = 10
    q, k, v, do = (rng.standard_normal((T, 8)) for _ in range(4))
    for w in (T - 1, T, 5 * T):
        np.testing.assert_array_equal(oracle.causal_attention(q, k, v, w)[0],
                                      oracle.causal_attention(q, k, v)[0])
        for a, b in zip(oracle.causal_attention_backward(q, k, v, do, w),
                        oracle.causal_attention_backward(q, k, v, do)):
            np.testing.assert_array_equal(a, b)


def test_window_equal_keys_give_moving_average():
    # identical keys: uniform weights over the visible keys t-w..t
    rng = np.random.default_rng(13)
    T, w = 11, 3
    q = rng.standard_normal((T, 8))
    k = np.tile(rng.standard_normal((1, 8)), (T, 1))
    v = rng.standard_normal((T, 8))
    o, _ = oracle.causal_attention(q, k, v, window=w)
    expect = np.stack([v[max(0, t - w):t + 1].mean(0) for t in range(T)])
    np.testing.assert_allclose(o, expect, atol=1e-14)


@pytest.mark.parametrize("w", [1, 2, 5])
def test_window_matches_per_query_softmax_over_the_sliced_keys(w):
    # brute force: each query's softmax written out over its own key slice
    rng = np.random.default_rng(20 + w)
    T, hd = 9, 8
    q, k, v = (rng.standard_normal((T, hd)) for _ in range(3))
    o, _ = oracle.causal_attention(q, k, v, window=w)
    for t in range(T):
        lo = max(0, t - w)
        s = [float(q[t] @ k[u]) / math.sqrt(hd) for u in range(lo, t + 1)]
        e = [math.exp(x - max(s)) for x in s]
        ref = sum(ei * v[lo + j] for j, ei in enumerate(e)) / sum(e)
        np.testing.assert_allclose(o[t], ref, rtol=1e-13, atol=1e-14)


def test_window_receptive_field_of_stacked_layers():
    # with windows w1, w2 a token reaches the logits of positions j .. j + w1 + w2 only
    cfg = micro_cfg(L=2, d=16, H=1, V=16, T=12)
    cfg["windows"] = [2, 3]
    params, tok, _ = make(cfg, B=1, std=0.5)
    z0 = oracle.logits_of(params, tok, cfg)
    j = 3
    tok2 = tok.copy()
    tok2[0, j] = (tok[0, j] + 1) % cfg["vocab"]
    z1 = oracle.logits_of(params, tok2, cfg)
    changed = np.any(z0 != z1, axis=-1)[0]
    assert not changed[:j].any() and not changed[j + 6:].any()
    assert changed[j:j + 6].all()


# --------------------------------------------------------------- gradients
def _fd_check(cfg, B, std, names=None, max_coords=None, seed=0):
    params, tok, tgt = make(cfg, B, seed=seed, std=std)
    _, g = oracle.loss_and_grads(params, tok, tgt, cfg)
    h = 1e-5
    rng = np.random.default_rng(seed)
    for name in names or params:
        W = params[name]
        idx = list(np.ndindex(W.shape))
        if name == "E":
            used = set(tok.reshape(-1).tolist())
            idx = [ij for ij in idx if ij[0] in used] + [ij for ij in idx if ij[0] not in used][:3]
        if max_coords and len(idx) > max_coords:
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
        err = np.max(np.abs(fd - an)) / scale
        assert err <= 1e-6, (name, err)


def test_fd_gradients_one_layer_every_coordinate():
    _fd_check(micro_cfg(L=1, d=16, H=1, V=16, T=8), B=2, std=0.4)


def test_fd_gradients_two_layers_two_heads_sampled():
    _fd_check(micro_cfg(L=2, d=32, H=2, V=64, T=8), B=2, std=0.3, max_coords=40, seed=3)


def test_fd_gradients_sliding_window_layers():
    cfg = micro_cfg(L=2, d=32, H=2, V=32, T=10)
    cfg["windows"] = [3, None]
    _fd_check(cfg, B=2, std=0.3, max_coords=40, seed=7)


def test_fd_gradients_grouped_query_attention():
    cfg = micro_cfg(L=2, d=32, H=4, V=32, T=8)      # head dim 8, 4 query heads
    cfg["n_kv_head"] = 2
    _fd_check(cfg, B=2, std=0.3, max_coords=40, seed=8)


def test_grouped_query_attention_equals_heads_with_copied_key_value_weights():
    # GQA with Wk, Wv = the MHA model whose key/value weight rows are repeated
    # per group: same loss; the GQA gradient of Wk (Wv) is the MHA gradient
    # summed over the copies
    H, Hkv, hd = 4, 2, 8
    g = H // Hkv
    cfg = micro_cfg(L=1, d=H * hd, H=H, V=24, T=7)
    gcfg = dict(cfg, n_kv_head=Hkv)
    pg, tok, tgt = make(gcfg, B=2, seed=4, std=0.3)
    pm = dict(pg)
    for n in ("0.Wk", "0.Wv"):
        W = pg[n].reshape(Hkv, hd, -1)
        pm[n] = np.repeat(W, g, axis=0).reshape(H * hd, -1)
    lg, gg = oracle.loss_and_grads(pg, tok, tgt, gcfg)
    lm, gm = oracle.loss_and_grads(pm, tok, tgt, cfg)
    assert lg == pytest.approx(lm, rel=1e-13)
    for n in ("0.Wk", "0.Wv"):
        summed = gm[n].reshape(Hkv, g, hd, -1).sum(axis=1).reshape(Hkv * hd, -1)
        np.testing.assert_allclose(gg[n], summed, rtol=1e-11, atol=1e-14)
    for n in ("0.Wq", "0.Wo", "0.W1", "0.W2", "E", "Wh"):
        np.testing.assert_allclose(gg[n], gm[n], rtol=1e-11, atol=1e-14)


def test_fd_gradients_tiny_shape_sampled():
    # the tiny configuration's shapes (d 128, one head of 128, vocab 512) at T = 16
    cfg = micro_cfg(L=2, d=128, H=1, V=512, T=16, F=512)
    _fd_check(cfg, B=2, std=0.05, max_coords=12, seed=5)


def test_accumulation_of_half_batches_equals_full_batch():
    cfg = micro_cfg(L=2, d=32, H=2, V=64, T=8)
    params, tok, tgt = make(cfg, B=4, std=0.3)
    l_full, g_full = oracle.loss_and_grads(params, tok, tgt, cfg)
    l_a, g_a = oracle.loss_and_grads(params, tok[:2], tgt[:2], cfg, grad_scale=0.5)
    l_b, g_b = oracle.loss_and_grads(params, tok[2:], tgt[2:], cfg, grad_scale=0.5)
    assert 0.5 * (l_a + l_b) == pytest.approx(l_full, abs=1e-13)
    for n in g_full:
        np.testing.assert_allclose(g_a[n] + g_b[n], g_full[n], rtol=0,
                                   atol=1e-12 * max(1e-30, np.max(np.abs(g_full[n]))))


@pytest.mark.filterwarnings("ignore:The number of unique classes")
def test_zero_layer_model_is_softmax_regression_on_normalised_embeddings():
    """With no blocks the model is multinomial logistic regression of the
    next token on the normalised embedding row: its loss is the library's
    log-loss of softmax(N(E[tok]) Wh^T), and the lm_head gradient is the
    regression's (softmax - onehot)^T features / n (checked against finite
    differences of that library loss)."""
    from sklearn.metrics import log_loss
    V, d = 50, 32
    cfg = dict(n_layer=0, d_model=d, n_head=1, head_dim=d, d_ff=64, vocab=V, seq_len=8,
               rope_base=10000.0, norm_eps=1e-6)
    params = {k: v.astype(np.float64) for k, v in
              synthetic.normal_params(4, param_shapes(cfg), 0.5).items()}
    tok, tgt = synthetic.token_rows(5, 3, 8, V, "uniform")
    loss, grads = oracle.loss_and_grads(params, tok, tgt, cfg)
    x = params["E"][tok.reshape(-1)]
    feats = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6)

    def lib_loss(Wh):
        z = feats @ Wh.T
        prob = np.exp(z - z.max(1, keepdims=True))
        prob /= prob.sum(1, keepdims=True)
        return log_loss(tgt.reshape(-1), prob, labels=np.arange(V))

    assert loss == pytest.approx(lib_loss(params["Wh"]), rel=1e-12)
    rng = np.random.default_rng(6)
    h = 1e-6
    for _ in range(20):
        i, j = rng.integers(V), rng.integers(d)
        Wp, Wm = params["Wh"].copy(), params["Wh"].copy()
        Wp[i, j] += h
        Wm[i, j] -= h
        fd = (lib_loss(Wp) - lib_loss(Wm)) / (2 * h)
        assert grads["Wh"][i, j] == pytest.approx(fd, rel=1e-5, abs=1e-9)
