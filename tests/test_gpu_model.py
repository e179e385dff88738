"""Model-level parity on the GPU: nc_fwd_bwd (loss and every gradient) and
nc_optimizer_step (every parameter update) against the fp64 oracle on the
same seeded inputs, plus invariants that hold at any size."""

import math

import numpy as np
import pytest
import torch
from dataclasses import replace

import oracle
from gpt_pretraining_step_gemms_amd import nc, synthetic
from gpt_pretraining_step_gemms_amd.configs import (TINY, D12, D20, CONFIGS, ModelConfig,
                                                    OptimConfig, with_batch, sliding_windows,
                                                    NS_QUINTIC_JORDAN)
from parity import cosine, max_rel

pytestmark = pytest.mark.gpu

# bf16 model with ragged GEMM tiles (d = 384, vocab = 4160), 2 query blocks per row
SMALL_BF16 = ModelConfig(name="small", n_layer=2, d_model=384, n_head=3, head_dim=128,
                         d_ff=1536, vocab=4160, seq_len=256, micro_batch=2, accum_steps=1,
                         dtype="bf16", token_dist="zipf")

TOL = {  # loss rel, grad/update cosine, grad/update max-rel
    "fp32": (1e-4, 1 - 1e-8, 1e-4),
    "bf16": (1e-2, 0.999, 5e-2),
    # fp8 forward products: the GPU's operands drift from the oracle's by a few
    # bf16 roundings, so about 4 % of the e4m3 codes fall on the other side of a
    # rounding boundary and move by one step (6-12 % of the value); that gives
    # output errors of about 2 % per product, compounding over the layers to a
    # few per cent in the gradients: cosine >= 0.99 (a relative difference of at
    # most 14 %) and max-rel <= 0.15.  The fp8 kernels themselves are checked to
    # the byte (quantiser) and to 2e-4 (GEMM) in the kernel tests.
    "fp8": (1e-2, 0.99, 0.15),
}


def setup(cfg, B, seed=0, ocfg=OptimConfig()):
    m = nc.Model(cfg, ocfg, max_micro_batch=B)
    params = synthetic.normal_params(seed, m.shapes(), cfg.init_std)
    m.set_params(params)
    tok, tgt = synthetic.token_rows(seed + 1, B, cfg.seq_len, cfg.vocab, cfg.token_dist)
    return m, params, tok, tgt


def gpu_tokens(a):
    return torch.from_numpy(a).to("cuda")


def run_gpu(m, tok, tgt, grad_scale=1.0):
    m.zero_grads()
    loss = m.fwd_bwd(gpu_tokens(tok), gpu_tokens(tgt), grad_scale)
    torch.cuda.synchronize()
    return float(loss.item()), {n: m.get(n, nc.NC_GRAD) for n in m.names()}


def check_step(cfg, B, seed=0, windows=None, ocfg=None):
    tol_l, tol_c, tol_r = TOL["fp8" if cfg.fp8_forward else cfg.dtype]
    ocfg = ocfg or OptimConfig()
    m, params, tok, tgt = setup(cfg, B, seed, ocfg)
    print(f"[parity] {cfg.name} B={B} seed={seed} windows={windows}", flush=True)
    ocfg_model = cfg.as_oracle_cfg()
    if windows is not None:
        m.set_attention_windows(windows)
        ocfg_model["windows"] = [None if w < 0 else w for w in windows]
    loss, grads = run_gpu(m, tok, tgt)
    loss_o, grads_o = oracle.loss_and_grads(params, tok, tgt, ocfg_model)
    assert abs(loss - loss_o) / abs(loss_o) <= tol_l, (loss, loss_o)
    worst = []
    for n in grads_o:
        c, r = cosine(grads[n], grads_o[n]), max_rel(grads[n], grads_o[n])
        worst.append((c, r, n))
        assert c >= tol_c and r <= tol_r, (n, c, r)
    # optimizer: the oracle's update applied to the GPU's gradients
    m.optimizer_step()
    torch.cuda.synchronize()
    new_o, _ = oracle.train_step(params, {n: g.astype(np.float64) for n, g in grads.items()}, {},
                                 1, ocfg.as_dict())
    upd = []
    for n in params:
        dW = m.get(n).astype(np.float64) - params[n]
        dW_o = new_o[n] - params[n]
        c, r = cosine(dW, dW_o), max_rel(dW, dW_o)
        upd.append((c, r, n))
        assert c >= tol_c and r <= tol_r, ("update", n, c, r)
    print(f"[parity] loss gpu {loss:.6f} oracle {loss_o:.6f}; worst grad cos "
          f"{min(worst)[0]:.6f} max-rel {max(w[1] for w in worst):.3e}; worst update cos "
          f"{min(upd)[0]:.6f} max-rel {max(u[1] for u in upd):.3e}", flush=True)
    m.close()


def test_tiny_fp32_full_step():
    check_step(TINY, B=4)


def test_small_bf16_full_step():
    check_step(SMALL_BF16, B=2, seed=3)


def test_tiny_fp32_sliding_windows():
    check_step(TINY, B=4, seed=4, windows=[8, -1])


def test_small_bf16_sliding_windows():
    check_step(SMALL_BF16, B=2, seed=5, windows=[127, 40])


def test_d12_shape_sssl_pattern_one_row():
    """The d12 shape with the short/short/short/long window pattern (short
    window of 1024 keys) on one 2048-token row."""
    cfg = with_batch(D12, micro_batch=1)
    check_step(cfg, B=1, seed=9, windows=sliding_windows(cfg.n_layer, cfg.seq_len, "SSSL"))


@pytest.mark.parametrize("name", ["tiny", "small", "d12", "d20"])
def test_constant_quintic_schedule_full_step(name):
    """The full step with the constant-quintic Newton-Schulz table (the
    default table is the Polar Express schedule)."""
    cfg = {"tiny": TINY, "small": SMALL_BF16, "d12": with_batch(D12, micro_batch=1),
           "d20": with_batch(D20, micro_batch=1)}[name]
    B = {"tiny": 4, "small": 2}.get(name, 1)
    check_step(cfg, B, seed=21, ocfg=OptimConfig(ns_coeffs=tuple(NS_QUINTIC_JORDAN)))


@pytest.mark.parametrize("name", ["tiny", "small", "d12"])
def test_normuon_two_steps(name):
    """Two full steps with NorMuon's per-neuron normalisation: the second one
    exercises the second-moment state the first one left."""
    cfg = {"tiny": TINY, "small": SMALL_BF16, "d12": with_batch(D12, micro_batch=1)}[name]
    B = {"tiny": 4, "small": 2}.get(name, 1)
    tol_l, tol_c, tol_r = TOL[cfg.dtype]
    ocfg = OptimConfig(normuon=True)
    m, params, tok, tgt = setup(cfg, B, 31, ocfg)
    hp = ocfg.as_dict()
    cur = {n: p.astype(np.float64) for n, p in params.items()}
    state = {}
    for step in (1, 2):
        print(f"[normuon] {cfg.name} step {step}", flush=True)
        _, grads = run_gpu(m, tok, tgt)
        m.optimizer_step()
        torch.cuda.synchronize()
        new_o, state = oracle.train_step(cur, {n: g.astype(np.float64) for n, g in grads.items()},
                                         state, step, hp)
        after = {n: m.get(n).astype(np.float64) for n in params}
        worst = []
        for n in params:
            dW, dW_o = after[n] - cur[n], new_o[n] - cur[n]
            c, r = cosine(dW, dW_o), max_rel(dW, dW_o)
            worst.append((c, r, n))
            assert c >= tol_c and r <= tol_r, ("update", step, n, c, r)
        print(f"[normuon] step {step}: worst update cos {min(worst)[0]:.6f} "
              f"max-rel {max(w[1] for w in worst):.3e}", flush=True)
        cur = after
    m.close()


TINY_GQA = ModelConfig(name="tiny_gqa", n_layer=2, d_model=256, n_head=2, head_dim=128,
                       d_ff=512, vocab=512, seq_len=64, micro_batch=2, accum_steps=1,
                       dtype="fp32", token_dist="uniform", n_kv_head=1)


@pytest.mark.parametrize("name", ["tiny_gqa", "small_gqa", "d12_gqa"])
def test_grouped_query_attention_full_step(name):
    """Loss, every gradient and every update with fewer key/value heads than
    query heads (fp32: 2 heads over 1; small bf16: 3 over 1; d12: 6 over 2)."""
    cfg = {"tiny_gqa": TINY_GQA, "small_gqa": replace(SMALL_BF16, n_kv_head=1),
           "d12_gqa": replace(with_batch(D12, micro_batch=1), n_kv_head=2)}[name]
    check_step(cfg, B=cfg.micro_batch, seed=41, ocfg=OptimConfig(normuon=(name == "small_gqa")))


def test_grouped_heads_with_sliding_windows_full_step():
    """Grouped key/value heads and per-layer windows together (fp32, 2 query
    heads over 1, windows 8 and 40 keys)."""
    check_step(TINY_GQA, B=2, seed=43, windows=[8, 40])


@pytest.mark.parametrize("name", ["small", "d12"])
def test_fp8_forward_full_step(name):
    """Forward block products in fp8 e4m3 (tensorwise scales, quantised on the
    device) against the oracle's e4m3 emulation of the same products; the
    backward stays bf16 with the unquantised operands on both sides (bounds:
    TOL["fp8"])."""
    cfg = {"small": replace(SMALL_BF16, fp8_forward=True),
           "d12": replace(with_batch(D12, micro_batch=1), fp8_forward=True)}[name]
    check_step(cfg, B=cfg.micro_batch, seed=51)


def test_d12_shape_one_row():
    check_step(with_batch(D12, micro_batch=1), B=1, seed=7)


@pytest.mark.parametrize("name,seed", [("d20", 11), ("d24", 12), ("d26", 13)])
def test_large_shape_one_row(name, seed):
    """The d20, d24 and d26 model shapes (one 2048-token row against the fp64
    oracle: loss, every gradient, every Muon/AdamW update)."""
    check_step(with_batch(CONFIGS[name], micro_batch=1), B=1, seed=seed)


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16])
def test_zero_head_loss_is_ln_vocab_and_other_grads_vanish(cfg):
    m, params, tok, tgt = setup(cfg, B=2, seed=2)
    m.set_params({"Wh": np.zeros((cfg.vocab, cfg.d_model), np.float32)})
    loss, grads = run_gpu(m, tok, tgt)
    assert loss == pytest.approx(math.log(cfg.vocab), abs=2e-6)
    for n, g in grads.items():
        if n != "Wh":
            assert not np.any(g), n
    # softmax rows sum to one: sum_v dWh[v, :] = 0 up to the rounding of dz to the
    # activation type: |sum_v dz[n, v]| <= 2^-8 sum_v |dz[n, v]| = 2^-7 / N per row
    # (fp32: each entry carries ~2^-24 sqrt(N) relative accumulation error)
    tol = 2e-5 if cfg.dtype == "fp32" else 1e-2
    gwh = grads["Wh"].astype(np.float64)
    assert np.max(np.abs(gwh.sum(0))) <= tol * np.max(np.abs(gwh))
    m.close()


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16])
def test_accumulation_matches_large_batch_and_is_deterministic(cfg):
    m, params, tok, tgt = setup(cfg, B=2, seed=4)
    loss_full, g_full = run_gpu(m, tok, tgt)
    loss_again, g_again = run_gpu(m, tok, tgt)
    assert loss_full == loss_again
    for n in g_full:
        assert np.array_equal(g_full[n], g_again[n]), n        # bitwise run-to-run
    m.zero_grads()
    losses = []
    for r in range(2):
        losses.append(float(m.fwd_bwd(gpu_tokens(tok[r:r + 1]), gpu_tokens(tgt[r:r + 1]), 0.5).item()))
    torch.cuda.synchronize()
    assert 0.5 * sum(losses) == pytest.approx(loss_full, rel=1e-5)
    tol_c = 1 - 1e-10 if cfg.dtype == "fp32" else 0.9999
    for n in g_full:
        g_acc = m.get(n, nc.NC_GRAD)
        assert cosine(g_acc, g_full[n]) >= tol_c, n
        assert max_rel(g_acc, g_full[n]) <= (1e-5 if cfg.dtype == "fp32" else 2e-2), n
    m.close()


def test_init_params_statistics_and_nonfinite_detection():
    cfg = SMALL_BF16
    m = nc.Model(cfg, OptimConfig(), max_micro_batch=1)
    m.init_params(seed=123, std=0.02)
    w1 = m.get("1.W1")
    assert abs(w1.mean()) < 3 * 0.02 / math.sqrt(w1.size)
    assert abs(w1.std() - 0.02) < 3 * 0.02 / math.sqrt(2 * w1.size)
    m.init_params(seed=123, std=0.02)
    assert np.array_equal(m.get("1.W1"), w1)
    m.zero_grads()
    assert m.check_finite()
    bad = m.get("0.Wo")
    bad[3, 5] = np.nan
    m.set_params({"0.Wo": bad})
    assert not m.check_finite()
    m.close()
