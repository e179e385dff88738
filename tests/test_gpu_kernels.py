"""Kernel-level parity on the GPU: the GEMM family (every operand layout and
epilogue, batched, split-K, ragged tiles, a full-size sampled case) against
numpy matmuls of the same (bf16-rounded) inputs, and causal attention
forward/backward against the oracle's attention."""

import numpy as np
import pytest
import torch

import oracle
from gpt_pretraining_step_gemms_amd import nc
from parity import cosine, max_rel

pytestmark = pytest.mark.gpu

BF, F32 = torch.bfloat16, torch.float32


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dtype)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rounded(a, dtype):
    """The values the GPU sees for a float array stored as `dtype`."""
    return host(dev(a, dtype))


def stored(logical, layout):
    return logical if layout == nc.NC_K_CONTIGUOUS else np.ascontiguousarray(logical.T)


# K = 200: the generic kernel (K not a multiple of 32); K = 320: the pipelined
# kernel (depth 64 with 16 x 16 x 32 MFMAs for K-contiguous x K-contiguous,
# depth 32 with 32 x 32 x 16 MFMAs otherwise); K = 288: K-contiguous at depth 32.
@pytest.mark.parametrize("K", [200, 288, 320])
@pytest.mark.parametrize("dtype", [BF, F32])
@pytest.mark.parametrize("al,bl", [(0, 0), (0, 1), (1, 1), (1, 0)])
def test_gemm_layouts_ragged(dtype, al, bl, K):
    M, N = 264, 136                  # one full 256 tile + ragged edges in M and N
    rng = np.random.default_rng(10 + 2 * al + bl + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((N, K)).astype(np.float32)
    As, Bs = stored(A, al), stored(B, bl)
    dA, dB = dev(As, dtype), dev(Bs, dtype)
    C = torch.zeros(M, N, dtype=F32, device="cuda")
    nc.gemm(dA, al, dB, bl, C, M, N, K, nc.EPI_STORE_F32, lda=As.shape[1], ldb=Bs.shape[1])
    torch.cuda.synchronize()
    ref = stored(host(dA), al) @ stored(host(dB), bl).T
    assert max_rel(host(C), ref) < 2e-6


# K = 96: depth 32, 32 x 32 x 16 MFMAs; K = 128: the half-stage ring, 16 x 16 x 32
@pytest.mark.parametrize("K", [96, 128])
@pytest.mark.parametrize("epi", ["store", "relu2", "acc_f32"])
def test_gemm_unaligned_output_rows(epi, K):
    """N = 131 (ldc not a multiple of 8): the epilogue's per-element path."""
    M, N = 300, 131
    rng = np.random.default_rng(8 + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((N, K)).astype(np.float32)
    dA, dB = dev(A, BF), dev(B, BF)
    acc = host(dA) @ host(dB).T
    if epi == "store":
        C = torch.empty(M, N, dtype=BF, device="cuda")
        nc.gemm(dA, 0, dB, 0, C, M, N, K, nc.EPI_STORE, alpha=2.0)
        torch.cuda.synchronize()
        assert max_rel(host(C), 2.0 * acc) < 2 ** -8
    elif epi == "relu2":
        G = torch.empty(M, N, dtype=BF, device="cuda")
        nc.gemm(dA, 0, dB, 0, G, M, N, K, nc.EPI_RELU2)
        torch.cuda.synchronize()
        assert max_rel(host(G), np.maximum(acc, 0) ** 2) < 2 ** -8
    else:
        C0 = rng.standard_normal((M, N)).astype(np.float32)
        C = dev(C0, F32)
        nc.gemm(dA, 0, dB, 0, C, M, N, K, nc.EPI_ACC_F32)
        torch.cuda.synchronize()
        assert max_rel(host(C), C0 + acc) < 2e-6


# K = 136: generic kernel; 192: pipelined, depth 64, 16 x 16 x 32 MFMAs; 224:
# pipelined, depth 32, 32 x 32 x 16 MFMAs (M and N ragged against 256 tiles)
@pytest.mark.parametrize("K", [136, 192, 224])
def test_gemm_epilogues_bf16(K):
    M, N = 320, 264
    rng = np.random.default_rng(3 + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((N, K)).astype(np.float32)
    dA, dB = dev(A, BF), dev(B, BF)
    acc = host(dA) @ host(dB).T
    # store (bf16 out, alpha)
    C = torch.empty(M, N, dtype=BF, device="cuda")
    nc.gemm(dA, 0, dB, 0, C, M, N, K, nc.EPI_STORE, alpha=0.5)
    # accumulate into fp32
    C0 = rng.standard_normal((M, N)).astype(np.float32)
    Cacc = dev(C0, F32)
    nc.gemm(dA, 0, dB, 0, Cacc, M, N, K, nc.EPI_ACC_F32)
    # ReLU^2 forward: g = max(h,0)^2
    G = torch.empty(M, N, dtype=BF, device="cuda")
    nc.gemm(dA, 0, dB, 0, G, M, N, K, nc.EPI_RELU2)
    G2 = torch.empty(M, N, dtype=BF, device="cuda")     # acc = alpha A B^T in every epilogue
    nc.gemm(dA, 0, dB, 0, G2, M, N, K, nc.EPI_RELU2, alpha=-0.5)
    # ReLU^2 backward (from the stored activation g >= 0, some entries 0) and the
    # Newton-Schulz polynomial read an auxiliary input
    aux = dev(rng.standard_normal((M, N)), BF)
    gst = dev(np.maximum(rng.standard_normal((M, N)), 0) ** 2, BF)
    R = torch.empty(M, N, dtype=BF, device="cuda")
    nc.gemm(dA, 0, dB, 0, R, M, N, K, nc.EPI_RELU2_BWD, aux_in=gst, alpha=0.75)
    Pn = torch.empty(M, N, dtype=BF, device="cuda")
    nc.gemm(dA, 0, dB, 0, Pn, M, N, K, nc.EPI_POLY, aux_in=aux, p0=1.5, p1=-0.25, alpha=2.0)
    aux32 = dev(rng.standard_normal((M, N)), F32)
    D32 = torch.empty(M, N, dtype=F32, device="cuda")
    Dh = torch.empty(M, N, dtype=BF, device="cuda")
    nc.gemm(dA, 0, dB, 0, D32, M, N, K, nc.EPI_DUAL, aux_in=aux32, aux_out=Dh, p0=3.0, p1=0.5,
            alpha=0.25)
    torch.cuda.synchronize()
    tol = 2 ** -8
    assert max_rel(host(C), 0.5 * acc) < tol
    assert max_rel(host(Cacc), C0 + acc) < 2e-6
    assert max_rel(host(G), np.maximum(acc, 0) ** 2) < tol
    assert max_rel(host(G2), np.maximum(-0.5 * acc, 0) ** 2) < tol
    assert max_rel(host(R), 2 * np.sqrt(host(gst)) * 0.75 * acc) < tol
    assert max_rel(host(Pn), 1.5 * host(aux) - 0.25 * 2.0 * acc) < tol
    dual = 3.0 * host(aux32) + 0.5 * 0.25 * acc
    assert max_rel(host(D32), dual) < 2e-6
    assert max_rel(host(Dh), dual) < tol


@pytest.mark.parametrize("K", [256, 288])
def test_gemm_batched_k_contiguous(K):
    # batched K-contiguous products (the Newton-Schulz shape) on both pipelined paths
    batch, M, N = 3, 264, 520
    rng = np.random.default_rng(5 + K)
    A = rng.standard_normal((batch, M, K)).astype(np.float32)
    B = rng.standard_normal((batch, N, K)).astype(np.float32)
    dA, dB = dev(A, BF), dev(B, BF)
    C = torch.zeros(batch, M, N, dtype=F32, device="cuda")
    nc.gemm(dA, 0, dB, 0, C, M, N, K, nc.EPI_STORE_F32, lda=K, ldb=K, ldc=N, batch=batch,
            sA=M * K, sB=N * K, sC=M * N)
    torch.cuda.synchronize()
    ref = np.einsum("bmk,bnk->bmn", host(dA), host(dB))
    assert max_rel(host(C), ref) < 2e-6


@pytest.mark.parametrize("al,bl", [(0, 0), (0, 1), (1, 1)])
def test_gemm_degenerate_shapes(al, bl):
    # more splits than 64-deep k-steps (empty splits write zero partials), and
    # a product smaller than one 256 x 256 tile, on the pipelined kernels
    rng = np.random.default_rng(21 + 2 * al + bl)
    for M, N, K, splits in [(264, 136, 128, 4), (8, 16, 64, 1), (24, 8, 192, 5)]:
        A = rng.standard_normal((M, K)).astype(np.float32)
        B = rng.standard_normal((N, K)).astype(np.float32)
        As, Bs = stored(A, al), stored(B, bl)
        dA, dB = dev(As, BF), dev(Bs, BF)
        C0 = rng.standard_normal((M, N)).astype(np.float32)
        C = dev(C0, F32)
        ws = torch.empty(splits * M * N, dtype=F32, device="cuda") if splits > 1 else None
        nc.gemm(dA, al, dB, bl, C, M, N, K, nc.EPI_ACC_F32, lda=As.shape[1], ldb=Bs.shape[1],
                splits=splits, workspace=ws)
        torch.cuda.synchronize()
        ref = C0 + stored(host(dA), al) @ stored(host(dB), bl).T
        assert max_rel(host(C), ref) < 2e-6, (M, N, K, splits)


@pytest.mark.parametrize("splits", [1, 4])
def test_gemm_batched_and_split_k(splits):
    batch, M, N, K = 3, 136, 200, 1024
    rng = np.random.default_rng(4)
    A = rng.standard_normal((batch, K, M)).astype(np.float32)   # MN-contiguous operands
    B = rng.standard_normal((batch, K, N)).astype(np.float32)
    C0 = rng.standard_normal((batch, M, N)).astype(np.float32)
    dA, dB, C = dev(A, BF), dev(B, BF), dev(C0, F32)
    ws = torch.empty(splits * batch * M * N, dtype=F32, device="cuda") if splits > 1 else None
    nc.gemm(dA, 1, dB, 1, C, M, N, K, nc.EPI_ACC_F32, lda=M, ldb=N, ldc=N, batch=batch,
            sA=K * M, sB=K * N, sC=M * N, splits=splits, workspace=ws)
    torch.cuda.synchronize()
    ref = C0 + np.einsum("bkm,bkn->bmn", host(dA), host(dB))
    assert max_rel(host(C), ref) < 2e-6


@pytest.mark.parametrize("shape", ["qkv_fwd", "wgrad"])
def test_gemm_full_size_sampled(shape):
    """d20 shapes: QKV forward (65536 x 3840 x 1280) and the QKV weight gradient
    (3840 x 1280 over 65536 tokens, split-K); sampled rows checked exactly."""
    rng = np.random.default_rng(5)
    if shape == "qkv_fwd":
        M, N, K, al, bl, splits = 65536, 3840, 1280, 0, 0, 1
    else:
        M, N, K, al, bl, splits = 3840, 1280, 65536, 1, 1, 8
    A = torch.randn((M, K) if al == 0 else (K, M), device="cuda").to(BF)
    B = torch.randn((N, K) if bl == 0 else (K, N), device="cuda").to(BF)
    C = torch.zeros(M, N, dtype=F32, device="cuda")
    ws = torch.empty(splits * M * N, dtype=F32, device="cuda") if splits > 1 else None
    nc.gemm(A, al, B, bl, C, M, N, K, nc.EPI_ACC_F32, lda=A.shape[1], ldb=B.shape[1],
            splits=splits, workspace=ws)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(M, 48, replace=False))
    rows = np.concatenate([rows, [0, M - 1]])
    Bl = host(B) if bl == 0 else host(B).T
    if al == 0:
        Ar = host(A[torch.from_numpy(rows).cuda()])
    else:
        Ar = host(A[:, torch.from_numpy(rows).cuda()]).T
    ref = Ar @ Bl.T
    got = host(C[torch.from_numpy(rows).cuda()])
    assert max_rel(got, ref) < 2e-6


# ------------------------------------------------------------------ attention
def _attn_inputs(B, T, H, dtype, seed):
    rng = np.random.default_rng(seed)
    qkv = dev(rng.standard_normal((B * T, 3 * H * 128)), dtype)
    dO = dev(rng.standard_normal((B * T, H * 128)), dtype)
    return qkv, dO


def _heads(x, B, T, H, col0):
    """[B*T, ...] token-major columns col0 .. col0 + H*128 -> [B, H, T, 128]"""
    a = host(x)[:, col0:col0 + H * 128]
    return a.reshape(B, T, H, 128).transpose(0, 2, 1, 3)


@pytest.mark.parametrize("dtype,B,T,H", [(BF, 2, 256, 2), (BF, 1, 2048, 2), (BF, 2, 384, 1), (BF, 3, 128, 2),
                                         (BF, 4, 640, 2), (F32, 2, 64, 1), (F32, 1, 100, 2)])
def test_attention_forward_backward_vs_oracle(dtype, B, T, H):
    d = H * 128
    qkv, dO = _attn_inputs(B, T, H, dtype, seed=T + H)
    o = torch.empty(B * T, d, dtype=dtype, device="cuda")
    lse = torch.empty(B, H, T, dtype=F32, device="cuda")
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    nc.attention_fwd(q, k, v, o, lse, B, T, H, ld_qkv=3 * d, ld_o=d)
    dqkv = torch.zeros_like(qkv)
    D = torch.empty(2, B, H, T, dtype=F32, device="cuda")
    nc.attention_bwd(q, k, v, o, dO, lse, D, dqkv[:, :d], dqkv[:, d:2 * d], dqkv[:, 2 * d:],
                     B, T, H, ld_qkv=3 * d, ld_o=d, ld_d=3 * d)
    torch.cuda.synchronize()
    Q, K, Vv = (_heads(qkv, B, T, H, c) for c in (0, d, 2 * d))
    o_ref, p = oracle.causal_attention(Q, K, Vv)
    s = Q @ np.swapaxes(K, -1, -2) / np.sqrt(128.0)
    s = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, s)
    lse_ref = np.log(np.sum(np.exp(s - s.max(-1, keepdims=True)), -1)) + s.max(-1)
    dq_r, dk_r, dv_r = oracle.causal_attention_backward(Q, K, Vv, _heads(dO, B, T, H, 0))
    got_o = _heads(o, B, T, H, 0)
    bf = dtype == BF
    assert max_rel(got_o, o_ref) < (2e-2 if bf else 1e-5)
    assert np.max(np.abs(host(lse) - lse_ref)) < (2e-3 if bf else 1e-5)
    for name, got, ref in [("dq", _heads(dqkv, B, T, H, 0), dq_r),
                           ("dk", _heads(dqkv, B, T, H, d), dk_r),
                           ("dv", _heads(dqkv, B, T, H, 2 * d), dv_r)]:
        assert cosine(got, ref) > (0.999 if bf else 1 - 1e-9), name
        assert max_rel(got, ref) < (3e-2 if bf else 1e-5), name


def _band_lse(Q, K, w):
    T = Q.shape[-2]
    s = Q @ np.swapaxes(K, -1, -2) / np.sqrt(128.0)
    t, u = np.arange(T)[:, None], np.arange(T)[None, :]
    s = np.where((u > t) | (u < t - w), -np.inf, s)
    return np.log(np.sum(np.exp(s - s.max(-1, keepdims=True)), -1)) + s.max(-1)


@pytest.mark.parametrize("dtype,B,T,H,w", [
    (BF, 1, 512, 2, 0), (BF, 1, 512, 2, 1), (BF, 1, 512, 2, 31), (BF, 1, 512, 2, 63),
    (BF, 1, 512, 2, 64), (BF, 1, 512, 2, 100), (BF, 1, 512, 2, 128), (BF, 1, 512, 2, 200),
    (BF, 1, 512, 2, 383), (BF, 1, 512, 2, 511), (BF, 2, 384, 1, 127), (BF, 1, 2048, 1, 1024),
    (BF, 4, 640, 2, 100), (BF, 8, 256, 2, 64),
    (F32, 2, 64, 1, 0), (F32, 2, 64, 1, 5), (F32, 1, 100, 2, 17), (F32, 1, 100, 2, 99)])
def test_attention_sliding_window_vs_oracle(dtype, B, T, H, w):
    """Query t sees keys t-w .. t: forward, log-sum-exp and all three
    gradients against the oracle's banded attention."""
    d = H * 128
    qkv, dO = _attn_inputs(B, T, H, dtype, seed=1000 + T + w)
    o = torch.empty(B * T, d, dtype=dtype, device="cuda")
    lse = torch.empty(B, H, T, dtype=F32, device="cuda")
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    print(f"[attn window] {dtype} B={B} T={T} H={H} w={w}", flush=True)
    nc.attention_fwd(q, k, v, o, lse, B, T, H, ld_qkv=3 * d, ld_o=d, window=w)
    dqkv = torch.zeros_like(qkv)
    D = torch.empty(2, B, H, T, dtype=F32, device="cuda")
    nc.attention_bwd(q, k, v, o, dO, lse, D, dqkv[:, :d], dqkv[:, d:2 * d], dqkv[:, 2 * d:],
                     B, T, H, ld_qkv=3 * d, ld_o=d, ld_d=3 * d, window=w)
    torch.cuda.synchronize()
    Q, K, Vv = (_heads(qkv, B, T, H, c) for c in (0, d, 2 * d))
    o_ref, _ = oracle.causal_attention(Q, K, Vv, window=w)
    dq_r, dk_r, dv_r = oracle.causal_attention_backward(Q, K, Vv, _heads(dO, B, T, H, 0), window=w)
    bf = dtype == BF
    assert max_rel(_heads(o, B, T, H, 0), o_ref) < (2e-2 if bf else 1e-5)
    assert np.max(np.abs(host(lse) - _band_lse(Q, K, w))) < (2e-3 if bf else 1e-5)
    for name, got, ref in [("dq", _heads(dqkv, B, T, H, 0), dq_r),
                           ("dk", _heads(dqkv, B, T, H, d), dk_r),
                           ("dv", _heads(dqkv, B, T, H, 2 * d), dv_r)]:
        if not np.any(ref):
            # w = 0: one visible key, no gradient reaches the scores; what is
            # left is the rounding of dP - D (both sums of the same products)
            assert np.max(np.abs(got)) < (2e-2 if bf else 1e-5), name
            continue
        assert cosine(got, ref) > (0.999 if bf else 1 - 1e-9), name
        assert max_rel(got, ref) < (3e-2 if bf else 1e-5), name


@pytest.mark.parametrize("w", [-1, 1024])
def test_attention_many_heads_sampled(w):
    """16 (row, head) pairs of 2048 tokens (each XCD's share of the grid
    holds whole heads, the layout of the full-size launches): sampled heads
    against the oracle."""
    B, T, H = 8, 2048, 2
    d = H * 128
    qkv, dO = _attn_inputs(B, T, H, BF, seed=77 + w)
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    o = torch.empty(B * T, d, dtype=BF, device="cuda")
    lse = torch.empty(B, H, T, dtype=F32, device="cuda")
    print(f"[attn heads] B={B} T={T} H={H} w={w}", flush=True)
    nc.attention_fwd(q, k, v, o, lse, B, T, H, 3 * d, d, window=w)
    dqkv = torch.zeros_like(qkv)
    D = torch.empty(2, B, H, T, dtype=F32, device="cuda")
    nc.attention_bwd(q, k, v, o, dO, lse, D, dqkv[:, :d], dqkv[:, d:2 * d], dqkv[:, 2 * d:],
                     B, T, H, 3 * d, d, 3 * d, window=w)
    torch.cuda.synchronize()
    win = None if w < 0 else w
    heads = {c: _heads(x, B, T, H, c0) for c, (x, c0) in
             {"q": (qkv, 0), "k": (qkv, d), "v": (qkv, 2 * d), "o": (o, 0), "dO": (dO, 0),
              "dq": (dqkv, 0), "dk": (dqkv, d), "dv": (dqkv, 2 * d)}.items()}
    for b, h in [(0, 0), (2, 1), (5, 0), (7, 1)]:
        Q, K, Vv = heads["q"][b, h], heads["k"][b, h], heads["v"][b, h]
        o_ref, _ = oracle.causal_attention(Q, K, Vv, window=win)
        assert max_rel(heads["o"][b, h], o_ref) < 2e-2, (b, h)
        assert np.max(np.abs(host(lse)[b, h] - _band_lse(Q, K, T if win is None else win))) < 2e-3
        refs = oracle.causal_attention_backward(Q, K, Vv, heads["dO"][b, h], window=win)
        for name, ref in zip(("dq", "dk", "dv"), refs):
            got = heads[name][b, h]
            assert cosine(got, ref) > 0.999 and max_rel(got, ref) < 3e-2, (b, h, name)


@pytest.mark.parametrize("dtype,B,T,H,Hkv,w", [
    (BF, 2, 256, 4, 2, -1), (BF, 1, 512, 6, 1, -1), (BF, 8, 256, 4, 1, -1),
    (BF, 2, 384, 4, 2, 100), (BF, 8, 256, 2, 1, 64), (F32, 2, 64, 2, 1, -1),
    (F32, 1, 100, 4, 2, 17)])
def test_attention_grouped_query_vs_oracle(dtype, B, T, H, Hkv, w):
    """H query heads over Hkv key/value heads (query head h reads head
    h // (H / Hkv)): forward, log-sum-exp and gradients against the oracle,
    dk and dv summed over each key/value head's query heads."""
    g = H // Hkv
    d, dk = H * 128, Hkv * 128
    rng = np.random.default_rng(500 + H * 10 + Hkv + max(w, 0))
    qkv = dev(rng.standard_normal((B * T, d + 2 * dk)), dtype)
    dO = dev(rng.standard_normal((B * T, d)), dtype)
    q, k, v = qkv[:, :d], qkv[:, d:d + dk], qkv[:, d + dk:]
    o = torch.empty(B * T, d, dtype=dtype, device="cuda")
    lse = torch.empty(B, H, T, dtype=F32, device="cuda")
    print(f"[attn gqa] {dtype} B={B} T={T} H={H} Hkv={Hkv} w={w}", flush=True)
    ld = d + 2 * dk
    nc.attention_fwd(q, k, v, o, lse, B, T, H, ld, d, window=w, n_kv_head=Hkv)
    dqkv = torch.zeros_like(qkv)
    D = torch.empty(2, B, H, T, dtype=F32, device="cuda")
    nc.attention_bwd(q, k, v, o, dO, lse, D, dqkv[:, :d], dqkv[:, d:d + dk], dqkv[:, d + dk:],
                     B, T, H, ld, d, ld, window=w, n_kv_head=Hkv)
    torch.cuda.synchronize()
    win = None if w < 0 else w
    Q = _heads(qkv, B, T, H, 0)
    K, Vv = (_heads(qkv, B, T, Hkv, c) for c in (d, d + dk))
    Kr, Vr = np.repeat(K, g, axis=1), np.repeat(Vv, g, axis=1)
    o_ref, _ = oracle.causal_attention(Q, Kr, Vr, window=win)
    dq_r, dk_r, dv_r = oracle.causal_attention_backward(Q, Kr, Vr, _heads(dO, B, T, H, 0),
                                                        window=win)
    dk_r = dk_r.reshape(B, Hkv, g, T, 128).sum(2)
    dv_r = dv_r.reshape(B, Hkv, g, T, 128).sum(2)
    bf = dtype == BF
    assert max_rel(_heads(o, B, T, H, 0), o_ref) < (2e-2 if bf else 1e-5)
    assert np.max(np.abs(host(lse) - _band_lse(Q, Kr, T if win is None else win))) < (
        2e-3 if bf else 1e-5)
    for name, got, ref in [("dq", _heads(dqkv, B, T, H, 0), dq_r),
                           ("dk", _heads(dqkv, B, T, Hkv, d), dk_r),
                           ("dv", _heads(dqkv, B, T, Hkv, d + dk), dv_r)]:
        assert cosine(got, ref) > (0.999 if bf else 1 - 1e-9), name
        assert max_rel(got, ref) < (3e-2 if bf else 1e-5), name


@pytest.mark.parametrize("w", [-1, 1024])
def test_attention_d20_launch_sampled(w):
    """The attention launches of a d20 micro-batch as the step runs them (32
    rows x 10 heads x 2048 tokens, q/k/v inside one [N, 3d] row): sampled
    (row, head) pairs against the oracle."""
    B, T, H = 32, 2048, 10
    d = H * 128
    rng = np.random.default_rng(90 + max(w, 0))
    qkv = dev(rng.standard_normal((B * T, 3 * d), dtype=np.float32), BF)
    dO = dev(rng.standard_normal((B * T, d), dtype=np.float32), BF)
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    o = torch.empty(B * T, d, dtype=BF, device="cuda")
    lse = torch.empty(B, H, T, dtype=F32, device="cuda")
    print(f"[attn d20] w={w}", flush=True)
    nc.attention_fwd(q, k, v, o, lse, B, T, H, 3 * d, d, window=w)
    dqkv = torch.empty_like(qkv)
    D = torch.empty(2, B, H, T, dtype=F32, device="cuda")
    nc.attention_bwd(q, k, v, o, dO, lse, D, dqkv[:, :d], dqkv[:, d:2 * d], dqkv[:, 2 * d:],
                     B, T, H, 3 * d, d, 3 * d, window=w)
    torch.cuda.synchronize()
    win = None if w < 0 else w
    for b, h in [(0, 0), (13, 7), (31, 9)]:
        rows = slice(b * T, (b + 1) * T)
        cols = lambda c0: slice(c0 + h * 128, c0 + (h + 1) * 128)
        Q, K, Vv = (host(qkv[rows, cols(c)]).astype(np.float64) for c in (0, d, 2 * d))
        o_ref, _ = oracle.causal_attention(Q, K, Vv, window=win)
        assert max_rel(host(o[rows, cols(0)]), o_ref) < 2e-2, (b, h)
        assert np.max(np.abs(host(lse)[b, h] - _band_lse(Q, K, T if win is None else win))) < 2e-3
        refs = oracle.causal_attention_backward(Q, K, Vv, host(dO[rows, cols(0)]).astype(np.float64),
                                                window=win)
        for name, c0, ref in zip(("dq", "dk", "dv"), (0, d, 2 * d), refs):
            got = host(dqkv[rows, cols(c0)])
            assert cosine(got, ref) > 0.999 and max_rel(got, ref) < 3e-2, (b, h, name)


def test_attention_window_covering_the_row_is_bitwise_causal():
    B, T, H = 1, 384, 2
    d = H * 128
    qkv, dO = _attn_inputs(B, T, H, BF, seed=5)
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    res = []
    for w in (-1, T - 1, T, 10 * T):
        o = torch.empty(B * T, d, dtype=BF, device="cuda")
        lse = torch.empty(B, H, T, dtype=F32, device="cuda")
        nc.attention_fwd(q, k, v, o, lse, B, T, H, 3 * d, d, window=w)
        dqkv = torch.zeros_like(qkv)
        D = torch.empty(2, B, H, T, dtype=F32, device="cuda")
        nc.attention_bwd(q, k, v, o, dO, lse, D, dqkv[:, :d], dqkv[:, d:2 * d], dqkv[:, 2 * d:],
                         B, T, H, 3 * d, d, 3 * d, window=w)
        res.append((o, lse, dqkv))
    torch.cuda.synchronize()
    for r in res[1:]:
        for a, b in zip(res[0], r):
            assert torch.equal(a, b)


def test_attention_causality_bitwise():
    """Changing key/value rows at t* >= t leaves outputs of queries t < t* unchanged."""
    B, T, H = 1, 256, 2
    d = H * 128
    qkv, _ = _attn_inputs(B, T, H, BF, seed=1)
    outs = []
    for trial in range(2):
        x = qkv.clone()
        if trial:
            x[200:, d:] = torch.randn_like(x[200:, d:])
        o = torch.empty(B * T, d, dtype=BF, device="cuda")
        lse = torch.empty(B, H, T, dtype=F32, device="cuda")
        nc.attention_fwd(x[:, :d], x[:, d:2 * d], x[:, 2 * d:], o, lse, B, T, H, 3 * d, d)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0][:200], outs[1][:200])
    assert not torch.equal(outs[0][200:], outs[1][200:])


# ------------------------------------------------------------------------ fp8
from oracle import fp8 as ofp8  # noqa: E402


def test_fp8_quantize_all_zero_input():
    x = torch.zeros(4096, dtype=F32, device="cuda")
    q = torch.full((4096,), 0x55, dtype=torch.uint8, device="cuda")
    amax_scale = torch.empty(2, dtype=F32, device="cuda")
    ws = torch.empty(1024, dtype=F32, device="cuda")
    nc.fp8_quantize(x, q, amax_scale, ws)
    torch.cuda.synchronize()
    assert host(amax_scale).tolist() == [0.0, 1.0]
    assert not q.any()


@pytest.mark.parametrize("dtype", [F32, BF])
def test_fp8_quantize_nan_reaches_every_code(dtype):
    """One NaN in the tensor: amax and scale NaN and every code 0x7F, as in
    the oracle's codec (a NaN must not become a finite e4m3 value)."""
    n = 20000 + 3
    x = np.random.default_rng(3).standard_normal(n).astype(np.float32)
    x[12345] = np.nan
    xd = dev(x, dtype)
    q = torch.zeros(n, dtype=torch.uint8, device="cuda")
    amax_scale = torch.empty(2, dtype=F32, device="cuda")
    ws = torch.empty(1024, dtype=F32, device="cuda")
    nc.fp8_quantize(xd, q, amax_scale, ws)
    torch.cuda.synchronize()
    codes, amax, scale = ofp8.quantize_tensorwise(host(xd).astype(np.float32))
    assert np.isnan(amax) and np.isnan(scale)
    got_amax, got_scale = host(amax_scale)
    assert np.isnan(got_amax) and np.isnan(got_scale)
    assert np.array_equal(q.cpu().numpy(), codes)


@pytest.mark.parametrize("dtype,n", [(F32, 1000), (F32, 300001), (BF, 65536 + 7)])
def test_fp8_quantize_bit_exact(dtype, n):
    """Tensorwise e4m3 quantisation: amax and scale exact, every byte equal to
    the oracle's (same fp32 products; rounding decided on the same values)."""
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n).astype(np.float32) * rng.uniform(0.01, 5.0)
    x[:7] = [0.0, -0.0, 1e-12, -3e-9, 1e-4, 2.5, -2.5]
    xd = dev(x, dtype)
    xs = host(xd).astype(np.float32)                 # the values the GPU sees
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    amax_scale = torch.empty(2, dtype=F32, device="cuda")
    ws = torch.empty(1024, dtype=F32, device="cuda")
    nc.fp8_quantize(xd, q, amax_scale, ws)
    torch.cuda.synchronize()
    codes, amax, scale = ofp8.quantize_tensorwise(xs)
    got_amax, got_scale = host(amax_scale)
    assert got_amax == amax and got_scale == scale
    got = q.cpu().numpy()
    assert np.array_equal(got, codes), np.flatnonzero(got != codes)[:10]


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (300, 520, 256), (1024, 768, 1280),
                                   (70, 40, 384), (513, 1000, 2048)])
def test_fp8_gemm_vs_oracle(M, N, K):
    """C = alpha A B^T on e4m3 codes against the fp64 product of the decoded
    values.  The products are exact, but the fp8 MFMA's internal sums round
    more coarsely than fp32 (about 4e-5 of the largest output at K = 128 on
    gfx950, against 1e-7 for fp32 sums): the bound is 2e-4, while a wrong
    pairing of k positions gives errors of order one."""
    rng = np.random.default_rng(M + N + K)
    a, _, sa = ofp8.quantize_tensorwise(rng.standard_normal((M, K)))
    b, _, sb = ofp8.quantize_tensorwise(0.02 * rng.standard_normal((N, K)))
    alpha = 1.0 / (sa * sb)
    ref = ofp8.fp8_matmul(a, b, alpha)
    A8 = torch.from_numpy(a).cuda()
    B8 = torch.from_numpy(b).cuda()
    print(f"[fp8 gemm] M={M} N={N} K={K}", flush=True)
    Cf = torch.empty(M, N, dtype=F32, device="cuda")
    nc.gemm_fp8(A8, B8, Cf, M, N, K, alpha, epilogue=nc.EPI_STORE_F32)
    Cb = torch.empty(M, N, dtype=BF, device="cuda")
    nc.gemm_fp8(A8, B8, Cb, M, N, K, alpha, epilogue=nc.EPI_STORE)
    torch.cuda.synchronize()
    err = max_rel(host(Cf), ref)
    print(f"[fp8 gemm] max-rel {err:.2e}", flush=True)
    assert err < 2e-4
    assert max_rel(host(Cb), ref) < 2 ** -8


def test_fp8_gemm_accumulate_and_relu2_epilogues():
    """The residual-add (C += acc, fp32) and ReLU^2 (bf16 max(acc, 0)^2)
    epilogues on fp8 operands."""
    M, N, K = 300, 520, 384
    rng = np.random.default_rng(12)
    a, _, sa = ofp8.quantize_tensorwise(rng.standard_normal((M, K)))
    b, _, sb = ofp8.quantize_tensorwise(0.02 * rng.standard_normal((N, K)))
    alpha = 1.0 / (sa * sb)
    acc = ofp8.fp8_matmul(a, b, alpha)
    A8, B8 = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    c0 = rng.standard_normal((M, N)).astype(np.float32)
    C = torch.from_numpy(c0).cuda()
    nc.gemm_fp8(A8, B8, C, M, N, K, alpha, epilogue=nc.EPI_ACC_F32)
    G = torch.empty(M, N, dtype=BF, device="cuda")
    nc.gemm_fp8(A8, B8, G, M, N, K, alpha, epilogue=nc.EPI_RELU2)
    torch.cuda.synchronize()
    assert np.max(np.abs(host(C) - (c0 + acc))) < 2e-4 * np.max(np.abs(acc)) + 1e-6
    g_ref = np.maximum(acc, 0.0) ** 2
    assert max_rel(host(G), g_ref) < 2 ** -7


def test_fp8_gemm_rejects_unsupported_shapes():
    A8 = torch.zeros(64, 192, dtype=torch.uint8, device="cuda")
    C = torch.empty(64, 64, dtype=F32, device="cuda")
    with pytest.raises(nc.NcError):                  # K not a multiple of 128
        nc.gemm_fp8(A8, A8, C, 64, 64, 192, 1.0, epilogue=nc.EPI_STORE_F32)


def test_fp8_gemm_mlp_up_shape_sampled():
    """The MLP up-projection shape of a d20 micro-batch in fp8: sampled rows."""
    M, N, K = 65536, 5120, 1280
    g = torch.Generator(device="cuda").manual_seed(5)
    A8 = torch.randint(0, 256, (M, K), dtype=torch.uint8, device="cuda", generator=g)
    B8 = torch.randint(0, 256, (N, K), dtype=torch.uint8, device="cuda", generator=g)
    for t in (A8, B8):                               # no NaN codes; keep magnitudes modest
        t &= 0xB7
    C = torch.empty(M, N, dtype=F32, device="cuda")
    nc.gemm_fp8(A8, B8, C, M, N, K, 0.25, epilogue=nc.EPI_STORE_F32)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 40000, M - 1])
    a = A8[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = ofp8.fp8_matmul(a, B8.cpu().numpy(), 0.25)
    assert max_rel(host(C[torch.from_numpy(rows).cuda()]), ref) < 2e-4


@pytest.mark.parametrize("dtype,n", [(F32, 1000), (F32, 300001), (BF, 65536 + 7)])
def test_fp8_quantize_e5m2_bit_exact(dtype, n):
    """Tensorwise e5m2 (gradients): amax, scale 57344 / amax and every byte
    equal to the oracle's table-search codec."""
    rng = np.random.default_rng(n + 1)
    x = rng.standard_normal(n).astype(np.float32) * rng.uniform(1e-7, 1e-3)
    x[:6] = [0.0, -0.0, 1e-30, -2e-12, 3e-5, -3e-5]
    xd = dev(x, dtype)
    xs = host(xd).astype(np.float32)
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    amax_scale = torch.empty(2, dtype=F32, device="cuda")
    ws = torch.empty(1024, dtype=F32, device="cuda")
    nc.fp8_quantize(xd, q, amax_scale, ws, fmt=nc.FP8_E5M2)
    torch.cuda.synchronize()
    codes, amax, scale = ofp8.quantize_tensorwise(xs, ofp8.E5M2)
    assert tuple(host(amax_scale)) == (amax, scale)
    got = q.cpu().numpy()
    assert np.array_equal(got, codes), np.flatnonzero(got != codes)[:10]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("R,C,both", [(64, 64, True), (192, 320, True), (2048, 1280, True),
                                      (512, 5120, False)])
def test_fp8_quantize_transposed_codes(fmt, R, C, both):
    """The 2-D quantiser: codes in x's layout and transposed, byte for byte the
    oracle's codes and their transpose (and the transposed ones alone)."""
    rng = np.random.default_rng(R + C + fmt)
    x = (rng.standard_normal((R, C)) * (1e-4 if fmt else 1.0)).astype(np.float32)
    xd = dev(x, BF)
    xs = host(xd).astype(np.float32)
    q = torch.zeros(R, C, dtype=torch.uint8, device="cuda") if both else None
    qt = torch.zeros(C, R, dtype=torch.uint8, device="cuda")
    amax_scale = torch.empty(2, dtype=F32, device="cuda")
    ws = torch.empty(1024, dtype=F32, device="cuda")
    print(f"[fp8 quantize 2d] fmt={fmt} R={R} C={C}", flush=True)
    nc.fp8_quantize(xd, q, amax_scale, ws, fmt=fmt, qt=qt, rows=R, cols=C)
    torch.cuda.synchronize()
    codes, amax, scale = ofp8.quantize_tensorwise(xs, ofp8.E5M2 if fmt else ofp8.E4M3)
    assert tuple(host(amax_scale)) == (amax, scale)
    if both:
        assert np.array_equal(q.cpu().numpy(), codes)
    assert np.array_equal(qt.cpu().numpy(), codes.T)


def _e5m2_e4m3_operands(rng, M, N, K, a_std=1e-4):
    a, _, sa = ofp8.quantize_tensorwise(a_std * rng.standard_normal((M, K)), ofp8.E5M2)
    b, _, sb = ofp8.quantize_tensorwise(0.02 * rng.standard_normal((N, K)), ofp8.E4M3)
    return a, b, 1.0 / (sa * sb)


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (300, 520, 256), (70, 40, 384),
                                   (513, 1000, 2048)])
def test_fp8_gemm_e5m2_a_vs_oracle(M, N, K):
    """A in e5m2 (a gradient), B in e4m3: C = alpha A B^T against the fp64
    product of the decoded values (same bound as the e4m3 x e4m3 product; a
    wrong format code would misread every A byte)."""
    rng = np.random.default_rng(M * 7 + N + K)
    a, b, alpha = _e5m2_e4m3_operands(rng, M, N, K)
    ref = ofp8.fp8_matmul(a, b, alpha, ofp8.E5M2, ofp8.E4M3)
    A8, B8 = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    print(f"[fp8 gemm e5m2] M={M} N={N} K={K}", flush=True)
    Cf = torch.empty(M, N, dtype=F32, device="cuda")
    nc.gemm_fp8(A8, B8, Cf, M, N, K, alpha, epilogue=nc.EPI_STORE_F32, a_format=nc.FP8_E5M2)
    torch.cuda.synchronize()
    err = max_rel(host(Cf), ref)
    print(f"[fp8 gemm e5m2] max-rel {err:.2e}", flush=True)
    assert err < 2e-4


@pytest.mark.parametrize("splits", [2, 5])
def test_fp8_gemm_split_k_and_relu2_backward(splits):
    """Split-K on fp8 operands (fp32 partials summed in a fixed order, added to
    C) equals the unsplit product to the kernel's rounding, and the ReLU^2
    backward epilogue 2 sqrt(g) acc reads its bf16 aux rows."""
    M, N, K = 320, 384, 2048
    rng = np.random.default_rng(splits)
    a, b, alpha = _e5m2_e4m3_operands(rng, M, N, K)
    ref = ofp8.fp8_matmul(a, b, alpha, ofp8.E5M2, ofp8.E4M3)
    A8, B8 = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    c0 = rng.standard_normal((M, N)).astype(np.float32)
    C = torch.from_numpy(c0).cuda()
    ws = torch.empty(splits * M * N, dtype=F32, device="cuda")
    nc.gemm_fp8(A8, B8, C, M, N, K, alpha, epilogue=nc.EPI_ACC_F32, a_format=nc.FP8_E5M2,
                splits=splits, workspace=ws)
    C1 = torch.from_numpy(c0).cuda()
    nc.gemm_fp8(A8, B8, C1, M, N, K, alpha, epilogue=nc.EPI_ACC_F32, a_format=nc.FP8_E5M2)
    g = np.abs(rng.standard_normal((M, N))).astype(np.float32)
    gd = dev(g, BF)
    D = torch.empty(M, N, dtype=BF, device="cuda")
    nc.gemm_fp8(A8, B8, D, M, N, K, alpha, epilogue=nc.EPI_RELU2_BWD, a_format=nc.FP8_E5M2,
                aux_in=gd)
    torch.cuda.synchronize()
    scale = np.max(np.abs(ref))
    assert np.max(np.abs(host(C) - (c0 + ref))) < 2e-4 * scale + 1e-6
    assert np.max(np.abs(host(C) - host(C1))) < 2e-4 * scale + 1e-6
    d_ref = 2.0 * np.sqrt(host(gd).astype(np.float64)) * ref
    assert max_rel(host(D), d_ref) < 2 ** -7


def test_fp8_gemm_weight_gradient_shape_sampled():
    """The weight-gradient shape of a d20 micro-batch (dW2: [1280, 5120],
    K = 65536 tokens) in fp8 with the split count the step uses: sampled
    rows against the decoded product."""
    M, N, K = 1280, 5120, 65536
    splits = 5                                       # what the split cost model picks here
    g = torch.Generator(device="cuda").manual_seed(9)
    A8 = torch.randint(0, 256, (M, K), dtype=torch.uint8, device="cuda", generator=g)
    B8 = torch.randint(0, 256, (N, K), dtype=torch.uint8, device="cuda", generator=g)
    A8 &= 0xB3                                       # e5m2: no inf/NaN codes, modest magnitudes
    B8 &= 0xB7                                       # e4m3: no NaN codes
    C = torch.zeros(M, N, dtype=F32, device="cuda")
    ws = torch.empty(splits * M * N, dtype=F32, device="cuda")
    print(f"[fp8 dW shape] splits={splits}", flush=True)
    nc.gemm_fp8(A8, B8, C, M, N, K, 1.0, epilogue=nc.EPI_ACC_F32, a_format=nc.FP8_E5M2,
                splits=splits, workspace=ws)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 640, M - 1])
    a = A8[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = ofp8.fp8_matmul(a, B8.cpu().numpy(), 1.0, ofp8.E5M2, ofp8.E4M3)
    assert max_rel(host(C[torch.from_numpy(rows).cuda()]), ref) < 2e-4
