"""nc_op_gemm_noalloc (split-K partials in the library's fixed device
scratch) against nc_op_gemm with a caller workspace: two calls in a row, the
second smaller, each bit for bit equal to the workspace entry point's
result (same kernels, same order of the split sums), and a request beyond
the scratch's 16 MiB refused before any launch."""

import numpy as np
import pytest
import torch

from gpt_pretraining_step_gemms_amd import nc

pytestmark = pytest.mark.gpu

BF, F32 = torch.bfloat16, torch.float32


def _case(M, N, K, splits, seed, epi):
    g = torch.Generator(device="cuda").manual_seed(seed)
    # weight-gradient layout: both operands MN-contiguous ([K, M] and [K, N])
    A = torch.randn(K, M, device="cuda", generator=g).to(BF)
    B = torch.randn(K, N, device="cuda", generator=g).to(BF)
    C0 = torch.randn(M, N, device="cuda", generator=g)
    ws = torch.empty(splits * M * N, dtype=F32, device="cuda")
    ref = C0.clone()
    nc.gemm(A, nc.NC_MN_CONTIGUOUS, B, nc.NC_MN_CONTIGUOUS, ref, M, N, K, epi, lda=M, ldb=N,
            splits=splits, workspace=ws)
    out = C0.clone()
    nc.gemm_noalloc(A, nc.NC_MN_CONTIGUOUS, B, nc.NC_MN_CONTIGUOUS, out, M, N, K, epi, lda=M,
                    ldb=N, splits=splits)
    torch.cuda.synchronize()
    return out, ref, A, B, C0


def test_noalloc_gemm_matches_workspace_gemm_on_two_calls():
    for (M, N, K, splits, seed, epi) in [(1152, 768, 8192, 4, 1, nc.EPI_ACC_F32),
                                         (264, 136, 2048, 3, 2, nc.EPI_STORE_F32)]:
        print(f"[no-alloc] M={M} N={N} K={K} splits={splits}", flush=True)
        out, ref, A, B, C0 = _case(M, N, K, splits, seed, epi)
        assert torch.equal(out, ref)
        # and against a plain product (fp32 sums of the same bf16 inputs)
        exact = (A.double().T @ B.double()).cpu().numpy()
        if epi == nc.EPI_ACC_F32:
            exact = exact + C0.double().cpu().numpy()
        err = np.max(np.abs(out.double().cpu().numpy() - exact)) / np.max(np.abs(exact))
        assert err < 2e-6, err


def test_noalloc_gemm_without_split_and_refusal_beyond_the_scratch():
    M, N, K = 300, 520, 256
    A = torch.randn(M, K, device="cuda").to(BF)
    B = torch.randn(N, K, device="cuda").to(BF)
    C = torch.empty(M, N, dtype=F32, device="cuda")
    R = torch.empty(M, N, dtype=F32, device="cuda")
    nc.gemm_noalloc(A, 0, B, 0, C, M, N, K, nc.EPI_STORE_F32)
    nc.gemm(A, 0, B, 0, R, M, N, K, nc.EPI_STORE_F32)
    torch.cuda.synchronize()
    assert torch.equal(C, R)
    # 5 splits of a [2048, 1024] fp32 slab = 40 MiB > 16 MiB: refused
    Mb, Nb, Kb = 2048, 1024, 4096
    Ab = torch.zeros(Kb, Mb, dtype=BF, device="cuda")
    Bb = torch.zeros(Kb, Nb, dtype=BF, device="cuda")
    Cb = torch.zeros(Mb, Nb, dtype=F32, device="cuda")
    with pytest.raises(nc.NcError) as e:
        nc.gemm_noalloc(Ab, 1, Bb, 1, Cb, Mb, Nb, Kb, nc.EPI_ACC_F32, lda=Mb, ldb=Nb, splits=5)
    assert e.value.status == nc.NC_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert not Cb.any()
