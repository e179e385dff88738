"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function declared in include/*.h, plans arenas, validates
configurations and reports call-order errors before touching the device."""

import ctypes
import glob
import os
import re

import pytest

from gpt_pretraining_step_gemms_amd import nc
from gpt_pretraining_step_gemms_amd.configs import CONFIGS, D26, TINY, OptimConfig, from_depth
from oracle.model import param_shapes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"^\s*(?:nc_status|void|const char\s*\*)\s*(nc_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = nc.load()
    names = declared_functions()
    assert len(names) >= 18
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_plan_sizes_fit_hbm_and_grow_with_batch():
    for cfg in CONFIGS.values():
        pb, ab = nc.plan(cfg)
        assert pb > 0 and ab > 0
        assert pb % 256 == 0 and ab % 256 == 0
    p1, a1 = nc.plan(D26, max_micro_batch=16)
    p2, a2 = nc.plan(D26, max_micro_batch=64)
    assert p1 == p2 and a2 > 2.5 * a1
    hbm = 288 * 10 ** 9
    assert p2 + a2 < 0.6 * hbm            # d26 at 64 rows fits one MI355X easily
    p3, a3 = nc.plan(D26, max_micro_batch=128)
    assert p3 + a3 < 0.96 * hbm           # 128 rows fit (only g = relu(h)^2 is kept per layer)
    p4, a4 = nc.plan(D26, max_micro_batch=160)
    assert p4 + a4 > hbm                  # ... and 160 rows do not


def _status_of_plan(cfg, ocfg=OptimConfig()):
    lib = nc.load()
    m, o = nc.model_cfg_c(cfg), nc.optim_cfg_c(ocfg)
    return lib.nc_plan(ctypes.byref(m), ctypes.byref(o), None, None)


def test_invalid_configurations_are_rejected():
    from dataclasses import replace
    assert _status_of_plan(TINY) == nc.NC_OK
    assert _status_of_plan(replace(TINY, head_dim=64, n_head=2)) == nc.NC_ERR_UNSUPPORTED
    assert _status_of_plan(replace(TINY, vocab=500)) == nc.NC_ERR_UNSUPPORTED
    assert _status_of_plan(replace(TINY, dtype="bf16")) == nc.NC_ERR_UNSUPPORTED  # T=64 not % 128
    assert _status_of_plan(replace(TINY, d_model=0)) == nc.NC_ERR_INVALID_ARG
    # the fp8 products take K in steps of 128: d_ff = 1536 + 64 is refused at plan time
    small = replace(TINY, dtype="bf16", seq_len=128, d_ff=1536)
    assert _status_of_plan(replace(small, fp8_forward=True)) == nc.NC_OK
    assert _status_of_plan(replace(small, d_ff=1600, fp8_forward=True)) == nc.NC_ERR_UNSUPPORTED
    assert _status_of_plan(replace(small, d_ff=1600)) == nc.NC_OK
    # fp8 backward products reuse the forward's codes and sum tokens in steps of 128
    assert _status_of_plan(replace(small, fp8_forward=True, fp8_backward=True)) == nc.NC_OK
    assert _status_of_plan(replace(small, fp8_backward=True)) == nc.NC_ERR_UNSUPPORTED
    assert _status_of_plan(replace(small, seq_len=192, fp8_forward=True,
                                   fp8_backward=True)) == nc.NC_ERR_UNSUPPORTED
    _, a8b = nc.plan(replace(small, fp8_forward=True, fp8_backward=True))
    _, a8 = nc.plan(replace(small, fp8_forward=True))
    N, d, F = 4 * 128, 128, 1536            # the kept transposed codes: L [3d + F, N] bytes
    assert a8b - a8 >= 2 * N * (3 * d + F)
    o = OptimConfig(ns_coeffs=((1.0, 0.0, 0.0),) * 8)
    assert _status_of_plan(TINY, o) == nc.NC_OK
    c = nc.optim_cfg_c(o)
    c.ns_steps = 9
    m = nc.model_cfg_c(TINY)
    assert nc.load().nc_plan(ctypes.byref(m), ctypes.byref(c), None, None) == nc.NC_ERR_INVALID_ARG


def test_call_order_and_arena_errors_without_device():
    lib = nc.load()
    m, o = nc.model_cfg_c(TINY), nc.optim_cfg_c(OptimConfig())
    ctx = ctypes.c_void_p()
    assert lib.nc_create(ctypes.byref(m), ctypes.byref(o), ctypes.byref(ctx)) == nc.NC_OK
    try:
        fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every check fails first
        assert lib.nc_fwd_bwd(ctx, fake, fake, 1, 1.0, fake) == nc.NC_ERR_STATE
        assert lib.nc_optimizer_step(ctx, 1.0) == nc.NC_ERR_STATE
        assert lib.nc_zero_grads(ctx) == nc.NC_ERR_STATE
        assert lib.nc_bind(ctx, None, 0, None, 0, None) == nc.NC_ERR_INVALID_ARG
        assert lib.nc_bind(ctx, ctypes.c_void_p((1 << 20) + 4), 1 << 40, fake, 1 << 40, None) \
            == nc.NC_ERR_INVALID_ARG                      # misaligned
        assert lib.nc_bind(ctx, fake, 16, fake, 16, None) == nc.NC_ERR_OUT_OF_MEMORY
        assert b"arena too small" in lib.nc_last_error(ctx)
        assert lib.nc_status_str(nc.NC_ERR_STATE) == b"bad call order"
    finally:
        lib.nc_destroy(ctx)


SMALL_BF16 = dict(name="small", n_layer=2, d_model=384, n_head=3, head_dim=128, d_ff=1536,
                  vocab=4160, seq_len=256, micro_batch=2, accum_steps=1, dtype="bf16",
                  token_dist="zipf")


@pytest.mark.parametrize("name", ["tiny", "small", "d12", "d20", "d24", "d26", "small_gqa",
                                  "d20_gqa", "d26_gqa", "small_fp8", "d20_fp8", "d26_gqa_fp8",
                                  "tiny_feat", "small_feat", "d20_feat", "d20_gqa_feat",
                                  "small_fp8_feat", "small_fp8b", "d20_fp8b", "d26_gqa_fp8b",
                                  "small_fp8b_feat"])
def test_every_launch_of_a_step_stays_inside_the_arenas(name):
    """Dry run of nc_fwd_bwd + nc_optimizer_step: every GEMM operand extent is
    checked against the planned arenas (no device access)."""
    from dataclasses import replace as dc_replace
    from gpt_pretraining_step_gemms_amd.configs import ModelConfig
    base = name.replace("_gqa", "").replace("_fp8b", "").replace("_fp8", "").replace("_feat", "")
    cfg = ModelConfig(**SMALL_BF16) if base == "small" else CONFIGS[base]
    if "_gqa" in name:
        cfg = dc_replace(cfg, n_kv_head=1)
    if "_fp8" in name:
        cfg = dc_replace(cfg, fp8_forward=True, fp8_backward="_fp8b" in name)
    if "_feat" in name:
        cfg = dc_replace(cfg, value_embeds=True, resid_lambdas=True, smear=True, backout=True)
    lib = nc.load()
    for maxb, b in [(cfg.micro_batch, cfg.micro_batch), (cfg.micro_batch, 1), (1, 1)]:
        o = nc.optim_cfg_c(OptimConfig(normuon="_feat" not in name))
        m = nc.model_cfg_c(cfg, maxb)
        ctx = ctypes.c_void_p()
        assert lib.nc_create(ctypes.byref(m), ctypes.byref(o), ctypes.byref(ctx)) == nc.NC_OK
        try:
            s = lib.nc_validate_launches(ctx, b)
            assert s == nc.NC_OK, lib.nc_last_error(ctx)
        finally:
            lib.nc_destroy(ctx)


def test_parameter_registry_matches_model_shapes():
    lib = nc.load()
    cfg = from_depth(12, micro_batch=1, accum_steps=1)
    m, o = nc.model_cfg_c(cfg), nc.optim_cfg_c(OptimConfig())
    ctx = ctypes.c_void_p()
    assert lib.nc_create(ctypes.byref(m), ctypes.byref(o), ctypes.byref(ctx)) == nc.NC_OK
    try:
        n = ctypes.c_int32()
        lib.nc_param_count(ctx, ctypes.byref(n))
        infos = []
        for i in range(n.value):
            info = nc.ParamInfoC()
            assert lib.nc_param_desc(ctx, i, ctypes.byref(info)) == nc.NC_OK
            infos.append(info)
        shapes = {i.name.decode(): (i.rows, i.cols) for i in infos}
        assert shapes == param_shapes(cfg.as_oracle_cfg())
        pb, _ = nc.plan(cfg)
        spans = sorted((i.param_offset, i.param_offset + 4 * i.rows * i.cols) for i in infos)
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))   # no overlap
        assert spans[-1][1] <= pb
        groups = {i.name.decode(): i.group for i in infos}
        assert groups["E"] == groups["Wh"] == 0 and groups["3.W1"] == 1
        # Wq, Wk, Wv of a layer are adjacent rows of one [3d, d] matrix
        q, k, v = (infos[1 + j] for j in range(3))
        assert k.param_offset - q.param_offset == 4 * cfg.d_model ** 2
        assert v.param_offset - k.param_offset == 4 * cfg.d_model ** 2
        assert lib.nc_param_desc(ctx, n.value, ctypes.byref(nc.ParamInfoC())) == nc.NC_ERR_INVALID_ARG
        fb, opt = ctypes.c_double(), ctypes.c_double()
        lib.nc_flops(ctx, 32, ctypes.byref(fb), ctypes.byref(opt))
        L, d, V, T = 12, 768, 32768, 2048
        assert fb.value == pytest.approx(6 * 32 * T * (12 * L * d * d + V * d) + 6 * 32 * T * L * d * T)
    finally:
        lib.nc_destroy(ctx)


@pytest.mark.parametrize("n_kv,cg", [(0, 32), (2, 8), (1, 64)])
def test_feature_parameter_registry_matches_model_shapes(n_kv, cg):
    """Value embeddings, residual/x0 lambdas, smear and backout: the registry
    lists the oracle's parameters with its shapes, every span inside the
    parameter arena without overlap, the gates in the Muon group next to the
    block matrices and the tables and scalars in the AdamW group; the FLOP
    count of the products is that of the plain model."""
    from dataclasses import replace as dc_replace
    lib = nc.load()
    plain = dc_replace(from_depth(12, micro_batch=1, accum_steps=1), n_kv_head=n_kv)
    cfg = dc_replace(plain, value_embeds=True, resid_lambdas=True, smear=True, backout=True,
                     ve_gate_channels=cg)
    m, o = nc.model_cfg_c(cfg), nc.optim_cfg_c(OptimConfig())
    ctx = ctypes.c_void_p()
    assert lib.nc_create(ctypes.byref(m), ctypes.byref(o), ctypes.byref(ctx)) == nc.NC_OK
    try:
        n = ctypes.c_int32()
        lib.nc_param_count(ctx, ctypes.byref(n))
        infos = []
        for i in range(n.value):
            info = nc.ParamInfoC()
            assert lib.nc_param_desc(ctx, i, ctypes.byref(info)) == nc.NC_OK
            infos.append(info)
        shapes = {i.name.decode(): (i.rows, i.cols) for i in infos}
        assert shapes == param_shapes(cfg.as_oracle_cfg())
        assert shapes["11.Wg"] == (cfg.kv_heads, cg) and "10.Wg" not in shapes
        assert shapes["smear_gate"] == (1, 24) and shapes["resid_lambdas"] == (1, 12)
        pb, _ = nc.plan(cfg)
        spans = sorted((i.param_offset, i.param_offset + 4 * i.rows * i.cols) for i in infos)
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
        assert spans[-1][1] <= pb
        groups = {i.name.decode(): i.group for i in infos}
        for k, g in groups.items():
            adam = k in ("E", "Wh", "resid_lambdas", "x0_lambdas", "smear_lambda",
                         "backout_lambda") or k.startswith("ve.")
            assert g == (0 if adam else 1), (k, g)
        fb, opt = ctypes.c_double(), ctypes.c_double()
        lib.nc_flops(ctx, 1, ctypes.byref(fb), ctypes.byref(opt))
        mp = nc.model_cfg_c(plain)
        ctx2 = ctypes.c_void_p()
        assert lib.nc_create(ctypes.byref(mp), ctypes.byref(o), ctypes.byref(ctx2)) == nc.NC_OK
        fb2 = ctypes.c_double()
        lib.nc_flops(ctx2, 1, ctypes.byref(fb2), ctypes.byref(opt))
        lib.nc_destroy(ctx2)
        assert fb.value == fb2.value
    finally:
        lib.nc_destroy(ctx)
    bad = [(dict(ve_gate_channels=12), nc.NC_ERR_UNSUPPORTED),
           (dict(ve_gate_channels=72), nc.NC_ERR_UNSUPPORTED),
           (dict(ve_gate_channels=-8), nc.NC_ERR_INVALID_ARG)]
    for b, err in bad:
        mb = nc.model_cfg_c(dc_replace(cfg, **b))
        ctx = ctypes.c_void_p()
        assert lib.nc_create(ctypes.byref(mb), ctypes.byref(o), ctypes.byref(ctx)) == err
    # the NorMuon option does not cover the gate groups
    on = nc.optim_cfg_c(OptimConfig(normuon=True))
    ctx = ctypes.c_void_p()
    assert lib.nc_create(ctypes.byref(m), ctypes.byref(on), ctypes.byref(ctx)) != nc.NC_OK


def test_grouped_query_registry_and_flops():
    """n_kv_head < n_head: Wk, Wv narrower, the six matrices of a layer still
    contiguous (Wq | Wk | Wv form the fused QKV weight), FLOPs counted with
    the narrower products; n_kv_head must divide n_head."""
    from dataclasses import replace as dc_replace
    lib = nc.load()
    cfg = dc_replace(from_depth(12, micro_batch=1, accum_steps=1), n_kv_head=2)
    d, dk, F, L, V, T = 768, 256, 3072, 12, 32768, 2048
    m, o = nc.model_cfg_c(cfg), nc.optim_cfg_c(OptimConfig())
    ctx = ctypes.c_void_p()
    assert lib.nc_create(ctypes.byref(m), ctypes.byref(o), ctypes.byref(ctx)) == nc.NC_OK
    try:
        n = ctypes.c_int32()
        lib.nc_param_count(ctx, ctypes.byref(n))
        infos = []
        for i in range(n.value):
            info = nc.ParamInfoC()
            assert lib.nc_param_desc(ctx, i, ctypes.byref(info)) == nc.NC_OK
            infos.append(info)
        shapes = {i.name.decode(): (i.rows, i.cols) for i in infos}
        assert shapes == param_shapes(cfg.as_oracle_cfg())
        assert shapes["0.Wk"] == (dk, d) and shapes["0.Wv"] == (dk, d)
        layer = infos[1:7]
        for a, b in zip(layer, layer[1:]):
            assert b.param_offset == a.param_offset + 4 * a.rows * a.cols
        fb, opt = ctypes.c_double(), ctypes.c_double()
        lib.nc_flops(ctx, 1, ctypes.byref(fb), ctypes.byref(opt))
        per_tok = 6 * (L * (2 * d * d + 2 * dk * d + 2 * d * F) + V * d) + 6 * L * d * T
        assert fb.value == pytest.approx(T * per_tok)
        ns = 5 * L * (2 * (6 * d ** 3) + 2 * (4 * dk * dk * d + 2 * dk ** 3) +
                      2 * (4 * d * d * F + 2 * d ** 3))
        assert opt.value == pytest.approx(ns)
    finally:
        lib.nc_destroy(ctx)
    for bad in (4, 5, -1):           # 6 heads: 4 and 5 do not divide it
        mb = nc.model_cfg_c(dc_replace(cfg, n_kv_head=bad))
        ctx = ctypes.c_void_p()
        assert lib.nc_create(ctypes.byref(mb), ctypes.byref(o), ctypes.byref(ctx)) == nc.NC_ERR_INVALID_ARG


def test_attention_windows_set_and_counted_in_flops():
    """nc_set_attention_windows (host only): rejects entries below -1, and
    nc_flops counts a windowed layer at its mean number of visible keys."""
    import ctypes
    from gpt_pretraining_step_gemms_amd.configs import sliding_windows
    cfg = TINY
    lib = nc.load()
    m, o = nc.model_cfg_c(cfg), nc.optim_cfg_c(OptimConfig())
    ctx = ctypes.c_void_p()
    assert lib.nc_create(ctypes.byref(m), ctypes.byref(o), ctypes.byref(ctx)) == nc.NC_OK
    fb, opt = ctypes.c_double(), ctypes.c_double()

    def flops():
        assert lib.nc_flops(ctx, 2, ctypes.byref(fb), ctypes.byref(opt)) == nc.NC_OK
        return fb.value

    T, d, L = cfg.seq_len, cfg.d_model, cfg.n_layer
    causal = flops()
    Wn = (ctypes.c_int32 * L)
    assert lib.nc_set_attention_windows(ctx, Wn(-2, 3)) == nc.NC_ERR_INVALID_ARG
    assert flops() == causal
    w = 8
    assert lib.nc_set_attention_windows(ctx, Wn(w, -1)) == nc.NC_OK
    visible = sum(min(t, w) + 1 for t in range(T))          # pairs (t, u) with t-w <= u <= t
    expect = causal - 12.0 * 2 * T * d * (T / 2 - visible / T)
    assert flops() == pytest.approx(expect, rel=1e-12)
    assert lib.nc_set_attention_windows(ctx, Wn(T, 10 * T)) == nc.NC_OK
    assert flops() == causal                                 # windows past the row = causal
    assert lib.nc_set_attention_windows(ctx, Wn(w, -1)) == nc.NC_OK
    assert lib.nc_set_attention_windows(ctx, None) == nc.NC_OK
    assert flops() == causal
    assert sliding_windows(5, 64, "SSL") == [32, 32, -1, 32, 32]
    with pytest.raises(ValueError):
        sliding_windows(4, 64, "SXL")
    lib.nc_destroy(ctx)


def test_normuon_options_validated_and_planned():
    from dataclasses import replace as dc_replace
    base = OptimConfig()
    pb0, _ = nc.plan(TINY, base)
    pb1, _ = nc.plan(TINY, dc_replace(base, normuon=True))
    L, d, F = TINY.n_layer, TINY.d_model, TINY.d_ff
    assert pb1 >= pb0 + L * (5 * d + F) * 4          # one second-moment value per block row
    for beta2 in (-0.1, 1.0, float("nan")):
        with pytest.raises(nc.NcError):
            nc.plan(TINY, dc_replace(base, normuon=True, normuon_beta2=beta2))
    nc.plan(TINY, dc_replace(base, normuon=False, normuon_beta2=5.0))   # ignored when off


def test_op_argument_errors_return_before_any_launch():
    """The single-kernel entry points reject bad arguments synchronously,
    before touching the device (placeholder pointers are never dereferenced)."""
    lib = nc.load()
    fake = ctypes.c_void_p(0x100000)
    fp = ctypes.c_void_p(0x200000)
    BIG = 1 << 40
    # fp8 GEMM: format, epilogue, leading dimensions, K, split-K
    def g8(K, lda, ldb, ldc, epi, fmt=nc.FP8_E4M3, aux=None, splits=1, ws=None, ws_bytes=0):
        return lib.nc_op_gemm_fp8(fmt, fake, BIG, lda, fake, BIG, ldb, fake, BIG, ldc, 64, 64, K,
                                  epi, aux, BIG if aux else 0, 1.0, splits, ws, ws_bytes, None)
    assert g8(256, 256, 256, 64, nc.EPI_POLY) == nc.NC_ERR_INVALID_ARG
    assert g8(256, 256, 256, 64, nc.EPI_RELU2_BWD) == nc.NC_ERR_INVALID_ARG      # no aux_in
    assert g8(256, 256, 256, 64, nc.EPI_STORE, fmt=2) == nc.NC_ERR_INVALID_ARG
    assert g8(256, 128, 256, 64, nc.EPI_STORE) == nc.NC_ERR_INVALID_ARG
    assert g8(192, 192, 192, 64, nc.EPI_STORE) == nc.NC_ERR_UNSUPPORTED
    assert g8(256, 264, 256, 64, nc.EPI_STORE) == nc.NC_ERR_UNSUPPORTED
    assert g8(256, 256, 256, 64, nc.EPI_STORE, splits=2, ws=fp, ws_bytes=BIG) == nc.NC_ERR_INVALID_ARG
    assert g8(256, 256, 256, 64, nc.EPI_ACC_F32, splits=2) == nc.NC_ERR_INVALID_ARG   # no workspace
    assert g8(256, 256, 256, 64, nc.EPI_ACC_F32, splits=2, ws=fp,
              ws_bytes=2 * 64 * 64 * 4 - 4) == nc.NC_ERR_INVALID_ARG
    assert g8(256, 256, 256, 64, nc.EPI_STORE, splits=0) == nc.NC_ERR_INVALID_ARG
    assert lib.nc_op_gemm_fp8(0, None, BIG, 256, fake, BIG, 256, fake, BIG, 64, 64, 64, 256, 0,
                              None, 0, 1.0, 1, None, 0, None) == nc.NC_ERR_INVALID_ARG
    # fp8 quantiser: dtype, format, sizes, a destination, the transposed layout's limits
    def q(dt, rows, cols, ws, fmt=nc.FP8_E4M3, qd=fake, qt=None):
        return lib.nc_op_fp8_quantize(dt, fmt, fake, BIG, rows, cols, fp, 8, qd, BIG, qt,
                                      BIG if qt else 0, ws, 4096, None)
    assert q(nc.NC_FP32, 0, 16, fp) == nc.NC_ERR_INVALID_ARG
    assert q(nc.NC_FP32, 1, 0, fp) == nc.NC_ERR_INVALID_ARG
    assert q(7, 1, 16, fp) == nc.NC_ERR_INVALID_ARG
    assert q(nc.NC_FP32, 1, 16, None) == nc.NC_ERR_INVALID_ARG
    assert q(nc.NC_BF16, 1, 16, fp, fmt=3) == nc.NC_ERR_INVALID_ARG
    assert q(nc.NC_BF16, 64, 64, fp, qd=None) == nc.NC_ERR_INVALID_ARG            # no output
    assert q(nc.NC_FP32, 64, 64, fp, qt=fake) == nc.NC_ERR_UNSUPPORTED           # fp32, transposed
    assert q(nc.NC_BF16, 64, 96, fp, qt=fake) == nc.NC_ERR_UNSUPPORTED           # cols % 64
    assert q(nc.NC_BF16, 1 << 40, 1 << 40, fp) == nc.NC_ERR_INVALID_ARG          # size overflow
    # attention: key/value heads must divide the query heads; window >= -1; bf16 T % 128
    def fwd(H, hkv, win, T=256, dt=nc.NC_BF16):
        return lib.nc_op_attention_fwd(dt, fake, BIG, fake, BIG, fake, BIG, 3 * 128 * H, fake, BIG,
                                       128 * H, fp, BIG, 1, T, H, hkv, win, None)
    assert fwd(4, 3, -1) == nc.NC_ERR_INVALID_ARG
    assert fwd(4, 0, -1) == nc.NC_ERR_INVALID_ARG
    assert fwd(4, 2, -2) == nc.NC_ERR_INVALID_ARG
    assert fwd(4, 2, 10, T=200) == nc.NC_ERR_UNSUPPORTED
    assert lib.nc_op_attention_bwd(nc.NC_BF16, fake, BIG, fake, BIG, fake, BIG, 384, fake, BIG,
                                   fake, BIG, 128, fp, BIG, fp, BIG, fake, BIG, fake, BIG, fake,
                                   BIG, 384, 1, 256, 1, 1, -3, None) == nc.NC_ERR_INVALID_ARG


def test_op_operand_extents_are_checked_before_any_launch():
    """Every op entry point takes the bytes owned behind each operand and
    refuses a layout that reaches past them, before any launch.  One case is
    the layout mistake of a grouped-query buffer read with the full-width
    strides (v at column 2 d, row stride 3 d): it must be refused."""
    lib = nc.load()
    fake = ctypes.c_void_p(0x100000)
    BIG = 1 << 40
    B, T, H, hkv = 32, 2048, 10, 2
    d, dk = H * 128, hkv * 128
    rows = B * T
    qkv_bytes = rows * (d + 2 * dk) * 2            # the grouped-query buffer
    # right layout: q at 0, k at d, v at d + dk, stride d + 2 dk
    def fwd(v_bytes, ld, o_bytes=BIG, lse_bytes=B * H * T * 4):
        return lib.nc_op_attention_fwd(nc.NC_BF16, fake, qkv_bytes, fake, qkv_bytes - d * 2, fake,
                                       v_bytes, ld, fake, o_bytes, d, fake, lse_bytes, B, T, H,
                                       hkv, -1, None)
    good_ld = d + 2 * dk
    assert fwd(qkv_bytes - (d + dk) * 2, 3 * d) == nc.NC_ERR_INVALID_ARG   # full-width stride
    assert fwd(qkv_bytes - 2 * d * 2, 3 * d) == nc.NC_ERR_INVALID_ARG      # and v at 2 d
    assert fwd(qkv_bytes - (d + dk) * 2, good_ld, o_bytes=rows * d * 2 - 2) == nc.NC_ERR_INVALID_ARG
    assert fwd(qkv_bytes - (d + dk) * 2, good_ld, lse_bytes=B * H * T * 4 - 4) == nc.NC_ERR_INVALID_ARG
    assert fwd(qkv_bytes - (d + dk) * 2, d - 8) == nc.NC_ERR_INVALID_ARG   # rows overlap
    # backward: every one of the ten operands is checked
    # exactly the bytes each one needs: ((rows - 1) ld + heads 128) elements
    need_q, need_kv = ((rows - 1) * good_ld + d) * 2, ((rows - 1) * good_ld + dk) * 2
    ext = dict(q=need_q, k=need_kv, v=need_kv, o=rows * d * 2, dO=rows * d * 2,
               lse=B * H * T * 4, D=2 * B * H * T * 4, dq=need_q, dk=need_kv, dv=need_kv)
    def bwd(**short):
        e = {k: v - short.get(k, 0) for k, v in ext.items()}
        return lib.nc_op_attention_bwd(nc.NC_BF16, fake, e["q"], fake, e["k"], fake, e["v"], good_ld,
                                       fake, e["o"], fake, e["dO"], d, fake, e["lse"], fake, e["D"],
                                       fake, e["dq"], fake, e["dk"], fake, e["dv"], good_ld, B, T, H,
                                       hkv, -1, None)
    for name in ext:
        assert bwd(**{name: 2}) == nc.NC_ERR_INVALID_ARG, name
    # GEMM: A K-contiguous [M, K] needs ((M - 1) lda + K) elements; batch strides count
    M, N, K = 300, 200, 256
    def gemm(a_bytes=BIG, c_bytes=BIG, lda=K, batch=1, sA=0, epi=nc.EPI_STORE_F32, aux=0,
             ws_bytes=0, splits=1):
        return lib.nc_op_gemm(nc.NC_BF16, fake, a_bytes, lda, 0, fake, BIG, K, 0, fake, c_bytes, N,
                              M, N, K, batch, sA, 0, 0, epi, fake if aux else None, aux,
                              fake if aux else None, aux, 1.0, 0.0, 0.0, splits,
                              fake if ws_bytes else None, ws_bytes, None)
    need_a = ((M - 1) * K + K) * 2
    assert gemm(a_bytes=need_a - 2) == nc.NC_ERR_INVALID_ARG
    assert gemm(a_bytes=need_a, batch=2, sA=M * K) == nc.NC_ERR_INVALID_ARG
    assert gemm(c_bytes=M * N * 4 - 4) == nc.NC_ERR_INVALID_ARG         # fp32 output
    assert gemm(lda=K - 8) == nc.NC_ERR_INVALID_ARG
    assert gemm(epi=nc.EPI_RELU2_BWD, aux=M * N * 2 - 2) == nc.NC_ERR_INVALID_ARG
    assert gemm(splits=4, ws_bytes=4 * M * N * 4 - 4) == nc.NC_ERR_INVALID_ARG
    # epilogue 7 (the QKV product's QK-norm + rotary) is the step's own, not an op's
    assert gemm(epi=7) == nc.NC_ERR_INVALID_ARG
    assert lib.nc_op_gemm_noalloc(nc.NC_BF16, fake, BIG, K, 0, fake, BIG, K, 0, fake, BIG, N, M, N,
                                  K, 1, 0, 0, 0, 7, None, 0, None, 0, 1.0, 0.0, 0.0, 1,
                                  None) == nc.NC_ERR_INVALID_ARG
    # fp8 GEMM and quantiser
    g8 = lambda a_bytes=BIG, c_bytes=BIG, epi=nc.EPI_STORE, aux=None, aux_bytes=0: \
        lib.nc_op_gemm_fp8(0, fake, a_bytes, 256, fake, BIG, 256, fake, c_bytes, 64, 64, 64, 256,
                           epi, aux, aux_bytes, 1.0, 1, None, 0, None)
    assert g8(a_bytes=64 * 256 - 1) == nc.NC_ERR_INVALID_ARG
    assert g8(c_bytes=64 * 64 * 4 - 4, epi=nc.EPI_STORE_F32) == nc.NC_ERR_INVALID_ARG
    assert g8(epi=nc.EPI_RELU2_BWD, aux=fake, aux_bytes=64 * 64 * 2 - 2) == nc.NC_ERR_INVALID_ARG
    assert g8(epi=7) == nc.NC_ERR_INVALID_ARG
    qz = lambda xb, qb, ab=8, wb=4096, qtb=0: lib.nc_op_fp8_quantize(
        nc.NC_BF16, 0, fake, xb, 1000, 1, fake, ab, fake, qb, fake if qtb else None, qtb, fake, wb,
        None)
    assert qz(1999, BIG) == nc.NC_ERR_INVALID_ARG
    assert qz(BIG, 999) == nc.NC_ERR_INVALID_ARG
    assert qz(BIG, BIG, ab=4) == nc.NC_ERR_INVALID_ARG
    assert qz(BIG, BIG, wb=4092) == nc.NC_ERR_INVALID_ARG
    assert qz(BIG, BIG, qtb=999) == nc.NC_ERR_INVALID_ARG
