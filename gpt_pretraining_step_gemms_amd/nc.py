"""ctypes binding of libncgpt.so (include/nc.h, include/nc_ops.h).

Argument marshalling only: every step of the forward/backward pass and of the
optimizer runs in the library's HIP kernels.  torch provides the device
memory (two uint8 arenas) and the stream; torch is imported first so the
library binds to the HIP runtime torch already loaded.
"""

import ctypes
import os

import numpy as np
import torch  # noqa: F401  (loads the HIP runtime the library links against)

from .configs import ModelConfig, OptimConfig

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libncgpt.so")
_lib = None

NC_OK, NC_ERR_INVALID_ARG, NC_ERR_UNSUPPORTED, NC_ERR_OUT_OF_MEMORY = 0, 1, 2, 3
NC_ERR_HIP, NC_ERR_STATE, NC_ERR_NONFINITE = 4, 5, 6
NC_FP32, NC_BF16 = 0, 1
NC_PARAM, NC_GRAD, NC_MOMENTUM, NC_ADAM_M, NC_ADAM_V = 0, 1, 2, 3, 4
NC_K_CONTIGUOUS, NC_MN_CONTIGUOUS = 0, 1
NC_FEAT_VALUE_EMBEDS, NC_FEAT_RESID_LAMBDAS, NC_FEAT_SMEAR, NC_FEAT_BACKOUT = 1, 2, 4, 8
FP8_E4M3, FP8_E5M2 = 0, 1
EPI_STORE, EPI_STORE_F32, EPI_ACC_F32, EPI_RELU2, EPI_RELU2_BWD, EPI_POLY, EPI_DUAL = range(7)


class NcError(RuntimeError):
    def __init__(self, status, msg=""):
        super().__init__(f"nc status {status}: {msg}")
        self.status = status


class ModelCfgC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layer", "d_model", "n_head", "head_dim", "d_ff", "vocab", "seq_len",
                 "max_micro_batch", "dtype")] + [("rope_base", ctypes.c_float),
                                                 ("norm_eps", ctypes.c_float),
                                                 ("n_kv_head", ctypes.c_int32),
                                                 ("fp8_forward", ctypes.c_int32),
                                                 ("features", ctypes.c_int32),
                                                 ("ve_gate_channels", ctypes.c_int32),
                                                 ("fp8_backward", ctypes.c_int32)]


class OptimCfgC(ctypes.Structure):
    _fields_ = [("muon_lr", ctypes.c_float), ("muon_momentum", ctypes.c_float),
                ("muon_wd", ctypes.c_float), ("ns_eps", ctypes.c_float),
                ("ns_steps", ctypes.c_int32), ("muon_nesterov", ctypes.c_int32),
                ("ns_coeffs", (ctypes.c_float * 3) * 8),
                ("adam_lr_embed", ctypes.c_float), ("adam_lr_head", ctypes.c_float),
                ("adam_beta1", ctypes.c_float), ("adam_beta2", ctypes.c_float),
                ("adam_eps", ctypes.c_float), ("adam_wd", ctypes.c_float),
                ("normuon", ctypes.c_int32), ("normuon_beta2", ctypes.c_float),
                ("adam_lr_scalar", ctypes.c_float)]


class ParamInfoC(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("group", ctypes.c_int32), ("param_offset", ctypes.c_int64),
                ("grad_offset", ctypes.c_int64), ("state0_offset", ctypes.c_int64),
                ("state1_offset", ctypes.c_int64)]


def lib_path():
    return _LIB_PATH


def load():
    """Loads libncgpt.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: run __graft_entry__.build() "
                          "(python -m gpt_pretraining_step_gemms_amd.build) first")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "nc_plan": [ctypes.POINTER(ModelCfgC), ctypes.POINTER(OptimCfgC),
                    ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
        "nc_create": [ctypes.POINTER(ModelCfgC), ctypes.POINTER(OptimCfgC), ctypes.POINTER(P)],
        "nc_bind": [P, P, SZ, P, SZ, P],
        "nc_init_params": [P, ctypes.c_uint64, F32],
        "nc_zero_grads": [P],
        "nc_set_attention_windows": [P, P],
        "nc_fwd_bwd": [P, P, P, I32, F32, P],
        "nc_optimizer_step": [P, F32],
        "nc_param_count": [P, ctypes.POINTER(I32)],
        "nc_param_desc": [P, I32, ctypes.POINTER(ParamInfoC)],
        "nc_set_param": [P, I32, P, I32],
        "nc_get_tensor": [P, I32, I32, P, I32],
        "nc_check_finite": [P, ctypes.POINTER(I32)],
        "nc_check_inputs": [P, ctypes.POINTER(I32)],
        "nc_validate_launches": [P, I32],
        "nc_flops": [P, I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)],
        "nc_op_gemm": [I32, P, SZ, I64, I32, P, SZ, I64, I32, P, SZ, I64, I32, I32, I32, I32,
                       I64, I64, I64, I32, P, SZ, P, SZ, F32, F32, F32, I32, P, SZ, P],
        "nc_op_gemm_noalloc": [I32, P, SZ, I64, I32, P, SZ, I64, I32, P, SZ, I64, I32, I32, I32,
                               I32, I64, I64, I64, I32, P, SZ, P, SZ, F32, F32, F32, I32, P],
        "nc_op_gemm_fp8": [I32, P, SZ, I64, P, SZ, I64, P, SZ, I64, I32, I32, I32, I32, P, SZ,
                           F32, I32, P, SZ, P],
        "nc_op_fp8_quantize": [I32, I32, P, SZ, I64, I64, P, SZ, P, SZ, P, SZ, P, SZ, P],
        "nc_op_attention_fwd": [I32, P, SZ, P, SZ, P, SZ, I64, P, SZ, I64, P, SZ, I32, I32, I32,
                                I32, I32, P],
        "nc_op_attention_bwd": [I32, P, SZ, P, SZ, P, SZ, I64, P, SZ, P, SZ, I64, P, SZ, P, SZ,
                                P, SZ, P, SZ, P, SZ, I64, I32, I32, I32, I32, I32, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.nc_status_str.argtypes = [ctypes.c_int]
    lib.nc_status_str.restype = ctypes.c_char_p
    lib.nc_last_error.argtypes = [P]
    lib.nc_last_error.restype = ctypes.c_char_p
    lib.nc_destroy.argtypes = [P]
    lib.nc_destroy.restype = None
    _lib = lib
    return lib


def model_cfg_c(cfg: ModelConfig, max_micro_batch=None):
    return ModelCfgC(cfg.n_layer, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.d_ff, cfg.vocab,
                     cfg.seq_len, max_micro_batch or cfg.micro_batch,
                     NC_BF16 if cfg.dtype == "bf16" else NC_FP32, cfg.rope_base, cfg.norm_eps,
                     cfg.n_kv_head, int(bool(cfg.fp8_forward)), features_of(cfg),
                     cfg.ve_gate_channels, int(bool(cfg.fp8_backward)))


def features_of(cfg: ModelConfig):
    return ((NC_FEAT_VALUE_EMBEDS if cfg.value_embeds else 0) |
            (NC_FEAT_RESID_LAMBDAS if cfg.resid_lambdas else 0) |
            (NC_FEAT_SMEAR if cfg.smear else 0) | (NC_FEAT_BACKOUT if cfg.backout else 0))


def optim_cfg_c(o: OptimConfig):
    c = OptimCfgC()
    c.muon_lr, c.muon_momentum, c.muon_wd, c.ns_eps = o.muon_lr, o.muon_momentum, o.muon_wd, o.ns_eps
    coeffs = list(o.ns_coeffs)
    if len(coeffs) > 8:
        raise ValueError("at most 8 Newton-Schulz iterations")
    c.ns_steps = len(coeffs)
    c.muon_nesterov = int(bool(o.muon_nesterov))
    for i, (a, b, cc) in enumerate(coeffs):
        c.ns_coeffs[i][0], c.ns_coeffs[i][1], c.ns_coeffs[i][2] = a, b, cc
    c.adam_lr_embed, c.adam_lr_head = o.adam_lr_embed, o.adam_lr_head
    c.adam_beta1, c.adam_beta2, c.adam_eps, c.adam_wd = o.adam_beta1, o.adam_beta2, o.adam_eps, o.adam_wd
    c.normuon, c.normuon_beta2 = int(bool(o.normuon)), o.normuon_beta2
    c.adam_lr_scalar = o.adam_lr_scalar
    return c


def _check(status, ctx=None, what=""):
    if status != NC_OK:
        lib = load()
        msg = lib.nc_last_error(ctx).decode() if ctx else ""
        raise NcError(status, f"{what}: {lib.nc_status_str(status).decode()} {msg}")


def plan(cfg: ModelConfig, ocfg: OptimConfig = OptimConfig(), max_micro_batch=None):
    lib = load()
    pb, ab = ctypes.c_size_t(), ctypes.c_size_t()
    m, o = model_cfg_c(cfg, max_micro_batch), optim_cfg_c(ocfg)
    _check(lib.nc_plan(ctypes.byref(m), ctypes.byref(o), ctypes.byref(pb), ctypes.byref(ab)),
           what="nc_plan")
    return pb.value, ab.value


def _ptr(t):
    return ctypes.c_void_p(None if t is None else t.data_ptr())


class Model:
    """One GPT (weights, gradients, optimizer state) bound to torch-owned arenas."""

    def __init__(self, cfg: ModelConfig, ocfg: OptimConfig = OptimConfig(), max_micro_batch=None,
                 device="cuda"):
        self.lib = load()
        self.cfg, self.ocfg = cfg, ocfg
        self.max_b = max_micro_batch or cfg.micro_batch
        self._m, self._o = model_cfg_c(cfg, self.max_b), optim_cfg_c(ocfg)
        self.ctx = ctypes.c_void_p()
        _check(self.lib.nc_create(ctypes.byref(self._m), ctypes.byref(self._o), ctypes.byref(self.ctx)),
               what="nc_create")
        pb, ab = plan(cfg, ocfg, self.max_b)
        self.param_bytes, self.act_bytes = pb, ab
        self.device = torch.device(device)
        self.param_arena = torch.empty(pb, dtype=torch.uint8, device=self.device)
        self.act_arena = torch.empty(ab, dtype=torch.uint8, device=self.device)
        self.stream = torch.cuda.current_stream(self.device)
        _check(self.lib.nc_bind(self.ctx, _ptr(self.param_arena), pb, _ptr(self.act_arena), ab,
                                ctypes.c_void_p(self.stream.cuda_stream)), self.ctx, "nc_bind")
        n = ctypes.c_int32()
        _check(self.lib.nc_param_count(self.ctx, ctypes.byref(n)), self.ctx)
        self.params = []
        for i in range(n.value):
            info = ParamInfoC()
            _check(self.lib.nc_param_desc(self.ctx, i, ctypes.byref(info)), self.ctx)
            self.params.append(info)
        self.index = {p.name.decode(): i for i, p in enumerate(self.params)}
        self.loss = torch.zeros(1, dtype=torch.float32, device=self.device)

    # ----------------------------------------------------------- tensors
    def _view(self, off, info):
        n = info.rows * info.cols
        return self.param_arena[off:off + 4 * n].view(torch.float32).view(info.rows, info.cols)

    def param(self, name):
        """Zero-copy fp32 view of a parameter's master weights."""
        info = self.params[self.index[name]]
        return self._view(info.param_offset, info)

    def grad(self, name):
        info = self.params[self.index[name]]
        return self._view(info.grad_offset, info)

    def names(self):
        return list(self.index)

    def shapes(self):
        return {p.name.decode(): (p.rows, p.cols) for p in self.params}

    def set_params(self, arrays):
        for name, a in arrays.items():
            a = np.ascontiguousarray(a, dtype=np.float32)
            info = self.params[self.index[name]]
            assert a.shape == (info.rows, info.cols), (name, a.shape)
            _check(self.lib.nc_set_param(self.ctx, self.index[name],
                                         a.ctypes.data_as(ctypes.c_void_p), 0), self.ctx, name)

    def get(self, name, which=NC_PARAM):
        info = self.params[self.index[name]]
        out = np.empty((info.rows, info.cols), dtype=np.float32)
        _check(self.lib.nc_get_tensor(self.ctx, self.index[name], which,
                                      out.ctypes.data_as(ctypes.c_void_p), 0), self.ctx, name)
        return out

    # ---------------------------------------------------------------- step
    def init_params(self, seed, std=0.02):
        _check(self.lib.nc_init_params(self.ctx, seed, std), self.ctx, "init")

    def set_attention_windows(self, windows):
        """Per-layer attention window (None or -1: plain causal); None for all
        layers plain causal."""
        if windows is None:
            _check(self.lib.nc_set_attention_windows(self.ctx, None), self.ctx, "windows")
            return
        assert len(windows) == self.cfg.n_layer
        arr = (ctypes.c_int32 * len(windows))(*[-1 if w is None else int(w) for w in windows])
        _check(self.lib.nc_set_attention_windows(self.ctx, arr), self.ctx, "windows")

    def zero_grads(self):
        _check(self.lib.nc_zero_grads(self.ctx), self.ctx, "zero_grads")

    def fwd_bwd(self, tokens, targets, grad_scale=1.0, loss_out=None):
        """tokens, targets: int32 device tensors [B, seq_len].  Returns the device
        loss tensor (mean cross-entropy of this micro-batch)."""
        assert tokens.dtype == torch.int32 and targets.dtype == torch.int32
        assert tokens.is_contiguous() and targets.is_contiguous()
        B = tokens.shape[0]
        out = self.loss if loss_out is None else loss_out
        _check(self.lib.nc_fwd_bwd(self.ctx, _ptr(tokens), _ptr(targets), B, grad_scale, _ptr(out)),
               self.ctx, "fwd_bwd")
        return out

    def optimizer_step(self, lr_mult=1.0):
        _check(self.lib.nc_optimizer_step(self.ctx, lr_mult), self.ctx, "optimizer_step")

    def check_finite(self):
        flag = ctypes.c_int32()
        s = self.lib.nc_check_finite(self.ctx, ctypes.byref(flag))
        if s not in (NC_OK, NC_ERR_NONFINITE):
            _check(s, self.ctx, "check_finite")
        return flag.value == 0

    def check_inputs(self):
        """(ok, flags): whether every token and target id since the last call
        was in [0, vocab); flags bit 0 = a bad token id, bit 1 = a bad target."""
        flag = ctypes.c_int32()
        s = self.lib.nc_check_inputs(self.ctx, ctypes.byref(flag))
        if s not in (NC_OK, NC_ERR_INVALID_ARG):
            _check(s, self.ctx, "check_inputs")
        return flag.value == 0, flag.value

    def flops(self, B=None):
        fb, opt = ctypes.c_double(), ctypes.c_double()
        _check(self.lib.nc_flops(self.ctx, B or self.max_b, ctypes.byref(fb), ctypes.byref(opt)),
               self.ctx)
        return fb.value, opt.value

    def close(self):
        if self.ctx:
            self.lib.nc_destroy(self.ctx)
            self.ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------ single ops
def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return NC_BF16
    if t.dtype == torch.float32:
        return NC_FP32
    raise TypeError(t.dtype)


def extent(t):
    """Bytes of device memory the caller owns from t's first element to the
    end of its storage (what the op entry points check layouts against)."""
    if t is None:
        return 0
    st = t.untyped_storage()
    return st.nbytes() - (t.data_ptr() - st.data_ptr())


def _opt(t):
    return (_ptr(t), extent(t)) if t is not None else (None, 0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def gemm(A, a_layout, B, b_layout, C, M, N, K, epilogue=EPI_STORE, aux_in=None, aux_out=None,
         alpha=1.0, p0=0.0, p1=0.0, lda=None, ldb=None, ldc=None, batch=1, sA=0, sB=0, sC=0,
         splits=1, workspace=None, dtype=None):
    lib = load()
    dt = dtype if dtype is not None else _dtype_code(A)
    lda = lda if lda is not None else A.shape[-1]
    ldb = ldb if ldb is not None else B.shape[-1]
    ldc = ldc if ldc is not None else C.shape[-1]
    ai, ao, ws = _opt(aux_in), _opt(aux_out), _opt(workspace)
    s = lib.nc_op_gemm(dt, _ptr(A), extent(A), lda, a_layout, _ptr(B), extent(B), ldb, b_layout,
                       _ptr(C), extent(C), ldc, M, N, K, batch, sA, sB, sC, epilogue, ai[0], ai[1],
                       ao[0], ao[1], alpha, p0, p1, splits, ws[0], ws[1], _stream())
    _check(s, what="nc_op_gemm")


def gemm_noalloc(A, a_layout, B, b_layout, C, M, N, K, epilogue=EPI_STORE, aux_in=None,
                 aux_out=None, alpha=1.0, p0=0.0, p1=0.0, lda=None, ldb=None, ldc=None, batch=1,
                 sA=0, sB=0, sC=0, splits=1, dtype=None):
    """gemm() through nc_op_gemm_noalloc: split-K partials in the library's
    fixed device scratch instead of a caller workspace."""
    lib = load()
    dt = dtype if dtype is not None else _dtype_code(A)
    lda = lda if lda is not None else A.shape[-1]
    ldb = ldb if ldb is not None else B.shape[-1]
    ldc = ldc if ldc is not None else C.shape[-1]
    ai, ao = _opt(aux_in), _opt(aux_out)
    s = lib.nc_op_gemm_noalloc(dt, _ptr(A), extent(A), lda, a_layout, _ptr(B), extent(B), ldb,
                               b_layout, _ptr(C), extent(C), ldc, M, N, K, batch, sA, sB, sC,
                               epilogue, ai[0], ai[1], ao[0], ao[1], alpha, p0, p1, splits,
                               _stream())
    _check(s, what="nc_op_gemm_noalloc")


def attention_fwd(q, k, v, o, lse, B, T, H, ld_qkv, ld_o, window=-1, n_kv_head=None):
    lib = load()
    s = lib.nc_op_attention_fwd(_dtype_code(q), _ptr(q), extent(q), _ptr(k), extent(k), _ptr(v),
                                extent(v), ld_qkv, _ptr(o), extent(o), ld_o, _ptr(lse),
                                extent(lse), B, T, H, n_kv_head or H, window, _stream())
    _check(s, what="nc_op_attention_fwd")


def attention_bwd(q, k, v, o, dO, lse, D, dq, dk, dv, B, T, H, ld_qkv, ld_o, ld_d, window=-1,
                  n_kv_head=None):
    lib = load()
    s = lib.nc_op_attention_bwd(_dtype_code(q), _ptr(q), extent(q), _ptr(k), extent(k), _ptr(v),
                                extent(v), ld_qkv, _ptr(o), extent(o), _ptr(dO), extent(dO), ld_o,
                                _ptr(lse), extent(lse), _ptr(D), extent(D), _ptr(dq), extent(dq),
                                _ptr(dk), extent(dk), _ptr(dv), extent(dv), ld_d, B, T, H,
                                n_kv_head or H, window, _stream())
    _check(s, what="nc_op_attention_bwd")


def gemm_fp8(A8, B8, C, M, N, K, alpha, epilogue=EPI_STORE, lda=None, ldb=None, ldc=None,
             a_format=FP8_E4M3, aux_in=None, splits=1, workspace=None):
    """C = alpha * A8 B8^T for K-contiguous uint8 fp8 operands (A e4m3 or e5m2,
    B e4m3)."""
    lib = load()
    s = lib.nc_op_gemm_fp8(a_format, _ptr(A8), extent(A8), lda or A8.shape[-1], _ptr(B8),
                           extent(B8), ldb or B8.shape[-1], _ptr(C), extent(C),
                           ldc or C.shape[-1], M, N, K, epilogue, _ptr(aux_in), extent(aux_in),
                           alpha, splits, _ptr(workspace), extent(workspace), _stream())
    _check(s, what="nc_op_gemm_fp8")


def fp8_quantize(x, q, amax_scale, workspace, fmt=FP8_E4M3, qt=None, rows=None, cols=None):
    """Tensorwise fp8 codes of x [rows, cols] (default: one row of x.numel()):
    q in x's layout and/or qt transposed; amax_scale (2 floats) = amax, scale."""
    lib = load()
    if rows is None:
        rows, cols = (1, x.numel()) if qt is None else (x.shape[0], x.numel() // x.shape[0])
    s = lib.nc_op_fp8_quantize(_dtype_code(x), fmt, _ptr(x), extent(x), rows, cols,
                               _ptr(amax_scale), extent(amax_scale), _ptr(q), extent(q),
                               _ptr(qt), extent(qt), _ptr(workspace), extent(workspace),
                               _stream())
    _check(s, what="nc_op_fp8_quantize")
