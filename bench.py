"""Training-step throughput of the GPT pretraining step on one MI355X.

A step is: zero the gradients, K accumulated micro-batches of forward +
backward (nc_fwd_bwd), one optimizer step (AdamW + Muon).  Workload: the d20
model (20 layers, width 1280, 10 heads of 128, MLP 5120, vocabulary 32768,
sequence 2048), micro-batch 32 rows, 8 micro-batches = 524,288 tokens per
step, Zipf(1.1) synthetic token ids, N(0, 0.02^2) weights, bf16 matrix-core
inputs with fp32 master weights and accumulation.

Prints one JSON line: tokens/s, MFU against the bf16 dense MFMA peak, the
roofline of the dominant kernel (the bf16 GEMM at the MLP up-projection
shape, timed with HIP events on its stream) and the CPU oracle's throughput
on a bounded sample.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15          # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12           # MI355X HBM3E, B/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="d20")
    ap.add_argument("--micro-batch", type=int, default=None)
    ap.add_argument("--accum", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--window-pattern", default=None,
                    help='sliding-window attention pattern over the layers, e.g. "SSSL" '
                         '(S: short window, L: whole causal context); default: none')
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="key/value heads for grouped-query attention (default: one per head)")
    ap.add_argument("--fp8-forward", action="store_true",
                    help="forward block products in fp8 e4m3 (tensorwise scales; backward bf16)")
    ap.add_argument("--fp8-backward", action="store_true",
                    help="with --fp8-forward: the backward block products in fp8 too "
                         "(gradients e5m2)")
    ap.add_argument("--model-features", default="",
                    help='comma list of the further model mechanisms: ve (value embeddings), '
                         'resid (residual/x0 lambdas), smear, backout; or "all"')
    ap.add_argument("--normuon", action="store_true",
                    help="NorMuon per-neuron normalisation after Newton-Schulz")
    ap.add_argument("--short-window", type=int, default=None,
                    help="keys before the query in an S layer (default seq_len / 2)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the dominant-kernel timing loop (for profiling it alone)")
    ap.add_argument("--roofline-iters", type=int, default=20)
    ap.add_argument("--roofline-fp8", action="store_true",
                    help="only the fp8 GEMM at the MLP up-projection shape (tensorwise e4m3)")
    ap.add_argument("--attention-only", action="store_true",
                    help="only the bf16 attention forward and backward of one layer and "
                         "micro-batch (the op entry points, 3 warm-up + --roofline-iters calls)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --roofline-only: also run a 1 GiB copy kernel (counter scale)")
    return ap.parse_args()


def roofline_gemm(cfg, iters):
    """bf16 MFMA GEMM at the MLP up-projection shape of one micro-batch:
    [B*T, d] x [F, d]^T with the ReLU^2 epilogue (g = max(h, 0)^2 in bf16)."""
    import torch
    from gpt_pretraining_step_gemms_amd import nc
    M, N, K = cfg.micro_batch * cfg.seq_len, cfg.d_ff, cfg.d_model
    A = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    B = (0.02 * torch.randn(N, K, device="cuda")).to(torch.bfloat16)
    G = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        nc.gemm(A, 0, B, 0, G, M, N, K, nc.EPI_RELU2)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(iters):
        nc.gemm(A, 0, B, 0, G, M, N, K, nc.EPI_RELU2)
    t1.record(stream)
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) / 1e3 / iters
    flops = 2.0 * M * N * K
    return {"kernel": "gemm_bf16_pipe_kernel<KCont, KCont> (MLP up + ReLU^2 epilogue)",
            "shape": [M, N, K], "avg_launch_us": sec * 1e6,
            "bound": "mfma", "achieved": flops / sec / 1e12, "peak": PEAK_BF16 / 1e12,
            "unit": "TFLOP/s", "frac": flops / sec / PEAK_BF16,
            "traffic": measured_traffic(2 * (M * K + N * K + M * N))}


def attention_only(cfg, iters):
    """bf16 causal attention of one layer and micro-batch ([B*T, 3d] token-major
    q | k | v, head dim 128) through the op entry points: the forward, then the
    backward (dQ kernel, then dK/dV kernel), each timed with HIP events on the
    launch stream.  FLOPs are the algorithmic causal counts, 2 N T d (forward)
    and 5 N T d (backward)."""
    import torch
    from gpt_pretraining_step_gemms_amd import nc
    B, T, H = cfg.micro_batch, cfg.seq_len, cfg.n_head
    d = H * 128
    g = torch.Generator(device="cuda").manual_seed(5)
    qkv = torch.randn(B * T, 3 * d, device="cuda", generator=g).to(torch.bfloat16)
    dO = (1e-3 * torch.randn(B * T, d, device="cuda", generator=g)).to(torch.bfloat16)
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    o = torch.empty(B * T, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, T, dtype=torch.float32, device="cuda")
    dqkv = torch.empty_like(qkv)
    D = torch.empty(2, B, H, T, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fwd = lambda: nc.attention_fwd(q, k, v, o, lse, B, T, H, 3 * d, d)
    bwd = lambda: nc.attention_bwd(q, k, v, o, dO, lse, D, dqkv[:, :d], dqkv[:, d:2 * d],
                                   dqkv[:, 2 * d:], B, T, H, 3 * d, d, 3 * d)
    out = {"shape": {"B": B, "T": T, "H": H, "head_dim": 128}}
    N = B * T
    for name, f, flops in (("forward", fwd, 2.0 * N * T * d), ("backward", bwd, 5.0 * N * T * d)):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(iters):
            f()
        t1.record(stream)
        torch.cuda.synchronize()
        sec = t0.elapsed_time(t1) / 1e3 / iters
        out[name] = {"avg_call_us": sec * 1e6, "achieved_tflops": flops / sec / 1e12,
                     "frac": flops / sec / PEAK_BF16}
    return out


PEAK_FP8 = 5.0e15           # MI355X dense fp8 MFMA, FLOP/s


def roofline_gemm_fp8(cfg, iters):
    """fp8 e4m3 GEMM at the MLP up-projection shape of one micro-batch, both
    operands quantised with one scale per tensor, bf16 output."""
    import torch
    from gpt_pretraining_step_gemms_amd import nc
    M, N, K = cfg.micro_batch * cfg.seq_len, cfg.d_ff, cfg.d_model
    A = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    B = (0.02 * torch.randn(N, K, device="cuda")).to(torch.bfloat16)
    A8 = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    B8 = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    sa = torch.empty(2, device="cuda")
    sb = torch.empty(2, device="cuda")
    ws = torch.empty(1024, device="cuda")
    nc.fp8_quantize(A, A8, sa, ws)
    nc.fp8_quantize(B, B8, sb, ws)
    alpha = 1.0 / (sa[1].item() * sb[1].item())
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        nc.gemm_fp8(A8, B8, C, M, N, K, alpha)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(iters):
        nc.gemm_fp8(A8, B8, C, M, N, K, alpha)
    t1.record(stream)
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) / 1e3 / iters
    flops = 2.0 * M * N * K
    return {"kernel": "gemm_bf16_pipe_kernel<KCont, KCont, ..., fp8> (e4m3, bf16 output)",
            "shape": [M, N, K], "avg_launch_us": sec * 1e6, "bound": "mfma",
            "achieved": flops / sec / 1e12, "peak": PEAK_FP8 / 1e12, "unit": "TFLOP/s",
            "frac": flops / sec / PEAK_FP8}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_mlp_up_relu2_d20_traffic.txt")
GEMM_SOURCE = os.path.join(ROOT, "gpt_pretraining_step_gemms_amd", "csrc", "gemm.hip")


def measured_traffic(algorithmic_bytes):
    """HBM bytes per launch of the roofline GEMM from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel's readings), or
    None when the GEMM source has changed since the counters were taken or
    the counters belong to another shape (their algorithmic bytes differ)."""
    import hashlib
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line)
        sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
        if fields["gemm.hip sha256"].strip() != sha:
            return None
        if int(fields["algorithmic bytes per launch"]) != algorithmic_bytes:
            return None
        return float(fields["hbm bytes per launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(nbytes=1 << 30):
    """A plain elementwise copy of known size (read nbytes, write nbytes):
    the reference that scales the HBM byte counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def feature_text(cfg):
    names = [n for on, n in ((cfg.value_embeds, "value embeddings on every second layer"),
                             (cfg.resid_lambdas, "residual/x0 lambdas"),
                             (cfg.smear, "smear"), (cfg.backout, "backout")) if on]
    return (", " + ", ".join(names)) if names else ""


def cpu_baseline(cfg, windows=None, ocfg=None):
    """The fp64 numpy oracle on a bounded sample of the same workload:
      * forward + backward of one 2048-token row of the model;
      * the optimizer on layer 0's six block matrices (Muon with Newton-Schulz)
        and on E and Wh (AdamW);
      * the whole tiny-config step (fwd + bwd + optimizer), timed on its own.
    The step time is extrapolated linearly from the sample: (micro-batch rows
    x accumulation steps) row passes + n_layer times the per-layer optimizer +
    the AdamW part; value = tokens per step / that time (labelled as
    extrapolated)."""
    import numpy as np
    import threadpoolctl
    import oracle
    from oracle.model import param_shapes
    from gpt_pretraining_step_gemms_amd import synthetic
    from gpt_pretraining_step_gemms_amd.configs import TINY, OptimConfig
    hp = (ocfg or OptimConfig()).as_dict()
    mcfg = cfg.as_oracle_cfg()
    if windows is not None:
        mcfg["windows"] = [None if w < 0 else w for w in windows]
    params = {k: v.astype(np.float64) for k, v in
              synthetic.normal_params(0, param_shapes(mcfg), cfg.init_std).items()}
    tok, tgt = synthetic.token_rows(1000, 1, cfg.seq_len, cfg.vocab, cfg.token_dist)
    t0 = time.perf_counter()
    _, grads = oracle.loss_and_grads(params, tok, tgt, mcfg)
    t_row = time.perf_counter() - t0
    layer0 = [n for n in params if n.startswith("0.")]
    t0 = time.perf_counter()
    oracle.train_step({n: params[n] for n in layer0}, grads, {}, 1, hp)
    t_layer = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.train_step({n: params[n] for n in ("E", "Wh")}, grads, {}, 1, hp)
    t_adamw = time.perf_counter() - t0
    del grads
    # the tiny configuration's whole step
    tcfg = TINY.as_oracle_cfg()
    tparams = {k: v.astype(np.float64) for k, v in
               synthetic.normal_params(0, param_shapes(tcfg), TINY.init_std).items()}
    ttok, ttgt = synthetic.token_rows(1, TINY.micro_batch, TINY.seq_len, TINY.vocab,
                                      TINY.token_dist)
    t0 = time.perf_counter()
    _, tgrads = oracle.loss_and_grads(tparams, ttok, ttgt, tcfg)
    oracle.train_step(tparams, tgrads, {}, 1, hp)
    t_tiny = time.perf_counter() - t0
    rows = cfg.micro_batch * cfg.accum_steps
    t_step = rows * t_row + cfg.n_layer * t_layer + t_adamw
    blas = [p for p in threadpoolctl.threadpool_info() if p["user_api"] == "blas"]
    threads = max((p["num_threads"] for p in blas), default=1)
    return {"value": cfg.tokens_per_step / t_step, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{cfg.name}: fwd+bwd of one {cfg.seq_len}-token row {t_row:.1f} s, "
                      f"optimizer of layer 0's 6 matrices {t_layer:.1f} s, AdamW of E and Wh "
                      f"{t_adamw:.1f} s; step time extrapolated to {rows} rows + "
                      f"{cfg.n_layer} layers = {t_step:.0f} s; numpy fp64 (OpenBLAS, "
                      f"{threads} threads)",
            "extrapolated": True,
            "host": {"logical_cpus": os.cpu_count(), "cpu_model": _cpu_model()},
            "tiny_full_step": {"seconds": t_tiny, "tokens_per_s": TINY.tokens_per_step / t_tiny,
                               "what": "tiny config fwd+bwd+optimizer, whole step"}}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(gradient accumulation replaces data parallelism)", file=sys.stderr)
        sys.exit(2)
    import torch
    from gpt_pretraining_step_gemms_amd import nc, synthetic
    from gpt_pretraining_step_gemms_amd.configs import (CONFIGS, OptimConfig, with_batch,
                                                        sliding_windows, NS_POLAR_EXPRESS)

    cfg = CONFIGS[args.config]
    cfg = with_batch(cfg, micro_batch=args.micro_batch, accum_steps=args.accum)
    from dataclasses import replace as dc_replace
    if args.kv_heads:
        cfg = dc_replace(cfg, n_kv_head=args.kv_heads)
    if args.fp8_forward:
        cfg = dc_replace(cfg, fp8_forward=True, fp8_backward=args.fp8_backward)
    elif args.fp8_backward:
        print("bench.py: --fp8-backward needs --fp8-forward", file=sys.stderr)
        sys.exit(2)
    feats = {f.strip() for f in args.model_features.split(",") if f.strip()}
    if "all" in feats:
        feats = {"ve", "resid", "smear", "backout"}
    unknown = feats - {"ve", "resid", "smear", "backout"}
    if unknown:
        print(f"bench.py: unknown --model-features {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)
    cfg = dc_replace(cfg, value_embeds="ve" in feats, resid_lambdas="resid" in feats,
                     smear="smear" in feats, backout="backout" in feats)
    if args.roofline_fp8:
        print(json.dumps({"roofline_fp8": roofline_gemm_fp8(cfg, args.roofline_iters)}))
        return
    if args.attention_only:
        print(json.dumps({"attention": attention_only(cfg, args.roofline_iters)}))
        return
    if args.roofline_only:
        r = roofline_gemm(cfg, args.roofline_iters)
        if args.copy_calibration:
            copy_calibration()
        print(json.dumps({"roofline": r}))
        return

    ocfg = OptimConfig(normuon=args.normuon)
    model = nc.Model(cfg, ocfg, max_micro_batch=cfg.micro_batch)
    model.init_params(seed=0, std=cfg.init_std)
    windows = None
    if args.window_pattern:
        windows = sliding_windows(cfg.n_layer, cfg.seq_len, args.window_pattern, args.short_window)
        model.set_attention_windows(windows)
    K = cfg.accum_steps
    toks, tgts = [], []
    for k in range(K):
        t, y = synthetic.token_rows(1000 + k, cfg.micro_batch, cfg.seq_len, cfg.vocab, cfg.token_dist)
        toks.append(torch.from_numpy(t).cuda())
        tgts.append(torch.from_numpy(y).cuda())
    losses = torch.zeros(K, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        model.zero_grads()
        for k in range(K):
            model.fwd_bwd(toks[k], tgts[k], 1.0 / K, loss_out=losses[k:k + 1])
        model.optimizer_step()

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup step {i} loss {losses.mean().item():.4f}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    # one event per step boundary on the bound stream (the first and last bracket
    # the timed region; the ones between give each step's own time)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    w0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    sec = ev[0].elapsed_time(ev[-1]) / 1e3 / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    print(f"[bench] {args.steps} steps, {sec * 1e3:.1f} ms/step (wall {wall:.1f} s), "
          f"last loss {losses.mean().item():.4f}", file=sys.stderr, flush=True)
    tokens = cfg.tokens_per_step
    fb_flops, ns_flops = model.flops(cfg.micro_batch)
    step_flops = K * fb_flops
    tps = tokens / sec
    mfu = step_flops / sec / PEAK_BF16
    finite = model.check_finite()
    model.close()
    del model
    torch.cuda.empty_cache()

    roof = roofline_gemm(cfg, args.roofline_iters)
    print(f"[bench] roofline {roof['achieved']:.0f} TFLOP/s ({roof['frac']:.3f} of peak)",
          file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(cfg, windows=windows, ocfg=ocfg)
    attention = "causal attention"
    if windows is not None:
        attention = (f"sliding-window attention, pattern {args.window_pattern.upper()} "
                     f"(S layers see {max(windows)} earlier keys)")

    d = cfg.d_model
    ns_name = ("Polar Express schedule" if tuple(ocfg.ns_coeffs) == tuple(NS_POLAR_EXPRESS)
               else "custom table") + (", NorMuon" if ocfg.normuon else "")
    out = {
        "metric": "training tokens/sec and MFU (% bf16 MFMA peak) per GPT step, 1 MI355X",
        "value": tps,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "step_ms": {"min": per_step[0], "median": per_step[len(per_step) // 2],
                    "max": per_step[-1]},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (Zipf(1.1) token ids, N(0, 0.02^2) random-init weights)",
        "config": {"workload": f"{cfg.name} GPT pretraining step: {cfg.n_layer} layers, d {d}, "
                               f"{cfg.n_head}x128 heads"
                               f"{f' over {cfg.kv_heads} key/value heads' if cfg.kv_heads != cfg.n_head else ''}"
                               f"{', forward block products in fp8 e4m3' if cfg.fp8_forward else ''}"
                               f"{', backward block products in fp8 (gradients e5m2)' if cfg.fp8_backward else ''}"
                               f"{feature_text(cfg)}"
                               f", {attention}, MLP {cfg.d_ff} ReLU^2, "
                               f"vocab {cfg.vocab}, "
                               f"seq {cfg.seq_len}, micro-batch {cfg.micro_batch} x {K} accumulated "
                               f"= {tokens} tokens/step, Muon ({len(ocfg.ns_coeffs)} Newton-Schulz "
                               f"steps, {ns_name}) + AdamW",
                   "global_batch": cfg.micro_batch * K, "seq_len": cfg.seq_len,
                   "parallelism": "1 GPU, gradient accumulation"},
        "mfu": mfu,
        "mfu_with_newton_schulz": (step_flops + ns_flops) / sec / PEAK_BF16,
        # attention counted as 12 L d T per token (the common non-causal convention)
        "mfu_palm_convention": None if windows is not None else
        (step_flops + 6.0 * cfg.n_layer * d * cfg.seq_len * tokens) / sec / PEAK_BF16,
        "flops_per_token": fb_flops / (cfg.micro_batch * cfg.seq_len),
        "params_finite": finite,
        "roofline": {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "roofline_kernel": {k: roof[k] for k in ("kernel", "shape", "avg_launch_us")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
