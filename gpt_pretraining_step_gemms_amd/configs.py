"""Model and optimizer configurations of the GPT pretraining step.

The depth knob sets every shape: width d = 64 * depth, head dim 128 (so
d / 128 heads), MLP hidden 4 d, vocabulary 32,768 (the tokenizer of
apidog.com, "Cara Melatih ChatGPT Sendiri dengan Budget 50 Dolar", section
"Langkah 3: Latih Tokenizer"), sequence length 2048.  The tiny model is a
correctness case computed in fp32 end to end.
"""

from dataclasses import dataclass, field, asdict, replace

from .polar_express import polar_express_table

# Newton-Schulz coefficient tables (a, b, c) per iteration: data, not code.
# Constant quintic from K. Jordan's public Muon write-up (the optimizer the
# nanochat pages name), five iterations.
NS_QUINTIC_JORDAN = [(3.4445, -4.7750, 2.0315)] * 5
# Textbook order-5 Newton-Schulz polar iteration (Higham, Functions of
# Matrices, ch. 8): p(s) = (15 s - 10 s^3 + 3 s^5) / 8.
NS_TEXTBOOK = [(15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)]
# The Polar Express schedule the pages name (five rows; the pages print the
# first two), rebuilt by its published construction in polar_express.py.
NS_POLAR_EXPRESS = polar_express_table()


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layer: int
    d_model: int
    n_head: int
    head_dim: int
    d_ff: int
    vocab: int
    seq_len: int
    micro_batch: int
    accum_steps: int
    dtype: str            # "fp32" | "bf16"
    token_dist: str       # "uniform" | "zipf"
    rope_base: float = 10000.0
    norm_eps: float = 1e-6
    init_std: float = 0.02
    n_kv_head: int = 0    # key/value heads for grouped-query attention (0: n_head)
    fp8_forward: bool = False   # forward block products in fp8 e4m3, tensorwise scales
    fp8_backward: bool = False  # and their backward products (gradients e5m2)
    # the pages' further model mechanisms (off in the benchmark configurations)
    value_embeds: bool = False  # gated value embeddings on every other layer
    resid_lambdas: bool = False # per-layer scaling of the stream and of the embedding output
    smear: bool = False         # gated mix-in of the previous token's embedding
    backout: bool = False       # subtract the mid-depth stream after the last layer
    ve_gate_channels: int = 32  # leading channels of the block input that drive a value gate

    @property
    def kv_heads(self):
        return self.n_kv_head or self.n_head

    def as_oracle_cfg(self):
        return dict(n_layer=self.n_layer, d_model=self.d_model, n_head=self.n_head,
                    head_dim=self.head_dim, d_ff=self.d_ff, vocab=self.vocab,
                    seq_len=self.seq_len, rope_base=self.rope_base, norm_eps=self.norm_eps,
                    n_kv_head=self.kv_heads, fp8_forward=self.fp8_forward,
                    fp8_backward=self.fp8_backward,
                    value_embeds=self.value_embeds, resid_lambdas=self.resid_lambdas,
                    smear=self.smear, backout=self.backout,
                    ve_gate_channels=self.ve_gate_channels)

    @property
    def tokens_per_step(self):
        return self.micro_batch * self.seq_len * self.accum_steps

    def n_params(self):
        d, F, V, L = self.d_model, self.d_ff, self.vocab, self.n_layer
        dk = self.kv_heads * self.head_dim
        return L * (2 * d * d + 2 * dk * d + 2 * d * F) + 2 * V * d


@dataclass(frozen=True)
class OptimConfig:
    muon_lr: float = 0.02
    muon_momentum: float = 0.95
    muon_wd: float = 0.0
    ns_eps: float = 1e-7
    muon_nesterov: bool = False
    ns_coeffs: tuple = tuple(NS_POLAR_EXPRESS)
    adam_lr_embed: float = 3e-3
    adam_lr_head: float = 3e-3
    adam_lr_scalar: float = 3e-3        # scalar parameters (residual, smear, backout lambdas)
    adam_beta1: float = 0.9
    adam_beta2: float = 0.95
    adam_eps: float = 1e-8
    adam_wd: float = 0.0
    normuon: bool = False       # NorMuon per-neuron normalisation after Newton-Schulz
    normuon_beta2: float = 0.95

    def as_dict(self):
        d = asdict(self)
        d["ns_coeffs"] = [tuple(c) for c in self.ns_coeffs]
        return d


def from_depth(depth, micro_batch, accum_steps, name=None):
    d = 64 * depth
    return ModelConfig(name=name or f"d{depth}", n_layer=depth, d_model=d,
                       n_head=d // 128, head_dim=128, d_ff=4 * d, vocab=32768,
                       seq_len=2048, micro_batch=micro_batch, accum_steps=accum_steps,
                       dtype="bf16", token_dist="zipf")


TINY = ModelConfig(name="tiny", n_layer=2, d_model=128, n_head=1, head_dim=128,
                   d_ff=512, vocab=512, seq_len=64, micro_batch=4, accum_steps=1,
                   dtype="fp32", token_dist="uniform")
D12 = from_depth(12, micro_batch=32, accum_steps=1)
D20 = from_depth(20, micro_batch=32, accum_steps=8)
D24 = from_depth(24, micro_batch=16, accum_steps=16)
# d26: 1,048,576 tokens per step with the largest micro-batch whose arenas fit
# one MI355X: 128 rows (about 274 GB of parameter and activation arenas)
# x 4 accumulated micro-batches.
D26 = from_depth(26, micro_batch=128, accum_steps=4)

CONFIGS = {c.name: c for c in (TINY, D12, D20, D24, D26)}


def sliding_windows(n_layer, seq_len, pattern, short=None):
    """Per-layer attention windows from a pattern of "S" (short window) and
    "L" (the whole causal context) letters, repeated over the layers from the
    first one.  apidog.com, "1. Model GPT (nanochat/gpt.py)", names such a
    configurable pattern ("SSSL") without a window size; the short window
    here defaults to half the sequence (keys t - seq_len/2 .. t).  Returns a
    list with -1 for "L" layers."""
    pattern = pattern.upper()
    if not pattern or set(pattern) - {"S", "L"}:
        raise ValueError(f"window pattern {pattern!r}: letters S and L only")
    short = seq_len // 2 if short is None else int(short)
    if short < 0:
        raise ValueError("short window must be >= 0")
    return [short if pattern[i % len(pattern)] == "S" else -1 for i in range(n_layer)]


def with_batch(cfg, micro_batch=None, accum_steps=None, seq_len=None):
    kw = {}
    if micro_batch is not None:
        kw["micro_batch"] = micro_batch
    if accum_steps is not None:
        kw["accum_steps"] = accum_steps
    if seq_len is not None:
        kw["seq_len"] = seq_len
    return replace(cfg, **kw)
