"""CPU fp64 oracle for one GPT pretraining step — TEST INFRASTRUCTURE ONLY.

This package is the slow, plain definition that the HIP path is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never
does.  It shares no code with the HIP path: it takes plain numpy arrays
(weights, token ids) and returns plain numpy arrays.

Sources (web pages on nanochat; cited by title and section):

* [APIDOG] apidog.com, "Cara Melatih ChatGPT Sendiri dengan Budget 50 Dolar",
  section "Bagaimana nanochat Bekerja": "1. Model GPT (nanochat/gpt.py)"
  (feature list: RoPE, QK normalisation, untied weights, ReLU^2),
  "2. Pengoptimal Muon (nanochat/optim.py)" (Newton-Schulz loop),
  "3. Manajemen Presisi (nanochat/common.py)" (bias-free Linear, fp32 masters),
  "Langkah 3: Latih Tokenizer" (32,768-token vocabulary).
* [DEVTO] dev.to, "วิธีฝึก ChatGPT ส่วนตัว งบ 50 ดอลลาร์", section
  "2. ตัวปรับปรุง Muon" (table: embeddings and lm_head -> AdamW, 2-D
  matrices -> Muon) and "3. การจัดการความแม่นยำ" (dtype table).
* [HADA] vi.news.hada.io, "NanoChat - ChatGPT tốt nhất bạn có thể mua với
  100 USD": single GPU runs use gradient accumulation with nearly identical
  results.

Where the pages are silent, the reading taken is stated in the function that
applies it.  Pins: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, invariants, textbook routines (SVD, polar
decomposition) and central finite differences.  Parity unpinned (no value
printed by the pages and no closed form; covered only by the structural pins
above and by the GPU-against-oracle tests):
* the absolute loss and gradient values of the d12..d26 shapes;
* Newton-Schulz coefficient rows three to five of the Polar Express schedule
  (an input here, like a learning rate; rows one and two are pinned to the
  printed ones, the later rows follow the same construction);
* ``optim.normuon_update``: the reading of the NorMuon fragment (per-output-row
  second moment, norm-preserving rescale) is checked against its own
  invariants, not against values from the pages;
* ``fp8``: the e5m2 format for gradients and which products run in fp8 are
  readings; the codecs themselves are pinned against the format definitions.
"""

from .model import (  # noqa: F401
    rmsnorm, rmsnorm_backward, rope_tables, rope, rope_inverse,
    causal_attention, causal_attention_backward, layer_windows, forward, loss_and_grads,
    logits_of,
)
from .optim import (  # noqa: F401
    adamw_step, newton_schulz, muon_step, normuon_update, muon_normuon_step, train_step,
)
