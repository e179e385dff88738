"""MI355X-native GPT pretraining step (gfx950 HIP kernels behind a C ABI).

Importing the package loads nothing native; ``gpt_pretraining_step_gemms_amd.nc``
loads ``libncgpt.so`` (the C-ABI library built by ``__graft_entry__.build()``)
and raises if it is missing.
"""

from .configs import CONFIGS, ModelConfig, OptimConfig  # noqa: F401
