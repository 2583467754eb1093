"""CPU oracle for the LoRA hot path — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 definitions of every operation the HIP library computes,
written from the API pages they come from:

* "nemo_automodel.components._peft.lora_kernel" (NeMo Automodel API docs):
  the single-adapter forward (lora_forward_kernel / lora_forward_wrapper) and
  backward (lora_da_dx_kernel / lora_da_dx_update_wrapper, lora_db_kernel /
  lora_db_update_wrapper);
* "mstar.engine.resources.lora.ops" (M* engine API docs): the slot-addressed
  multi-adapter ops shrink, expand_fused and gather_shrink of LoraOpsBackend.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The GPU library never calls it, and it shares no
code with the GPU library.

Every function here is pinned by tests that do not re-use its own formula
(closed forms, finite differences, identities, brute force on tiny inputs,
hand-worked examples); see ``tests/test_oracle_*.py``.
"""
from .lora_oracle import (  # noqa: F401
    lora_fwd,
    lora_bwd_dx_da,
    lora_bwd_db,
    group_tokens,
    active_mask,
    token_ranks,
    shrink,
    expand_fused,
    gather_shrink,
    apply_linear,
    rel_frobenius,
    bf16_bits_to_f64,
    round_to_bf16,
)
