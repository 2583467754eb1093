"""MI355X (gfx950) LoRA low-rank-adapter hot path.

The computation lives in the HIP library ``liblora_mi355x.so`` (C ABI in
include/lora.h); this package is its Python binding. See ``ops`` for the
functions: lora_fwd, lora_bwd_dx_da, lora_bwd_dx_da_accumulate, lora_bwd_db,
lora_addressing_build, lora_shrink, lora_expand_fused, lora_apply_linear,
lora_apply_linear_noalloc, lora_gather_shrink, lora_workspace_bytes, and the kernel-timing calls
lora_timing_begin/pause/resume/read/reserve. Importing
``lora_rank_adapter_amd.torch_ops`` registers the same operations as torch
custom ops (namespace ``lora_amd``) with fake implementations for tracing and
torch.compile, and a differentiable ``lora_delta``.
"""
from ._lib import LoraError, load as load_library, library_path  # noqa: F401
from ._lib import LORA_OP_FWD, LORA_OP_BWD_DX_DA, LORA_OP_BWD_DB  # noqa: F401
from .ops import (  # noqa: F401
    Addressing,
    lora_fwd,
    lora_bwd_dx_da,
    lora_bwd_dx_da_accumulate,
    lora_bwd_db,
    lora_addressing_build,
    lora_shrink,
    lora_expand_fused,
    lora_apply_linear,
    lora_apply_linear_noalloc,
    lora_gather_shrink,
    lora_workspace_bytes,
    lora_timing_begin,
    lora_timing_pause,
    lora_timing_resume,
    lora_timing_read,
    lora_timing_reserve,
)
