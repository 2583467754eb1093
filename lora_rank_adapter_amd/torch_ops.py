"""PyTorch custom ops over the LoRA library (namespace ``lora_amd``).

On the M* ops page the shrink and the expand are custom ops, each one opaque
node under torch.compile; the expand lists y among its mutated arguments, so
functionalization orders the reads of y before and after the in-place update
correctly; the pair also exists as one op for a linear target, and the fake
(shape) implementations are checked on a CPU. The same here, over the
HIP library: each op's only kernel is the library call on a CUDA (ROCm)
device; there is no CPU kernel, so calling an op with CPU tensors raises
NotImplementedError instead of computing anything elsewhere. The fake
implementations give the output shapes and dtypes for tracing.

Ops (the addressing arrays are passed as the tensors of lora_addressing):
  addressing(token_slot, ranks, num_slots, r_max) -> (counts, offsets, sorted_tokens)
  shrink(x, a, token_slot, counts, offsets, sorted_tokens, ranks, num_slices, r_max) -> h
  expand_(h, b, token_slot, counts, offsets, sorted_tokens, ranks, scalings, y, out_slices, r_max)   [y += ...]
  apply_(x, y, a, b, token_slot, counts, offsets, sorted_tokens, ranks, scalings, out_slices, r_max) [y += ...]
  gather_shrink(ids, a, token_slot, counts, offsets, sorted_tokens, ranks, r_max) -> h
  lora_fwd_(x, lora_A, lora_B, res, scale)                 [res += scale * (x @ lora_A) @ lora_B]
  lora_bwd_dx_da(xt, dy, lora_B, lora_A, scale) -> (dx, dA)
  lora_bwd_dx_da_accumulate_(xt, dy, lora_B, lora_A, scale, dx) -> dA  [dx += scale * (dy @ lora_B) @ lora_A]
  lora_bwd_db(lora_A, xt, dy, scale) -> dB
  lora_delta(x, A_w, B_w, scale) -> scale * (x @ A_w^T) @ B_w^T  (float32, differentiable)

h from shrink and gather_shrink is zero where the op leaves it unspecified
(inactive tokens, columns past a slot's rank), and sorted_tokens from
addressing is -1 past the active tokens, so every output is fully defined. lora_delta takes the adapter
weights in nn.Linear layout (A_w r x K, B_w L x r); its backward casts the
incoming float32 gradient to x's dtype for the backward kernels (which take dy
in the input dtype) and returns gradients in the dtypes and layouts of x, A_w
and B_w.
"""
from __future__ import annotations

import torch

from . import ops

_NS = "lora_amd"


def _addr(token_slot, counts, offsets, sorted_tokens):
    return ops.Addressing.from_arrays(token_slot, offsets.shape[0] - 1, counts, offsets, sorted_tokens)


# ---------------------------------------------------------------------------
# multi adapter
# ---------------------------------------------------------------------------

@torch.library.custom_op(f"{_NS}::addressing", mutates_args=(), device_types="cuda")
def addressing(token_slot: torch.Tensor, ranks: torch.Tensor, num_slots: int,
               r_max: int) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    # entries of sorted_tokens past the active tokens are not written by the
    # grouping pass; they hold -1 here so the op's outputs are fully defined
    dev = token_slot.device
    T = token_slot.shape[0]
    a = ops.Addressing.from_arrays(token_slot, num_slots, torch.zeros(max(num_slots, 1), dtype=torch.int32, device=dev),
                                   torch.empty(num_slots + 1, dtype=torch.int32, device=dev),
                                   torch.full((max(T, 1),), -1, dtype=torch.int32, device=dev))
    ops.lora_addressing_build(a, ranks, r_max)
    return a.counts, a.offsets, a.sorted_tokens


@addressing.register_fake
def _(token_slot, ranks, num_slots, r_max):
    T = token_slot.shape[0]
    return (token_slot.new_empty(max(num_slots, 1)), token_slot.new_empty(num_slots + 1),
            token_slot.new_empty(max(T, 1)))


@torch.library.custom_op(f"{_NS}::shrink", mutates_args=(), device_types="cuda")
def shrink(x: torch.Tensor, a: torch.Tensor, token_slot: torch.Tensor, counts: torch.Tensor,
           offsets: torch.Tensor, sorted_tokens: torch.Tensor, ranks: torch.Tensor, num_slices: int,
           r_max: int) -> torch.Tensor:
    h = torch.zeros((x.shape[0], num_slices, r_max), dtype=torch.float32, device=x.device)
    return ops.lora_shrink(x, a, _addr(token_slot, counts, offsets, sorted_tokens), ranks, num_slices, r_max, h=h)


@shrink.register_fake
def _(x, a, token_slot, counts, offsets, sorted_tokens, ranks, num_slices, r_max):
    return x.new_empty((x.shape[0], num_slices, r_max), dtype=torch.float32)


@torch.library.custom_op(f"{_NS}::expand_", mutates_args=("y",), device_types="cuda")
def expand_(h: torch.Tensor, b: torch.Tensor, token_slot: torch.Tensor, counts: torch.Tensor,
            offsets: torch.Tensor, sorted_tokens: torch.Tensor, ranks: torch.Tensor, scalings: torch.Tensor,
            y: torch.Tensor, out_slices: list[int], r_max: int) -> None:
    ops.lora_expand_fused(h, b, _addr(token_slot, counts, offsets, sorted_tokens), ranks, scalings, y, out_slices,
                          r_max)


@expand_.register_fake
def _(h, b, token_slot, counts, offsets, sorted_tokens, ranks, scalings, y, out_slices, r_max):
    return None


@torch.library.custom_op(f"{_NS}::apply_", mutates_args=("y",), device_types="cuda")
def apply_(x: torch.Tensor, y: torch.Tensor, a: torch.Tensor, b: torch.Tensor, token_slot: torch.Tensor,
           counts: torch.Tensor, offsets: torch.Tensor, sorted_tokens: torch.Tensor, ranks: torch.Tensor,
           scalings: torch.Tensor, out_slices: list[int], r_max: int) -> None:
    ops.lora_apply_linear(x, y, a, b, _addr(token_slot, counts, offsets, sorted_tokens), ranks, scalings,
                          out_slices, r_max)


@apply_.register_fake
def _(x, y, a, b, token_slot, counts, offsets, sorted_tokens, ranks, scalings, out_slices, r_max):
    return None


@torch.library.custom_op(f"{_NS}::gather_shrink", mutates_args=(), device_types="cuda")
def gather_shrink(ids: torch.Tensor, a: torch.Tensor, token_slot: torch.Tensor, counts: torch.Tensor,
                  offsets: torch.Tensor, sorted_tokens: torch.Tensor, ranks: torch.Tensor,
                  r_max: int) -> torch.Tensor:
    h = torch.zeros((ids.shape[0], 1, r_max), dtype=torch.float32, device=ids.device)
    return ops.lora_gather_shrink(ids, a, _addr(token_slot, counts, offsets, sorted_tokens), ranks, r_max, h=h)


@gather_shrink.register_fake
def _(ids, a, token_slot, counts, offsets, sorted_tokens, ranks, r_max):
    return ids.new_empty((ids.shape[0], 1, r_max), dtype=torch.float32)


# ---------------------------------------------------------------------------
# single adapter
# ---------------------------------------------------------------------------

@torch.library.custom_op(f"{_NS}::lora_fwd_", mutates_args=("res",), device_types="cuda")
def lora_fwd_(x: torch.Tensor, lora_A: torch.Tensor, lora_B: torch.Tensor, res: torch.Tensor, scale: float) -> None:
    ops.lora_fwd(x, lora_A, lora_B, res, scale)


@lora_fwd_.register_fake
def _(x, lora_A, lora_B, res, scale):
    return None


@torch.library.custom_op(f"{_NS}::lora_bwd_dx_da", mutates_args=(), device_types="cuda")
def lora_bwd_dx_da(xt: torch.Tensor, dy: torch.Tensor, lora_B: torch.Tensor, lora_A: torch.Tensor,
                   scale: float) -> tuple[torch.Tensor, torch.Tensor]:
    return ops.lora_bwd_dx_da(xt, dy, lora_B, lora_A, scale)


@lora_bwd_dx_da.register_fake
def _(xt, dy, lora_B, lora_A, scale):
    K, M = xt.shape
    return dy.new_empty((M, K), dtype=torch.float32), dy.new_empty((K, lora_B.shape[1]), dtype=torch.float32)


@torch.library.custom_op(f"{_NS}::lora_bwd_dx_da_accumulate_", mutates_args=("dx",), device_types="cuda")
def lora_bwd_dx_da_accumulate_(xt: torch.Tensor, dy: torch.Tensor, lora_B: torch.Tensor, lora_A: torch.Tensor,
                               scale: float, dx: torch.Tensor) -> torch.Tensor:
    return ops.lora_bwd_dx_da_accumulate(xt, dy, lora_B, lora_A, scale, dx)[1]


@lora_bwd_dx_da_accumulate_.register_fake
def _(xt, dy, lora_B, lora_A, scale, dx):
    return dy.new_empty((xt.shape[0], lora_B.shape[1]), dtype=torch.float32)


@torch.library.custom_op(f"{_NS}::lora_bwd_db", mutates_args=(), device_types="cuda")
def lora_bwd_db(lora_A: torch.Tensor, xt: torch.Tensor, dy: torch.Tensor, scale: float) -> torch.Tensor:
    return ops.lora_bwd_db(lora_A, xt, dy, scale)


@lora_bwd_db.register_fake
def _(lora_A, xt, dy, scale):
    return dy.new_empty((lora_A.shape[0], dy.shape[1]), dtype=torch.float32)


@torch.library.custom_op(f"{_NS}::lora_delta", mutates_args=(), device_types="cuda")
def lora_delta(x: torch.Tensor, A_w: torch.Tensor, B_w: torch.Tensor, scale: float) -> torch.Tensor:
    y = torch.zeros((x.shape[0], B_w.shape[0]), dtype=torch.float32, device=x.device)
    return ops.lora_fwd(x, A_w.t(), B_w.t(), y, scale)


@lora_delta.register_fake
def _(x, A_w, B_w, scale):
    return x.new_empty((x.shape[0], B_w.shape[0]), dtype=torch.float32)


def _delta_setup(ctx, inputs, output):
    x, A_w, B_w, scale = inputs
    ctx.save_for_backward(x, A_w, B_w)
    ctx.scale = scale


def _delta_backward(ctx, grad):
    x, A_w, B_w = ctx.saved_tensors
    dy = grad.to(x.dtype).contiguous()
    gx = gA = gB = None
    if ctx.needs_input_grad[0] or ctx.needs_input_grad[1]:
        dx, dA = torch.ops.lora_amd.lora_bwd_dx_da(x.t(), dy, B_w, A_w, ctx.scale)
        gx = dx.to(x.dtype) if ctx.needs_input_grad[0] else None
        gA = dA.t().to(A_w.dtype) if ctx.needs_input_grad[1] else None
    if ctx.needs_input_grad[2]:
        gB = torch.ops.lora_amd.lora_bwd_db(A_w, x.t(), dy, ctx.scale).t().to(B_w.dtype)
    return gx, gA, gB, None


torch.library.register_autograd(f"{_NS}::lora_delta", _delta_backward, setup_context=_delta_setup)
