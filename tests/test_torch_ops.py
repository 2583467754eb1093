"""CPU checks of the torch custom ops (lora_rank_adapter_amd.torch_ops).

No GPU is used: the fake (shape) implementations are exercised on fake CUDA
tensors, the schemas are checked for the in-place annotations the M* ops page
asks for (the expand adds into y and says so), tracing keeps one node per op,
and every op refuses CPU tensors (the library's kernels are its only
implementation). torch.library.opcheck and torch.compile over the ops run in
the GPU tests.
"""
import types

import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode
from torch.fx.experimental.proxy_tensor import make_fx

import lora_rank_adapter_amd.torch_ops  # registers the ops

OPS = torch.ops.lora_amd
T, K, S, R_MAX, SLICES = 40, 64, 5, 16, [32, 16, 16]


def _fake_multi(mode):
    with mode:
        x = torch.empty(T, K, dtype=torch.bfloat16, device="cuda")
        a = torch.empty(S, len(SLICES) * R_MAX, K, dtype=torch.bfloat16, device="cuda")
        b = torch.empty(S, sum(SLICES), R_MAX, dtype=torch.bfloat16, device="cuda")
        ts = torch.empty(T, dtype=torch.int32, device="cuda")
        ranks = torch.empty(S, dtype=torch.int32, device="cuda")
        sc = torch.empty(S, dtype=torch.float32, device="cuda")
        y = torch.empty(T, sum(SLICES), dtype=torch.float32, device="cuda")
    return x, a, b, ts, ranks, sc, y


def _written(op):
    return [a.name for a in op.default._schema.arguments if a.alias_info is not None and a.alias_info.is_write]


def test_schemas_declare_in_place_outputs():
    assert _written(OPS.expand_) == ["y"]
    assert _written(OPS.apply_) == ["y"]
    assert _written(OPS.lora_fwd_) == ["res"]
    assert _written(OPS.lora_bwd_dx_da_accumulate_) == ["dx"]
    for name in ("addressing", "shrink", "gather_shrink", "lora_bwd_dx_da", "lora_bwd_db", "lora_delta"):
        assert _written(getattr(OPS, name)) == [], name


def test_fake_shapes_multi_adapter():
    mode = FakeTensorMode()
    x, a, b, ts, ranks, sc, y = _fake_multi(mode)
    with mode:
        counts, offsets, sorted_tokens = OPS.addressing(ts, ranks, S, R_MAX)
        assert (counts.shape, offsets.shape, sorted_tokens.shape) == ((S,), (S + 1,), (T,))
        assert counts.dtype == offsets.dtype == sorted_tokens.dtype == torch.int32
        h = OPS.shrink(x, a, ts, counts, offsets, sorted_tokens, ranks, len(SLICES), R_MAX)
        assert h.shape == (T, len(SLICES), R_MAX) and h.dtype == torch.float32 and h.device.type == "cuda"
        OPS.expand_(h, b, ts, counts, offsets, sorted_tokens, ranks, sc, y, SLICES, R_MAX)
        OPS.apply_(x, y, a, b, ts, counts, offsets, sorted_tokens, ranks, sc, SLICES, R_MAX)
        ids = torch.empty(T, dtype=torch.int32, device="cuda")
        tab = torch.empty(S, R_MAX, 1000, dtype=torch.bfloat16, device="cuda")
        g = OPS.gather_shrink(ids, tab, ts, counts, offsets, sorted_tokens, ranks, R_MAX)
        assert g.shape == (T, 1, R_MAX) and g.dtype == torch.float32


def test_fake_shapes_single_adapter_and_backward_formula():
    """Output shapes of the single-adapter ops, and the gradients the
    differentiable lora_delta hands back (its backward run on fake tensors:
    the autograd engine itself needs a device context)."""
    M, K_, L_, r = 24, 48, 40, 8
    with FakeTensorMode():
        x = torch.empty(M, K_, dtype=torch.bfloat16, device="cuda")
        A_w = torch.empty(r, K_, dtype=torch.bfloat16, device="cuda")
        B_w = torch.empty(L_, r, dtype=torch.bfloat16, device="cuda")
        y = OPS.lora_delta(x, A_w, B_w, 2.0)
        assert y.shape == (M, L_) and y.dtype == torch.float32
        ctx = types.SimpleNamespace(saved_tensors=(x, A_w, B_w), needs_input_grad=(True, True, True, False),
                                    scale=2.0)
        gx, gA, gB, gs = lora_rank_adapter_amd.torch_ops._delta_backward(ctx, torch.empty_like(y))
        assert gx.shape == x.shape and gx.dtype == x.dtype
        assert gA.shape == A_w.shape and gA.dtype == A_w.dtype
        assert gB.shape == B_w.shape and gB.dtype == B_w.dtype
        assert gs is None
        dy = torch.empty(M, L_, dtype=torch.bfloat16, device="cuda")
        dx, dA = OPS.lora_bwd_dx_da(x.t(), dy, B_w, A_w, 2.0)
        assert dx.shape == (M, K_) and dA.shape == (K_, r) and dx.dtype == dA.dtype == torch.float32
        dA2 = OPS.lora_bwd_dx_da_accumulate_(x.t(), dy, B_w, A_w, 2.0, torch.empty(M, K_, device="cuda"))
        assert dA2.shape == (K_, r) and dA2.dtype == torch.float32
        dB = OPS.lora_bwd_db(A_w, x.t(), dy, 2.0)
        assert dB.shape == (r, L_) and dB.dtype == torch.float32
        res = torch.empty(M, L_, dtype=torch.float32, device="cuda")
        OPS.lora_fwd_(x, A_w.t(), B_w.t(), res, 2.0)


def _serving_step(x, a, b, ts, ranks, sc, y):
    counts, offsets, sorted_tokens = OPS.addressing(ts, ranks, S, R_MAX)
    h = OPS.shrink(x, a, ts, counts, offsets, sorted_tokens, ranks, len(SLICES), R_MAX)
    OPS.expand_(h, b, ts, counts, offsets, sorted_tokens, ranks, sc, y, SLICES, R_MAX)
    return y


def test_trace_keeps_one_node_per_op():
    mode = FakeTensorMode()
    args = _fake_multi(mode)
    gm = make_fx(_serving_step, tracing_mode="fake")(*args)
    targets = [n.target for n in gm.graph.nodes if n.op == "call_function"]
    names = [str(t) for t in targets]
    assert names.count("lora_amd.addressing.default") == 1
    assert names.count("lora_amd.shrink.default") == 1
    assert names.count("lora_amd.expand_.default") == 1
    assert names.index("lora_amd.shrink.default") < names.index("lora_amd.expand_.default")


@pytest.mark.parametrize("name", ["addressing", "shrink", "gather_shrink", "lora_delta", "lora_bwd_db"])
def test_cpu_tensors_are_refused(name):
    """Every op has only the library's kernel: CPU tensors raise instead of
    running anywhere else."""
    i32 = torch.zeros(4, dtype=torch.int32)
    calls = {
        "addressing": lambda: OPS.addressing(i32, torch.zeros(2, dtype=torch.int32), 2, 16),
        "shrink": lambda: OPS.shrink(torch.zeros(4, 8), torch.zeros(2, 16, 8), i32, i32[:2], i32[:3], i32,
                                     i32[:2], 1, 16),
        "gather_shrink": lambda: OPS.gather_shrink(i32, torch.zeros(2, 16, 8), i32, i32[:2], i32[:3], i32,
                                                   i32[:2], 16),
        "lora_delta": lambda: OPS.lora_delta(torch.zeros(4, 8), torch.zeros(2, 8), torch.zeros(6, 2), 1.0),
        "lora_bwd_db": lambda: OPS.lora_bwd_db(torch.zeros(2, 8), torch.zeros(8, 4), torch.zeros(4, 6), 1.0),
    }
    with pytest.raises(NotImplementedError):
        calls[name]()
