"""The torch custom ops (lora_rank_adapter_amd.torch_ops) on the GPU.

torch.library.opcheck runs every op (schema and mutation claims, fake
implementation against the real outputs, autograd registration, AOT dispatch
with dynamic shapes); the ops must give the same bits as the direct library
calls; the serving step compiled with torch.compile (AOT autograd with
functionalization, no Inductor) must give the same bits as eager; the
differentiable lora_delta must match the oracle's forward and gradients.
"""
import numpy as np
import pytest
import torch

import lora_rank_adapter_amd as L
import lora_rank_adapter_amd.torch_ops  # registers the ops
import oracle
import synth
from tests.gpu_util import DEV, dev, f32, host, note, same_bits, tol

pytestmark = pytest.mark.gpu

OPS = torch.ops.lora_amd
T, K, SLICES, S, R_MAX = 70, 256, [128, 32, 32], 6, 32


def _multi(seed=5):
    rng = np.random.default_rng(seed)
    ts, ranks = synth.decode_routing(T, S, R_MAX, (0, 8, 16, 32), 0.1, rng)
    ts[3] = -1
    m = synth.multi_lora(ts, ranks, K, SLICES, R_MAX, rng=rng, name="ops")
    return m, dict(x=dev(m.x, "bf16"), a=dev(m.a, "bf16"), b=dev(m.b, "bf16"),
                   ts=torch.from_numpy(m.token_slot).to(DEV), ranks=torch.from_numpy(m.ranks).to(DEV),
                   sc=f32(m.scalings), y=f32(m.y0))


def _serving_step(x, a, b, ts, ranks, sc, y):
    counts, offsets, sorted_tokens = OPS.addressing(ts, ranks, S, R_MAX)
    h = OPS.shrink(x, a, ts, counts, offsets, sorted_tokens, ranks, len(SLICES), R_MAX)
    OPS.expand_(h, b, ts, counts, offsets, sorted_tokens, ranks, sc, y, SLICES, R_MAX)
    return y


def test_ops_match_direct_calls_bitwise():
    m, d = _multi()
    note("custom ops vs direct calls")
    addr = L.lora_addressing_build(L.Addressing(d["ts"], S), d["ranks"], R_MAX)
    h_ref = torch.zeros((T, len(SLICES), R_MAX), device=DEV)
    L.lora_shrink(d["x"], d["a"], addr, d["ranks"], len(SLICES), R_MAX, h=h_ref)
    y_ref = d["y"].clone()
    L.lora_expand_fused(h_ref, d["b"], addr, d["ranks"], d["sc"], y_ref, SLICES, R_MAX)

    counts, offsets, sorted_tokens = OPS.addressing(d["ts"], d["ranks"], S, R_MAX)
    h = OPS.shrink(d["x"], d["a"], d["ts"], counts, offsets, sorted_tokens, d["ranks"], len(SLICES), R_MAX)
    y1 = d["y"].clone()
    OPS.expand_(h, d["b"], d["ts"], counts, offsets, sorted_tokens, d["ranks"], d["sc"], y1, SLICES, R_MAX)
    y2 = d["y"].clone()
    OPS.apply_(d["x"], y2, d["a"], d["b"], d["ts"], counts, offsets, sorted_tokens, d["ranks"], d["sc"], SLICES,
               R_MAX)
    torch.cuda.synchronize()
    assert torch.equal(counts, addr.counts) and torch.equal(offsets, addr.offsets)
    n = int(offsets[-1])
    assert torch.equal(sorted_tokens[:n], addr.sorted_tokens[:n])
    assert same_bits(host(y1), host(y_ref))
    assert same_bits(host(y2), host(y_ref))
    act = oracle.active_mask(m.token_slot, m.ranks, R_MAX)
    h_o = oracle.shrink(m.x, m.a, m.token_slot, m.ranks, len(SLICES), R_MAX)
    want = oracle.expand_fused(h_o, m.b, m.token_slot, m.ranks, m.scalings, m.y0, SLICES, R_MAX)
    got = host(y1)
    assert same_bits(got[~act], m.y0[~act])
    assert oracle.rel_frobenius(got[act] - m.y0[act], want[act] - m.y0[act]) <= tol("bf16")


def test_compiled_serving_step_matches_eager():
    m, d = _multi(6)
    note("torch.compile(aot_eager) serving step")
    y_e = d["y"].clone()
    _serving_step(d["x"], d["a"], d["b"], d["ts"], d["ranks"], d["sc"], y_e)
    compiled = torch.compile(_serving_step, backend="aot_eager", fullgraph=True)
    y_c = d["y"].clone()
    out = compiled(d["x"], d["a"], d["b"], d["ts"], d["ranks"], d["sc"], y_c)
    torch.cuda.synchronize()
    assert same_bits(host(y_c), host(y_e)), "the compiled step must add into y like the eager one"
    assert same_bits(host(out), host(y_e))


def test_opcheck_multi_adapter_ops():
    m, d = _multi(7)
    counts, offsets, sorted_tokens = OPS.addressing(d["ts"], d["ranks"], S, R_MAX)
    h = OPS.shrink(d["x"], d["a"], d["ts"], counts, offsets, sorted_tokens, d["ranks"], len(SLICES), R_MAX)
    ids = torch.randint(-2, 300, (T,), dtype=torch.int32, device=DEV)
    tab = torch.randn((S, 300, R_MAX), device=DEV).to(torch.bfloat16).permute(0, 2, 1)
    cases = [
        (OPS.addressing, (d["ts"], d["ranks"], S, R_MAX)),
        (OPS.shrink, (d["x"], d["a"], d["ts"], counts, offsets, sorted_tokens, d["ranks"], len(SLICES), R_MAX)),
        (OPS.expand_, (h, d["b"], d["ts"], counts, offsets, sorted_tokens, d["ranks"], d["sc"], d["y"].clone(),
                       SLICES, R_MAX)),
        (OPS.apply_, (d["x"], d["y"].clone(), d["a"], d["b"], d["ts"], counts, offsets, sorted_tokens, d["ranks"],
                      d["sc"], SLICES, R_MAX)),
        (OPS.gather_shrink, (ids, tab, d["ts"], counts, offsets, sorted_tokens, d["ranks"], R_MAX)),
    ]
    for op, args in cases:
        note(f"opcheck {op}")
        torch.library.opcheck(op, args)


def test_opcheck_single_adapter_ops():
    M, K_, L_, r, s = 96, 128, 80, 8, 2.0
    c = synth.single_adapter(M, K_, L_, r, seed=77, dtype="bf16", scale=s)
    x = dev(c.X, "bf16")
    A_w = dev(np.ascontiguousarray(c.A.T), "bf16")
    B_w = dev(np.ascontiguousarray(c.B.T), "bf16")
    dy = dev(c.dY, "bf16")
    cases = [
        (OPS.lora_fwd_, (x, A_w.t(), B_w.t(), torch.zeros((M, L_), device=DEV), s)),
        (OPS.lora_bwd_dx_da, (x.t(), dy, B_w, A_w, s)),
        (OPS.lora_bwd_dx_da_accumulate_, (x.t(), dy, B_w, A_w, s, torch.randn((M, K_), device=DEV))),
        (OPS.lora_bwd_db, (A_w, x.t(), dy, s)),
        (OPS.lora_delta, (x.clone().requires_grad_(), A_w.clone().requires_grad_(), B_w.clone().requires_grad_(),
                          s)),
    ]
    for op, args in cases:
        note(f"opcheck {op}")
        torch.library.opcheck(op, args)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lora_delta_forward_and_gradients(dtype):
    M, K_, L_, r, s = 200, 264, 136, 16, 0.5
    note(f"lora_delta autograd {dtype}")
    c = synth.single_adapter(M, K_, L_, r, seed=88, dtype=dtype, scale=s)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = dev(c.X, dtype).requires_grad_()
    A_w = dev(np.ascontiguousarray(c.A.T), dtype).requires_grad_()
    B_w = dev(np.ascontiguousarray(c.B.T), dtype).requires_grad_()
    y = OPS.lora_delta(x, A_w, B_w, s)
    # the upstream gradient in the input dtype (the backward kernels take dy in it)
    y.backward(dev(c.dY, dtype).to(torch.float32))
    torch.cuda.synchronize()
    zero = np.zeros((M, L_), np.float32)
    want_y = oracle.lora_fwd(c.X, c.A, c.B, zero, s)
    odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, s)
    odB = oracle.lora_bwd_db(c.A.T, c.X.T, c.dY, s)
    assert x.grad.dtype == tdt and A_w.grad.dtype == tdt and B_w.grad.dtype == tdt
    # bf16 gradients carry one rounding of their own (2^-9 relative)
    gtol = tol(dtype) + (4e-3 if dtype == "bf16" else 0.0)
    assert oracle.rel_frobenius(host(y.detach()), want_y) <= tol(dtype)
    assert oracle.rel_frobenius(host(x.grad.float()), odx) <= gtol
    assert oracle.rel_frobenius(host(A_w.grad.float()).T, odA) <= gtol
    assert oracle.rel_frobenius(host(B_w.grad.float()).T, odB) <= gtol


def test_dx_accumulate_op_matches_direct_call_bitwise():
    M, K_, L_, r, s = 150, 264, 200, 16, 0.5
    note("dx accumulate op vs direct call")
    c = synth.single_adapter(M, K_, L_, r, seed=79, dtype="bf16", scale=s)
    x = dev(c.X, "bf16")
    A_w = dev(np.ascontiguousarray(c.A.T), "bf16")
    B_w = dev(np.ascontiguousarray(c.B.T), "bf16")
    dy = dev(c.dY, "bf16")
    dx0 = torch.randn((M, K_), device=DEV)
    d1 = dx0.clone()
    _, dA1 = L.lora_bwd_dx_da_accumulate(x.t(), dy, B_w, A_w, s, d1)
    d2 = dx0.clone()
    dA2 = OPS.lora_bwd_dx_da_accumulate_(x.t(), dy, B_w, A_w, s, d2)
    torch.cuda.synchronize()
    assert same_bits(host(d2), host(d1)) and same_bits(host(dA2), host(dA1))
