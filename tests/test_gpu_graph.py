"""HIP graph capture of the multi-adapter decode sequence and of a
single-adapter training step.

The M* ops page requires the ops to run with no host synchronisation and no
data-dependent shapes; that is what lets a serving loop capture the grouping
pass, shrink and expand_fused of a decode step once and replay them for every
batch with new routing and activations. The graph is replayed several times
with eager work and synchronisations in between; every replay must equal the
eager sequence bit for bit (same kernels, same order) and the oracle within
the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import lora_rank_adapter_amd as L
import oracle
import synth
from tests.gpu_util import DEV, dev, f32, host, note, same_bits, tol

pytestmark = pytest.mark.gpu

T, K, SLICES, S, R_MAX = 96, 512, (256, 64, 64), 9, 32
CHOICES = (0, 8, 16, 32)


def _draw(seed):
    rng = np.random.default_rng(seed)
    ts, ranks = synth.decode_routing(T, S, R_MAX, CHOICES, 0.1, rng)
    ts[3] = -1
    ts[5] = S
    return synth.multi_lora(ts, ranks, K, SLICES, R_MAX, rng=rng, name=f"graph-{seed}")


def _run(addr, ranks, x, a, b, sc, h, y):
    L.lora_addressing_build(addr, ranks, R_MAX)
    L.lora_shrink(x, a, addr, ranks, len(SLICES), R_MAX, h=h)
    L.lora_expand_fused(h, b, addr, ranks, sc, y, SLICES, R_MAX)


def test_decode_sequence_graph_replays():
    cases = [_draw(900 + i) for i in range(4)]
    m0 = cases[0]
    # static buffers the graph is captured on
    ts_d = torch.from_numpy(m0.token_slot).to(DEV)
    rk_d = torch.from_numpy(m0.ranks).to(DEV)
    x_d = dev(m0.x, "bf16")
    a_d = dev(m0.a, "bf16")
    b_d = dev(m0.b, "bf16")
    sc_d = f32(m0.scalings)
    h_d = torch.zeros((T, len(SLICES), R_MAX), dtype=torch.float32, device=DEV)
    y_d = f32(m0.y0)
    addr = L.Addressing(ts_d, S)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(addr, rk_d, x_d, a_d, b_d, sc_d, h_d, y_d)   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(addr, rk_d, x_d, a_d, b_d, sc_d, h_d, y_d)

    for rep in range(2):
        for i, m in enumerate(cases):
            note(f"graph replay {rep}.{i}")
            # eager work between replays: new routing, activations and adapters
            ts_d.copy_(torch.from_numpy(m.token_slot))
            rk_d.copy_(torch.from_numpy(m.ranks))
            x_d.copy_(dev(m.x, "bf16"))
            a_d.copy_(dev(m.a, "bf16"))
            b_d.copy_(dev(m.b, "bf16"))
            sc_d.copy_(f32(m.scalings))
            y_d.copy_(f32(m.y0))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = host(y_d)

            # the same sequence, eagerly, on buffers of its own
            y_e = f32(m.y0)
            h_e = torch.zeros_like(h_d)
            addr_e = L.Addressing(torch.from_numpy(m.token_slot).to(DEV), S)
            _run(addr_e, torch.from_numpy(m.ranks).to(DEV), dev(m.x, "bf16"), dev(m.a, "bf16"), dev(m.b, "bf16"),
                 f32(m.scalings), h_e, y_e)
            torch.cuda.synchronize()
            assert same_bits(got, host(y_e)), f"replay {rep}.{i} differs from the eager sequence"

            act = oracle.active_mask(m.token_slot, m.ranks, R_MAX)
            h_o = oracle.shrink(m.x, m.a, m.token_slot, m.ranks, len(SLICES), R_MAX)
            want = oracle.expand_fused(h_o, m.b, m.token_slot, m.ranks, m.scalings, m.y0, SLICES, R_MAX)
            assert same_bits(got[~act], m.y0[~act]), "rows of inactive tokens were written"
            assert oracle.rel_frobenius(got[act] - m.y0[act], want[act] - m.y0[act]) <= tol("bf16")


# (M, K, L, r): the fused forward and dX kernels; the split dX schedule (band
# expand beside dA's partials, contraction over 8200 outputs) and dB's 8-wave
# weight-gradient workgroups
STEP_SHAPES = [(512, 256, 512, 16), (1024, 512, 8200, 64)]


@pytest.mark.parametrize("shape", STEP_SHAPES, ids=lambda s: "M{}-K{}-L{}-r{}".format(*s))
def test_training_step_graph_replays(shape):
    """A single-adapter training step (lora_fwd, lora_bwd_dx_da, lora_bwd_db
    on nn.Linear-layout bf16 weights, read in place) captured once and
    replayed with new activations, gradients and weights: the library
    allocates nothing, never synchronises and launches on the caller's
    stream, so every replay equals the eager step bit for bit."""
    M, K, L_, r = shape
    s = 0.5
    draws = [synth.single_adapter(M, K, L_, r, seed=950 + i, dtype="bf16", scale=s, y0="normal") for i in range(3)]
    c0 = draws[0]
    x_d = dev(c0.X, "bf16")
    dy_d = dev(c0.dY, "bf16")
    a_d = dev(np.ascontiguousarray(c0.A.T), "bf16")   # lora_A weight, r x K
    b_d = dev(np.ascontiguousarray(c0.B.T), "bf16")   # lora_B weight, L x r
    y_d = f32(c0.Y0)
    dx_d = torch.empty((M, K), dtype=torch.float32, device=DEV)
    da_d = torch.empty((K, r), dtype=torch.float32, device=DEV)
    db_d = torch.empty((r, L_), dtype=torch.float32, device=DEV)
    ws = [torch.empty(max(1, L.lora_workspace_bytes(op, M, K, L_, r, torch.bfloat16)), dtype=torch.uint8, device=DEV)
          for op in (L.LORA_OP_FWD, L.LORA_OP_BWD_DX_DA, L.LORA_OP_BWD_DB)]

    def step(x, dy, a, b, y, dx, da, db):
        L.lora_fwd(x, a.t(), b.t(), y, s, workspace=ws[0])
        L.lora_bwd_dx_da(x.t(), dy, b, a, s, dx=dx, dA=da, workspace=ws[1])
        L.lora_bwd_db(a, x.t(), dy, s, dB=db, workspace=ws[2])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(x_d, dy_d, a_d, b_d, y_d, dx_d, da_d, db_d)   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(x_d, dy_d, a_d, b_d, y_d, dx_d, da_d, db_d)

    for rep in range(2):
        for i, c in enumerate(draws):
            note(f"training-step graph replay {shape} {rep}.{i}")
            x_d.copy_(dev(c.X, "bf16"))
            dy_d.copy_(dev(c.dY, "bf16"))
            a_d.copy_(dev(np.ascontiguousarray(c.A.T), "bf16"))
            b_d.copy_(dev(np.ascontiguousarray(c.B.T), "bf16"))
            y_d.copy_(f32(c.Y0))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = [host(t) for t in (y_d, dx_d, da_d, db_d)]

            outs = [f32(c.Y0), torch.empty_like(dx_d), torch.empty_like(da_d), torch.empty_like(db_d)]
            step(dev(c.X, "bf16"), dev(c.dY, "bf16"), dev(np.ascontiguousarray(c.A.T), "bf16"),
                 dev(np.ascontiguousarray(c.B.T), "bf16"), *outs)
            torch.cuda.synchronize()
            for name, g, e in zip(("Y", "dX", "dA", "dB"), got, outs):
                assert same_bits(g, host(e)), f"replay {rep}.{i}: {name} differs from the eager step"
            if rep == 0 and i == 0:
                want = oracle.lora_fwd(c.X, c.A, c.B, c.Y0, s)
                assert oracle.rel_frobenius(got[0] - c.Y0, want - c.Y0) <= tol("bf16")
                odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, s)
                assert oracle.rel_frobenius(got[1], odx) <= tol("bf16")
                assert oracle.rel_frobenius(got[2], odA) <= tol("bf16")
                assert oracle.rel_frobenius(got[3], oracle.lora_bwd_db(c.A.T, c.X.T, c.dY, s)) <= tol("bf16")
