"""Full-size parity of the single-adapter calls, every output element checked,
through the schedules the library picks by default at these shapes.

Two kinds of inputs at the two bf16 workload shapes (8192 x 4096 x 4096,
rank 16; 16384 x 4096 x 14336, rank 64):

* sparse signed inputs (each element 0, +1 or -1) whose every partial sum,
  in any order, is an exact float32 value: the GPU must equal the oracle bit
  for bit in Y, dX (overwritten and accumulated), dA and dB. The bounds that
  make this hold are checked on the host before the GPU runs.
* the workloads' normal inputs: relative Frobenius error <= 2e-3 for the
  whole output and for every 64-row tile of it, so one wrong tile cannot hide
  in the whole-matrix norm.

These are the defaults being exercised: the split dX schedule at both
shapes (a 134 MB dX at 8192 x 4096, a contraction over 14336 features at
16384 x 14336), with dX's column-band expand and dA's weight-gradient
partials in one launch, 32 token chunks in the weight-gradient kernels at
8192 tokens; the fused forward at 8192 x 4096 and the split forward (a
940 MB Y) at 16384 x 14336.
"""
import ctypes

import numpy as np
import pytest
import torch

import lora_rank_adapter_amd as L
from lora_rank_adapter_amd import _lib
import oracle
import synth
from tests.gpu_util import dev, exactness_bounds, f32, host, note, same_bits

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SHAPES = {
    "M8192-K4096-L4096-r16": (8192, 4096, 4096, 16, 2.0, 2),
    "M16384-K4096-L14336-r64": (16384, 4096, 14336, 64, 0.5, 3),
}
# nonzero probability of X, A, B, dY in the integer-exact inputs
DENSITY = (1.0 / 32, 1.0 / 4, 1.0 / 4, 1.0 / 32)
TILE = 64
TOL = 2e-3


def _upload(c):
    X = dev(c.X, "bf16")
    A_w = dev(np.ascontiguousarray(c.A.T), "bf16")   # lora_A weight, r x K
    B_w = dev(np.ascontiguousarray(c.B.T), "bf16")   # lora_B weight, L x r
    dY = dev(c.dY, "bf16")
    return X, A_w, B_w, dY


@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_full_size_integer_exact_bitwise(shape):
    M, K, L_, r, s, seed = SHAPES[shape]
    note(f"full-size integer-exact {shape}: drawing inputs")
    c = synth.single_adapter(M, K, L_, r, seed=100 + seed, dtype="bf16", scale=s, y0="normal",
                             int_exact=True, density=DENSITY)
    b = exactness_bounds(c)
    # |h|, |dYB| < 2^15 (hi + lo exact, scale a power of two); outputs < 2^22
    assert b["h"] < 2 ** 15 and b["dyb"] < 2 ** 15, b
    assert max(b["y"], b["dx"], b["dA"], b["dB"]) < 2 ** 22, b
    X, A_w, B_w, dY = _upload(c)
    dx0 = np.random.default_rng(seed).integers(-8, 9, size=(M, K)).astype(np.float32)

    note(f"full-size integer-exact {shape}: forward")
    y = f32(c.Y0)
    L.lora_fwd(X, A_w.t(), B_w.t(), y, s)
    torch.cuda.synchronize()
    want = oracle.lora_fwd(c.X, c.A, c.B, c.Y0, s).astype(np.float32)
    assert same_bits(host(y), want), "Y"
    del y, want

    note(f"full-size integer-exact {shape}: lora_bwd_dx_da and the accumulating variant")
    dx, dA = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, s)
    dxa = f32(dx0)
    _, dA2 = L.lora_bwd_dx_da_accumulate(X.t(), dY, B_w, A_w, s, dxa)
    torch.cuda.synchronize()
    odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, s)
    assert same_bits(host(dx), odx.astype(np.float32)), "dX"
    assert same_bits(host(dxa), (dx0 + odx).astype(np.float32)), "dX accumulated"
    assert same_bits(host(dA), odA.astype(np.float32)), "dA"
    assert same_bits(host(dA2), odA.astype(np.float32)), "dA (accumulating call)"
    del dx, dxa, odx

    note(f"full-size integer-exact {shape}: lora_bwd_db")
    dB = L.lora_bwd_db(A_w, X.t(), dY, s)
    torch.cuda.synchronize()
    assert same_bits(host(dB), oracle.lora_bwd_db(c.A.T, c.X.T, c.dY, s).astype(np.float32)), "dB"


def _tile_errors(got, want):
    """Relative Frobenius error of the whole matrix and the largest one over
    its 64-row tiles."""
    whole = oracle.rel_frobenius(got, want)
    worst = 0.0
    for t0 in range(0, got.shape[0], TILE):
        worst = max(worst, oracle.rel_frobenius(got[t0:t0 + TILE], want[t0:t0 + TILE]))
    return whole, worst


@pytest.mark.parametrize("cfg", ["config2", "config3"])
def test_full_size_every_row(cfg):
    c = getattr(synth, cfg)()
    note(f"full size {c.name}: forward")
    X, A_w, B_w, dY = _upload(c)
    y = torch.zeros((c.M, c.L), dtype=torch.float32, device=X.device)
    L.lora_fwd(X, A_w.t(), B_w.t(), y, c.scale)
    torch.cuda.synchronize()
    whole, worst = _tile_errors(host(y), oracle.lora_fwd(c.X, c.A, c.B, c.Y0, c.scale))
    assert whole <= TOL and worst <= TOL, ("Y", whole, worst)
    del y

    note(f"full size {c.name}: backward")
    dx, dA = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, c.scale)
    dB = L.lora_bwd_db(A_w, X.t(), dY, c.scale)
    torch.cuda.synchronize()
    odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, c.scale)
    whole, worst = _tile_errors(host(dx), odx)
    assert whole <= TOL and worst <= TOL, ("dX", whole, worst)
    # dA is K x r and dB is r x L: tiles of 64 rows of dA, whole dB
    whole, worst = _tile_errors(host(dA), odA)
    assert whole <= TOL and worst <= TOL, ("dA", whole, worst)
    odB = oracle.lora_bwd_db(c.A.T, c.X.T, c.dY, c.scale)
    whole, worst = _tile_errors(host(dB).T.copy(), odB.T.copy())
    assert whole <= TOL and worst <= TOL, ("dB", whole, worst)


def test_forward_without_workspace():
    """With the weights in their in-place layouts and a contraction of at most
    8192 features the forward uses no workspace: the C entry point takes NULL
    and gives the bits of a call with one."""
    note("forward with a NULL workspace")
    c = synth.single_adapter(1000, 2048, 1536, 16, seed=9, dtype="bf16", scale=2.0, y0="normal")
    X, A_w, B_w, _ = _upload(c)
    lib = _lib.load()
    from lora_rank_adapter_amd.ops import mat, _stream
    y_ws = f32(c.Y0)
    L.lora_fwd(X, A_w.t(), B_w.t(), y_ws, c.scale)
    y0 = f32(c.Y0)
    st = lib.lora_fwd(ctypes.byref(mat(X)), ctypes.byref(mat(A_w.t())), ctypes.byref(mat(B_w.t())),
                      ctypes.byref(mat(y0)), c.scale, None, 0, _stream(X.device))
    torch.cuda.synchronize()
    assert st == 0
    assert same_bits(host(y0), host(y_ws))
    # a packed weight needs the workspace: refused before any launch, y untouched
    y1 = f32(c.Y0)
    A_kr = dev(c.A, "bf16")                      # K x r contiguous: not an in-place layout
    st = lib.lora_fwd(ctypes.byref(mat(X)), ctypes.byref(mat(A_kr)), ctypes.byref(mat(B_w.t())),
                      ctypes.byref(mat(y1)), c.scale, None, 0, _stream(X.device))
    torch.cuda.synchronize()
    assert st == -6 and same_bits(host(y1), c.Y0)
