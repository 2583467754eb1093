"""Helpers of the GPU parity tests: upload seeded inputs, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth

DEV = torch.device("cuda:0")
TOL_BF16 = 2e-3   # relative Frobenius error, bf16 inputs / fp32 accumulate and outputs
TOL_F32 = 1e-5    # relative Frobenius error, fp32 inputs and outputs


def tol(dtype: str) -> float:
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def note(msg: str) -> None:
    """Print and flush what names the case before a GPU step."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy values (exact in ``dtype``) -> device tensor of that dtype."""
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))


def _max_nnz(a, axis):
    return int((a != 0).sum(axis=axis).max())


def exactness_bounds(c):
    """Largest magnitude any partial sum of a single-adapter case can reach,
    from nonzero counts, when every input value is 0 or +-1 and Y0 lies in
    {-2..2} (the sparse integer-exact inputs of synth.single_adapter); a rank
    intermediate must also be exact as a bf16 hi + lo pair (at most 16
    significant bits). Keys: h = |X A|, dyb = |dY B^T|, and the outputs."""
    s = abs(c.scale)
    h = min(_max_nnz(c.X, 1), _max_nnz(c.A, 0))
    dyb = min(_max_nnz(c.dY, 1), _max_nnz(c.B, 1))
    return {"h": h, "dyb": dyb,
            "y": 2 + s * h * _max_nnz(c.B, 0),
            "dx": 8 + 2 * s * dyb * _max_nnz(c.A, 1),   # also covers dx added twice / onto dx0 in [-8, 8]
            "dA": s * dyb * _max_nnz(c.X, 0),
            "dB": s * h * _max_nnz(c.dY, 0)}


def host_bf16(t: torch.Tensor) -> np.ndarray:
    """A bfloat16 device tensor -> its values as float64 (exact widening)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_spacing(v: np.ndarray) -> np.ndarray:
    """Spacing of the bfloat16 grid at |v|: 2^(e-7) in the binade [2^e,
    2^(e+1)), 2^-133 below 2^-126."""
    a = np.abs(np.asarray(v, np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, -126)
    return np.ldexp(1.0, e - 7)


def check_bf16_output(got: np.ndarray, exact: np.ndarray, rounded: np.ndarray, mag: np.ndarray, what: str,
                      max_mismatch: float = 2.0 ** -7) -> None:
    """A bfloat16 output updated in place against the exact result. The
    device adds a float32 sum (rank intermediates as bf16 hi + lo pairs, each
    within 2^-18 of its value) and rounds once, so every element must be
    finite and within one bfloat16 spacing of the exact value plus the float32
    path's own error, bounded here by 2^-16 * mag (mag: the elementwise sum of
    the magnitudes added, |y0| + |s| |X| |A| |B|); and it must equal the exact
    value rounded once to nearest even (``rounded``) except for at most a
    fraction ``max_mismatch``: where the float32 sum lands on the other side
    of a rounding midpoint than the exact value. Midpoints lie 2^-8 of a
    value apart and the path's error is within 2^-16 of it, so at most about
    2 * 2^-16 / 2^-8 = 2^-7 of the elements can cross one (measured: 1.6e-3
    with the bf16 hi + lo rank intermediate, 1.5e-4 for plain float32)."""
    got = np.asarray(got, np.float64)
    exact = np.asarray(exact, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    bound = bf16_spacing(exact) + 2.0 ** -16 * np.asarray(mag, np.float64)
    err = np.abs(got - exact)
    assert (err <= bound).all(), (what, float((err / bound).max()))
    mism = float((got != np.asarray(rounded, np.float64)).mean()) if got.size else 0.0
    assert mism <= max_mismatch, (what, mism)
