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
