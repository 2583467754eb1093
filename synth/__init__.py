"""Seeded synthetic inputs for the LoRA ops.

This module is shared by the CPU oracle's tests, the GPU parity tests, the
smoke check and the benchmark. It holds none of the LoRA arithmetic: only
random draws, rounding of the drawn values to bfloat16, and the shapes and
value laws of the workloads.

Workloads (sizes and value laws of the single-adapter and multi-adapter
cases; seeds are the case numbers 1-5):

1. single adapter, fp32: X 256x512 ~N(0,1), A 512x8 ~N(0,1/512),
   B 8x512 ~N(0,1/8), dY 256x512 ~N(0,1), s = 2.0, Y0 = 0.
2. single adapter, bf16 in / fp32 out: M = 8192, K = L = 4096, r = 16,
   X, dY ~N(0,1), A ~N(0,1/K), B ~N(0,1/r), s = 2.0.
3. single adapter, bf16, MLP-up shape: M = 16384, K = 4096, L = 14336,
   r = 64, same laws, s = 0.5.
4. multi-adapter decode, bf16: T = 256, K = 4096, output slices
   [4096, 1024, 1024], 32 slots, r_max = 64.
5. multi-adapter prefill, bf16: 64 requests with log-normal lengths
   (median 256, sigma 0.5, capped at 2048), 128 slots, r_max = 128,
   K = 8192, output slices [8192, 1024, 1024]; plus an embedding table
   (vocabulary 128256) for the one-hot shrink with 5% of ids set to -1.

Arrays are returned as float32 numpy arrays whose values are exactly
representable in the stated dtype ("bf16" values went through round to
nearest even). ``bf16_bits`` gives the 16-bit patterns to upload.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BF16_QNAN_BITS = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# bfloat16 helpers (input preparation only)
# ----------------------------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN inputs map to the canonical quiet NaN 0x7FC0.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = BF16_QNAN_BITS
    return rounded


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    return bf16_to_f32(bf16_bits(a))


def _normal(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# single adapter (forward and backward)
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class SingleAdapterCase:
    """Inputs of one single-adapter forward+backward case (logical shapes).

    X: M x K, A: K x r, B: r x L, dY: M x L, Y0: M x L (fp32), scale s.
    """
    X: np.ndarray
    A: np.ndarray
    B: np.ndarray
    dY: np.ndarray
    Y0: np.ndarray
    scale: float
    dtype: str
    name: str = ""

    @property
    def M(self):
        return self.X.shape[0]

    @property
    def K(self):
        return self.X.shape[1]

    @property
    def L(self):
        return self.B.shape[1]

    @property
    def r(self):
        return self.A.shape[1]


def single_adapter(M: int, K: int, L: int, r: int, *, seed: int, dtype: str = "bf16",
                   scale: float = 2.0, y0: str = "zero", int_exact: bool = False,
                   density=None, name: str = "") -> SingleAdapterCase:
    """Draw X, A, B, dY (and Y0) in that order from ``default_rng(seed)``.

    Laws: X, dY ~ N(0,1); A ~ N(0, 1/K); B ~ N(0, 1/r); Y0 = 0 or ~N(0,1).
    ``int_exact`` draws every input uniformly from {-2,...,2} instead (exact in
    bf16; with small enough shapes every fp32 partial sum is then exact).
    ``density`` = (d_X, d_A, d_B, d_dY) with ``int_exact`` draws sparse
    values instead: each element is nonzero with its matrix's probability,
    then +1 or -1 with equal odds (Y0 stays on {-2,...,2}); full-size shapes
    keep their sums small this way.
    """
    rng = np.random.default_rng(seed)
    if int_exact and density is not None:
        dens = iter(density)

        def draw(shape, _sigma):
            p = next(dens, None)
            if p is None:      # Y0
                return rng.integers(-2, 3, size=shape).astype(np.float32)
            nz = rng.random(shape, dtype=np.float32) < np.float32(p)
            sign = rng.integers(0, 2, size=shape, dtype=np.int8)
            return np.where(nz, np.where(sign == 1, np.float32(1.0), np.float32(-1.0)),
                            np.float32(0.0)).astype(np.float32)
    elif int_exact:
        def draw(shape, _sigma):
            return rng.integers(-2, 3, size=shape).astype(np.float32)
    else:
        def draw(shape, sigma):
            return _normal(rng, shape, sigma)
    X = _cast(draw((M, K), 1.0), dtype)
    A = _cast(draw((K, r), 1.0 / math.sqrt(K)), dtype)
    B = _cast(draw((r, L), 1.0 / math.sqrt(r)), dtype)
    dY = _cast(draw((M, L), 1.0), dtype)
    if y0 == "zero":
        Y0 = np.zeros((M, L), np.float32)
    elif y0 == "normal":
        Y0 = draw((M, L), 1.0).astype(np.float32)
    else:
        raise ValueError(y0)
    return SingleAdapterCase(X, A, B, dY, Y0, float(scale), dtype, name)


def config1() -> SingleAdapterCase:
    return single_adapter(256, 512, 512, 8, seed=1, dtype="f32", scale=2.0, name="cfg1-fp32-256x512x512-r8")


def config2(y0: str = "zero") -> SingleAdapterCase:
    return single_adapter(8192, 4096, 4096, 16, seed=2, dtype="bf16", scale=2.0, y0=y0,
                          name="cfg2-bf16-M8192-K4096-L4096-r16")


def config3() -> SingleAdapterCase:
    return single_adapter(16384, 4096, 14336, 64, seed=3, dtype="bf16", scale=0.5,
                          name="cfg3-bf16-M16384-K4096-L14336-r64")


# ----------------------------------------------------------------------------
# multi-adapter serving
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class MultiLoraCase:
    """Inputs of one slot-addressed multi-adapter case.

    token_slot: int32[T]; ranks: int32[S]; scalings: float32[S];
    x: T x K; a: S x (n*r_max) x K (rows i*r_max + j hold slice i, rank row j;
    rows j >= rank are NaN padding); b: S x sum(out_slices) x r_max (columns
    j >= rank are NaN padding); y0: T x sum(out_slices) fp32, rows of inactive
    tokens hold -0.0.
    """
    token_slot: np.ndarray
    ranks: np.ndarray
    scalings: np.ndarray
    x: np.ndarray
    a: np.ndarray
    b: np.ndarray
    y0: np.ndarray
    out_slices: tuple
    r_max: int
    name: str = ""

    @property
    def T(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def S(self):
        return self.ranks.shape[0]

    @property
    def num_slices(self):
        return len(self.out_slices)


def _active_rows(token_slot, ranks, r_max):
    S = ranks.shape[0]
    ok = (token_slot >= 0) & (token_slot < S)
    rho = np.zeros(token_slot.shape, np.int64)
    rho[ok] = np.clip(ranks[token_slot[ok]], 0, r_max)
    return ok & (rho > 0)


def multi_lora(token_slot: np.ndarray, ranks: np.ndarray, K: int, out_slices, r_max: int, *,
               rng: np.random.Generator, int_exact: bool = False, name: str = "") -> MultiLoraCase:
    """Draw scalings, x, a, b, y0 (in that order) for a given routing.

    Laws: scalings ~ U[0.5, 2]; x ~ N(0,1); a ~ N(0, 1/K); b[s] ~ N(0, 1/rank_s);
    y0 ~ N(0,1). Padding (rank rows/columns past a slot's rank, and whole
    rank-0 slots) is NaN. ``int_exact`` draws x, a, b, y0 from {-2..2} and
    scalings from {0.5, 1, 2}.
    """
    token_slot = np.asarray(token_slot, np.int32)
    ranks = np.asarray(ranks, np.int32)
    T = token_slot.shape[0]
    S = ranks.shape[0]
    n = len(out_slices)
    O = int(sum(out_slices))
    if int_exact:
        scalings = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), size=S).astype(np.float32)
        x = rng.integers(-2, 3, size=(T, K)).astype(np.float32)
        a = rng.integers(-2, 3, size=(S, n * r_max, K)).astype(np.float32)
        b = rng.integers(-2, 3, size=(S, O, r_max)).astype(np.float32)
        y0 = rng.integers(-2, 3, size=(T, O)).astype(np.float32)
    else:
        scalings = rng.uniform(0.5, 2.0, size=S).astype(np.float32)
        x = round_bf16(_normal(rng, (T, K), 1.0))
        a = _normal(rng, (S, n * r_max, K), 1.0 / math.sqrt(K))
        b = rng.standard_normal((S, O, r_max), dtype=np.float32)
        for s in range(S):
            rho = int(np.clip(ranks[s], 0, r_max))
            if rho > 0:
                b[s] *= np.float32(1.0 / math.sqrt(rho))
        a = round_bf16(a)
        b = round_bf16(b)
        y0 = _normal(rng, (T, O), 1.0)
    for s in range(S):
        rho = int(np.clip(ranks[s], 0, r_max))
        for i in range(n):
            a[s, i * r_max + rho:(i + 1) * r_max, :] = np.nan
        b[s, :, rho:] = np.nan
    active = _active_rows(token_slot, ranks, r_max)
    y0[~active, :] = -0.0
    return MultiLoraCase(token_slot, ranks, scalings, x, a, b, y0, tuple(int(o) for o in out_slices),
                         int(r_max), name)


def decode_routing(T: int, S: int, r_max: int, rank_choices, zero_p: float, rng: np.random.Generator):
    """Slot 0 is the zero adapter (rank 0); ranks[1:] uniform on ``rank_choices``;
    each token goes to slot 0 with probability ``zero_p``, else uniformly to 1..S-1."""
    ranks = np.zeros(S, np.int32)
    ranks[1:] = rng.choice(np.asarray(rank_choices, np.int32), size=S - 1)
    u = rng.random(T)
    other = rng.integers(1, S, size=T)
    token_slot = np.where(u < zero_p, 0, other).astype(np.int32)
    return token_slot, ranks


def prefill_routing(n_requests: int, S: int, rank_choices, rng: np.random.Generator,
                    median: float = 256.0, sigma: float = 0.5, cap: int = 2048):
    """Request lengths clip(round(exp(N(ln median, sigma^2))), 1, cap), tokens of a
    request contiguous, each request on a slot uniform on 0..S-1, ranks uniform
    on ``rank_choices``."""
    lengths = np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, size=n_requests))), 1, cap).astype(np.int64)
    req_slot = rng.integers(0, S, size=n_requests).astype(np.int32)
    ranks = rng.choice(np.asarray(rank_choices, np.int32), size=S).astype(np.int32)
    token_slot = np.repeat(req_slot, lengths).astype(np.int32)
    return token_slot, ranks, lengths


def config4() -> MultiLoraCase:
    rng = np.random.default_rng(4)
    token_slot, ranks = decode_routing(256, 32, 64, (0, 8, 16, 32, 64), 0.1, rng)
    return multi_lora(token_slot, ranks, 4096, (4096, 1024, 1024), 64, rng=rng,
                      name="cfg4-decode-T256-K4096-qkv-S32-rmax64")


def config5_routing():
    rng = np.random.default_rng(5)
    token_slot, ranks, lengths = prefill_routing(64, 128, (8, 16, 32, 64, 128), rng)
    return token_slot, ranks, lengths, rng


def config5() -> MultiLoraCase:
    token_slot, ranks, _lengths, rng = config5_routing()
    return multi_lora(token_slot, ranks, 8192, (8192, 1024, 1024), 128, rng=rng,
                      name="cfg5-prefill-K8192-qkv-S128-rmax128")


# ----------------------------------------------------------------------------
# embedding table for the one-hot shrink
# ----------------------------------------------------------------------------

def gather_ids(T: int, V: int, rng: np.random.Generator, invalid_p: float = 0.05) -> np.ndarray:
    """ids uniform on [0, V); a fraction ``invalid_p`` set to -1."""
    ids = rng.integers(0, V, size=T).astype(np.int32)
    ids[rng.random(T) < invalid_p] = -1
    return ids


def gather_table_bits(S: int, r_max: int, V: int, ranks: np.ndarray, seed: int,
                      chunk_rows: int = 4096) -> np.ndarray:
    """Embedding adapter table as bf16 bits, physical shape S x V x r_max (rank
    index contiguous); logical a[s][j, v] = table[s, v, j]. Values ~N(0,1),
    columns j >= rank(s) are NaN padding. Drawn in row chunks to bound memory.
    """
    rng = np.random.default_rng(seed)
    out = np.empty((S, V, r_max), np.uint16)
    for s in range(S):
        rho = int(np.clip(ranks[s], 0, r_max))
        for v0 in range(0, V, chunk_rows):
            v1 = min(V, v0 + chunk_rows)
            vals = rng.standard_normal((v1 - v0, r_max), dtype=np.float32)
            vals[:, rho:] = np.nan
            out[s, v0:v1, :] = bf16_bits(vals)
    return out
