"""Float64 CPU oracle for the LoRA operations — TEST INFRASTRUCTURE ONLY.

Each function is the plain definition of one operation, computed in float64
(every float32 or bfloat16 input converts exactly to float64). Matrix
products use numpy's float64 matmul as a library primitive; nothing is
blocked, fused or reordered beyond what the definitions state.

Notation of the pages is kept in each function's frame. Readings of points
the pages leave open are stated where they are used:

* scale is applied once per output, in float64 (the pages pass it both to
  kernels and wrappers; where it is applied is mathematically irrelevant);
* the forward always adds into ``res`` (an absent ``res`` is a zero matrix);
* dx, dlora_A and d_lora_B are overwritten, not accumulated;
* ``LoraAddressing`` is read as the per-token slot id ``token_slot[t]``; a
  token is active iff 0 <= slot < S and its slot's rank, clamped to
  [0, r_max], is positive;
* entries the multi-adapter expand does not read are written as zeros here
  (the M* page says its reference writes zeros there);
* h has layout T x num_slices x r_max; a stacks the slices along its rows
  (S x num_slices*r_max x K); b concatenates the output slices along its rows
  (S x sum(out_slices) x r_max); one rank and one scaling per slot.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 values (exact widening)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """float64 values -> the nearest bfloat16 values (ties to the even
    significand), returned as float64. bfloat16 keeps float32's exponent
    range with 8 significant bits: in the binade [2^e, 2^(e+1)) the values
    are spaced 2^(e-7), and below 2^-126 (subnormals) 2^-133. A result at or
    beyond 2^128 is infinite; NaN stays NaN, zeros keep their sign. This is
    the single rounding a bfloat16 output in place stores: the exact value
    rounded once."""
    v = _f64(v)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0.0)
    a = np.abs(v[fin])
    _, ex = np.frexp(a)                      # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -126)             # binade exponent, floored at the normal range
    spacing = np.ldexp(1.0, e - 7)
    n = np.rint(a / spacing)                 # round half to even (a / spacing is exact)
    r = n * spacing
    r[r >= 2.0 ** 128] = np.inf
    out[fin] = np.copysign(r, v[fin])
    return out


def rel_frobenius(got, want) -> float:
    """||got - want||_F / ||want||_F in float64; if ||want||_F == 0 the error is
    0 when got equals want exactly and +inf otherwise."""
    g = _f64(got)
    w = _f64(want)
    den = np.linalg.norm(w.ravel())
    num = np.linalg.norm((g - w).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


# ----------------------------------------------------------------------------
# Single adapter: "nemo_automodel.components._peft.lora_kernel"
# ----------------------------------------------------------------------------

def lora_fwd(x, lora_A, lora_B, res, scale):
    """Forward, in the frame of the lora_forward_kernel / lora_forward_wrapper
    entries: x is M x K, lora_A is K x N, lora_B is N x L (N = rank), res is
    M x L. Three matrices are multiplied in a row and the product is added
    into res (lora_forward_kernel); inner_kernel supplies the first, scaled
    product and block_vector_mul the second one together with the add.

    Returns res + scale * (x @ lora_A) @ lora_B as a new float64 array.
    """
    x = _f64(x)
    A = _f64(lora_A)
    B = _f64(lora_B)
    out = _f64(res).copy()
    h = float(scale) * (x @ A)       # inner_kernel: M x N, stays with the caller
    out += h @ B                     # block_vector_mul: added into D
    return out


def lora_bwd_dx_da(xt, dy, lora_B, lora_A, scale):
    """Gradients of x and lora_A, in the frame of the lora_da_dx_kernel /
    lora_da_dx_update_wrapper entries: xt is the input transposed (S x M,
    S = in-features), dy is M x K (K = out-features), lora_B is K x N, lora_A
    is N x L (L = in-features, N = rank).

    lora_da_dx_kernel produces the rank-sized product of dy and lora_B and,
    from it, the input gradient; the gradient of lora_A is a sum over the M
    tokens of xt times that product, which the wrapper entry carries out.

    Returns (dx, dlora_A): dx = scale * DYB @ lora_A (M x L) and
    dlora_A = scale * xt @ DYB (S x N, i.e. in-features x rank).
    """
    xt = _f64(xt)
    dy = _f64(dy)
    B = _f64(lora_B)
    A = _f64(lora_A)
    s = float(scale)
    dyb = dy @ B                     # DYB = DY x B, M x N
    dx = s * (dyb @ A)               # DX = DY * B * A, M x L
    dA = s * (xt @ dyb)              # reduced over the tokens: S x N
    return dx, dA


def lora_bwd_db(lora_A, xt, dy, scale):
    """Gradient of lora_B, in the frame of the lora_db_kernel /
    lora_db_update_wrapper entries: lora_A is M x K (M = rank, K =
    in-features), xt is K x N (N = tokens), dy is N x S (S = out-features).

    The kernel forms AXT = A x X^T (rank x tokens); the wrapper multiplies it
    by dy. Returns d_lora_B = scale * AXT @ dy (M x S, i.e. rank x out).
    """
    A = _f64(lora_A)
    xt = _f64(xt)
    dy = _f64(dy)
    axt = A @ xt                     # AXT = A x X^T, rank x tokens
    return float(scale) * (axt @ dy)


# ----------------------------------------------------------------------------
# Multi-adapter serving: "mstar.engine.resources.lora.ops", LoraOpsBackend
# ----------------------------------------------------------------------------

def _clamped_ranks(ranks, r_max):
    return [min(max(int(v), 0), int(r_max)) for v in np.asarray(ranks).ravel()]


def token_ranks(token_slot, ranks, r_max) -> np.ndarray:
    """Effective rank of each token: the rank of its slot clamped to
    [0, r_max] when the slot id lies in [0, S), else 0.

    The page names the addressing and the per-slot ranks but not what an
    out-of-range slot id or rank means; the reading taken is that such a
    token, or a token on a rank-0 slot (the zero adapter), adds no term, and
    that a rank outside [0, r_max] is clamped into it."""
    token_slot = np.asarray(token_slot).ravel()
    rho = _clamped_ranks(ranks, r_max)
    S = len(rho)
    out = np.zeros(token_slot.shape[0], dtype=np.int64)
    for t, s in enumerate(token_slot.tolist()):
        if 0 <= s < S:
            out[t] = rho[s]
    return out


def active_mask(token_slot, ranks, r_max) -> np.ndarray:
    """True for the tokens that contribute: effective rank (see
    :func:`token_ranks`) above zero."""
    return token_ranks(token_slot, ranks, r_max) > 0


def group_tokens(token_slot, ranks, r_max):
    """Token-to-slot grouping: a stable counting sort of the active tokens by slot.

    Returns (counts[S], offsets[S+1], sorted_tokens[n_active], n_active):
    counts[s] = number of active tokens on slot s; offsets = exclusive prefix
    sum of counts with offsets[S] = n_active; sorted_tokens lists the active
    tokens ordered by slot, ascending token index within a slot.
    """
    token_slot = np.asarray(token_slot).ravel().tolist()
    rho = _clamped_ranks(ranks, r_max)
    S = len(rho)
    counts = [0] * S
    for s in token_slot:                       # histogram
        if 0 <= s < S and rho[s] > 0:
            counts[s] += 1
    offsets = [0] * (S + 1)                    # exclusive scan
    for s in range(S):
        offsets[s + 1] = offsets[s] + counts[s]
    cursor = offsets[:S]
    sorted_tokens = [0] * offsets[S]
    for t, s in enumerate(token_slot):         # stable scatter, ascending t
        if 0 <= s < S and rho[s] > 0:
            sorted_tokens[cursor[s]] = t
            cursor[s] += 1
    return (np.asarray(counts, np.int32), np.asarray(offsets, np.int32),
            np.asarray(sorted_tokens, np.int32), offsets[S])


def shrink(x, a, token_slot, ranks, num_slices, r_max, tokens=None):
    """h[t] = x[t] @ a[slot(t)]^T per slice (LoraOpsBackend.shrink).

    For an active token t on slot s with rank rho and slice i < num_slices:
    h[t, i, j] = sum_k x[t, k] * a[s, i*r_max + j, k] for j < rho. Every other
    entry (inactive tokens, j >= rho) is unspecified on the page and written
    as 0 here. Only rows listed in ``tokens`` are computed (all if None).

    Returns a float64 array T x num_slices x r_max.
    """
    x = np.asarray(x)
    T = x.shape[0]
    n = int(num_slices)
    r_max = int(r_max)
    rho = _clamped_ranks(ranks, r_max)
    S = len(rho)
    slots = np.asarray(token_slot).ravel()
    h = np.zeros((T, n, r_max), np.float64)
    cache = {}
    for t in (range(T) if tokens is None else tokens):
        s = int(slots[t])
        if not (0 <= s < S and rho[s] > 0):
            continue
        if s not in cache:
            cache[s] = _f64(a[s])
        a_s = cache[s]
        xt = _f64(x[t])
        for i in range(n):
            rows = a_s[i * r_max:i * r_max + rho[s], :]
            h[t, i, :rho[s]] = rows @ xt
    return h


def expand_fused(h, b, token_slot, ranks, scalings, y, out_slices, r_max, tokens=None):
    """y[t, slice i] += scalings[slot(t)] * h[t, slice i] @ b[slot(t), slice i]^T
    (LoraOpsBackend.expand_fused).

    For an active token t on slot s with rank rho, slice i with columns
    [off_i, off_i + O_i) of y: y[t, off_i + c] += sc[s] * sum_{j < rho}
    h[t, i, j] * b[s, off_i + c, j]. Columns of h and b at j >= rho are not
    read. Inactive tokens leave their y row unchanged.

    Returns the updated rows (all rows, or those listed in ``tokens``, in that
    order) as a new float64 array.
    """
    r_max = int(r_max)
    rho = _clamped_ranks(ranks, r_max)
    S = len(rho)
    slots = np.asarray(token_slot).ravel()
    sc = _f64(scalings).ravel()
    offs = np.concatenate([[0], np.cumsum(np.asarray(out_slices, np.int64))])
    rows = range(np.asarray(y).shape[0]) if tokens is None else list(tokens)
    out = np.empty((len(rows), np.asarray(y).shape[1]), np.float64)
    cache = {}
    for row, t in enumerate(rows):
        out[row] = _f64(y[t])
        s = int(slots[t])
        if not (0 <= s < S and rho[s] > 0):
            continue
        if s not in cache:
            cache[s] = _f64(b[s])
        b_s = cache[s]
        for i in range(len(out_slices)):
            o0, o1 = int(offs[i]), int(offs[i + 1])
            hi = _f64(h[t, i, :rho[s]])
            out[row, o0:o1] += sc[s] * (b_s[o0:o1, :rho[s]] @ hi)
    return out


def gather_shrink(ids, a, token_slot, ranks, r_max, tokens=None, a_is_bf16_bits=False):
    """Column ids[t] of the token's adapter (LoraOpsBackend.gather_shrink):
    what the shrink would give for a one-hot input row.

    ``a`` is indexable as a[s, j, v] (S x r_max x V, any strides). For an
    active token t on slot s with rank rho: h[t, 0, j] = a[s, j, ids[t]] for
    j < rho when 0 <= ids[t] < V; an id outside [0, V) selects no column, so
    those entries are +0.0. Other entries are written as 0.

    Returns a float64 array T x 1 x r_max.
    """
    ids = np.asarray(ids).ravel()
    T = ids.shape[0]
    r_max = int(r_max)
    V = a.shape[2]
    rho = _clamped_ranks(ranks, r_max)
    S = len(rho)
    slots = np.asarray(token_slot).ravel()
    h = np.zeros((T, 1, r_max), np.float64)
    for t in (range(T) if tokens is None else tokens):
        s = int(slots[t])
        if not (0 <= s < S and rho[s] > 0):
            continue
        v = int(ids[t])
        if 0 <= v < V:
            col = a[s, :rho[s], v]
            h[t, 0, :rho[s]] = bf16_bits_to_f64(col) if a_is_bf16_bits else _f64(col)
        else:
            h[t, 0, :rho[s]] = 0.0
    return h


def apply_linear(x, y, a, b, token_slot, ranks, scalings, out_slices, r_max, tokens=None):
    """Shrink then expand into y for one linear target
    (LoraOpsBackend.apply_linear_): the expand_fused of the shrink of x.
    Returns the updated rows of y as in :func:`expand_fused`."""
    h = shrink(x, a, token_slot, ranks, len(out_slices), r_max, tokens=tokens)
    return expand_fused(h, b, token_slot, ranks, scalings, y, out_slices, r_max, tokens=tokens)
