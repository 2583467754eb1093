"""Pins for the CPU oracle: checks that tie it to the pages' definitions and
to mathematics, without re-using the oracle's own formulas.

Each ``pin_*`` takes the oracle functions it checks as arguments, so the same
checks run on the real oracle (they must pass) and on deliberately broken
copies of it (at least one must fail), see ``test_oracle_mutants.py``.
All raise AssertionError on failure.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _arr(v):
    """JSON lists -> float64 array; null -> NaN, "-0.0" -> negative zero."""
    def conv(e):
        if isinstance(e, list):
            return [conv(x) for x in e]
        if e is None:
            return float("nan")
        if isinstance(e, str):
            return float(e)
        return float(e)
    return np.asarray(conv(v), dtype=np.float64)


def _close(got, want, tol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    den = max(np.linalg.norm(want.ravel()), 1e-300)
    err = np.linalg.norm((got - want).ravel()) / den
    assert err <= tol, f"{what}: relative error {err:.3e} > {tol:.1e}"


def _bitwise(got, want, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), f"{what}: not bitwise equal"


# ---------------------------------------------------------------------------
# hand-worked examples
# ---------------------------------------------------------------------------

def pin_golden_single(fwd, dxda, db):
    g = _load("fwd_bwd_tiny.json")
    X, A, B, Y0, dY = (_arr(g[k]) for k in ("X", "A", "B", "Y0", "dY"))
    s = g["scale"]
    _bitwise(fwd(X, A, B, Y0, s), _arr(g["Y"]), "golden Y")
    dx, dA = dxda(X.T, dY, B.T, A.T, s)
    _bitwise(dx, _arr(g["dX"]), "golden dX")
    _bitwise(dA, _arr(g["dA"]), "golden dA")
    _bitwise(db(A.T, X.T, dY, s), _arr(g["dB"]), "golden dB")


def pin_golden_multi(shrink, expand, group):
    g = _load("multi_tiny.json")
    x, a, b, y0 = (_arr(g[k]) for k in ("x", "a", "b", "y0"))
    ts = np.asarray(g["token_slot"], np.int32)
    ranks = np.asarray(g["ranks"], np.int32)
    h = shrink(x, a, ts, ranks, g["num_slices"], g["r_max"])
    _bitwise(h, _arr(g["h"]), "golden h")
    y = expand(h, b, ts, ranks, np.asarray(g["scalings"], np.float64), y0, g["out_slices"], g["r_max"])
    _bitwise(y, _arr(g["y"]), "golden y")
    counts, offsets, sorted_tokens, n_active = group(ts, ranks, g["r_max"])
    assert list(counts) == g["counts"] and list(offsets) == g["offsets"]
    assert list(sorted_tokens[:n_active]) == g["sorted_tokens"] and n_active == g["n_active"]


def pin_golden_gather(gather):
    g = _load("gather_tiny.json")
    a = _arr(g["a"])
    h = gather(np.asarray(g["ids"], np.int32), a, np.asarray(g["token_slot"], np.int32),
               np.asarray(g["ranks"], np.int32), g["r_max"])
    spec = np.asarray(g["specified"], bool)
    want = _arr(g["h"])
    _bitwise(h[spec], want[spec], "golden gather h")
    assert not np.signbit(h[spec]).any(), "gather: an out-of-range id must give +0.0"


def pin_golden_grouping(group):
    g = _load("grouping_tiny.json")
    counts, offsets, sorted_tokens, n_active = group(np.asarray(g["token_slot"], np.int32),
                                                     np.asarray(g["ranks"], np.int32), g["r_max"])
    assert list(counts) == g["counts"], counts
    assert list(offsets) == g["offsets"], offsets
    assert list(sorted_tokens[:n_active]) == g["sorted_tokens"], sorted_tokens
    assert n_active == g["n_active"]


# ---------------------------------------------------------------------------
# single adapter: closed forms, special cases, finite differences, identities
# ---------------------------------------------------------------------------

def _rand_single(rng, M, K, L, r):
    X = rng.standard_normal((M, K))
    A = rng.standard_normal((K, r)) / math.sqrt(K)
    B = rng.standard_normal((r, L)) / math.sqrt(r)
    Y0 = rng.standard_normal((M, L))
    dY = rng.standard_normal((M, L))
    return X, A, B, Y0, dY


def pin_fwd_dense_identity(fwd, seed=11):
    """Y - Y0 equals X @ W with the dense W = s * A @ B formed first."""
    rng = np.random.default_rng(seed)
    for (M, K, L, r, s) in [(37, 53, 29, 5, 2.0), (64, 40, 96, 16, 0.5), (5, 7, 3, 2, -1.25)]:
        X, A, B, Y0, _ = _rand_single(rng, M, K, L, r)
        W = s * (A @ B)
        _close(fwd(X, A, B, Y0, s) - Y0, X @ W, 1e-12, "fwd dense identity")


def pin_fwd_special_cases(fwd, seed=12):
    rng = np.random.default_rng(seed)
    M, K, L = 9, 6, 5
    X, _, B, Y0, _ = _rand_single(rng, M, K, L, K)
    # r = K with A = I: the forward reduces to the plain product s X B.
    _close(fwd(X, np.eye(K), B, Y0, 2.0) - Y0, 2.0 * (X @ B), 1e-13, "A = I")
    # r = L with B = I: the forward reduces to s X A.
    A = rng.standard_normal((K, L))
    _close(fwd(X, A, np.eye(L), Y0, 0.5) - Y0, 0.5 * (X @ A), 1e-13, "B = I")
    # A = 0 or B = 0: the output equals res bitwise.
    _bitwise(fwd(X, np.zeros((K, 3)), rng.standard_normal((3, L)), Y0, 3.0), Y0, "A = 0")
    _bitwise(fwd(X, rng.standard_normal((K, 3)), np.zeros((3, L)), Y0, 3.0), Y0, "B = 0")
    # linear in the scale
    A3 = rng.standard_normal((K, 3))
    B3 = rng.standard_normal((3, L))
    d1 = fwd(X, A3, B3, Y0, 1.0) - Y0
    _close(fwd(X, A3, B3, Y0, -3.5) - Y0, -3.5 * d1, 1e-13, "scale linearity")


def _grads(dxda, db, X, A, B, dY, s):
    dx, dA = dxda(X.T, dY, B.T, A.T, s)
    dB = db(A.T, X.T, dY, s)
    return np.asarray(dx), np.asarray(dA), np.asarray(dB)


def pin_bwd_finite_differences(fwd, dxda, db, seed=13):
    """f(X, A, B) = <dY, s X A B> is linear in each argument, so the central
    difference with a step E of size 1 equals <grad, E> exactly (up to
    float64 rounding)."""
    rng = np.random.default_rng(seed)
    for (M, K, L, r, s) in [(11, 7, 5, 3, 2.0), (6, 13, 9, 4, 0.5)]:
        X, A, B, _, dY = _rand_single(rng, M, K, L, r)
        zero = np.zeros((M, L))

        def f(X_, A_, B_):
            return float(np.sum(dY * np.asarray(fwd(X_, A_, B_, zero, s))))

        dx, dA, dB = _grads(dxda, db, X, A, B, dY, s)
        assert dx.shape == X.shape and dA.shape == A.shape and dB.shape == B.shape, "gradient shapes"
        for name, base, grad, wrap in (
            ("dX", X, dx, lambda P: f(P, A, B)),
            ("dA", A, dA, lambda P: f(X, P, B)),
            ("dB", B, dB, lambda P: f(X, A, P)),
        ):
            for _ in range(3):
                E = rng.standard_normal(base.shape)
                fd = (wrap(base + E) - wrap(base - E)) / 2.0
                ip = float(np.sum(grad * E))
                scale_ref = max(abs(fd), 1e-3 * np.linalg.norm(grad) * np.linalg.norm(E))
                assert abs(fd - ip) <= 1e-10 * scale_ref, f"{name}: FD {fd} vs <grad,E> {ip}"


def pin_bwd_euler(fwd, dxda, db, seed=14):
    """Degree-1 homogeneity in each argument: <dX,X> = <dA,A> = <dB,B> = <dY, Y-Y0>."""
    rng = np.random.default_rng(seed)
    M, K, L, r, s = 19, 23, 17, 6, 0.75
    X, A, B, _, dY = _rand_single(rng, M, K, L, r)
    dx, dA, dB = _grads(dxda, db, X, A, B, dY, s)
    f = float(np.sum(dY * np.asarray(fwd(X, A, B, np.zeros((M, L)), s))))
    for name, v in (("X", np.sum(dx * X)), ("A", np.sum(dA * A)), ("B", np.sum(dB * B))):
        assert abs(v - f) <= 1e-10 * max(abs(f), 1.0), f"Euler identity for {name}: {v} vs {f}"


def pin_bwd_dense_chain(dxda, db, seed=15):
    """Gradients through the dense W = s A B: dW = X^T dY, dA = dW B^T, dB = A^T dW
    (dW carries s), dX = dY W^T."""
    rng = np.random.default_rng(seed)
    M, K, L, r, s = 31, 12, 20, 5, 2.0
    X, A, B, _, dY = _rand_single(rng, M, K, L, r)
    dx, dA, dB = _grads(dxda, db, X, A, B, dY, s)
    W = s * (A @ B)
    dW = X.T @ dY
    _close(dx, dY @ W.T, 1e-12, "dX = dY W^T")
    _close(dA, s * (dW @ B.T), 1e-12, "dA = s dW B^T")
    _close(dB, s * (A.T @ dW), 1e-12, "dB = s A^T dW")


def pin_single_brute_force(fwd, dxda, db, seed=16):
    """Literal nested sums on tiny shapes (pure Python, float64)."""
    rng = np.random.default_rng(seed)
    for (M, K, L, r) in [(1, 1, 1, 1), (2, 3, 1, 2), (3, 2, 7, 3), (7, 3, 2, 1)]:
        X, A, B, Y0, dY = _rand_single(rng, M, K, L, r)
        s = 1.5
        Y = [[Y0[m][l] + s * sum(sum(X[m][k] * A[k][j] for k in range(K)) * B[j][l] for j in range(r))
              for l in range(L)] for m in range(M)]
        _close(fwd(X, A, B, Y0, s), Y, 1e-14, "brute fwd")
        dyb = [[sum(dY[m][l] * B[j][l] for l in range(L)) for j in range(r)] for m in range(M)]
        dXw = [[s * sum(dyb[m][j] * A[k][j] for j in range(r)) for k in range(K)] for m in range(M)]
        dAw = [[s * sum(X[m][k] * dyb[m][j] for m in range(M)) for j in range(r)] for k in range(K)]
        xa = [[sum(X[m][k] * A[k][j] for k in range(K)) for j in range(r)] for m in range(M)]
        dBw = [[s * sum(xa[m][j] * dY[m][l] for m in range(M)) for l in range(L)] for j in range(r)]
        dx, dA, dB = _grads(dxda, db, X, A, B, dY, s)
        _close(dx, dXw, 1e-14, "brute dX")
        _close(dA, dAw, 1e-14, "brute dA")
        _close(dB, dBw, 1e-14, "brute dB")


def pin_single_integer_exact(fwd, dxda, db, seed=17):
    """Integer inputs: every result is an exact integer/power-of-two fraction,
    computed here with Python's exact integer arithmetic."""
    rng = np.random.default_rng(seed)
    M, K, L, r = 9, 14, 11, 4
    X = rng.integers(-2, 3, (M, K))
    A = rng.integers(-2, 3, (K, r))
    B = rng.integers(-2, 3, (r, L))
    dY = rng.integers(-2, 3, (M, L))
    Y0 = rng.integers(-2, 3, (M, L))
    s = 2
    xa = [[sum(int(X[m, k]) * int(A[k, j]) for k in range(K)) for j in range(r)] for m in range(M)]
    Y = [[int(Y0[m, l]) + s * sum(xa[m][j] * int(B[j, l]) for j in range(r)) for l in range(L)] for m in range(M)]
    _bitwise(fwd(X, A, B, Y0, s), np.asarray(Y, np.float64), "exact fwd")
    dyb = [[sum(int(dY[m, l]) * int(B[j, l]) for l in range(L)) for j in range(r)] for m in range(M)]
    dAw = [[s * sum(int(X[m, k]) * dyb[m][j] for m in range(M)) for j in range(r)] for k in range(K)]
    dBw = [[s * sum(xa[m][j] * int(dY[m, l]) for m in range(M)) for l in range(L)] for j in range(r)]
    dXw = [[s * sum(dyb[m][j] * int(A[k, j]) for j in range(r)) for k in range(K)] for m in range(M)]
    dx, dA, dB = _grads(dxda, db, X, A, B, dY, s)
    _bitwise(dx, np.asarray(dXw, np.float64), "exact dX")
    _bitwise(dA, np.asarray(dAw, np.float64), "exact dA")
    _bitwise(dB, np.asarray(dBw, np.float64), "exact dB")


# ---------------------------------------------------------------------------
# multi-adapter
# ---------------------------------------------------------------------------

def _rand_multi(rng, T, K, out_slices, S, r_max, ranks=None, slot_range=None):
    n = len(out_slices)
    O = sum(out_slices)
    if ranks is None:
        ranks = rng.integers(0, r_max + 1, S)
    ranks = np.asarray(ranks, np.int32)
    lo, hi = slot_range if slot_range else (-1, S + 1)
    ts = rng.integers(lo, hi, T).astype(np.int32)
    x = rng.standard_normal((T, K))
    a = rng.standard_normal((S, n * r_max, K))
    b = rng.standard_normal((S, O, r_max))
    for s in range(S):
        rho = min(max(int(ranks[s]), 0), r_max)
        for i in range(n):
            a[s, i * r_max + rho:(i + 1) * r_max] = np.nan
        b[s, :, rho:] = np.nan
    sc = rng.uniform(0.5, 2.0, S)
    y0 = rng.standard_normal((T, O))
    for t, act in enumerate(_active(ts, ranks, r_max)):
        if not act:
            y0[t] = -0.0          # a stray "+= 0" on an untouched row would flip the sign
    return ts, ranks, x, a, b, sc, y0


def _active(ts, ranks, r_max):
    S = len(ranks)
    return [0 <= s < S and min(max(int(ranks[s]), 0), r_max) > 0 for s in ts.tolist()]


def pin_multi_brute_force(shrink, expand, seed=21):
    """Literal sums over the definitions on tiny cases with padding = NaN,
    out-of-range slots and rank-0 slots."""
    rng = np.random.default_rng(seed)
    for (T, K, out_slices, S, r_max) in [(7, 3, (2, 1), 3, 2), (17, 5, (3,), 4, 3), (2, 1, (1, 1, 2), 1, 1)]:
        ts, ranks, x, a, b, sc, y0 = _rand_multi(rng, T, K, out_slices, S, r_max)
        n = len(out_slices)
        act = _active(ts, ranks, r_max)
        h = np.asarray(shrink(x, a, ts, ranks, n, r_max))
        y = np.asarray(expand(h, b, ts, ranks, sc, y0, out_slices, r_max))
        offs = [sum(out_slices[:i]) for i in range(n + 1)]
        for t in range(T):
            if not act[t]:
                _bitwise(y[t], y0[t], "inactive row untouched")
                assert not h[t].any(), "the oracle writes zeros in unspecified rows of h"
                continue
            s = int(ts[t])
            rho = min(int(ranks[s]), r_max)
            assert not h[t, :, rho:].any(), "the oracle writes zeros past a slot's rank"
            for i in range(n):
                for j in range(rho):
                    want = sum(x[t][k] * a[s][i * r_max + j][k] for k in range(K))
                    assert abs(h[t, i, j] - want) <= 1e-13 * (1 + abs(want)), "brute shrink"
                for c in range(offs[i], offs[i + 1]):
                    want = y0[t][c] + sc[s] * sum(
                        sum(x[t][k] * a[s][i * r_max + j][k] for k in range(K)) * b[s][c][j] for j in range(rho))
                    assert abs(y[t, c] - want) <= 1e-13 * (1 + abs(want)), "brute expand"
        assert np.isfinite(y).all(), "NaN padding leaked into y"


def pin_multi_reduces_to_single(fwd, shrink, expand, seed=22):
    """All tokens on one slot of rank r with one slice: the multi-adapter
    shrink+expand equals the single-adapter forward with a = A^T, b = B^T,
    scaling = s."""
    rng = np.random.default_rng(seed)
    T, K, L, r = 13, 9, 7, 3
    X, A, B, Y0, _ = _rand_single(rng, T, K, L, r)
    s = 1.75
    a = A.T[None, :, :]
    b = B.T[None, :, :]
    ts = np.zeros(T, np.int32)
    h = shrink(X, a, ts, [r], 1, r)
    y = expand(h, b, ts, [r], [s], Y0, (L,), r)
    _close(y, fwd(X, A, B, Y0, s), 1e-13, "multi == single")


def pin_gather_is_onehot_shrink(gather, shrink, seed=23):
    """gather_shrink equals the shrink of the one-hot of the id; an id outside
    [0, V) has a zero one-hot and gives +0.0."""
    rng = np.random.default_rng(seed)
    T, V, S, r_max = 12, 6, 3, 4
    ranks = np.asarray([3, 0, 4], np.int32)
    ts = rng.integers(-1, S + 1, T).astype(np.int32)
    ids = rng.integers(-2, V + 2, T).astype(np.int32)
    a = rng.standard_normal((S, r_max, V))
    for s in range(S):
        a[s, ranks[s]:, :] = np.nan
    onehot = np.zeros((T, V))
    for t, v in enumerate(ids.tolist()):
        if 0 <= v < V:
            onehot[t, v] = 1.0
    a_nan_free = np.nan_to_num(a, nan=0.0)   # the one-hot times a NaN row is NaN; only j < rank is compared
    want = np.asarray(shrink(onehot, a_nan_free, ts, ranks, 1, r_max))
    got = np.asarray(gather(ids, a, ts, ranks, r_max))
    act = _active(ts, ranks, r_max)
    for t in range(T):
        if act[t]:
            rho = int(ranks[ts[t]])
            _bitwise(got[t, 0, :rho], want[t, 0, :rho] + 0.0, "gather vs one-hot shrink")
            if not (0 <= ids[t] < V):
                assert not np.signbit(got[t, 0, :rho]).any(), "out-of-range id must give +0.0"


def pin_grouping_is_stable_sort(group, seed=24):
    """The grouping equals Python's stable sort of the active tokens by slot,
    and the histogram sums to the number of active tokens."""
    rng = np.random.default_rng(seed)
    for (T, S, r_max) in [(1, 1, 1), (50, 5, 4), (300, 17, 8), (0, 3, 2)]:
        ranks = rng.integers(-1, r_max + 3, S).astype(np.int32)
        ts = rng.integers(-2, S + 2, T).astype(np.int32)
        counts, offsets, sorted_tokens, n_active = group(ts, ranks, r_max)
        act = [t for t in range(T) if 0 <= ts[t] < S and min(max(int(ranks[ts[t]]), 0), r_max) > 0]
        want = sorted(act, key=lambda t: int(ts[t]))   # Python's sort is stable
        assert list(sorted_tokens[:n_active]) == want, "stable order"
        assert n_active == len(act) and int(np.sum(counts)) == n_active
        assert offsets[0] == 0 and all(offsets[s + 1] - offsets[s] == counts[s] for s in range(S))
        for s in range(S):
            seg = list(sorted_tokens[offsets[s]:offsets[s + 1]])
            assert all(int(ts[t]) == s for t in seg)


def pin_golden_active(token_ranks, active_mask, group):
    """Hand-worked addressing with a negative rank, a rank above r_max, a
    rank-0 slot and slot ids S, -1, -7 and 1000."""
    g = _load("active_tiny.json")
    ts = np.asarray(g["token_slot"], np.int32)
    ranks = np.asarray(g["ranks"], np.int32)
    assert [int(v) for v in token_ranks(ts, ranks, g["r_max"])] == g["token_ranks"], "golden token ranks"
    assert [bool(v) for v in active_mask(ts, ranks, g["r_max"])] == g["active"], "golden active mask"
    counts, offsets, sorted_tokens, n_active = group(ts, ranks, g["r_max"])
    assert list(counts) == g["counts"] and list(offsets) == g["offsets"], "golden grouping"
    assert list(sorted_tokens[:n_active]) == g["sorted_tokens"] and n_active == g["n_active"]


def _literal_rank(ts_t, ranks, r_max):
    """The reading written out with Python conditionals, one token at a time."""
    S = len(ranks)
    if ts_t < 0 or ts_t >= S:
        return 0
    v = int(ranks[ts_t])
    if v < 0:
        return 0
    if v > r_max:
        return r_max
    return v


def pin_active_mask(token_ranks, active_mask, group, seed=25):
    """Effective ranks against the reading written out per token with plain
    conditionals, on random slot ids and ranks well outside their ranges; the
    active mask against the grouping (a token is active iff the grouping lists
    it)."""
    rng = np.random.default_rng(seed)
    cases = []
    for (T, S, r_max) in [(1, 1, 1), (64, 6, 4), (400, 33, 16), (0, 2, 3)]:
        wild = rng.integers(-2 * r_max - 3, 2 * r_max + 4, S).astype(np.int32)
        inside = rng.integers(1, r_max + 1, S).astype(np.int32)     # every slot active
        for ranks in (wild, inside):
            ts = rng.integers(-S - 3, 2 * S + 3, T).astype(np.int32)
            edge = np.asarray([S, -1, -S, S - 1, 0, S + 1, -S - 1], np.int32)[:T]
            ts[:edge.shape[0]] = edge                                # the bounds of [0, S)
            cases.append((T, S, r_max, ranks, ts))
    for (T, S, r_max, ranks, ts) in cases:
        rho = [int(v) for v in token_ranks(ts, ranks, r_max)]
        assert rho == [_literal_rank(int(t), ranks, r_max) for t in ts.tolist()], "effective ranks"
        act = np.asarray(active_mask(ts, ranks, r_max), bool)
        assert act.shape == (T,)
        assert list(act) == [v > 0 for v in rho], "active iff effective rank > 0"
        _, _, sorted_tokens, n_active = group(ts, ranks, r_max)
        assert sorted(int(t) for t in sorted_tokens[:n_active]) == [t for t in range(T) if act[t]], \
            "active tokens = tokens the grouping lists"


def pin_golden_bf16(conv):
    """bf16 bit patterns -> values on the hand-worked golden patterns."""
    g = _load("bf16_bits.json")
    bits = np.asarray([int(c["bits"], 16) for c in g["cases"]], np.uint16)
    got = np.asarray(conv(bits), np.float64)
    for c, v in zip(g["cases"], got.tolist()):
        want = float(c["value"])
        if math.isnan(want):
            assert math.isnan(v), (c["bits"], v)
        else:
            assert v == want and math.copysign(1.0, v) == math.copysign(1.0, want), (c["bits"], v, want)


def pin_bf16_closed_form(conv):
    """Every one of the 65536 bf16 patterns against the format's closed form
    (sign, biased exponent, fraction), computed with math.ldexp."""
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):          # signalling-NaN patterns
        got = np.asarray(conv(every), np.float64)
    for b in range(65536):
        sgn, e, f = (b >> 15) & 1, (b >> 7) & 0xFF, b & 0x7F
        v = float(got[b])
        if e == 255:
            assert (math.isnan(v) if f else (v == (-math.inf if sgn else math.inf))), hex(b)
            continue
        mag = math.ldexp(f / 128.0, -126) if e == 0 else math.ldexp(1.0 + f / 128.0, e - 127)
        assert v == (-mag if sgn else mag) and math.copysign(1.0, v) == (-1.0 if sgn else 1.0), hex(b)


def pin_golden_bf16_round(rnd):
    """Rounding to bfloat16 on the hand-worked golden cases (ties, just off
    ties, overflow, subnormals, signed zero, NaN)."""
    g = _load("bf16_round.json")
    got = np.asarray(rnd(np.asarray([float(c["value"]) for c in g["cases"]])), np.float64)
    for c, v in zip(g["cases"], got.tolist()):
        want = float(c["rounded"])
        if math.isnan(want):
            assert math.isnan(v), (c["value"], v)
        else:
            assert v == want and math.copysign(1.0, v) == math.copysign(1.0, want), (c["value"], v, want)


def pin_bf16_round_grid(rnd, conv):
    """On the grid of every finite bfloat16 value (consecutive bit patterns
    widened by the pinned conv): each value rounds to itself, the midpoint of
    two neighbours to the one whose pattern is even, the float64 numbers next
    to a midpoint to the nearer neighbour, and past the largest finite value
    the midpoint to 2^128 and above gives infinity. Both signs."""
    pos = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)      # +0 .. largest finite
    vals = np.asarray(conv(pos), np.float64)
    top = np.append(vals, 2.0 ** 128)                                   # the next grid point
    even = (np.arange(top.shape[0] - 1) % 2) == 0                        # pattern parity of the lower one
    lo, hi = top[:-1], top[1:]
    mid = (lo + hi) / 2.0
    tie = np.where(even, lo, hi)
    tie[-1] = np.inf                                                     # 2^128 is infinity
    hi_or_inf = hi.copy()
    hi_or_inf[-1] = np.inf
    for sgn in (1.0, -1.0):
        _bitwise(np.asarray(rnd(sgn * vals), np.float64), sgn * vals, "grid values round to themselves")
        _bitwise(np.asarray(rnd(sgn * mid), np.float64), sgn * tie, "midpoints round to the even pattern")
        _bitwise(np.asarray(rnd(sgn * np.nextafter(mid, np.inf)), np.float64), sgn * hi_or_inf, "above a midpoint")
        _bitwise(np.asarray(rnd(sgn * np.nextafter(mid, -np.inf)), np.float64), sgn * lo, "below a midpoint")


def pin_bf16_round_f32(rnd):
    """For float32 inputs the rounding is the one float32 -> bfloat16
    conversion of torch (round to nearest even, a library routine): random
    float32 bit patterns over the whole range, subnormals and the edge of
    overflow included."""
    import torch
    rng = np.random.default_rng(31)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits[:4] = [0x7F7FFFFF, 0x7F7F8000, 0x007FFFFF, 0x00008000]          # overflow edge, subnormals
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    _bitwise(np.asarray(rnd(f.astype(np.float64)), np.float64), want, "float32 -> bfloat16 by torch")


def pin_golden_apply(apply):
    """apply_linear on the hand-worked multi-adapter example gives its y."""
    g = _load("multi_tiny.json")
    x, a, b, y0 = (_arr(g[k]) for k in ("x", "a", "b", "y0"))
    y = apply(x, y0, a, b, np.asarray(g["token_slot"], np.int32), np.asarray(g["ranks"], np.int32),
              np.asarray(g["scalings"], np.float64), g["out_slices"], g["r_max"])
    _bitwise(y, _arr(g["y"]), "golden apply_linear y")


def pin_apply_linear_brute(apply, seed=26):
    """Literal sums of the composed definition, y[t, off_i + c] = y0 +
    sc[s] * sum_j (sum_k x[t,k] a[s, i*r_max + j, k]) b[s, off_i + c, j], on
    tiny cases with NaN padding, out-of-range slots and clamped ranks."""
    rng = np.random.default_rng(seed)
    for (T, K, out_slices, S, r_max) in [(6, 4, (2, 3), 3, 2), (11, 3, (1, 1, 2), 4, 3)]:
        ranks = rng.integers(-1, r_max + 2, S).astype(np.int32)
        ts, ranks, x, a, b, sc, y0 = _rand_multi(rng, T, K, out_slices, S, r_max, ranks=ranks)
        y = np.asarray(apply(x, y0, a, b, ts, ranks, sc, out_slices, r_max))
        offs = [sum(out_slices[:i]) for i in range(len(out_slices) + 1)]
        for t in range(T):
            rho = _literal_rank(int(ts[t]), ranks, r_max)
            if rho == 0:
                _bitwise(y[t], y0[t], "apply_linear: inactive row untouched")
                continue
            s = int(ts[t])
            for i in range(len(out_slices)):
                for c in range(offs[i], offs[i + 1]):
                    acc = 0.0
                    for j in range(rho):
                        hj = 0.0
                        for k in range(K):
                            hj += x[t][k] * a[s][i * r_max + j][k]
                        acc += hj * b[s][c][j]
                    want = y0[t][c] + sc[s] * acc
                    assert abs(y[t, c] - want) <= 1e-13 * (1 + abs(want)), "brute apply_linear"
        assert np.isfinite(y).all(), "NaN padding leaked into y"


ALL_SINGLE = ("pin_golden_single", "pin_fwd_dense_identity", "pin_fwd_special_cases",
              "pin_bwd_finite_differences", "pin_bwd_euler", "pin_bwd_dense_chain",
              "pin_single_brute_force", "pin_single_integer_exact")
ALL_MULTI = ("pin_golden_multi", "pin_golden_gather", "pin_golden_grouping", "pin_multi_brute_force",
             "pin_multi_reduces_to_single", "pin_gather_is_onehot_shrink", "pin_grouping_is_stable_sort",
             "pin_golden_active", "pin_active_mask", "pin_golden_apply", "pin_apply_linear_brute")
ALL_FORMAT = ("pin_golden_bf16", "pin_bf16_closed_form", "pin_golden_bf16_round", "pin_bf16_round_grid",
              "pin_bf16_round_f32")


def run_all(o):
    """Run every pin against the namespace ``o`` (the oracle module or a mutant)."""
    pin_golden_single(o.lora_fwd, o.lora_bwd_dx_da, o.lora_bwd_db)
    pin_fwd_dense_identity(o.lora_fwd)
    pin_fwd_special_cases(o.lora_fwd)
    pin_bwd_finite_differences(o.lora_fwd, o.lora_bwd_dx_da, o.lora_bwd_db)
    pin_bwd_euler(o.lora_fwd, o.lora_bwd_dx_da, o.lora_bwd_db)
    pin_bwd_dense_chain(o.lora_bwd_dx_da, o.lora_bwd_db)
    pin_single_brute_force(o.lora_fwd, o.lora_bwd_dx_da, o.lora_bwd_db)
    pin_single_integer_exact(o.lora_fwd, o.lora_bwd_dx_da, o.lora_bwd_db)
    pin_golden_multi(o.shrink, o.expand_fused, o.group_tokens)
    pin_golden_gather(o.gather_shrink)
    pin_golden_grouping(o.group_tokens)
    pin_multi_brute_force(o.shrink, o.expand_fused)
    pin_multi_reduces_to_single(o.lora_fwd, o.shrink, o.expand_fused)
    pin_gather_is_onehot_shrink(o.gather_shrink, o.shrink)
    pin_grouping_is_stable_sort(o.group_tokens)
    pin_golden_active(o.token_ranks, o.active_mask, o.group_tokens)
    pin_active_mask(o.token_ranks, o.active_mask, o.group_tokens)
    pin_golden_apply(o.apply_linear)
    pin_apply_linear_brute(o.apply_linear)
    pin_golden_bf16(o.bf16_bits_to_f64)
    pin_bf16_closed_form(o.bf16_bits_to_f64)
    pin_golden_bf16_round(o.round_to_bf16)
    pin_bf16_round_grid(o.round_to_bf16, o.bf16_bits_to_f64)
    pin_bf16_round_f32(o.round_to_bf16)


def pin_calls(o):
    """(name, thunk) for every pin, bound to the namespace ``o``."""
    return [
        ("golden_single", lambda: pin_golden_single(o.lora_fwd, o.lora_bwd_dx_da, o.lora_bwd_db)),
        ("fwd_dense_identity", lambda: pin_fwd_dense_identity(o.lora_fwd)),
        ("fwd_special_cases", lambda: pin_fwd_special_cases(o.lora_fwd)),
        ("bwd_finite_differences", lambda: pin_bwd_finite_differences(o.lora_fwd, o.lora_bwd_dx_da, o.lora_bwd_db)),
        ("bwd_euler", lambda: pin_bwd_euler(o.lora_fwd, o.lora_bwd_dx_da, o.lora_bwd_db)),
        ("bwd_dense_chain", lambda: pin_bwd_dense_chain(o.lora_bwd_dx_da, o.lora_bwd_db)),
        ("single_brute_force", lambda: pin_single_brute_force(o.lora_fwd, o.lora_bwd_dx_da, o.lora_bwd_db)),
        ("single_integer_exact", lambda: pin_single_integer_exact(o.lora_fwd, o.lora_bwd_dx_da, o.lora_bwd_db)),
        ("golden_multi", lambda: pin_golden_multi(o.shrink, o.expand_fused, o.group_tokens)),
        ("golden_gather", lambda: pin_golden_gather(o.gather_shrink)),
        ("golden_grouping", lambda: pin_golden_grouping(o.group_tokens)),
        ("multi_brute_force", lambda: pin_multi_brute_force(o.shrink, o.expand_fused)),
        ("multi_reduces_to_single", lambda: pin_multi_reduces_to_single(o.lora_fwd, o.shrink, o.expand_fused)),
        ("gather_is_onehot_shrink", lambda: pin_gather_is_onehot_shrink(o.gather_shrink, o.shrink)),
        ("grouping_is_stable_sort", lambda: pin_grouping_is_stable_sort(o.group_tokens)),
        ("golden_active", lambda: pin_golden_active(o.token_ranks, o.active_mask, o.group_tokens)),
        ("active_mask", lambda: pin_active_mask(o.token_ranks, o.active_mask, o.group_tokens)),
        ("golden_apply", lambda: pin_golden_apply(o.apply_linear)),
        ("apply_linear_brute", lambda: pin_apply_linear_brute(o.apply_linear)),
        ("golden_bf16", lambda: pin_golden_bf16(o.bf16_bits_to_f64)),
        ("bf16_closed_form", lambda: pin_bf16_closed_form(o.bf16_bits_to_f64)),
        ("golden_bf16_round", lambda: pin_golden_bf16_round(o.round_to_bf16)),
        ("bf16_round_grid", lambda: pin_bf16_round_grid(o.round_to_bf16, o.bf16_bits_to_f64)),
        ("bf16_round_f32", lambda: pin_bf16_round_f32(o.round_to_bf16)),
    ]


def failing_pins(o):
    """Names of the pins that fail on ``o``."""
    out = []
    for name, call in pin_calls(o):
        try:
            with np.errstate(all="ignore"):
                call()
        except (AssertionError, ValueError, IndexError):
            out.append(name)
    return out
