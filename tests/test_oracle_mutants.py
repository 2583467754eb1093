"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them (CPU only). The real oracle is never modified."""
import types

import numpy as np
import pytest

import oracle
from oracle import lora_oracle as O
from tests import oracle_pins as P


def _ns(**over):
    base = {k: getattr(O, k) for k in ("lora_fwd", "lora_bwd_dx_da", "lora_bwd_db", "group_tokens",
                                       "shrink", "expand_fused", "gather_shrink", "token_ranks",
                                       "active_mask", "apply_linear", "bf16_bits_to_f64", "round_to_bf16")}
    base.update(over)
    return types.SimpleNamespace(**base)


def _f(a):
    return np.asarray(a, np.float64)


# --- single adapter mutants --------------------------------------------------

def fwd_no_scale(x, A, B, res, scale):
    return _f(res) + (_f(x) @ _f(A)) @ _f(B)


def fwd_overwrites(x, A, B, res, scale):
    return scale * (_f(x) @ _f(A)) @ _f(B)


def fwd_squared_scale(x, A, B, res, scale):
    return _f(res) + scale * scale * (_f(x) @ _f(A)) @ _f(B)


def fwd_drops_last_rank(x, A, B, res, scale):
    A = _f(A)[:, :-1]
    B = _f(B)[:-1, :]
    return _f(res) + scale * (_f(x) @ A) @ B


def dxda_no_scale_on_dA(xt, dy, B, A, scale):
    dyb = _f(dy) @ _f(B)
    return scale * (dyb @ _f(A)), _f(xt) @ dyb


def dxda_wrong_sign(xt, dy, B, A, scale):
    dyb = _f(dy) @ _f(B)
    return -scale * (dyb @ _f(A)), scale * (_f(xt) @ dyb)


def dxda_uses_dy_not_dyb(xt, dy, B, A, scale):
    # dA computed against a shifted copy of the token axis (an index mistake)
    dyb = _f(dy) @ _f(B)
    return scale * (dyb @ _f(A)), scale * (_f(xt) @ np.roll(dyb, 1, axis=0))


def db_no_scale(A, xt, dy, scale):
    return (_f(A) @ _f(xt)) @ _f(dy)


def db_transposed_tokens(A, xt, dy, scale):
    return scale * (_f(A) @ _f(xt)) @ _f(dy)[::-1]


# --- multi-adapter mutants ---------------------------------------------------

def group_unstable(token_slot, ranks, r_max):
    counts, offsets, st, n = O.group_tokens(token_slot, ranks, r_max)
    st = st.copy()
    for s in range(len(counts)):
        st[offsets[s]:offsets[s + 1]] = st[offsets[s]:offsets[s + 1]][::-1]
    return counts, offsets, st, n


def group_keeps_rank0(token_slot, ranks, r_max):
    ranks = np.maximum(np.asarray(ranks), 1)
    return O.group_tokens(token_slot, ranks, r_max)


def shrink_ignores_rank(x, a, token_slot, ranks, num_slices, r_max, tokens=None):
    return O.shrink(x, a, token_slot, [r_max] * len(ranks), num_slices, r_max, tokens)


def shrink_slice_offset_by_rank(x, a, token_slot, ranks, num_slices, r_max, tokens=None):
    # slices stacked at i*rank instead of i*r_max
    x = np.asarray(x)
    h = np.zeros((x.shape[0], num_slices, r_max))
    for t in range(x.shape[0]):
        s = int(token_slot[t])
        if not (0 <= s < len(ranks)) or min(int(ranks[s]), r_max) <= 0:
            continue
        rho = min(int(ranks[s]), r_max)
        for i in range(num_slices):
            h[t, i, :rho] = _f(a[s])[i * rho:i * rho + rho] @ _f(x[t])
    return h


def expand_no_scaling(h, b, token_slot, ranks, scalings, y, out_slices, r_max, tokens=None):
    return O.expand_fused(h, b, token_slot, ranks, np.ones(len(ranks)), y, out_slices, r_max, tokens)


def expand_touches_inactive(h, b, token_slot, ranks, scalings, y, out_slices, r_max, tokens=None):
    out = O.expand_fused(h, b, token_slot, ranks, scalings, y, out_slices, r_max, tokens)
    return out + 0.0   # turns -0.0 of untouched rows into +0.0


def expand_wrong_slice(h, b, token_slot, ranks, scalings, y, out_slices, r_max, tokens=None):
    h = np.asarray(h)[:, ::-1, :] if np.asarray(h).shape[1] > 1 else np.asarray(h)
    return O.expand_fused(h, b, token_slot, ranks, scalings, y, out_slices, r_max, tokens)


def gather_negative_zero(ids, a, token_slot, ranks, r_max, tokens=None, a_is_bf16_bits=False):
    h = O.gather_shrink(ids, a, token_slot, ranks, r_max, tokens, a_is_bf16_bits)
    for t, v in enumerate(np.asarray(ids).tolist()):
        if not (0 <= v < a.shape[2]):
            h[t] = -h[t] - 0.0
    return h


def gather_wraps_negative_ids(ids, a, token_slot, ranks, r_max, tokens=None, a_is_bf16_bits=False):
    ids = np.asarray(ids) % a.shape[2]
    return O.gather_shrink(ids, a, token_slot, ranks, r_max, tokens, a_is_bf16_bits)


# --- addressing, apply_linear and bf16 mutants -----------------------------

def ranks_slot_le_S(token_slot, ranks, r_max):
    # slot id S read as the last slot (an off-by-one bound)
    ts = np.asarray(token_slot).ravel().copy()
    S = len(np.asarray(ranks).ravel())
    ts[ts == S] = S - 1
    return O.token_ranks(ts, ranks, r_max)


def ranks_negative_slot_wraps(token_slot, ranks, r_max):
    # negative slot ids index from the end, as Python lists do
    ts = np.asarray(token_slot).ravel().copy()
    S = len(np.asarray(ranks).ravel())
    ts[(ts < 0) & (ts >= -S)] += S
    return O.token_ranks(ts, ranks, r_max)


def ranks_unclamped_above(token_slot, ranks, r_max):
    # a rank above r_max counted raw
    return O.token_ranks(token_slot, ranks, 10 ** 6)


def ranks_abs_negative(token_slot, ranks, r_max):
    # a negative rank taken by magnitude instead of clamped to 0
    return O.token_ranks(token_slot, np.abs(np.asarray(ranks)), r_max)


def active_zero_adapter(token_slot, ranks, r_max):
    # rank-0 slots counted as active (>= instead of >)
    ts = np.asarray(token_slot).ravel()
    S = len(np.asarray(ranks).ravel())
    return (ts >= 0) & (ts < S)


def active_mask_of(rank_fn):
    return lambda token_slot, ranks, r_max: rank_fn(token_slot, ranks, r_max) > 0


def apply_no_scaling(x, y, a, b, token_slot, ranks, scalings, out_slices, r_max, tokens=None):
    return O.apply_linear(x, y, a, b, token_slot, ranks, np.ones(len(ranks)), out_slices, r_max, tokens)


def apply_swapped_slices(x, y, a, b, token_slot, ranks, scalings, out_slices, r_max, tokens=None):
    h = O.shrink(x, a, token_slot, ranks, len(out_slices), r_max, tokens=tokens)
    if h.shape[1] > 1:
        h = h[:, ::-1, :]
    return O.expand_fused(h, b, token_slot, ranks, scalings, y, out_slices, r_max, tokens=tokens)


def apply_touches_inactive(x, y, a, b, token_slot, ranks, scalings, out_slices, r_max, tokens=None):
    return O.apply_linear(x, y, a, b, token_slot, ranks, scalings, out_slices, r_max, tokens) + 0.0


def bf16_shift15(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 15).view(np.float32).astype(np.float64)


def bf16_as_fp16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_drops_sign(bits):
    return np.abs(O.bf16_bits_to_f64(bits))


def _round_with(v, rule, floor_exp=True, overflow=True):
    """round_to_bf16 with one step replaced (for the mutants below)."""
    v = _f(v)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0.0)
    a = np.abs(v[fin])
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -126) if floor_exp else ex - 1
    spacing = np.ldexp(1.0, e - 7)
    r = rule(a / spacing) * spacing
    if overflow:
        r[r >= 2.0 ** 128] = np.inf
    else:
        r = np.minimum(r, 255 * 2.0 ** 120)
    out[fin] = np.copysign(r, v[fin])
    return out


def round_truncates(v):
    return _round_with(v, np.floor)


def round_ties_away(v):
    return _round_with(v, lambda n: np.floor(n + 0.5))


def round_saturates(v):
    return _round_with(v, np.rint, overflow=False)


def round_no_subnormals(v):
    return _round_with(v, np.rint, floor_exp=False)


def round_twice_via_f32(v):
    with np.errstate(over="ignore"):
        f = _f(v).astype(np.float32)
    return O.round_to_bf16(f.astype(np.float64))


MUTANTS = {
    "ranks_slot_le_S": dict(token_ranks=ranks_slot_le_S, active_mask=active_mask_of(ranks_slot_le_S)),
    "ranks_negative_slot_wraps": dict(token_ranks=ranks_negative_slot_wraps,
                                      active_mask=active_mask_of(ranks_negative_slot_wraps)),
    "ranks_unclamped_above": dict(token_ranks=ranks_unclamped_above),
    "ranks_abs_negative": dict(token_ranks=ranks_abs_negative, active_mask=active_mask_of(ranks_abs_negative)),
    "active_zero_adapter": dict(active_mask=active_zero_adapter),
    "apply_no_scaling": dict(apply_linear=apply_no_scaling),
    "apply_swapped_slices": dict(apply_linear=apply_swapped_slices),
    "apply_touches_inactive": dict(apply_linear=apply_touches_inactive),
    "bf16_shift15": dict(bf16_bits_to_f64=bf16_shift15),
    "bf16_as_fp16": dict(bf16_bits_to_f64=bf16_as_fp16),
    "bf16_drops_sign": dict(bf16_bits_to_f64=bf16_drops_sign),
    "round_truncates": dict(round_to_bf16=round_truncates),
    "round_ties_away": dict(round_to_bf16=round_ties_away),
    "round_saturates": dict(round_to_bf16=round_saturates),
    "round_no_subnormals": dict(round_to_bf16=round_no_subnormals),
    "round_twice_via_f32": dict(round_to_bf16=round_twice_via_f32),
    "fwd_no_scale": dict(lora_fwd=fwd_no_scale),
    "fwd_overwrites": dict(lora_fwd=fwd_overwrites),
    "fwd_squared_scale": dict(lora_fwd=fwd_squared_scale),
    "fwd_drops_last_rank": dict(lora_fwd=fwd_drops_last_rank),
    "dxda_no_scale_on_dA": dict(lora_bwd_dx_da=dxda_no_scale_on_dA),
    "dxda_wrong_sign": dict(lora_bwd_dx_da=dxda_wrong_sign),
    "dxda_token_index": dict(lora_bwd_dx_da=dxda_uses_dy_not_dyb),
    "db_no_scale": dict(lora_bwd_db=db_no_scale),
    "db_token_order": dict(lora_bwd_db=db_transposed_tokens),
    "group_unstable": dict(group_tokens=group_unstable),
    "group_keeps_rank0": dict(group_tokens=group_keeps_rank0),
    "shrink_ignores_rank": dict(shrink=shrink_ignores_rank),
    "shrink_slice_offset": dict(shrink=shrink_slice_offset_by_rank),
    "expand_no_scaling": dict(expand_fused=expand_no_scaling),
    "expand_touches_inactive": dict(expand_fused=expand_touches_inactive),
    "expand_wrong_slice": dict(expand_fused=expand_wrong_slice),
    "gather_negative_zero": dict(gather_shrink=gather_negative_zero),
    "gather_wraps_ids": dict(gather_shrink=gather_wraps_negative_ids),
}


def test_real_oracle_passes_every_pin():
    P.run_all(oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    """Every planted mistake fails at least one pin that is not a hand-worked
    example (so the catch does not rest on one fixture alone)."""
    failing = P.failing_pins(_ns(**MUTANTS[name]))
    assert any(not f.startswith("golden") for f in failing), failing
