"""bfloat16 outputs: the forward's Y (lora_fwd with a bfloat16 res, the
dtype argument of the NeMo lora_forward_wrapper entry) and the multi-adapter
y (lora_expand_fused and lora_apply_linear, the in-place y of the M*
LoraOpsBackend.expand_fused entry), updated in place; the backward's dX
(overwritten or accumulated), dA and dB (the dtype of the NeMo
lora_da_dx_update_wrapper and lora_db_update_wrapper outputs).

The stored value is the exact result rounded once to the nearest bfloat16
(oracle.round_to_bf16 of the float64 oracle). Integer inputs make the
device's float32 sum exact, so its one rounding must give those bits exactly;
on the workloads' normal inputs every element must lie within one bfloat16
spacing of the exact value plus the float32 path's error bound (2^-16 of the
magnitudes added), match the rounded oracle except where the float32 sum
crossed a rounding midpoint (at most 2^-7 of the elements), and keep the
relative Frobenius error within 2e-3. Rows of inactive tokens and
the padding columns of a strided output keep their bits.
"""
import numpy as np
import pytest
import torch

import lora_rank_adapter_amd as L
import oracle
import synth
from tests.gpu_util import DEV, check_bf16_output, dev, exactness_bounds, f32, host_bf16, note

pytestmark = pytest.mark.gpu

# M, K, L, r, scale, row stride of Y (None: contiguous)
FWD_SHAPES = {
    "fused-r16": (96, 256, 264, 16, 2.0, None),
    "fused-r64": (2000, 512, 1024, 64, 0.5, None),
    "fused-r128-shared-tile": (256, 512, 512, 128, 0.5, None),
    "fused-padded-rows": (300, 1024, 200, 8, 1.0, 208),
    "split-K8200": (130, 8200, 512, 32, 2.0, None),
}
# which forward schedule each shape reaches: the fused kernel (private or,
# at rank 128, shared output tiles) up to a contraction of 8192; beyond it
# the shrink kernel and the column-band expand
DENSITY = (1.0 / 8, 1.0 / 4, 1.0 / 4, 1.0 / 8)


def _bf16_y(y0: np.ndarray, ld=None) -> tuple[torch.Tensor, torch.Tensor]:
    """(storage, view) of a bfloat16 output holding y0 (values on the bf16
    grid); with ld, rows of ld elements whose tail holds a sentinel."""
    M, N = y0.shape
    if ld is None:
        t = dev(y0, "bf16")
        return t, t
    store = dev(np.full((M, ld), 7.0, np.float32), "bf16")
    view = store[:, :N]
    view.copy_(dev(y0, "bf16"))
    return store, view


@pytest.mark.parametrize("kind", ["normal", "exact"])
@pytest.mark.parametrize("shape", sorted(FWD_SHAPES))
def test_fwd_bf16_output(shape, kind):
    M, K, N, r, s, ld = FWD_SHAPES[shape]
    note(f"bf16 Y forward {shape} {kind}")
    c = synth.single_adapter(M, K, N, r, seed=40 + M, dtype="bf16", scale=s, y0="normal",
                             int_exact=kind == "exact", density=DENSITY if kind == "exact" else None)
    y0 = synth.round_bf16(c.Y0)
    X = dev(c.X, "bf16")
    A_w = dev(np.ascontiguousarray(c.A.T), "bf16")   # lora_A weight, r x K
    B_w = dev(np.ascontiguousarray(c.B.T), "bf16")   # lora_B weight, L x r
    store, y = _bf16_y(y0, ld)
    L.lora_fwd(X, A_w.t(), B_w.t(), y, s)
    torch.cuda.synchronize()
    exact = oracle.lora_fwd(c.X, c.A, c.B, y0, s)
    rounded = oracle.round_to_bf16(exact)
    got = host_bf16(y)
    if kind == "exact":
        assert np.array_equal(got, rounded), "Y: one rounding of an exact float32 sum"
    else:
        mag = oracle.lora_fwd(np.abs(c.X), np.abs(c.A), np.abs(c.B), np.abs(y0), abs(s))
        check_bf16_output(got, exact, rounded, mag, "Y")
        assert oracle.rel_frobenius(got, exact) <= 2e-3
    if ld is not None:
        assert (host_bf16(store)[:, N:] == 7.0).all(), "padding columns were written"


def test_fwd_bf16_output_refuses_f32_inputs():
    """A bfloat16 Y needs bfloat16 inputs: LORA_ERR_DTYPE, Y untouched."""
    note("bf16 Y with f32 inputs")
    x = torch.zeros((16, 64), device=DEV)
    a = torch.zeros((64, 8), device=DEV)
    b = torch.zeros((8, 32), device=DEV)
    y = torch.full((16, 32), 3.0, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(L.LoraError) as e:
        L.lora_fwd(x, a, b, y, 1.0)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())


# ---- multi-adapter --------------------------------------------------------

# name, T, K, out_slices, S, r_max, rank choices, zero-adapter probability;
# the expand and apply_linear schedule each reaches
MULTI = {
    "decode-stream": (200, 256, (128, 64, 64), 9, 40, (0, 3, 17, 40), 0.1),       # streaming expand
    "band": (0, 256, (256, 64, 64), 12, 64, (8, 16, 32, 64), 0.0),              # column-band expand (>= 512 tokens)
    "one-launch-r128": (640, 512, (1536, 256, 256), 16, 128, (0, 8, 100, 128), 0.1),   # one-launch apply_linear
    "wide-two-launch": (1000, 256, (3000, 500, 500), 16, 64, (0, 16, 40, 64), 0.1),   # too wide for one launch
}


def _multi(name, int_exact):
    T, K, out_slices, S, r_max, choices, zero_p = MULTI[name]
    rng = np.random.default_rng(2000 + len(name))
    if T == 0:
        ts, ranks, _ = synth.prefill_routing(20, S, choices, rng, median=150.0, sigma=0.5, cap=400)
    else:
        ts, ranks = synth.decode_routing(T, S, r_max, choices, zero_p, rng)
        ts[3], ts[5] = -1, S          # slot ids outside [0, S): inactive
        if name == "one-launch-r128":
            ranks[1], ranks[2] = -3, r_max + 5
    m = synth.multi_lora(ts, ranks, K, out_slices, r_max, rng=rng, int_exact=int_exact, name=name)
    m.y0[:] = synth.round_bf16(m.y0)    # y starts on the bf16 grid (inactive rows -0.0)
    return m


def _addr(m):
    ts = torch.from_numpy(m.token_slot).to(DEV)
    ranks = torch.from_numpy(m.ranks).to(DEV)
    return L.lora_addressing_build(L.Addressing(ts, m.S), ranks, m.r_max), ranks


def _check_multi(m, got, exact, kind, mag=None):
    act = oracle.active_mask(m.token_slot, m.ranks, m.r_max)
    y0_bits = synth.bf16_bits(m.y0)
    got_bits = synth.bf16_bits(got.astype(np.float32))
    assert np.array_equal(got_bits[~act], y0_bits[~act]), "rows of inactive tokens were written"
    rounded = oracle.round_to_bf16(exact)
    if kind == "exact":
        assert np.array_equal(got[act], rounded[act])
    else:
        check_bf16_output(got[act], exact[act], rounded[act], mag[act], "y")
        assert oracle.rel_frobenius(got[act], exact[act]) <= 2e-3


@pytest.mark.parametrize("kind", ["normal", "exact"])
@pytest.mark.parametrize("name", sorted(MULTI))
def test_expand_fused_bf16_y(name, kind):
    m = _multi(name, kind == "exact")
    note(f"bf16 y expand_fused {name} {kind} T={m.T}")
    addr, ranks = _addr(m)
    rng = np.random.default_rng(5)
    hin = rng.integers(-2, 3, size=(m.T, m.num_slices, m.r_max)).astype(np.float32) if kind == "exact" else \
        rng.standard_normal((m.T, m.num_slices, m.r_max)).astype(np.float32)
    y = dev(m.y0, "bf16")
    L.lora_expand_fused(f32(hin), dev(m.b, "bf16"), addr, ranks, f32(m.scalings), y, m.out_slices, m.r_max)
    torch.cuda.synchronize()
    exact = oracle.expand_fused(hin, m.b, m.token_slot, m.ranks, m.scalings, m.y0, m.out_slices, m.r_max)
    mag = oracle.expand_fused(np.abs(hin), np.abs(m.b), m.token_slot, m.ranks, np.abs(m.scalings), np.abs(m.y0),
                              m.out_slices, m.r_max)
    _check_multi(m, host_bf16(y), exact, kind, mag)


@pytest.mark.parametrize("kind", ["normal", "exact"])
@pytest.mark.parametrize("name", sorted(MULTI))
def test_apply_linear_bf16_y(name, kind):
    """One launch (the one-launch cases) or shrink then expand (the others)
    into a bfloat16 y."""
    m = _multi(name, kind == "exact")
    note(f"bf16 y apply_linear {name} {kind} T={m.T}")
    addr, ranks = _addr(m)
    x, a, b, sc = dev(m.x, "bf16"), dev(m.a, "bf16"), dev(m.b, "bf16"), f32(m.scalings)
    y = dev(m.y0, "bf16")
    L.lora_apply_linear(x, y, a, b, addr, ranks, sc, m.out_slices, m.r_max)
    torch.cuda.synchronize()
    exact = oracle.apply_linear(m.x, m.y0, m.a, m.b, m.token_slot, m.ranks, m.scalings, m.out_slices, m.r_max)
    mag = oracle.apply_linear(np.abs(m.x), np.abs(m.y0), np.abs(m.a), np.abs(m.b), m.token_slot, m.ranks,
                              np.abs(m.scalings), m.out_slices, m.r_max)
    _check_multi(m, host_bf16(y), exact, kind, mag)


def test_expand_general_kernel_bf16_y():
    """Rows of h that are not 16-byte aligned send a bfloat16 y through the
    general expand kernel: integer inputs, exact."""
    m = _multi("decode-stream", True)
    note(f"bf16 y general expand T={m.T}")
    addr, ranks = _addr(m)
    rng = np.random.default_rng(6)
    hin = rng.integers(-2, 3, size=(m.T, m.num_slices, m.r_max)).astype(np.float32)
    buf = torch.full((m.T, m.num_slices, m.r_max + 1), float("nan"), device=DEV)
    h = buf[:, :, :m.r_max]
    h.copy_(f32(hin))
    y = dev(m.y0, "bf16")
    L.lora_expand_fused(h, dev(m.b, "bf16"), addr, ranks, f32(m.scalings), y, m.out_slices, m.r_max)
    torch.cuda.synchronize()
    exact = oracle.expand_fused(hin, m.b, m.token_slot, m.ranks, m.scalings, m.y0, m.out_slices, m.r_max)
    _check_multi(m, host_bf16(y), exact, "exact")


def test_expand_bf16_y_refuses_f32_weights():
    """A bfloat16 y needs bfloat16 weights: LORA_ERR_DTYPE, y untouched."""
    note("bf16 y with f32 weights")
    m = _multi("decode-stream", True)
    addr, ranks = _addr(m)
    y = dev(m.y0, "bf16")
    with pytest.raises(L.LoraError) as e:
        L.lora_expand_fused(f32(np.zeros((m.T, m.num_slices, m.r_max), np.float32)), dev(m.b, "f32"), addr, ranks,
                            f32(m.scalings), y, m.out_slices, m.r_max)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(y), m.y0.astype(np.float64))


# ---- single-adapter backward ----------------------------------------------

# M, K, L, r, scale: the fused dX kernel (rank 16, 64) and the split schedule
# (a contraction over 8200 outputs: band expand beside dA's partials, dB's
# 8-wave weight-gradient workgroups)
BWD_SHAPES = {
    "fused-r20-packed": (150, 256, 264, 20, 1.0),   # rank not a multiple of 8: weights packed first
    "fused-r16": (96, 256, 264, 16, 2.0),
    "fused-r64": (300, 512, 520, 64, 0.5),
    "split-r64": (130, 264, 8200, 64, 0.5),
    "split-r128": (200, 512, 8200, 128, 1.0),
}
BWD_DENSITY = (1.0 / 8, 1.0 / 4, 1.0 / 4, 1.0 / 8)


@pytest.mark.parametrize("kind", ["normal", "exact"])
@pytest.mark.parametrize("shape", sorted(BWD_SHAPES))
def test_bwd_bf16_outputs(shape, kind):
    """dX (overwritten and accumulated into a bfloat16 base), dA and dB in
    bfloat16 (the dtype of the NeMo lora_da_dx_update_wrapper and
    lora_db_update_wrapper outputs): each element the float32 result rounded
    once."""
    M, K, N, r, s = BWD_SHAPES[shape]
    note(f"bf16 backward outputs {shape} {kind}")
    c = synth.single_adapter(M, K, N, r, seed=60 + r, dtype="bf16", scale=s, int_exact=kind == "exact",
                             density=BWD_DENSITY if kind == "exact" else None)
    if kind == "exact":
        # every float32 partial sum exact (checked before the GPU runs)
        b = exactness_bounds(c)
        assert b["dyb"] < 2 ** 15 and max(b["dx"], b["dA"], b["dB"]) < 2 ** 20, b
    X = dev(c.X, "bf16")
    dY = dev(c.dY, "bf16")
    A_w = dev(np.ascontiguousarray(c.A.T), "bf16")   # lora_A weight, r x K
    B_w = dev(np.ascontiguousarray(c.B.T), "bf16")   # lora_B weight, L x r
    rng = np.random.default_rng(7)
    base = synth.round_bf16(rng.integers(-3, 4, (M, K)).astype(np.float32) if kind == "exact"
                            else rng.standard_normal((M, K)).astype(np.float32))
    dx, dA = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, s, dtype=torch.bfloat16)
    dB = L.lora_bwd_db(A_w, X.t(), dY, s, dtype=torch.bfloat16)
    dxa = dev(base, "bf16")
    L.lora_bwd_dx_da_accumulate(X.t(), dY, B_w, A_w, s, dxa, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert dx.dtype == dA.dtype == dB.dtype == torch.bfloat16
    odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, s)
    odB = oracle.lora_bwd_db(c.A.T, c.X.T, c.dY, s)
    cases = [("dX", host_bf16(dx), odx), ("dA", host_bf16(dA), odA), ("dB", host_bf16(dB), odB),
             ("dX accumulated", host_bf16(dxa), base.astype(np.float64) + odx)]
    if kind == "exact":
        for name, got, exact in cases:
            assert np.array_equal(got, oracle.round_to_bf16(exact)), f"{name}: one rounding of an exact float32 value"
        return
    aX, adY, aA, aB = np.abs(c.X), np.abs(c.dY), np.abs(c.A), np.abs(c.B)
    mdx, mdA = oracle.lora_bwd_dx_da(aX.T, adY, aB.T, aA.T, abs(s))
    mdB = oracle.lora_bwd_db(aA.T, aX.T, adY, abs(s))
    mags = [mdx, mdA, mdB, np.abs(base).astype(np.float64) + mdx]
    for (name, got, exact), mag in zip(cases, mags):
        check_bf16_output(got, exact, oracle.round_to_bf16(exact), mag, name)
        assert oracle.rel_frobenius(got, exact) <= 2e-3, name


def test_bwd_bf16_outputs_refuse_f32_inputs():
    """bfloat16 backward outputs need bfloat16 inputs: LORA_ERR_DTYPE."""
    note("bf16 backward outputs with f32 inputs")
    M, K, N, r = 32, 64, 64, 8
    xt = torch.zeros((M, K), device=DEV).t()
    dy = torch.zeros((M, N), device=DEV)
    Bw = torch.zeros((N, r), device=DEV)
    Aw = torch.zeros((r, K), device=DEV)
    for kw in ({"dx": torch.zeros((M, K), device=DEV, dtype=torch.bfloat16)},
               {"dA": torch.zeros((K, r), device=DEV, dtype=torch.bfloat16)}):
        with pytest.raises(L.LoraError) as e:
            L.lora_bwd_dx_da(xt, dy, Bw, Aw, 1.0, **kw)
        assert e.value.status == -3
    with pytest.raises(L.LoraError) as e:
        L.lora_bwd_db(Aw, xt, dy, 1.0, dtype=torch.bfloat16)
    assert e.value.status == -3


def test_bwd_bf16_dx_padded_rows():
    """A bfloat16 dX with padded rows (row stride K + 8): the padding columns
    keep their bits, overwritten and accumulated; integer inputs, exact."""
    M, K, N, r, s = 130, 256, 264, 16, 2.0
    note("bf16 dX with padded rows")
    c = synth.single_adapter(M, K, N, r, seed=66, dtype="bf16", scale=s, int_exact=True, density=BWD_DENSITY)
    X, dY = dev(c.X, "bf16"), dev(c.dY, "bf16")
    A_w = dev(np.ascontiguousarray(c.A.T), "bf16")
    B_w = dev(np.ascontiguousarray(c.B.T), "bf16")
    store = dev(np.full((M, K + 8), 7.0, np.float32), "bf16")
    dx = store[:, :K]
    L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, s, dx=dx, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    odx, _ = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, s)
    assert np.array_equal(host_bf16(dx), oracle.round_to_bf16(odx))
    L.lora_bwd_dx_da_accumulate(X.t(), dY, B_w, A_w, s, dx, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(dx), oracle.round_to_bf16(oracle.round_to_bf16(odx) + odx))
    assert (host_bf16(store)[:, K:] == 7.0).all(), "padding columns were written"
