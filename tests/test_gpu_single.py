"""GPU parity of the single-adapter forward and backward against the CPU oracle.

Every case goes through the C ABI (ctypes binding). Tolerances: relative
Frobenius error <= 2e-3 for bf16 inputs, <= 1e-5 for fp32 inputs, measured on
the added delta for the in-place forward; bitwise equality for integer-valued
inputs whose every partial sum is exact in fp32.
"""
import numpy as np
import pytest
import torch

import lora_rank_adapter_amd as L
import oracle
import synth
from tests.gpu_util import dev, exactness_bounds, f32, host, note, same_bits, tol

pytestmark = pytest.mark.gpu

# (M, K, L, r, dtype, scale): ragged against every tile size (16-token blocks,
# 32/16-wide contraction steps, 4-wave feature split, 16-column output blocks,
# 256-column gradient slices, 32-token gradient stages).
CASES = [
    (200, 264, 1000, 16, "bf16", 2.0),
    (77, 128, 64, 1, "bf16", 0.5),
    (300, 512, 256, 5, "bf16", 1.0),
    (129, 1032, 520, 33, "bf16", 2.0),
    (64, 4096, 128, 64, "bf16", 0.5),
    (40, 256, 96, 128, "bf16", 2.0),
    (1, 8, 8, 7, "bf16", 1.5),
    (517, 2048, 1536, 100, "bf16", 0.25),
    (256, 512, 512, 8, "f32", 2.0),
    (70, 132, 300, 19, "f32", 0.5),
    (33, 4, 8, 128, "f32", 1.0),
]


def _ids(c):
    return "M{}-K{}-L{}-r{}-{}".format(*c[:5])


def _upload(c, dtype):
    X = dev(c.X, dtype)
    A_w = dev(np.ascontiguousarray(c.A.T), dtype)   # lora_A weight, r x K
    B_w = dev(np.ascontiguousarray(c.B.T), dtype)   # lora_B weight, L x r
    dY = dev(c.dY, dtype)
    return X, A_w, B_w, dY


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_fwd(case):
    M, K, L_, r, dtype, s = case
    note(f"fwd {case}")
    c = synth.single_adapter(M, K, L_, r, seed=100 + M, dtype=dtype, scale=s, y0="normal")
    X, A_w, B_w, _ = _upload(c, dtype)
    y = f32(c.Y0)
    L.lora_fwd(X, A_w.t(), B_w.t(), y, s)
    torch.cuda.synchronize()
    want = oracle.lora_fwd(c.X, c.A, c.B, c.Y0, s)
    err = oracle.rel_frobenius(host(y) - c.Y0, want - c.Y0)
    assert err <= tol(dtype), err


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_bwd(case):
    M, K, L_, r, dtype, s = case
    note(f"bwd {case}")
    c = synth.single_adapter(M, K, L_, r, seed=200 + M, dtype=dtype, scale=s)
    X, A_w, B_w, dY = _upload(c, dtype)
    dx, dA = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, s)
    dB = L.lora_bwd_db(A_w, X.t(), dY, s)
    torch.cuda.synchronize()
    odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, s)
    odB = oracle.lora_bwd_db(c.A.T, c.X.T, c.dY, s)
    for name, g, w in (("dX", dx, odx), ("dA", dA, odA), ("dB", dB, odB)):
        err = oracle.rel_frobenius(host(g), w)
        assert err <= tol(dtype), (name, err)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("s", [2.0, 0.5])
def test_integer_exact_bitwise(dtype, s):
    """Integer inputs in [-2, 2]: every fp32 partial sum (and the hi+lo split)
    is exact, so any summation order gives the oracle's value bit for bit."""
    note(f"integer-exact {dtype} s={s}")
    M, K, L_, r = 96, 256, 200, 16
    c = synth.single_adapter(M, K, L_, r, seed=31, dtype=dtype, scale=s, y0="normal", int_exact=True)
    X, A_w, B_w, dY = _upload(c, dtype)
    y = f32(c.Y0)
    L.lora_fwd(X, A_w.t(), B_w.t(), y, s)
    dx, dA = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, s)
    dB = L.lora_bwd_db(A_w, X.t(), dY, s)
    torch.cuda.synchronize()
    assert same_bits(host(y), oracle.lora_fwd(c.X, c.A, c.B, c.Y0, s).astype(np.float32))
    odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, s)
    assert same_bits(host(dx), odx.astype(np.float32))
    assert same_bits(host(dA), odA.astype(np.float32))
    assert same_bits(host(dB), oracle.lora_bwd_db(c.A.T, c.X.T, c.dY, s).astype(np.float32))


def test_weight_layouts_and_output_strides():
    """Weights given in the other orientation (packed by the library) and
    strided gradient outputs give the same results as the natural layouts."""
    note("layouts")
    M, K, L_, r, s = 150, 384, 272, 24, 2.0
    c = synth.single_adapter(M, K, L_, r, seed=41, dtype="bf16", scale=s, y0="normal")
    X, A_w, B_w, dY = _upload(c, "bf16")
    A_kr = dev(c.A, "bf16")          # K x r contiguous
    B_rl = dev(c.B, "bf16")          # r x L contiguous
    y1 = f32(c.Y0)
    y2 = f32(c.Y0)
    L.lora_fwd(X, A_w.t(), B_w.t(), y1, s)
    L.lora_fwd(X, A_kr, B_rl, y2, s)
    dx1, dA1 = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, s)
    dA_rk = torch.empty((r, K), dtype=torch.float32, device=X.device)   # dA stored r x K (lora_A layout)
    dx2, _ = L.lora_bwd_dx_da(X.t(), dY, B_rl.t(), A_kr.t(), s, dA=dA_rk.t())
    dB1 = L.lora_bwd_db(A_w, X.t(), dY, s)
    dB_lr = torch.empty((L_, r), dtype=torch.float32, device=X.device)  # dB stored L x r (lora_B layout)
    L.lora_bwd_db(A_kr.t(), X.t(), dY, s, dB=dB_lr.t())
    torch.cuda.synchronize()
    assert same_bits(host(y1), host(y2))
    assert same_bits(host(dx1), host(dx2))
    assert same_bits(host(dA1), host(dA_rk.t()))
    assert same_bits(host(dB1), host(dB_lr.t()))
    want = oracle.lora_fwd(c.X, c.A, c.B, c.Y0, s)
    assert oracle.rel_frobenius(host(y1) - c.Y0, want - c.Y0) <= 2e-3


# (M, K, L, r): the fused dX kernel at rank 8 (half of one rank block), 16
# and 64, the split schedule's shrink + band expand beside dA's partials at
# rank 8, 64 and 128
IN_PLACE_CASES = [(200, 264, 1000, 16), (130, 512, 296, 64), (2100, 264, 8200, 64), (700, 1032, 8200, 128),
                  (96, 256, 200, 8), (400, 512, 8208, 8)]


@pytest.mark.parametrize("case", IN_PLACE_CASES, ids=lambda c: "M{}-K{}-L{}-r{}".format(*c))
def test_bwd_weights_read_in_place(case):
    """bf16 weights in the nn.Linear layouts are read in place by the dX/dA
    call (lora_B's feature rows and lora_A's rank rows staged and read
    transposed); weights in padded rows, and weights whose rows do not start
    16-byte aligned (packed by the library instead), give the same bits."""
    M, K, L_, r = case
    note(f"weights in place {case}")
    c = synth.single_adapter(M, K, L_, r, seed=70 + r, dtype="bf16", scale=0.5)
    X, A_w, B_w, dY = _upload(c, "bf16")
    dx1, dA1 = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, 0.5)
    # rows padded to r + 8 and K + 8 elements (in place, other strides)
    B_pad = torch.zeros((L_, r + 8), dtype=B_w.dtype, device=X.device)
    B_pad[:, :r] = B_w
    A_pad = torch.zeros((r, K + 8), dtype=A_w.dtype, device=X.device)
    A_pad[:, :K] = A_w
    dx2, dA2 = L.lora_bwd_dx_da(X.t(), dY, B_pad[:, :r], A_pad[:, :K], 0.5)
    # rows starting 2 bytes past a 16-byte boundary: packed
    B_off = torch.zeros((L_ * r + 1,), dtype=B_w.dtype, device=X.device)
    B_off[1:] = B_w.reshape(-1)
    dx3, dA3 = L.lora_bwd_dx_da(X.t(), dY, B_off[1:].view(L_, r), A_w, 0.5)
    torch.cuda.synchronize()
    for got in ((dx2, dA2), (dx3, dA3)):
        assert same_bits(host(got[0]), host(dx1)), "dX"
        assert same_bits(host(got[1]), host(dA1)), "dA"
    odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, 0.5)
    assert oracle.rel_frobenius(host(dx1), odx) <= 2e-3
    assert oracle.rel_frobenius(host(dA1), odA) <= 2e-3


def test_bwd_in_place_weights_launch_no_pack():
    """The dX/dA call on nn.Linear-layout bf16 weights launches three kernels
    (fused shrink-expand, weight-gradient partials, reduce); weights that
    must be packed first add the pack launch."""
    note("in-place weights: launch count")
    M, K, L_, r = 600, 1024, 768, 16
    c = synth.single_adapter(M, K, L_, r, seed=62, dtype="bf16", scale=1.0)
    X, A_w, B_w, dY = _upload(c, "bf16")
    B_off = torch.zeros((L_ * r + 1,), dtype=B_w.dtype, device=X.device)
    B_off[1:] = B_w.reshape(-1)
    counts = []
    for b in (B_w, B_off[1:].view(L_, r)):
        torch.cuda.synchronize()
        L.lora_timing_begin()
        L.lora_bwd_dx_da(X.t(), dY, b, A_w, 1.0)
        L.lora_timing_pause()
        counts.append(L.lora_timing_read()[1])
    torch.cuda.synchronize()
    assert counts == [3, 4], counts


def test_deterministic_reruns():
    note("determinism")
    c = synth.single_adapter(333, 1024, 640, 48, seed=51, dtype="bf16", scale=0.5)
    X, A_w, B_w, dY = _upload(c, "bf16")
    outs = []
    for _ in range(2):
        y = torch.zeros((333, 640), dtype=torch.float32, device=X.device)
        L.lora_fwd(X, A_w.t(), B_w.t(), y, 0.5)
        dx, dA = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, 0.5)
        dB = L.lora_bwd_db(A_w, X.t(), dY, 0.5)
        torch.cuda.synchronize()
        outs.append([host(t) for t in (y, dx, dA, dB)])
    for a, b in zip(*outs):
        assert same_bits(a, b)


def test_kernel_timing_records_each_launch():
    """Timed launches (hipExtLaunchKernel with events) give the same bits as
    untimed ones, one record per kernel; pausing stops the records."""
    note("kernel timing")
    c = synth.single_adapter(600, 1024, 768, 16, seed=61, dtype="bf16", scale=2.0, y0="normal")
    X, A_w, B_w, dY = _upload(c, "bf16")
    y_plain = f32(c.Y0)
    L.lora_fwd(X, A_w.t(), B_w.t(), y_plain, 2.0)
    dx_plain, dA_plain = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, 2.0)
    torch.cuda.synchronize()
    y_timed = f32(c.Y0)
    torch.cuda.synchronize()
    L.lora_timing_begin()
    L.lora_fwd(X, A_w.t(), B_w.t(), y_timed, 2.0)
    L.lora_timing_pause()
    ms_fwd, n_fwd = L.lora_timing_read()
    assert n_fwd == 1 and 0.0 < ms_fwd < 1000.0
    L.lora_timing_resume()
    dx_t, dA_t = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, 2.0)
    L.lora_timing_pause()
    L.lora_fwd(X, A_w.t(), B_w.t(), f32(c.Y0), 2.0)   # untimed
    ms_all, n_all = L.lora_timing_read()
    assert n_all >= 3 and ms_all > ms_fwd               # dx/dA take at least two kernels
    assert same_bits(host(y_timed), host(y_plain))
    assert same_bits(host(dx_t), host(dx_plain))
    assert same_bits(host(dA_t), host(dA_plain))
    L.lora_timing_begin()
    L.lora_timing_pause()
    assert L.lora_timing_read() == (0.0, 0)


@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[5], CASES[7], CASES[8], CASES[9]], ids=_ids)
def test_bwd_dx_accumulate(case):
    """lora_bwd_dx_da_accumulate adds the input gradient into dx (a base
    layer's gradient of the same scale) and overwrites dA: compared with the
    oracle on the added delta, like the forward."""
    M, K, L_, r, dtype, s = case
    note(f"bwd dx accumulate {case}")
    c = synth.single_adapter(M, K, L_, r, seed=300 + M, dtype=dtype, scale=s)
    X, A_w, B_w, dY = _upload(c, dtype)
    odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, s)
    rms = float(np.sqrt(np.mean(odx * odx)))
    dx0 = (np.random.default_rng(M).standard_normal((M, K)) * rms).astype(np.float32)
    dx = f32(dx0)
    out, dA = L.lora_bwd_dx_da_accumulate(X.t(), dY, B_w, A_w, s, dx)
    torch.cuda.synchronize()
    assert out is dx
    assert oracle.rel_frobenius(host(dx) - dx0, odx) <= tol(dtype)
    assert oracle.rel_frobenius(host(dA), odA) <= tol(dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_dx_accumulate_integer_exact(dtype):
    """Integer inputs and an integer dx: every sum is exact, so dx must equal
    dx0 + the oracle's dX bit for bit."""
    note(f"bwd dx accumulate integer-exact {dtype}")
    M, K, L_, r, s = 96, 256, 200, 16, 2.0
    c = synth.single_adapter(M, K, L_, r, seed=32, dtype=dtype, scale=s, int_exact=True)
    X, A_w, B_w, dY = _upload(c, dtype)
    dx0 = np.random.default_rng(5).integers(-8, 9, size=(M, K)).astype(np.float32)
    dx = f32(dx0)
    _, dA = L.lora_bwd_dx_da_accumulate(X.t(), dY, B_w, A_w, s, dx)
    torch.cuda.synchronize()
    odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, s)
    assert same_bits(host(dx), (dx0 + odx).astype(np.float32))
    assert same_bits(host(dA), odA.astype(np.float32))


def test_bwd_dx_accumulate_empty_contraction():
    """L = 0: nothing to add, dx keeps its bits; dA is zero."""
    note("bwd dx accumulate, L = 0")
    dv = torch.device("cuda:0")
    bf = torch.bfloat16
    x = torch.randn((24, 64), device=dv).to(bf)
    a_w = torch.randn((8, 64), device=dv).to(bf)
    b_w = torch.empty((0, 8), dtype=bf, device=dv)
    dy = torch.empty((24, 0), dtype=bf, device=dv)
    dx0 = torch.randn((24, 64), device=dv)
    dx = dx0.clone()
    _, dA = L.lora_bwd_dx_da_accumulate(x.t(), dy, b_w, a_w, 1.0, dx, dA=torch.full((64, 8), 7.0, device=dv))
    torch.cuda.synchronize()
    assert torch.equal(dx, dx0) and not dA.any()


def test_empty_and_degenerate():
    note("empty")
    dv = torch.device("cuda:0")
    bf = torch.bfloat16
    # M = 0: forward is a no-op, gradients of the weights are zero
    x = torch.empty((0, 64), dtype=bf, device=dv)
    a_w = torch.randn((8, 64), device=dv).to(bf)
    b_w = torch.randn((32, 8), device=dv).to(bf)
    y = torch.empty((0, 32), dtype=torch.float32, device=dv)
    L.lora_fwd(x, a_w.t(), b_w.t(), y, 1.0)
    dy = torch.empty((0, 32), dtype=bf, device=dv)
    dx, dA = L.lora_bwd_dx_da(x.t(), dy, b_w, a_w, 1.0, dA=torch.full((64, 8), 7.0, device=dv))
    dB = L.lora_bwd_db(a_w, x.t(), dy, 1.0, dB=torch.full((8, 32), 7.0, device=dv))
    torch.cuda.synchronize()
    assert not dA.any() and not dB.any()
    # A = 0: the output is untouched bit for bit
    x = torch.randn((50, 64), device=dv).to(bf)
    y0 = torch.randn((50, 32), device=dv)
    y = y0.clone()
    L.lora_fwd(x, torch.zeros((8, 64), dtype=bf, device=dv).t(), b_w.t(), y, 3.0)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)


def test_bad_arguments_raise_before_launch():
    note("bad args")
    dv = torch.device("cuda:0")
    bf = torch.bfloat16
    x = torch.randn((16, 64), device=dv).to(bf)
    a_w = torch.randn((8, 64), device=dv).to(bf)
    b_w = torch.randn((32, 8), device=dv).to(bf)
    y = torch.zeros((16, 32), device=dv)
    with pytest.raises(L.LoraError) as e:
        L.lora_fwd(x, a_w.t(), b_w.t(), torch.zeros((16, 33), device=dv), 1.0)
    assert e.value.status == -2
    with pytest.raises(L.LoraError) as e:
        L.lora_fwd(x.float(), a_w.t(), b_w.t(), y, 1.0)
    assert e.value.status == -3
    with pytest.raises(L.LoraError) as e:
        L.lora_fwd(x.t().contiguous().t(), a_w.t(), b_w.t(), y, 1.0)   # column-major x
    assert e.value.status == -4
    big = torch.randn((129, 64), device=dv).to(bf)
    with pytest.raises(L.LoraError) as e:
        L.lora_fwd(x, big.t(), torch.randn((32, 129), device=dv).to(bf).t(), y, 1.0)
    assert e.value.status == -5
    assert torch.equal(y, torch.zeros_like(y))


def test_fp32_workload():
    """The fp32 workload (256 x 512 x 512, rank 8) in full: every row of Y and
    dX, all of dA and dB (the bf16 workloads: tests/test_gpu_fullsize.py)."""
    c = synth.config1()
    note(f"full size {c.name}")
    dtype = c.dtype
    X, A_w, B_w, dY = _upload(c, dtype)
    rows = np.arange(c.M)
    y = torch.zeros((c.M, c.L), dtype=torch.float32, device=X.device)
    L.lora_fwd(X, A_w.t(), B_w.t(), y, c.scale)
    torch.cuda.synchronize()
    want = oracle.lora_fwd(c.X[rows], c.A, c.B, c.Y0[rows], c.scale)
    assert oracle.rel_frobenius(host(y[torch.from_numpy(rows).to(X.device)]), want) <= tol(dtype)
    del y
    dx, dA = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, c.scale)
    dB = L.lora_bwd_db(A_w, X.t(), dY, c.scale)
    torch.cuda.synchronize()
    odx_rows, _ = oracle.lora_bwd_dx_da(c.X[rows].T, c.dY[rows], c.B.T, c.A.T, c.scale)
    rows_d = torch.from_numpy(rows).to(X.device)
    assert oracle.rel_frobenius(host(dx[rows_d]), odx_rows) <= tol(dtype)
    # the accumulating variant adds the same gradient once more
    base = host(dx[rows_d])
    L.lora_bwd_dx_da_accumulate(X.t(), dY, B_w, A_w, c.scale, dx, dA=torch.empty_like(dA))
    torch.cuda.synchronize()
    assert oracle.rel_frobenius(host(dx[rows_d]) - base, odx_rows) <= tol(dtype)
    # dA and dB contract over every token
    _, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, c.scale)
    assert oracle.rel_frobenius(host(dA), odA) <= tol(dtype)
    odB = oracle.lora_bwd_db(c.A.T, c.X.T, c.dY, c.scale)
    assert oracle.rel_frobenius(host(dB), odB) <= tol(dtype)


# Shapes that reach every branch of the library's schedule plan (chosen by
# shape alone): fused forward with 64-, 32- and 16-token tiles, fused dX with
# 32- and 16-token tiles, shrink tiles of 16, 32 and 64 tokens with 8 or 4
# waves, and the split schedule (shrink kernel + column-band expand; for dX
# the band expand and dA's partials in one launch) for contractions over more
# than 8192 features, forward outputs of 256 MB or more and dX outputs of
# 128 MB or more, with 32- and 16-token band tiles and token groups walking
# several tiles (ragged tails in every dimension), and dB's 8-wave
# weight-gradient workgroups (8192 or more outputs), in bf16 and f32.
PLAN_CASES = [
    (32768, 256, 264, 16, "bf16", 2.0),    # fused fwd 64-token tiles, fused dX 32-token tiles
    (16400, 512, 264, 40, "bf16", 0.5),    # fused fwd 32-token tiles, shrink 64-token tiles (4 waves)
    (9000, 264, 512, 100, "bf16", 1.0),    # rank 100 (8 rank blocks): shrink 32-token tiles, 4 waves
    (9000, 264, 512, 20, "bf16", 2.0),     # shrink 32-token tiles, 8 waves
    (1500, 8200, 2056, 128, "bf16", 0.5),  # split forward (long contraction), 16-token band tiles
    (1500, 2056, 8200, 128, "bf16", 2.0),  # split dX, same
    (4100, 8200, 1000, 16, "bf16", 1.0),   # split forward, 32-token band tiles
    (2100, 264, 8200, 64, "bf16", 0.5),    # split dX, 32-token band tiles
    (8200, 4096, 264, 16, "bf16", 2.0),    # split dX for a 134 MB dX (contraction 264)
    (300, 264, 8312, 16, "bf16", 1.0),     # dB over 8312 outputs: 8-wave weight-gradient workgroups, rank 16
    (16400, 256, 4104, 16, "bf16", 2.0),   # split forward for a 269 MB output (contraction 256)
    (3000, 8196, 300, 19, "f32", 0.5),     # split forward, f32
    (70, 132, 8196, 19, "f32", 2.0),       # split dX, f32
]
EXACT_DENSITY = (1.0 / 8, 1.0 / 4, 1.0 / 4, 1.0 / 8)


@pytest.mark.parametrize("case", PLAN_CASES, ids=_ids)
@pytest.mark.parametrize("kind", ["normal", "exact"])
def test_every_schedule_matches_oracle(case, kind):
    """Each branch of the schedule plan against the oracle: within tolerance
    for normal inputs, bit for bit for sparse signed inputs whose every
    partial sum is exact (checked before the GPU runs). Forward, dX (also
    accumulated), dA, dB."""
    M, K, L_, r, dtype, s = case
    note(f"schedule {kind} {case}")
    if kind == "exact":
        c = synth.single_adapter(M, K, L_, r, seed=600 + M, dtype=dtype, scale=s, y0="normal", int_exact=True,
                                 density=EXACT_DENSITY)
        b = exactness_bounds(c)
        assert b["h"] < 2 ** 15 and b["dyb"] < 2 ** 15, b
        assert max(b["y"], b["dx"], b["dA"], b["dB"]) < 2 ** 22, b
    else:
        c = synth.single_adapter(M, K, L_, r, seed=600 + M, dtype=dtype, scale=s, y0="normal")
    X, A_w, B_w, dY = _upload(c, dtype)
    y = f32(c.Y0)
    L.lora_fwd(X, A_w.t(), B_w.t(), y, s)
    dx, dA = L.lora_bwd_dx_da(X.t(), dY, B_w, A_w, s)
    dB = L.lora_bwd_db(A_w, X.t(), dY, s)
    dxa = dx.clone()
    L.lora_bwd_dx_da_accumulate(X.t(), dY, B_w, A_w, s, dxa)
    torch.cuda.synchronize()
    want = oracle.lora_fwd(c.X, c.A, c.B, c.Y0, s)
    odx, odA = oracle.lora_bwd_dx_da(c.X.T, c.dY, c.B.T, c.A.T, s)
    odB = oracle.lora_bwd_db(c.A.T, c.X.T, c.dY, s)
    if kind == "exact":
        assert same_bits(host(y), want.astype(np.float32)), "Y"
        assert same_bits(host(dx), odx.astype(np.float32)), "dX"
        assert same_bits(host(dxa), (2.0 * odx).astype(np.float32)), "dX accumulated"
        assert same_bits(host(dA), odA.astype(np.float32)), "dA"
        assert same_bits(host(dB), odB.astype(np.float32)), "dB"
        return
    assert oracle.rel_frobenius(host(y) - c.Y0, want - c.Y0) <= tol(dtype)
    assert oracle.rel_frobenius(host(dx), odx) <= tol(dtype)
    assert oracle.rel_frobenius(host(dxa) - host(dx), odx) <= tol(dtype)
    assert oracle.rel_frobenius(host(dA), odA) <= tol(dtype)
    assert oracle.rel_frobenius(host(dB), odB) <= tol(dtype)
