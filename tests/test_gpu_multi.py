"""GPU parity of the slot-addressed multi-adapter ops against the CPU oracle.

Grouping and gather_shrink are compared bit for bit; shrink and expand_fused
within a relative Frobenius error of 2e-3 (bf16 inputs) or 1e-5 (fp32),
on the entries the page specifies (active tokens, rank columns below the
slot's rank). Rows of inactive tokens must stay bitwise untouched and NaN
padding must never reach an output.
"""
import numpy as np
import pytest
import torch

import lora_rank_adapter_amd as L
import oracle
import synth
from tests.gpu_util import DEV, dev, f32, host, note, same_bits, tol

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0

# name, T, K, out_slices, S, r_max, rank choices, zero-adapter probability, dtype
CASES = [
    ("decode-small", 40, 256, (128, 64, 64), 6, 32, (0, 8, 16, 32), 0.1, "bf16"),
    ("ragged-ranks", 203, 520, (100, 28), 9, 40, (0, 3, 17, 40), 0.1, "bf16"),
    ("prefill-like", 1500, 1024, (512, 128, 128), 12, 128, (8, 16, 32, 64, 128), 0.0, "bf16"),
    ("fp32", 77, 64, (32, 16), 5, 16, (0, 4, 16), 0.2, "f32"),
    ("one-token", 1, 8, (4,), 1, 1, (1,), 0.0, "bf16"),
    ("prefill-long", 0, 512, (384, 128, 64), 12, 64, (8, 16, 32, 64), 0.0, "bf16"),
    ("fp32-prefill", 0, 256, (128, 64), 10, 32, (4, 16, 32), 0.0, "f32"),
    ("prefill-many-slots", 0, 256, (256, 64, 64), 176, 128, (8, 16, 64, 128), 0.0, "bf16"),
    ("decode-mid", 640, 512, (1536, 256, 256), 16, 128, (0, 8, 100, 128), 0.1, "bf16"),
    ("decode-wide", 1000, 256, (3000, 500, 500), 16, 64, (0, 16, 40, 64), 0.1, "bf16"),
    ("decode-1k", 1100, 256, (1024, 256), 8, 32, (0, 8, 32), 0.1, "bf16"),
    ("fp32-mid", 600, 64, (32, 16), 8, 16, (0, 4, 16), 0.2, "f32"),
    ("decode-many-slots", 400, 256, (128, 64), 1000, 32, (0, 8, 16, 32), 0.1, "bf16"),
]
# Which kernel each case reaches (the library picks by shape):
#   grouping: one token per thread (<= 1024 tokens): decode-small, ragged-ranks, fp32, one-token,
#             decode-mid, decode-wide, fp32-mid, decode-many-slots; one workgroup per 1024-token chunk: the others
#             (and test_grouping_schedules_bitwise for every grouping kernel);
#   shrink: row-split (bf16, >= 1024 tokens, a grid of >= 256 workgroups): prefill-many-slots;
#           pipelined, 64-token tiles, four rank blocks (>= 1024 tokens where the busiest CU streams
#             fewer rows so): prefill-like, prefill-long;
#           pipelined, 16-token tiles, four rank blocks (>= 512 tokens otherwise): fp32-prefill,
#             decode-mid, decode-wide, decode-1k, fp32-mid;
#           pipelined, 16-token tiles, one rank block, live units counted on the device (< 512
#             tokens): the others (decode-many-slots: a 1000-slot table, 16 chunks of the slot scan);
#           general (no buffer descriptors): test_shrink_general_kernel.
#   expand: column band (>= 512 tokens; 256-token pieces at r_max 128, 64 below): prefill-like,
#             prefill-long, fp32-prefill, prefill-many-slots, decode-mid, decode-wide, decode-1k, fp32-mid;
#           streaming (fewer): decode-small, ragged-ranks, fp32, one-token;
#           general (rows of h not 16-byte aligned): test_expand_general_kernel.
#   Every expand adds the MFMA chain of an element's rank blocks to y the same way, so all of them,
#   and both forms of apply_linear, give the same bits.
#   apply_linear: one launch (1024-column chunks): decode-mid (rank 128, two slots' ranks
#             outside [0, r_max]), decode-1k, fp32-mid;
#           shrink then expand: the others (decode-wide: a batch too wide for one launch).
ONE_LAUNCH = ("decode-mid", "decode-1k", "fp32-mid")
REQUESTS = {"prefill-like": 12, "fp32-prefill": 12, "prefill-long": 20, "prefill-many-slots": 16}


def _case(name, T, K, out_slices, S, r_max, choices, zero_p, dtype, seed=0, int_exact=False, wild_slots=True):
    rng = np.random.default_rng(1000 + seed + T)
    if name in REQUESTS:
        median, sigma = (150.0, 0.5) if name in ("prefill-long", "prefill-many-slots") else (120.0, 0.6)
        ts, ranks, _ = synth.prefill_routing(REQUESTS[name], S, choices, rng, median=median, sigma=sigma, cap=400)
        T = ts.shape[0]
    else:
        ts, ranks = synth.decode_routing(T, S, r_max, choices, zero_p, rng) if S > 1 else (
            np.zeros(T, np.int32), np.asarray([choices[0]], np.int32))
        if wild_slots and T >= 8:
            ts[3] = -1          # slot ids outside [0, S): inactive
            ts[5] = S
            ts[7] = 999
        if name == "decode-mid":
            ranks[1], ranks[2] = -3, r_max + 5     # clamped to 0 and r_max
    # bf16-rounded values are exact in fp32 too, so the fp32 cases reuse the same draws
    return synth.multi_lora(ts, ranks, K, out_slices, r_max, rng=rng, int_exact=int_exact, name=name)


def _addr(m):
    ts = torch.from_numpy(m.token_slot).to(DEV)
    ranks = torch.from_numpy(m.ranks).to(DEV)
    addr = L.lora_addressing_build(L.Addressing(ts, m.S), ranks, m.r_max)
    return addr, ranks


def _spec_mask(m):
    """Entries of h the page specifies: active tokens, j below the token's
    effective rank (the oracle's pinned token_ranks)."""
    rho = oracle.token_ranks(m.token_slot, m.ranks, m.r_max)
    act = rho > 0
    spec = np.arange(m.r_max)[None, None, :] < rho[:, None, None]
    spec = np.broadcast_to(spec, (m.T, m.num_slices, m.r_max)).copy()
    return act, spec


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouping_bitwise(case):
    m = _case(*case)
    note(f"grouping {case[0]} T={m.T} S={m.S}")
    addr, _ = _addr(m)
    torch.cuda.synchronize()
    counts, offsets, sorted_tokens, n = oracle.group_tokens(m.token_slot, m.ranks, m.r_max)
    assert np.array_equal(host(addr.counts)[:m.S], counts)
    assert np.array_equal(host(addr.offsets), offsets)
    assert np.array_equal(host(addr.sorted_tokens)[:n], sorted_tokens)


def _grouping_inputs(kind, rng):
    if kind == "small-max":
        T, S = 1024, 40
        ts = rng.integers(-1, S + 2, T).astype(np.int32)
    elif kind == "small-many-slots":
        T, S = 1000, 1000
        ts = rng.integers(-5, S + 5, T).astype(np.int32)
    elif kind == "small-one-token":
        T, S = 1, 3
        ts = np.asarray([2], np.int32)
    elif kind == "small-one-slot":
        T, S = 640, 8
        ts = np.full(T, 2, np.int32)
    elif kind == "small-all-inactive":
        T, S = 300, 8
        ts = np.full(T, -1, np.int32)
    elif kind == "chunk-multiple":
        T, S = 4096, 40
        ts = rng.integers(0, S, T).astype(np.int32)
    elif kind == "bursty":
        ts, _, _ = synth.prefill_routing(40, 96, (8, 16), rng, median=300.0, sigma=0.8, cap=2048)
        T, S = ts.shape[0], 96
    elif kind == "many-slots":
        T, S = 5000, 1000
        ts = rng.integers(-5, S + 5, T).astype(np.int32)
    elif kind == "max-chunked":
        T, S = 32768, 200
        ts = np.repeat(rng.integers(-2, S, 128), 256).astype(np.int32)
    elif kind == "all-inactive":
        T, S = 3000, 8
        ts = np.full(T, -1, np.int32)
    else:  # "beyond-chunked" (more tokens than the chunked kernel takes)
        T, S = 70000, 64
        ts = rng.integers(0, S + 2, T).astype(np.int32)
    ranks = rng.choice(np.asarray([0, 4, 16, 64], np.int32), S).astype(np.int32)
    if kind in ("small-one-token", "small-one-slot"):
        ranks[2] = 16
    return ts, ranks


@pytest.mark.parametrize("kind", ["small-max", "small-many-slots", "small-one-token", "small-one-slot",
                                  "small-all-inactive", "chunk-multiple", "bursty", "many-slots", "max-chunked",
                                  "all-inactive", "beyond-chunked"])
def test_grouping_schedules_bitwise(kind):
    """The three grouping kernels against the stable sort of the oracle: one
    token per thread up to 1024 tokens (the small-* kinds; small-max is the
    largest), one workgroup per 1024-token chunk up to 32768 tokens
    (max-chunked is the largest), one workgroup beyond (beyond-chunked)."""
    rng = np.random.default_rng(77)
    ts, ranks = _grouping_inputs(kind, rng)
    S = ranks.shape[0]
    note(f"grouping {kind} T={ts.shape[0]} S={S}")
    addr = L.lora_addressing_build(L.Addressing(torch.from_numpy(ts).to(DEV), S), torch.from_numpy(ranks).to(DEV), 64)
    torch.cuda.synchronize()
    counts, offsets, sorted_tokens, n = oracle.group_tokens(ts, ranks, 64)
    assert np.array_equal(host(addr.counts)[:S], counts)
    assert np.array_equal(host(addr.offsets), offsets)
    assert np.array_equal(host(addr.sorted_tokens)[:n], sorted_tokens)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shrink(case):
    m = _case(*case)
    dtype = case[-1]
    note(f"shrink {case[0]} T={m.T}")
    addr, ranks = _addr(m)
    h = torch.full((m.T, m.num_slices, m.r_max), SENTINEL, dtype=torch.float32, device=DEV)
    L.lora_shrink(dev(m.x, dtype), dev(m.a, dtype), addr, ranks, m.num_slices, m.r_max, h=h)
    torch.cuda.synchronize()
    want = oracle.shrink(m.x, m.a, m.token_slot, m.ranks, m.num_slices, m.r_max)
    got = host(h)
    act, spec = _spec_mask(m)
    assert np.all(got[~spec] == SENTINEL), "unspecified entries of h were written"
    assert np.isfinite(got[spec]).all()
    assert oracle.rel_frobenius(got[spec], want[spec]) <= tol(dtype)


@pytest.mark.parametrize("name", ["decode-small", "prefill-like", "fp32", "fp32-prefill", "prefill-many-slots",
                                  "decode-many-slots"])
def test_shrink_integer_exact(name):
    """Each shrink kernel (pipelined with 16- and 64-token tiles, row-split,
    bf16 and f32) bit for bit on integer inputs; unspecified entries of h
    untouched."""
    case = next(c for c in CASES if c[0] == name)
    m = _case(*case, int_exact=True)
    dtype = case[-1]
    note(f"shrink integer-exact {name} T={m.T}")
    addr, ranks = _addr(m)
    act, spec = _spec_mask(m)
    h = torch.full((m.T, m.num_slices, m.r_max), SENTINEL, dtype=torch.float32, device=DEV)
    L.lora_shrink(dev(m.x, dtype), dev(m.a, dtype), addr, ranks, m.num_slices, m.r_max, h=h)
    torch.cuda.synchronize()
    want = oracle.shrink(m.x, m.a, m.token_slot, m.ranks, m.num_slices, m.r_max)
    got = host(h)
    assert np.all(got[~spec] == SENTINEL)
    assert same_bits(got[spec], want[spec].astype(np.float32))


def _wide_stride_adapter(m, dtype):
    """The adapter as a view whose rank rows lie 2^27 (bf16) or 2^26 (f32)
    elements apart, so one slot's rows span more than a 2 GiB buffer
    descriptor; the memory between rows holds NaN."""
    es = 2 if dtype == "bf16" else 4
    s1 = ((1 << 31) // (es * m.num_slices * m.r_max) + 16) // 8 * 8   # 16-byte aligned rows
    s0 = m.K
    n_rows = m.num_slices * m.r_max
    size = (n_rows - 1) * s1 + (m.S - 1) * s0 + m.K
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    store = torch.full((size,), float("nan"), dtype=tdt, device=DEV)
    a_dev = store.as_strided((m.S, n_rows, m.K), (s0, s1, 1))
    a_dev.copy_(dev(m.a, dtype))
    return store, a_dev


@pytest.mark.parametrize("T", [203, 600, 2400])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shrink_general_kernel(dtype, T):
    """One slot's adapter rows spanning more than 2 GiB (a strided view): the
    shrink without buffer descriptors, bit for bit on integer inputs, with
    each of its tilings (203 tokens: 16-token tiles and one rank block; 600:
    four rank blocks; 2400 over 9 slots: 64-token tiles)."""
    note(f"shrink general kernel {dtype} T={T}")
    m = _case("ragged-ranks", T, 64, (100, 28), 9, 40, (0, 3, 17, 40), 0.1, dtype, int_exact=True)
    addr, ranks = _addr(m)
    act, spec = _spec_mask(m)
    store, a_dev = _wide_stride_adapter(m, dtype)
    h = torch.full((m.T, m.num_slices, m.r_max), SENTINEL, dtype=torch.float32, device=DEV)
    L.lora_shrink(dev(m.x, dtype), a_dev, addr, ranks, m.num_slices, m.r_max, h=h)
    torch.cuda.synchronize()
    del store, a_dev
    want = oracle.shrink(m.x, m.a, m.token_slot, m.ranks, m.num_slices, m.r_max)
    got = host(h)
    assert np.all(got[~spec] == SENTINEL)
    assert same_bits(got[spec], want[spec].astype(np.float32))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_expand_fused(case):
    m = _case(*case)
    dtype = case[-1]
    note(f"expand {case[0]} T={m.T}")
    addr, ranks = _addr(m)
    rng = np.random.default_rng(7)
    act, spec = _spec_mask(m)
    hin = rng.standard_normal((m.T, m.num_slices, m.r_max)).astype(np.float32)
    hin[~spec] = np.nan                      # the expand must not read unspecified entries
    y = f32(m.y0)
    L.lora_expand_fused(f32(hin), dev(m.b, dtype), addr, ranks, f32(m.scalings), y, m.out_slices, m.r_max)
    torch.cuda.synchronize()
    got = host(y)
    want = oracle.expand_fused(hin, m.b, m.token_slot, m.ranks, m.scalings, m.y0, m.out_slices, m.r_max)
    assert same_bits(got[~act], m.y0[~act]), "rows of inactive tokens were written"
    assert np.isfinite(got).all(), "NaN padding reached y"
    assert oracle.rel_frobenius(got[act] - m.y0[act], want[act] - m.y0[act]) <= tol(dtype)


def _expand_exact(m, dtype, h_view=None):
    addr, ranks = _addr(m)
    act, spec = _spec_mask(m)
    rng = np.random.default_rng(9)
    hin = rng.integers(-2, 3, size=(m.T, m.num_slices, m.r_max)).astype(np.float32)
    hin[~spec] = np.nan
    h = f32(hin) if h_view is None else h_view(hin)
    y = f32(m.y0)
    L.lora_expand_fused(h, dev(m.b, dtype), addr, ranks, f32(m.scalings), y, m.out_slices, m.r_max)
    torch.cuda.synchronize()
    want = oracle.expand_fused(hin, m.b, m.token_slot, m.ranks, m.scalings, m.y0, m.out_slices, m.r_max)
    assert same_bits(host(y), want.astype(np.float32))


@pytest.mark.parametrize("name", ["decode-small", "prefill-like", "fp32", "fp32-prefill", "prefill-long"])
def test_expand_integer_exact(name):
    """The streaming and column-band expand kernels (bf16 and f32 weights,
    rank blocks 1 to 8) bit for bit on integer inputs, NaN in every entry of h
    they must not read; the band cases have work-item counts that are not
    multiples of their XCD grouping."""
    case = next(c for c in CASES if c[0] == name)
    m = _case(*case, int_exact=True)
    note(f"expand integer-exact {name} T={m.T}")
    _expand_exact(m, case[-1])


@pytest.mark.parametrize("name", ["decode-small", "prefill-like"])
def test_expand_general_kernel(name):
    """Rows of h whose stride is not a multiple of 4 floats: the general
    expand kernel (element loads), 16- and 64-token tiles, bit for bit."""
    case = next(c for c in CASES if c[0] == name)
    m = _case(*case, int_exact=True)
    note(f"expand general kernel {name} T={m.T}")

    def odd_view(hin):
        buf = torch.full((m.T, m.num_slices, m.r_max + 1), float("nan"), device=DEV)
        view = buf[:, :, :m.r_max]
        view.copy_(f32(hin))
        return view
    _expand_exact(m, case[-1], odd_view)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shrink_then_expand(case):
    m = _case(*case)
    dtype = case[-1]
    note(f"apply {case[0]}")
    addr, ranks = _addr(m)
    h = L.lora_shrink(dev(m.x, dtype), dev(m.a, dtype), addr, ranks, m.num_slices, m.r_max)
    y = f32(m.y0)
    L.lora_expand_fused(h, dev(m.b, dtype), addr, ranks, f32(m.scalings), y, m.out_slices, m.r_max)
    torch.cuda.synchronize()
    want = oracle.apply_linear(m.x, m.y0, m.a, m.b, m.token_slot, m.ranks, m.scalings, m.out_slices, m.r_max)
    act, _ = _spec_mask(m)
    got = host(y)
    assert same_bits(got[~act], m.y0[~act])
    assert oracle.rel_frobenius(got[act] - m.y0[act], want[act] - m.y0[act]) <= tol(dtype)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_apply_linear(case):
    """lora_apply_linear gives the bits of the two separate calls, as one
    launch (its shrink takes the pipelined shrink's feature ranges and
    summation order) or as two, and the oracle's apply_linear within
    tolerance; inactive rows stay bitwise untouched."""
    m = _case(*case)
    dtype = case[-1]
    note(f"apply_linear {case[0]}")
    addr, ranks = _addr(m)
    x, a, b, sc = dev(m.x, dtype), dev(m.a, dtype), dev(m.b, dtype), f32(m.scalings)
    h_ref = L.lora_shrink(x, a, addr, ranks, m.num_slices, m.r_max)
    y_ref = f32(m.y0)
    L.lora_expand_fused(h_ref, b, addr, ranks, sc, y_ref, m.out_slices, m.r_max)
    y = f32(m.y0)
    L.lora_apply_linear(x, y, a, b, addr, ranks, sc, m.out_slices, m.r_max)
    torch.cuda.synchronize()
    got = host(y)
    assert same_bits(got, host(y_ref))
    want = oracle.apply_linear(m.x, m.y0, m.a, m.b, m.token_slot, m.ranks, m.scalings, m.out_slices, m.r_max)
    act, _ = _spec_mask(m)
    assert same_bits(got[~act], m.y0[~act])
    assert oracle.rel_frobenius(got[act] - m.y0[act], want[act] - m.y0[act]) <= tol(dtype)


@pytest.mark.parametrize("name", list(ONE_LAUNCH) + ["decode-small", "decode-wide", "prefill-like"])
def test_apply_linear_integer_exact(name):
    """lora_apply_linear bit for bit against the oracle on integer inputs:
    the one-launch kernel (ranks up to 128 and clamped ones, bf16 and f32,
    fewer and more than 1024 tokens) and the shrink-then-expand path; rows of
    inactive tokens untouched."""
    case = next(c for c in CASES if c[0] == name)
    m = _case(*case, int_exact=True)
    dtype = case[-1]
    note(f"apply_linear integer-exact {name} T={m.T}")
    addr, ranks = _addr(m)
    y = f32(m.y0)
    L.lora_apply_linear(dev(m.x, dtype), y, dev(m.a, dtype), dev(m.b, dtype), addr, ranks, f32(m.scalings),
                        m.out_slices, m.r_max)
    torch.cuda.synchronize()
    want = oracle.apply_linear(m.x, m.y0, m.a, m.b, m.token_slot, m.ranks, m.scalings, m.out_slices, m.r_max)
    assert same_bits(host(y), want.astype(np.float32))


def test_apply_linear_mixed_weight_dtype():
    """bf16 activations and adapter with f32 expand weights at a shape that
    would run as one launch: the shrink-then-expand path, the bits of the two
    separate calls."""
    m = _case(*next(c for c in CASES if c[0] == "decode-mid"))
    note(f"apply_linear mixed dtypes T={m.T}")
    addr, ranks = _addr(m)
    x, a, b, sc = dev(m.x, "bf16"), dev(m.a, "bf16"), dev(m.b, "f32"), f32(m.scalings)
    h_ref = L.lora_shrink(x, a, addr, ranks, m.num_slices, m.r_max)
    y_ref = f32(m.y0)
    L.lora_expand_fused(h_ref, b, addr, ranks, sc, y_ref, m.out_slices, m.r_max)
    y = f32(m.y0)
    L.lora_apply_linear(x, y, a, b, addr, ranks, sc, m.out_slices, m.r_max)
    torch.cuda.synchronize()
    assert same_bits(host(y), host(y_ref))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_integer_exact_bitwise(dtype):
    note(f"multi integer-exact {dtype}")
    m = _case("ragged-ranks", 203, 200, (100, 28), 9, 40, (0, 3, 17, 40), 0.1, dtype, int_exact=True)
    addr, ranks = _addr(m)
    h = L.lora_shrink(dev(m.x, dtype), dev(m.a, dtype), addr, ranks, m.num_slices, m.r_max)
    y = f32(m.y0)
    L.lora_expand_fused(h, dev(m.b, dtype), addr, ranks, f32(m.scalings), y, m.out_slices, m.r_max)
    torch.cuda.synchronize()
    act, spec = _spec_mask(m)
    hw = oracle.shrink(m.x, m.a, m.token_slot, m.ranks, m.num_slices, m.r_max)
    assert same_bits(host(h)[spec], hw[spec].astype(np.float32))
    want = oracle.expand_fused(hw, m.b, m.token_slot, m.ranks, m.scalings, m.y0, m.out_slices, m.r_max)
    assert same_bits(host(y), want.astype(np.float32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["rank-contiguous", "vocab-contiguous"])
def test_gather_shrink_bitwise(dtype, layout):
    note(f"gather {dtype} {layout}")
    rng = np.random.default_rng(77)
    T, S, r_max, V = 300, 7, 48, 1000
    ts, ranks = synth.decode_routing(T, S, r_max, (0, 5, 16, 48), 0.1, rng)
    ts[4] = -3
    ts[6] = S
    ids = synth.gather_ids(T, V, rng)
    ids[:4] = [V, V + 7, np.iinfo(np.int32).min, -1]
    table = rng.standard_normal((S, r_max, V)).astype(np.float32)
    for s in range(S):
        table[s, ranks[s]:, :] = np.nan
    table = synth.round_bf16(table)
    if layout == "rank-contiguous":
        a_dev = dev(np.ascontiguousarray(table.transpose(0, 2, 1)), dtype).permute(0, 2, 1)   # S x r_max x V view
    else:
        a_dev = dev(table, dtype)
    ranks_d = torch.from_numpy(ranks).to(DEV)
    addr = L.lora_addressing_build(L.Addressing(torch.from_numpy(ts).to(DEV), S), ranks_d, r_max)
    h = torch.full((T, 1, r_max), SENTINEL, dtype=torch.float32, device=DEV)
    L.lora_gather_shrink(torch.from_numpy(ids).to(DEV), a_dev, addr, ranks_d, r_max, h=h)
    torch.cuda.synchronize()
    want = oracle.gather_shrink(ids, table, ts, ranks, r_max)
    got = host(h)
    rho = oracle.token_ranks(ts, ranks, r_max)
    act = rho > 0
    spec = (np.arange(r_max)[None, None, :] < rho[:, None, None]).repeat(1, axis=1)
    assert same_bits(got[spec], want[spec].astype(np.float32))
    assert np.all(got[~spec] == SENTINEL)
    invalid = act & ((ids < 0) | (ids >= V))
    assert invalid.any()
    assert not np.signbit(got[invalid][spec[invalid]]).any(), "an out-of-range id must give +0.0"


def test_bad_arguments():
    note("multi bad args")
    ts = torch.zeros(4, dtype=torch.int32, device=DEV)
    ranks = torch.ones(1100, dtype=torch.int32, device=DEV)
    with pytest.raises(L.LoraError) as e:
        L.lora_addressing_build(L.Addressing(ts, 1100), ranks, 16)
    assert e.value.status == -8
    addr = L.lora_addressing_build(L.Addressing(ts, 2), ranks[:2], 16)
    h = torch.zeros((4, 2, 16), device=DEV)
    b = torch.zeros((2, 12, 16), device=DEV, dtype=torch.bfloat16)
    y = torch.zeros((4, 12), device=DEV)
    with pytest.raises(L.LoraError) as e:
        L.lora_expand_fused(h, b, addr, ranks[:2], torch.ones(2, device=DEV), y, (8, 8), 16)
    assert e.value.status == -2
    with pytest.raises(L.LoraError) as e:
        L.lora_expand_fused(h, b, addr, ranks[:2], torch.ones(2, device=DEV), y, (6, 6), 16)
    assert e.value.status == -2


def _full_size_check(m):
    note(f"full size {m.name} T={m.T}")
    addr, ranks = _addr(m)
    counts, offsets, sorted_tokens, n = oracle.group_tokens(m.token_slot, m.ranks, m.r_max)
    torch.cuda.synchronize()
    assert np.array_equal(host(addr.counts)[:m.S], counts)
    assert np.array_equal(host(addr.offsets), offsets)
    assert np.array_equal(host(addr.sorted_tokens)[:n], sorted_tokens)
    h = L.lora_shrink(dev(m.x, "bf16"), dev(m.a, "bf16"), addr, ranks, m.num_slices, m.r_max)
    y = f32(m.y0)
    L.lora_expand_fused(h, dev(m.b, "bf16"), addr, ranks, f32(m.scalings), y, m.out_slices, m.r_max)
    torch.cuda.synchronize()
    # sampled tokens: the ends, random ones, and the first and last token of
    # every slot the batch uses (so every slot's rank, clamped or not, is seen)
    rng = np.random.default_rng(1)
    per_slot = []
    for s in np.unique(m.token_slot):
        idx = np.nonzero(m.token_slot == s)[0]
        per_slot += [idx[0], idx[-1]]
    toks = np.unique(np.concatenate([[0, m.T - 1], rng.integers(0, m.T, 200), per_slot]))
    act, spec = _spec_mask(m)
    hw = oracle.shrink(m.x, m.a, m.token_slot, m.ranks, m.num_slices, m.r_max, tokens=toks)
    hg = host(h)
    assert oracle.rel_frobenius(hg[toks][spec[toks]], hw[toks][spec[toks]]) <= 2e-3
    want = oracle.expand_fused(hw, m.b, m.token_slot, m.ranks, m.scalings, m.y0, m.out_slices, m.r_max, tokens=toks)
    got = host(y)[toks]
    a_t = act[toks]
    assert same_bits(got[~a_t], m.y0[toks][~a_t])
    assert oracle.rel_frobenius(got[a_t] - m.y0[toks][a_t], want[a_t] - m.y0[toks][a_t]) <= 2e-3
    return act


@pytest.mark.slow
@pytest.mark.parametrize("cfg", ["config4", "config5"])
def test_full_size_shrink_expand(cfg):
    _full_size_check(getattr(synth, cfg)())


@pytest.mark.slow
def test_full_size_rank_clamp():
    """The prefill workload's routing with the ranks of four used slots moved
    outside [0, r_max] (-3, r_max + 5, 2^30, -2^30): ranks are clamped into
    [0, r_max], so two of those slots use all 128 rank rows and the tokens of
    the other two are inactive and leave y untouched."""
    ts, ranks, _lengths, rng = synth.config5_routing()
    used = np.unique(ts)
    ranks = ranks.copy()
    ranks[used[:4]] = [-3, 128 + 5, 1 << 30, -(1 << 30)]
    m = synth.multi_lora(ts, ranks, 8192, (8192, 1024, 1024), 128, rng=rng, name="cfg5-rank-clamp")
    act = _full_size_check(m)
    rho = oracle.token_ranks(m.token_slot, m.ranks, m.r_max)
    assert (rho[np.isin(m.token_slot, used[[1, 2]])] == 128).all()
    assert not act[np.isin(m.token_slot, used[[0, 3]])].any()


@pytest.mark.slow
def test_full_size_gather_shrink():
    """Vocabulary 128256, 128 slots of rank <= 128: a 4.2 GB table (64-bit offsets)."""
    ts, ranks, _lengths, rng = synth.config5_routing()
    T, S, r_max, V = ts.shape[0], 128, 128, 128256
    note(f"full size gather T={T} V={V}")
    ids = synth.gather_ids(T, V, rng)
    ids[:3] = [V, V + 7, np.iinfo(np.int32).min]
    bits = synth.gather_table_bits(S, r_max, V, ranks, seed=55)       # S x V x r_max, rank index contiguous
    a_dev = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16).permute(0, 2, 1)
    ts_d = torch.from_numpy(ts).to(DEV)
    ranks_d = torch.from_numpy(ranks).to(DEV)
    addr = L.lora_addressing_build(L.Addressing(ts_d, S), ranks_d, r_max)
    h = torch.full((T, 1, r_max), SENTINEL, dtype=torch.float32, device=DEV)
    L.lora_gather_shrink(torch.from_numpy(ids).to(DEV), a_dev, addr, ranks_d, r_max, h=h)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, 1, 2, T - 1], rng.integers(0, T, 300)]))
    want = oracle.gather_shrink(ids, bits.transpose(0, 2, 1), ts, ranks, r_max, tokens=toks, a_is_bf16_bits=True)
    got = host(h)
    for t in toks:
        rho = int(ranks[ts[t]])
        assert same_bits(got[t, 0, :rho], want[t, 0, :rho].astype(np.float32)), t
        assert np.all(got[t, 0, rho:] == SENTINEL)
