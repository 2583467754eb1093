"""The C ABI on the host (no GPU): the library loads, exports every symbol
include/lora.h declares, and rejects invalid arguments with the documented
status codes before launching anything."""
import ctypes
import os
import re

import pytest
import torch

import lora_rank_adapter_amd as L
from lora_rank_adapter_amd import _lib
from lora_rank_adapter_amd._lib import LoraAddressing, LoraMat, LoraT3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")

FAKE = 0x10000  # a 64 KiB-aligned non-NULL address; never dereferenced by these calls

# These checks hand the library fake device pointers and expect every call to be
# rejected (or to be an empty no-op) before any launch; they run only where no
# GPU is visible, so a check that wrongly reached a launch could never touch one.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="host-only checks (fake device pointers)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return L.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in include/lora.h but not exported"
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_version_and_status_strings(lib):
    assert lib.lora_abi_version() == 1
    for code in range(-8, 1):
        assert lib.lora_status_string(code)
    assert b"workspace" in lib.lora_status_string(-6)


def test_timing_calls_without_launches(lib):
    assert lib.lora_timing_begin() == 0
    assert lib.lora_timing_pause() == 0
    assert lib.lora_timing_resume() == 0
    total = ctypes.c_double(-1.0)
    n = ctypes.c_int64(-1)
    assert lib.lora_timing_read(ctypes.byref(total), ctypes.byref(n)) == 0
    assert (total.value, n.value) == (0.0, 0)
    assert lib.lora_timing_read(None, ctypes.byref(n)) == -1
    assert lib.lora_timing_read(ctypes.byref(total), None) == -1
    assert lib.lora_timing_pause() == 0


def test_workspace_bytes(lib):
    f = lib.lora_workspace_bytes
    assert f(1, 8192, 4096, 4096, 16, 1) > 0
    assert f(2, 8192, 4096, 4096, 16, 1) > 0
    assert f(0, 8192, 4096, 4096, 16, 1) > 0
    assert f(1, 8192, 4096, 4096, 0, 1) == 0        # rank 0
    assert f(1, 8192, 4096, 4096, 129, 1) == 0      # rank > 128
    assert f(1, -1, 4096, 4096, 16, 1) == 0
    assert f(7, 8192, 4096, 4096, 16, 1) == 0       # unknown op
    assert f(1, 8192, 4096, 4096, 16, 5) == 0       # unknown dtype
    assert f(1, 16384, 4096, 14336, 64, 1) >= f(1, 8192, 4096, 4096, 16, 1)
    # sizes no operand could have (x or the output beyond 2^47 elements) are
    # invalid, and sizing them must not overflow
    big = 1 << 47
    assert f(1, 1 << 20, 1 << 27, 1 << 27, 64, 1) > 0             # M x K = 2^47 elements
    assert f(1, 1 << 20, (1 << 27) + 8, 4096, 64, 1) == 0
    for op in (0, 1, 2):
        assert f(op, 1 << 40, 1 << 40, 1 << 40, 128, 1) == 0
        assert f(op, 1 << 62, 4096, 4096, 64, 1) == 0
        assert f(op, (1 << 63) - 1, (1 << 63) - 1, (1 << 63) - 1, 128, 0) == 0
        assert f(op, 1, big + 8, 8, 16, 1) == 0


def m(rows, cols, dtype=1, sr=None, sc=1, ptr=FAKE):
    return LoraMat(ptr, dtype, 0, rows, cols, cols if sr is None else sr, sc)


def fwd(lib, x, A, B, res, ws=None, nbytes=0):
    return lib.lora_fwd(ctypes.byref(x), ctypes.byref(A), ctypes.byref(B), ctypes.byref(res), 1.0, ws, nbytes, None)


def test_fwd_validation(lib):
    M, K, L_, r = 64, 128, 96, 16
    x = m(M, K)
    A = m(K, r, sr=1, sc=K)        # view of an r x K weight
    B = m(r, L_, sr=1, sc=r)       # view of an L x r weight
    res = m(M, L_, dtype=0)
    assert lib.lora_fwd(None, ctypes.byref(A), ctypes.byref(B), ctypes.byref(res), 1.0, None, 0, None) == -1
    assert fwd(lib, m(M, K, ptr=None), A, B, res) == -1
    assert fwd(lib, x, A, B, m(M, L_ + 4, dtype=0)) == -2                 # res shape
    assert fwd(lib, x, m(K + 8, r, sr=1, sc=K + 8), B, res) == -2          # A rows != K
    assert fwd(lib, m(M, K, dtype=0), m(K, r, 0, sr=1, sc=K), m(r, L_, 0, sr=1, sc=r),
               m(M, L_, dtype=1)) == -3                                    # bf16 res needs bf16 inputs
    assert fwd(lib, m(M, K, dtype=0), A, B, res) == -3                     # mixed input dtypes
    assert fwd(lib, m(M, K, dtype=7), m(K, r, 7), m(r, L_, 7), res) == -3
    assert fwd(lib, x, m(K, 0, sr=1, sc=K), m(0, L_, sr=1, sc=1), res) == -5
    assert fwd(lib, x, m(K, 129, sr=1, sc=K), m(129, L_, sr=1, sc=129), res) == -5
    assert fwd(lib, m(M, K, sr=1, sc=M), A, B, res) == -4                  # column-major x
    assert fwd(lib, m(M, K, ptr=FAKE + 2), A, B, res) == -4                # misaligned x
    assert fwd(lib, m(M, K, sr=K + 2), A, B, res) == -4                    # row pitch not 16-byte aligned
    assert fwd(lib, m(M, 132), m(132, r, sr=1, sc=132), B, res) == -2      # K not a multiple of 8 (bf16)
    assert fwd(lib, x, A, m(r, 98, sr=1, sc=r), m(M, 98, dtype=0)) == -2   # L not a multiple of 4
    # the forward needs its workspace when it packs a weight or runs the split
    # schedule (contractions longer than 8192); weights read in place with the
    # fused schedule need none (that call launches: covered by a GPU test)
    assert fwd(lib, x, m(K, r), B, res) == -6                               # A packed
    assert fwd(lib, x, A, m(r, L_), res) == -6                              # B packed
    assert fwd(lib, x, m(K, r), B, res, ctypes.c_void_p(FAKE), 16) == -6
    assert fwd(lib, x, m(K, r), B, res, ctypes.c_void_p(FAKE + 128), 1 << 20) == -6   # not 256-byte aligned
    Kl = 8200
    assert fwd(lib, m(M, Kl), m(Kl, r, sr=1, sc=Kl), B, res) == -6          # split schedule
    # operands that could not exist (beyond 2^47 bytes, or negative strides)
    assert fwd(lib, m(1 << 62, K), A, B, m(1 << 62, L_, dtype=0)) == -2
    assert fwd(lib, m(M, K, sr=1 << 50), A, B, res) == -2
    assert fwd(lib, m(M, K, sr=-K), A, B, res) == -2
    assert fwd(lib, x, m(K, r, sr=-1, sc=K), B, res) == -2
    assert fwd(lib, m(1 << 40, 1 << 40, sr=1 << 40), m(1 << 40, r, sr=1, sc=1 << 40), B, res) == -2
    # empty problems launch nothing and succeed
    assert fwd(lib, m(0, K), A, B, m(0, L_, dtype=0)) == 0
    assert fwd(lib, m(M, 0), m(0, r, sr=1, sc=1), B, res) == 0


def test_bwd_validation(lib):
    M, K, L_, r = 64, 128, 96, 16
    xt = m(K, M, sr=1, sc=K)        # view of row-major x
    dy = m(M, L_)
    Bw = m(L_, r)
    Aw = m(r, K)
    dx = m(M, K, dtype=0)
    dA = m(K, r, dtype=0)
    dB = m(r, L_, dtype=0)
    need = lib.lora_workspace_bytes(1, M, K, L_, r, 1)

    for fn in (lib.lora_bwd_dx_da, lib.lora_bwd_dx_da_accumulate):
        def dxda(xt_=xt, dy_=dy, B_=Bw, A_=Aw, dx_=dx, dA_=dA, ws=FAKE, nb=need):
            return fn(ctypes.byref(xt_), ctypes.byref(dy_), ctypes.byref(B_), ctypes.byref(A_), 1.0,
                      ctypes.byref(dx_), ctypes.byref(dA_), ctypes.c_void_p(ws) if ws else None, nb, None)

        assert dxda(ws=0) == -6
        assert dxda(nb=need - 1) == -6
        assert dxda(ws=FAKE + 64) == -6                       # workspace must be 256-byte aligned
        assert dxda(xt_=m(K, M)) == -4                        # xt must be a view of row-major x
        assert dxda(dy_=m(M, L_ + 8)) == -2
        # bfloat16 outputs need bfloat16 inputs
        xt32, dy32, B32, A32 = m(K, M, dtype=0, sr=1, sc=K), m(M, L_, dtype=0), m(L_, r, dtype=0), m(r, K, dtype=0)
        assert dxda(xt_=xt32, dy_=dy32, B_=B32, A_=A32, dA_=m(K, r, dtype=1)) == -3
        assert dxda(xt_=xt32, dy_=dy32, B_=B32, A_=A32, dx_=m(M, K, dtype=1)) == -3
        assert dxda(dx_=m(M, K, dtype=7)) == -3
        assert dxda(B_=m(L_, 200), A_=m(200, K)) == -2         # dA shape disagrees with rank 200
        assert dxda(B_=m(L_, 0), A_=m(0, K), dA_=m(K, 0, dtype=0)) == -5

    def db(A_=Aw, xt_=xt, dy_=dy, dB_=dB, ws=FAKE, nb=lib.lora_workspace_bytes(2, M, K, L_, r, 1)):
        return lib.lora_bwd_db(ctypes.byref(A_), ctypes.byref(xt_), ctypes.byref(dy_), 1.0, ctypes.byref(dB_),
                               ctypes.c_void_p(ws) if ws else None, nb, None)

    assert db(ws=0) == -6
    assert db(dB_=m(r, L_ + 4, dtype=0)) == -2
    assert db(A_=m(r, K, dtype=0), xt_=m(K, M, dtype=0, sr=1, sc=K), dy_=m(M, L_, dtype=0),
              dB_=m(r, L_, dtype=1)) == -3                                 # bf16 dB needs bf16 inputs
    assert db(dB_=m(r, L_, dtype=7)) == -3
    assert db(dy_=m(M, L_, sr=L_ + 1)) == -4


def test_multi_validation(lib):
    T, S, K, r_max = 32, 4, 64, 16
    addr = LoraAddressing(FAKE, T, S, FAKE, FAKE, FAKE)
    x = m(T, K)
    a = LoraT3(FAKE, 1, 0, S, 2 * r_max, K, 2 * r_max * K, K, 1)
    h = LoraT3(FAKE, 0, 0, T, 2, r_max, 2 * r_max, r_max, 1)

    def shrink(x_=x, a_=a, addr_=addr, n=2, rm=r_max, h_=h, ranks=FAKE):
        return lib.lora_shrink(ctypes.byref(x_), ctypes.byref(a_), ctypes.byref(addr_) if addr_ else None,
                               ctypes.c_void_p(ranks) if ranks else None, n, rm, ctypes.byref(h_), None)

    assert shrink(addr_=None) == -1
    assert shrink(ranks=0) == -1
    assert shrink(rm=0) == -5
    assert shrink(rm=129) == -5
    assert shrink(n=3) == -2
    assert shrink(h_=LoraT3(FAKE, 1, 0, T, 2, r_max, 2 * r_max, r_max, 1)) == -3
    assert shrink(a_=LoraT3(FAKE, 1, 0, S, 2 * r_max, K, 2 * r_max * K, 1, K)) == -4
    assert shrink(addr_=LoraAddressing(FAKE, T, 2000, FAKE, FAKE, FAKE)) == -8
    huge = 1 << 62
    assert shrink(x_=m(T, huge), a_=LoraT3(FAKE, 1, 0, S, 2 * r_max, huge, 2 * r_max * K, K, 1)) == -2
    assert shrink(a_=LoraT3(FAKE, 1, 0, S, 2 * r_max, K, huge, K, 1)) == -2
    assert shrink(h_=LoraT3(FAKE, 0, 0, T, 2, r_max, -2 * r_max, r_max, 1)) == -2
    assert shrink(x_=m(0, K), addr_=LoraAddressing(FAKE, 0, S, FAKE, FAKE, FAKE),
                  h_=LoraT3(FAKE, 0, 0, 0, 2, r_max, 2 * r_max, r_max, 1)) == 0

    b = LoraT3(FAKE, 1, 0, S, 48, r_max, 48 * r_max, r_max, 1)
    y = m(T, 48, dtype=0)
    sl = (ctypes.c_int64 * 2)(32, 16)

    def expand(h_=h, b_=b, y_=y, slices=sl, n=2, sc=FAKE):
        return lib.lora_expand_fused(ctypes.byref(h_), ctypes.byref(b_), ctypes.byref(addr), ctypes.c_void_p(FAKE),
                                     ctypes.c_void_p(sc) if sc else None, ctypes.byref(y_), slices, n, r_max, None)

    assert expand(sc=0) == -1
    assert expand(slices=(ctypes.c_int64 * 2)(30, 18)) == -2      # widths must be multiples of 4
    assert expand(slices=(ctypes.c_int64 * 2)(32, 20)) == -2      # must sum to y's width
    b32 = LoraT3(FAKE, 0, 0, S, 48, r_max, 48 * r_max, r_max, 1)
    assert expand(b_=b32, y_=m(T, 48, dtype=1)) == -3                 # bf16 y needs bf16 weights
    assert expand(y_=m(T, 48, dtype=7)) == -3
    assert expand(h_=LoraT3(FAKE, 0, 0, T, 2, r_max, 2 * r_max, 1, 2)) == -4      # rank index not contiguous
    assert expand(slices=(ctypes.c_int64 * 2)(1 << 62, 48 - (1 << 62))) == -2       # widths beyond any operand
    assert expand(b_=LoraT3(FAKE, 1, 0, S, 48, r_max, 1 << 60, r_max, 1)) == -2

    def apply(x_=x, y_=y, h_=h, slices=sl, n=2, b_=b):
        return lib.lora_apply_linear(ctypes.byref(x_), ctypes.byref(a), ctypes.byref(b_), ctypes.byref(addr),
                                     ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.byref(y_), slices, n, r_max,
                                     ctypes.byref(h_), None)

    # the shrink's and the expand's checks both run before any launch
    assert apply(h_=LoraT3(FAKE, 1, 0, T, 2, r_max, 2 * r_max, r_max, 1)) == -3       # h must be float32
    assert apply(slices=(ctypes.c_int64 * 2)(32, 20)) == -2                            # expand: widths vs y
    assert apply(b_=b32, y_=m(T, 48, dtype=1)) == -3                                   # expand: bf16 y, f32 b
    assert apply(x_=m(T, K + 8)) == -2                                                 # shrink: x vs a

    ah = LoraT3(FAKE, 1, 0, S, r_max, 1000, r_max * 1000, 1000, 1)
    h1 = LoraT3(FAKE, 0, 0, T, 1, r_max, r_max, r_max, 1)
    assert lib.lora_gather_shrink(None, ctypes.byref(ah), ctypes.byref(addr), ctypes.c_void_p(FAKE), r_max,
                                  ctypes.byref(h1), None) == -1
    assert lib.lora_gather_shrink(ctypes.c_void_p(FAKE), ctypes.byref(ah), ctypes.byref(addr), ctypes.c_void_p(FAKE),
                                  r_max, ctypes.byref(LoraT3(FAKE, 0, 0, T, 2, r_max, r_max, r_max, 1)), None) == -2
    assert lib.lora_addressing_build(ctypes.byref(LoraAddressing(FAKE, T, 1025, FAKE, FAKE, FAKE)),
                                     ctypes.c_void_p(FAKE), r_max, None) == -8
    assert lib.lora_addressing_build(ctypes.byref(addr), ctypes.c_void_p(FAKE), 0, None) == -5
