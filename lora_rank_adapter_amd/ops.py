"""Python binding of the C ABI, same names as include/lora.h.

Argument marshalling only: torch tensors are described to the library by
pointer, dtype, shape and strides, outputs and workspaces are allocated with
torch on the tensors' device, and the call goes to the HIP library on torch's
current stream. Every step of the computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import LoraAddressing, LoraMat, LoraT3, check

_DT = {torch.float32: _lib.LORA_F32, torch.bfloat16: _lib.LORA_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        return -1


def mat(t: torch.Tensor) -> LoraMat:
    if t.dim() != 2:
        raise ValueError(f"expected a 2-D tensor, got shape {tuple(t.shape)}")
    return LoraMat(t.data_ptr() or None, _dtype_code(t), 0, t.shape[0], t.shape[1], t.stride(0), t.stride(1))


def t3(t: torch.Tensor) -> LoraT3:
    if t.dim() != 3:
        raise ValueError(f"expected a 3-D tensor, got shape {tuple(t.shape)}")
    return LoraT3(t.data_ptr() or None, _dtype_code(t), 0, t.shape[0], t.shape[1], t.shape[2],
                  t.stride(0), t.stride(1), t.stride(2))


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    """torch's current stream on `device` as a raw pointer."""
    if _raw_stream is not None:
        idx = device.index if device.index is not None else torch.cuda.current_device()
        return ctypes.c_void_p(_raw_stream(idx))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def lora_workspace_bytes(op: int, M: int, K: int, L: int, r: int, dtype: torch.dtype) -> int:
    return int(_lib.load().lora_workspace_bytes(op, M, K, L, r, _DT[dtype]))


def _workspace(op, M, K, L, r, dtype, device, workspace):
    # a caller's workspace is passed with its size; the library checks it
    if workspace is None:
        need = lora_workspace_bytes(op, M, K, L, r, dtype)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, workspace.numel()


# ---------------------------------------------------------------------------
# single adapter
# ---------------------------------------------------------------------------

def lora_fwd(x: torch.Tensor, lora_A: torch.Tensor, lora_B: torch.Tensor, res: torch.Tensor, scale: float,
             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """res += scale * (x @ lora_A) @ lora_B, in place; returns res.
    x: M x K, lora_A: K x r, lora_B: r x L (views with any strides), res: M x L float32, or bfloat16 with
    bfloat16 inputs (the float32 sum rounded once)."""
    lib = _lib.load()
    M, K = x.shape
    r, L = lora_B.shape
    ws, nbytes = _workspace(_lib.LORA_OP_FWD, M, K, L, r, x.dtype, x.device, workspace)
    check("lora_fwd", lib.lora_fwd(ctypes.byref(mat(x)), ctypes.byref(mat(lora_A)), ctypes.byref(mat(lora_B)),
                                   ctypes.byref(mat(res)), float(scale), _ptr(ws), nbytes, _stream(x.device)))
    return res


def lora_bwd_dx_da(xt: torch.Tensor, dy: torch.Tensor, lora_B: torch.Tensor, lora_A: torch.Tensor, scale: float,
                   dx: torch.Tensor | None = None, dA: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, dtype: torch.dtype = torch.float32):
    """dx = scale * (dy @ lora_B) @ lora_A; dA = scale * xt @ (dy @ lora_B).
    xt: K x M (transposed view of row-major x), dy: M x L, lora_B: L x r, lora_A: r x K.
    Returns (dx [M x K], dA [K x r]): the given tensors, else new ones of `dtype` (float32, or bfloat16 with
    bfloat16 inputs: the float32 result rounded once)."""
    lib = _lib.load()
    K, M = xt.shape
    L = dy.shape[1]
    r = lora_B.shape[1]
    if dx is None:
        dx = torch.empty((M, K), dtype=dtype, device=dy.device)
    if dA is None:
        dA = torch.empty((K, r), dtype=dtype, device=dy.device)
    ws, nbytes = _workspace(_lib.LORA_OP_BWD_DX_DA, M, K, L, r, dy.dtype, dy.device, workspace)
    check("lora_bwd_dx_da", lib.lora_bwd_dx_da(
        ctypes.byref(mat(xt)), ctypes.byref(mat(dy)), ctypes.byref(mat(lora_B)), ctypes.byref(mat(lora_A)),
        float(scale), ctypes.byref(mat(dx)), ctypes.byref(mat(dA)), _ptr(ws), nbytes, _stream(dy.device)))
    return dx, dA


def lora_bwd_dx_da_accumulate(xt: torch.Tensor, dy: torch.Tensor, lora_B: torch.Tensor, lora_A: torch.Tensor,
                              scale: float, dx: torch.Tensor, dA: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None, dtype: torch.dtype = torch.float32):
    """dx += scale * (dy @ lora_B) @ lora_A (dx: M x K float32, or bfloat16 with bfloat16 inputs, added to
    in place); dA = scale * xt @ (dy @ lora_B) as in lora_bwd_dx_da (new of `dtype` when not given).
    Returns (dx, dA)."""
    lib = _lib.load()
    K, M = xt.shape
    L = dy.shape[1]
    r = lora_B.shape[1]
    if dA is None:
        dA = torch.empty((K, r), dtype=dtype, device=dy.device)
    ws, nbytes = _workspace(_lib.LORA_OP_BWD_DX_DA, M, K, L, r, dy.dtype, dy.device, workspace)
    check("lora_bwd_dx_da_accumulate", lib.lora_bwd_dx_da_accumulate(
        ctypes.byref(mat(xt)), ctypes.byref(mat(dy)), ctypes.byref(mat(lora_B)), ctypes.byref(mat(lora_A)),
        float(scale), ctypes.byref(mat(dx)), ctypes.byref(mat(dA)), _ptr(ws), nbytes, _stream(dy.device)))
    return dx, dA


def lora_bwd_db(lora_A: torch.Tensor, xt: torch.Tensor, dy: torch.Tensor, scale: float,
                dB: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """dB = scale * (lora_A @ xt) @ dy.  lora_A: r x K, xt: K x M, dy: M x L. Returns dB [r x L]: the given
    tensor, else a new one of `dtype` (float32, or bfloat16 with bfloat16 inputs)."""
    lib = _lib.load()
    r, K = lora_A.shape
    M = xt.shape[1]
    L = dy.shape[1]
    if dB is None:
        dB = torch.empty((r, L), dtype=dtype, device=dy.device)
    ws, nbytes = _workspace(_lib.LORA_OP_BWD_DB, M, K, L, r, dy.dtype, dy.device, workspace)
    check("lora_bwd_db", lib.lora_bwd_db(ctypes.byref(mat(lora_A)), ctypes.byref(mat(xt)), ctypes.byref(mat(dy)),
                                         float(scale), ctypes.byref(mat(dB)), _ptr(ws), nbytes, _stream(dy.device)))
    return dB


# ---------------------------------------------------------------------------
# multi adapter
# ---------------------------------------------------------------------------

class Addressing:
    """Device arrays of one batch's token-to-slot addressing (see lora_addressing in include/lora.h)."""

    def __init__(self, token_slot: torch.Tensor, S: int):
        if token_slot.dtype != torch.int32 or token_slot.dim() != 1:
            raise ValueError("token_slot must be a 1-D int32 tensor")
        dev = token_slot.device
        self.token_slot = token_slot
        self.T = int(token_slot.shape[0])
        self.S = int(S)
        self.counts = torch.empty(max(self.S, 1), dtype=torch.int32, device=dev)
        self.offsets = torch.empty(self.S + 1, dtype=torch.int32, device=dev)
        self.sorted_tokens = torch.empty(max(self.T, 1), dtype=torch.int32, device=dev)

    @classmethod
    def from_arrays(cls, token_slot: torch.Tensor, S: int, counts: torch.Tensor, offsets: torch.Tensor,
                    sorted_tokens: torch.Tensor) -> "Addressing":
        """An addressing over arrays the caller already holds (e.g. built by an earlier call)."""
        a = cls.__new__(cls)
        a.token_slot, a.T, a.S = token_slot, int(token_slot.shape[0]), int(S)
        a.counts, a.offsets, a.sorted_tokens = counts, offsets, sorted_tokens
        return a

    def struct(self) -> LoraAddressing:
        return LoraAddressing(_ptr(self.token_slot), self.T, self.S, _ptr(self.counts), _ptr(self.offsets),
                              _ptr(self.sorted_tokens))


def lora_addressing_build(addr: Addressing, ranks: torch.Tensor, r_max: int) -> Addressing:
    lib = _lib.load()
    check("lora_addressing_build", lib.lora_addressing_build(ctypes.byref(addr.struct()), _ptr(ranks), int(r_max),
                                                             _stream(addr.token_slot.device)))
    return addr


def lora_shrink(x: torch.Tensor, a: torch.Tensor, addr: Addressing, ranks: torch.Tensor, num_slices: int,
                r_max: int, h: torch.Tensor | None = None) -> torch.Tensor:
    """h[t, i, :rank] = x[t] @ a[slot(t), i*r_max : i*r_max+rank]^T. Returns h [T x num_slices x r_max] float32
    (entries of inactive tokens and past a slot's rank are left as they were)."""
    lib = _lib.load()
    if h is None:
        h = torch.zeros((x.shape[0], num_slices, r_max), dtype=torch.float32, device=x.device)
    check("lora_shrink", lib.lora_shrink(ctypes.byref(mat(x)), ctypes.byref(t3(a)), ctypes.byref(addr.struct()),
                                         _ptr(ranks), int(num_slices), int(r_max), ctypes.byref(t3(h)),
                                         _stream(x.device)))
    return h


def lora_expand_fused(h: torch.Tensor, b: torch.Tensor, addr: Addressing, ranks: torch.Tensor,
                      scalings: torch.Tensor, y: torch.Tensor, out_slices, r_max: int) -> torch.Tensor:
    """y[t, slice i] += scalings[slot(t)] * h[t, i, :rank] @ b[slot(t), slice i, :rank]^T, in place; returns y."""
    lib = _lib.load()
    n = len(out_slices)
    sl = (ctypes.c_int64 * n)(*[int(v) for v in out_slices])
    check("lora_expand_fused", lib.lora_expand_fused(
        ctypes.byref(t3(h)), ctypes.byref(t3(b)), ctypes.byref(addr.struct()), _ptr(ranks), _ptr(scalings),
        ctypes.byref(mat(y)), sl, n, int(r_max), _stream(y.device)))
    return y


def lora_apply_linear(x: torch.Tensor, y: torch.Tensor, a: torch.Tensor, b: torch.Tensor, addr: Addressing,
                      ranks: torch.Tensor, scalings: torch.Tensor, out_slices, r_max: int,
                      h: torch.Tensor | None = None) -> torch.Tensor:
    """y[t, slice i] += scalings[slot(t)] * (x[t] @ a[slot(t), slice i]^T) @ b[slot(t), slice i]^T, in place
    (one launch with the rank intermediate on chip, or shrink then expand through h [T x num_slices x r_max]
    float32, the library's choice by shape; h's contents afterwards are unspecified). Returns y."""
    lib = _lib.load()
    n = len(out_slices)
    if h is None:
        h = torch.empty((x.shape[0], n, r_max), dtype=torch.float32, device=x.device)
    sl = (ctypes.c_int64 * n)(*[int(v) for v in out_slices])
    check("lora_apply_linear", lib.lora_apply_linear(
        ctypes.byref(mat(x)), ctypes.byref(t3(a)), ctypes.byref(t3(b)), ctypes.byref(addr.struct()), _ptr(ranks),
        _ptr(scalings), ctypes.byref(mat(y)), sl, n, int(r_max), ctypes.byref(t3(h)), _stream(x.device)))
    return y


def lora_apply_linear_noalloc(x: torch.Tensor, y: torch.Tensor, a: torch.Tensor, b: torch.Tensor, addr: Addressing,
                              ranks: torch.Tensor, scalings: torch.Tensor, out_slices, r_max: int) -> torch.Tensor:
    """lora_apply_linear with the rank intermediate in the library's per-GPU
    scratch (no allocation in the library or here). Returns y."""
    lib = _lib.load()
    n = len(out_slices)
    sl = (ctypes.c_int64 * n)(*[int(v) for v in out_slices])
    check("lora_apply_linear_noalloc", lib.lora_apply_linear_noalloc(
        ctypes.byref(mat(x)), ctypes.byref(t3(a)), ctypes.byref(t3(b)), ctypes.byref(addr.struct()), _ptr(ranks),
        _ptr(scalings), ctypes.byref(mat(y)), sl, n, int(r_max), _stream(x.device)))
    return y


def lora_gather_shrink(ids: torch.Tensor, a: torch.Tensor, addr: Addressing, ranks: torch.Tensor, r_max: int,
                       h: torch.Tensor | None = None) -> torch.Tensor:
    """h[t, 0, j] = a[slot(t), j, ids[t]] for j < rank (+0.0 for ids outside [0, V)). Returns h [T x 1 x r_max]."""
    lib = _lib.load()
    if h is None:
        h = torch.zeros((ids.shape[0], 1, r_max), dtype=torch.float32, device=ids.device)
    check("lora_gather_shrink", lib.lora_gather_shrink(_ptr(ids), ctypes.byref(t3(a)), ctypes.byref(addr.struct()),
                                                       _ptr(ranks), int(r_max), ctypes.byref(t3(h)),
                                                       _stream(ids.device)))
    return h


def lora_timing_begin() -> None:
    """Start recording kernel durations (forgets earlier records)."""
    check("lora_timing_begin", _lib.load().lora_timing_begin())


def lora_timing_pause() -> None:
    """Stop recording; later launches run untimed."""
    check("lora_timing_pause", _lib.load().lora_timing_pause())


def lora_timing_resume() -> None:
    """Record again, keeping the earlier records."""
    check("lora_timing_resume", _lib.load().lora_timing_resume())


def lora_timing_reserve(pairs: int) -> None:
    """Create event pairs up front (on the current device) so that timed
    launches do not create events while being timed."""
    check("lora_timing_reserve", _lib.load().lora_timing_reserve(int(pairs)))


def lora_timing_read() -> tuple[float, int]:
    """Waits for the recorded kernels; returns (sum of their durations in ms, number of launches)."""
    total = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    check("lora_timing_read", _lib.load().lora_timing_read(ctypes.byref(total), ctypes.byref(n)))
    return total.value, n.value
