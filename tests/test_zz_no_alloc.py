"""lora_apply_linear_noalloc (the rank intermediate in the library's per-GPU
scratch array, no allocation) against lora_apply_linear with a caller
workspace, through the C ABI: the same kernels, so bit for bit, on two calls
in a row (the second with a smaller batch, so it runs over what the first
left in the scratch), and a batch too large for the scratch refused before
any launch."""
import numpy as np
import pytest
import torch

import lora_rank_adapter_amd as L
import oracle
import synth
from tests.gpu_util import DEV, dev, f32, host, note, same_bits

pytestmark = pytest.mark.gpu


def _batch(kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "prefill":
        ts, ranks, _ = synth.prefill_routing(12, 10, (8, 16, 32, 64), rng, median=120.0, sigma=0.6, cap=400)
        return synth.multi_lora(ts, ranks, 512, (256, 128, 64), 64, rng=rng, name=kind)
    ts, ranks = synth.decode_routing(96, 8, 64, (0, 8, 16, 64), 0.1, rng)
    return synth.multi_lora(ts, ranks, 512, (256, 128, 64), 64, rng=rng, name=kind)


def test_noalloc_matches_workspace_call():
    for kind, seed in (("prefill", 11), ("decode", 12)):
        m = _batch(kind, seed)
        note(f"apply_linear_noalloc {kind} T={m.T}")
        ts = torch.from_numpy(m.token_slot).to(DEV)
        ranks = torch.from_numpy(m.ranks).to(DEV)
        addr = L.lora_addressing_build(L.Addressing(ts, m.S), ranks, m.r_max)
        x, a, b, sc = dev(m.x, "bf16"), dev(m.a, "bf16"), dev(m.b, "bf16"), f32(m.scalings)
        y_ref = f32(m.y0)
        L.lora_apply_linear(x, y_ref, a, b, addr, ranks, sc, m.out_slices, m.r_max)
        y = f32(m.y0)
        L.lora_apply_linear_noalloc(x, y, a, b, addr, ranks, sc, m.out_slices, m.r_max)
        torch.cuda.synchronize()
        got = host(y)
        assert same_bits(got, host(y_ref)), kind
        rho = oracle.token_ranks(m.token_slot, m.ranks, m.r_max)
        act = rho > 0
        assert same_bits(got[~act], m.y0[~act])
        want = oracle.apply_linear(m.x, m.y0, m.a, m.b, m.token_slot, m.ranks, m.scalings, m.out_slices, m.r_max)
        assert oracle.rel_frobenius(got[act] - m.y0[act], want[act] - m.y0[act]) <= 2e-3


def test_noalloc_refuses_batches_beyond_the_scratch():
    """70000 tokens x 3 slices x rank 128 (107 MB of h) exceed the 32 MiB
    scratch: LORA_ERR_LIMIT, nothing launched, y untouched."""
    note("apply_linear_noalloc beyond the scratch")
    T, K, r_max = 70000, 8, 128
    ts = torch.zeros(T, dtype=torch.int32, device=DEV)
    ranks = torch.full((1,), 8, dtype=torch.int32, device=DEV)
    addr = L.Addressing(ts, 1)
    x = torch.zeros((T, K), dtype=torch.bfloat16, device=DEV)
    a = torch.zeros((1, 3 * r_max, K), dtype=torch.bfloat16, device=DEV)
    b = torch.zeros((1, 12, r_max), dtype=torch.bfloat16, device=DEV)
    y = torch.full((T, 12), 5.0, device=DEV)
    with pytest.raises(L.LoraError) as e:
        L.lora_apply_linear_noalloc(x, y, a, b, addr, ranks, torch.ones(1, device=DEV), (4, 4, 4), r_max)
    assert e.value.status == -8
    torch.cuda.synchronize()
    assert bool((y == 5.0).all())
