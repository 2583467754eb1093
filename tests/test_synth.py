"""The seeded input generator: bf16 rounding and the workload laws (CPU)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -1e-40, 65504.0])])
    got = synth.bf16_bits(v)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    back = synth.bf16_to_f32(got)
    assert np.array_equal(back, torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_nan_padding_bits():
    assert synth.bf16_bits(np.float32([np.nan]))[0] == 0x7FC0


def test_config1_shapes_and_laws():
    c = synth.config1()
    assert c.X.shape == (256, 512) and c.A.shape == (512, 8) and c.B.shape == (8, 512) and c.dY.shape == (256, 512)
    assert c.dtype == "f32" and c.scale == 2.0 and not c.Y0.any()
    assert abs(c.A.std() - 1 / np.sqrt(512)) < 0.1 / np.sqrt(512)
    assert abs(c.B.std() - 1 / np.sqrt(8)) < 0.1 / np.sqrt(8)


def test_seeded_determinism():
    a = synth.single_adapter(40, 24, 16, 4, seed=9)
    b = synth.single_adapter(40, 24, 16, 4, seed=9)
    assert np.array_equal(a.X, b.X) and np.array_equal(a.B, b.B)


def test_config4_routing_laws():
    c = synth.config4()
    assert c.T == 256 and c.S == 32 and c.r_max == 64 and c.out_slices == (4096, 1024, 1024)
    assert c.ranks[0] == 0 and set(np.unique(c.ranks[1:])) <= {0, 8, 16, 32, 64}
    frac0 = np.mean(c.token_slot == 0)
    assert 0.03 < frac0 < 0.2
    act = synth._active_rows(c.token_slot, c.ranks, c.r_max)
    assert np.all(np.signbit(c.y0[~act]))  # inactive rows hold -0.0
    s = int(c.token_slot[act][0])
    assert np.isnan(c.a[s, c.ranks[s]:c.r_max]).all() if c.ranks[s] < c.r_max else True


def test_config5_routing_laws():
    ts, ranks, lengths, _ = synth.config5_routing()
    assert len(lengths) == 64 and lengths.min() >= 1 and lengths.max() <= 2048
    assert 12000 < lengths.sum() < 26000
    assert set(np.unique(ranks)) <= {8, 16, 32, 64, 128}
    # tokens of a request are contiguous and share a slot
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    for s0, n in zip(starts, lengths):
        assert np.all(ts[s0:s0 + n] == ts[s0])
