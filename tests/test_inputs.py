"""The seeded input generators (CPU only)."""

import numpy as np
import torch

from memory_efficient_activation_amd import inputs


def test_bf16_encoding_matches_torch_cast():
    rng = np.random.default_rng(5)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1e-40, -3e38, 3.3e38, np.nan], np.float32)])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = inputs.f32_to_bf16_bits(a)
    fin = ~np.isnan(a)
    assert np.array_equal(got[fin], want[fin])
    assert np.isnan(inputs.bf16_bits_to_f32(got[~fin])).all()
    back = inputs.bf16_bits_to_f32(got[fin])
    assert np.array_equal(torch.from_numpy(back).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16),
                          got[fin])


def test_small_workloads_are_deterministic_and_shaped():
    for idx in (1, 2, 3, 4):
        a = inputs.make(idx, n=4096)
        b = inputs.make(idx, n=4096)
        assert a.xs[0].tobytes() == b.xs[0].tobytes()
        assert a.dys[0].tobytes() == b.dys[0].tobytes()
        assert a.xs[0].dtype == (np.uint16 if a.dtype == "bf16" else np.float32)
    w1 = inputs.make(1)
    assert w1.shapes == [(65536,)] and w1.alpha == 1.0
    assert abs(float(np.std(w1.xs[0])) - 3.0) < 0.05


def test_outlier_mixture_recipe():
    w = inputs.make(4, n=1 << 20)
    x = w.xs[0]
    out = np.abs(x) >= 20
    frac = out.mean()
    assert 0.009 < frac < 0.011
    assert np.abs(x).max() <= 90.0
    assert (x[out] > 0).mean() > 0.45 and (x[out] < 0).mean() > 0.45
    assert w.alpha == 1.5


def test_grouped_workload_shapes():
    shapes = inputs.CONFIG_SHAPES[5]
    assert len(shapes) == 7
    assert sum(int(np.prod(s)) for s in shapes) == 70_045_696


def test_exhaustive_bf16_count():
    b = inputs.exhaustive_bf16_finite()
    assert b.size == 65280
    assert np.isfinite(inputs.bf16_bits_to_f32(b)).all()


def test_densenet_bc100_channel_bookkeeping():
    """DenseNet-BC-100 at growth 12: 16 layers per block, block inputs 24,
    108 (= (24 + 16 * 12) / 2) and 150 (= (108 + 16 * 12) / 2) channels."""
    from memory_efficient_activation_amd import dense_inputs as di
    assert (100 - 4) // 6 == di.BLOCK_LAYERS
    assert di.BLOCKS[1][0] == (di.BLOCKS[0][0] + di.BLOCK_LAYERS * di.GROWTH) // 2
    assert di.BLOCKS[2][0] == (di.BLOCKS[1][0] + di.BLOCK_LAYERS * di.GROWTH) // 2
    assert sum(di.block_layer_channels(0, 15)) == 204
    assert di.block_layer_channels(2, 0) == [150]
    w = di.dense_layer([3, 2], 2, 5, "bf16", seed=1)
    assert [s.shape for s in w.sources] == [(2, 3, 5), (2, 2, 5)]
    assert w.dz.shape == (2, 5, 5) and w.dz.dtype == np.uint16
    assert w.gamma.dtype == np.float32 and w.gamma.shape == (5,)
    w2 = di.dense_layer([3, 2], 2, 5, "bf16", seed=1)
    assert all(np.array_equal(a, b) for a, b in zip(w.sources, w2.sources))
