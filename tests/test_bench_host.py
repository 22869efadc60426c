"""Host-side checks of bench.py (no GPU): a batch larger than the activations prepared
for it is refused before anything reaches the library, and the bench prepares enough
activation rows for every batch it is asked to time."""

import numpy as np
import pytest
import torch

import bench
import workloads as wl


def test_time_layer_refuses_a_batch_larger_than_its_activations():
    cfg = wl.CONFIGS["c3"]
    layer = {"x": torch.zeros((16, cfg.K), dtype=torch.float16)}
    with pytest.raises(ValueError, match="M=64"):
        bench.time_layer(cfg, 64, layer, 1, 0, sample_clocks=False)
    with pytest.raises(ValueError):
        bench.time_layer(cfg, 1, {"x": torch.zeros((1, cfg.K // 2), dtype=torch.float16)}, 1, 0,
                         sample_clocks=False)


def test_activations_cover_batches_beyond_the_configured_list():
    cfg = wl.CONFIGS["c3"]
    x = wl.activations(cfg, 64)
    assert x.shape == (64, cfg.K)
    np.testing.assert_array_equal(x[:16], wl.activations(cfg, 16))
