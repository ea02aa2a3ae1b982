"""The seeded input generator: deterministic, offset-addressable, with the stated statistics."""
import numpy as np
import torch

from layer_wise_obs_amd import synth


def test_activations_reproducible_and_offset_addressable():
    a = synth.activations(64, 48, 7, 1, 3, 20.0, relu=True, dtype=torch.bfloat16)
    b = synth.activations(64, 48, 7, 1, 3, 20.0, relu=True, dtype=torch.bfloat16)
    assert torch.equal(a, b)
    part = synth.activations(16, 48, 7, 1, 3, 20.0, relu=True, dtype=torch.bfloat16, token_offset=40)
    assert torch.equal(part, a[40:56])


def test_statistics_and_outliers():
    x = synth.activations(4096, 64, 11, 1, 2, 30.0, relu=False, dtype=torch.float32)
    oc = synth.outlier_channels(64, 2, 11, 1)
    assert len(oc) == 2
    normal = np.setdiff1d(np.arange(64), oc.numpy())
    v = x[:, normal].numpy()
    assert abs(v.mean()) < 0.02 and abs(v.std() - 1.0) < 0.02
    assert abs(x[:, oc].numpy().std() / 30.0 - 1.0) < 0.05
    r = synth.activations(4096, 64, 11, 1, 2, 30.0, relu=True, dtype=torch.float32)[:, normal]
    assert abs((r == 0).float().mean().item() - 0.5) < 0.02
    w = synth.weights(256, 256, 0.02, 3, 100, dtype=torch.float32)
    assert abs(w.std().item() - 0.02) < 0.001


def test_config_shapes():
    c3 = synth.config(3)
    assert (c3.layers[0].c, c3.layers[0].b) == (4096, 11008)
    assert c3.streams["down_in"].n == 262144 and c3.streams["down_in"].outlier_count == 110
    c5 = synth.config(5)
    assert c5.streams["down_in"].outlier_count == 287
    assert synth.config(1).block == 32
