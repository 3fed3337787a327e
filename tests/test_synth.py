"""Seeded input generators: reproducibility, shapes, byte counts (CPU only)."""
import numpy as np
import torch

from synth import (LayerSpec, make_layer, make_x, make_logits, zipf_bias, q2k_bytes_per_matrix,
                   mxfp4_bytes_per_matrix, derive_seed, WORKLOADS)


def test_seeds_reproducible_and_distinct():
    assert derive_seed(1, 0, "gate", 3) == derive_seed(1, 0, "gate", 3)
    assert derive_seed(1, 0, "gate", 3) != derive_seed(1, 0, "gate", 4)
    assert derive_seed(1, 0, "gate", 3) != derive_seed(1, 1, "gate", 3)
    a = make_x(4, 64, seed=3)
    b = make_x(4, 64, seed=3)
    assert torch.equal(a, b) and a.dtype == torch.bfloat16
    assert torch.equal(make_logits(4, 8, seed=3), make_logits(4, 8, seed=3))
    assert not torch.equal(make_logits(4, 8, seed=3, index=0), make_logits(4, 8, seed=3, index=1))


def test_tiny_layer_bytes():
    spec = WORKLOADS["tiny"]["spec"]
    L = make_layer(spec, device="cpu")
    L2 = make_layer(spec, device="cpu")
    assert torch.equal(L.gate, L2.gate) and torch.equal(L.down, L2.down)
    assert L.gate.shape == (8, q2k_bytes_per_matrix(128, 256)) == (8, 10752)
    assert L.down.shape == (8, 10752)
    assert L.sh_gate is None
    total = sum(L.weight_bytes().values())
    assert total == 258048


def test_full_size_byte_counts():
    assert q2k_bytes_per_matrix(2048, 7168) == 4816896
    assert 3 * q2k_bytes_per_matrix(2048, 7168) == 14450688
    c, s = mxfp4_bytes_per_matrix(2048, 7168)
    assert c + s == 7798784


def test_mxfp4_layer_shapes():
    L = make_layer(LayerSpec(256, 128, 2, 1, 64, "mxfp4"), device="cpu")
    assert L.gate.shape == (2, 128, 128) and L.gate_scales.shape == (2, 128, 8)
    assert L.down.shape == (2, 256, 64) and L.down_scales.shape == (2, 256, 4)
    assert L.sh_down.dtype == torch.bfloat16 and L.sh_down.shape == (256, 64)


def test_zipf_bias_skews_popularity():
    b = zipf_bias(256, 1.1, seed=1)
    p = np.exp(b)
    assert abs(p.sum() - 1) < 1e-12
    assert p.max() / p.min() > 256 ** 1.1 * 0.99
