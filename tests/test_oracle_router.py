"""Pins for the oracle's router projection (CPU only).

logits[t][e] = sum_h W_r[e][h] x[t][h] is checked against what fixes it
independently of the matrix product the oracle calls: a selection matrix
(one 1 per row) that must copy chosen activations out unchanged, which
catches a transposed operand or a wrong axis on non-square shapes; exact
rational sums on tiny inputs; exact scaling by powers of two; and routing of
logits built so that the expert order is known in advance.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import make_router_w, make_x


def _bf16_values(a):
    """float32 values rounded to bf16 (RNE) as float64, via bit patterns."""
    bits = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint32)
    return (r << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("T,E,H", [(3, 5, 16), (1, 8, 256), (7, 24, 40)])
def test_selection_matrix_copies_activations(T, E, H):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((T, H))
    pick = rng.choice(H, size=E, replace=E > H)
    w = np.zeros((E, H))
    w[np.arange(E), pick] = 1.0
    out = oracle.router_logits(x, w)
    assert out.shape == (T, E)
    assert np.array_equal(out, x[:, pick])


def test_exact_rational_sums_on_tiny_inputs():
    rng = np.random.default_rng(12)
    T, E, H = 3, 4, 12
    x = _bf16_values(rng.standard_normal((T, H)))
    w = _bf16_values(rng.standard_normal((E, H)) * 0.1)
    out = oracle.router_logits(x, w)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(w[e, h])) * Fraction(float(x[t, h])) for h in range(H))
            mag = sum(abs(Fraction(float(w[e, h])) * Fraction(float(x[t, h]))) for h in range(H))
            # fp64 summation of H exact products
            assert abs(Fraction(float(out[t, e])) - exact) <= H * Fraction(2) ** -53 * mag


def test_power_of_two_scaling_is_exact():
    x = make_x(5, 512, seed=13).float().numpy()
    w = make_router_w(16, 512, seed=14).float().numpy()
    a = oracle.router_logits(x, w)
    assert np.array_equal(oracle.router_logits(4.0 * x, w), 4.0 * a)
    assert np.array_equal(oracle.router_logits(x, 0.5 * w), 0.5 * a)


def test_known_expert_order_routes_through():
    """Rows W_r[e] = c_e * d for a direction d with d . x > 0: the logits are
    c_e * (d . x), so the top-k experts are those with the k largest c_e."""
    rng = np.random.default_rng(15)
    H, E, k = 64, 12, 3
    x = rng.standard_normal((1, H))
    d = np.sign(x[0]) * 0.25                      # d . x = 0.25 * sum |x| > 0
    c = rng.permutation(E).astype(np.float64) - 4.0
    w = c[:, None] * d[None, :]
    idx, _ = oracle.route(oracle.router_logits(x, w), k)
    assert idx[0].tolist() == list(np.argsort(-c)[:k])


def test_synthetic_router_scale():
    """N(0, 1/H) router rows on N(0,1) activations give unit-variance logits."""
    x = make_x(64, 1024, seed=16).float().numpy()
    w = make_router_w(64, 1024, seed=17).float().numpy()
    l = oracle.router_logits(x, w)
    assert 0.8 < l.std() < 1.2


def test_shape_errors():
    with pytest.raises(ValueError):
        oracle.router_logits(np.zeros((2, 8)), np.zeros((3, 9)))
