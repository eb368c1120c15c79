"""Pins of the oracle's prologue / epilogue activations (oracle/fused.py)
against special values and identities the definitions fix."""

import math

import numpy as np
import pytest

from oracle import fused


def test_l2_normalize_gives_unit_rows_and_keeps_directions():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 3, 7)) * 10.0
    y = fused.l2_normalize(x)
    norms = np.linalg.norm(y, axis=-1)
    # |y| = |x| / sqrt(|x|^2 + eps): one to within eps / (2 |x|^2)
    np.testing.assert_allclose(norms, np.linalg.norm(x, axis=-1) /
                               np.sqrt(np.sum(x * x, -1) + 1e-6), rtol=1e-15)
    assert np.all(np.abs(norms - 1.0) < 1e-6)
    # direction kept: y is a positive multiple of x
    np.testing.assert_allclose(y * np.linalg.norm(x, axis=-1, keepdims=True) / norms[..., None],
                               x, rtol=1e-12)
    # a zero row stays zero (no division by zero)
    assert np.all(fused.l2_normalize(np.zeros((2, 4))) == 0.0)


def test_sigmoid_special_values():
    assert fused.sigmoid(0.0) == 0.5
    np.testing.assert_allclose(fused.sigmoid(math.log(3.0)), 0.75, rtol=1e-15)
    np.testing.assert_allclose(fused.sigmoid(-math.log(3.0)), 0.25, rtol=1e-15)
    x = np.linspace(-20, 20, 41)
    np.testing.assert_allclose(fused.sigmoid(x) + fused.sigmoid(-x), 1.0, rtol=1e-15)


def test_softplus_special_values_and_identity():
    np.testing.assert_allclose(fused.softplus(0.0), math.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(fused.softplus(math.log(math.e - 1.0)), 1.0, rtol=1e-15)
    x = np.linspace(-30, 800, 200)
    # softplus(x) - softplus(-x) = x, also where e^x overflows
    np.testing.assert_allclose(fused.softplus(x) - fused.softplus(-x), x, rtol=1e-12, atol=1e-12)
    assert np.all(np.isfinite(fused.softplus(x)))


@pytest.mark.parametrize("kind,x,want", [
    ("softplus", 0.0, -math.log(2.0)),
    ("softplus", math.log(math.e - 1.0), -1.0),
    # GLA: a = sigmoid(x)^(1/16); at x = ln 3, sigmoid = 3/4
    ("gla", math.log(3.0), math.log(0.75) / 16.0),
    ("gla", 0.0, -math.log(2.0) / 16.0),
])
def test_log_decay_special_values(kind, x, want):
    np.testing.assert_allclose(fused.log_decay(np.array([x]), kind), [want], rtol=1e-14)
    assert fused.log_decay(np.array([x]), None)[0] == x
    # both transforms give a decay a in (0, 1)
    xs = np.linspace(-10, 10, 21)
    a = np.exp(fused.log_decay(xs, kind))
    assert np.all((a > 0) & (a < 1))


def test_silu_gate_special_values():
    assert fused.silu_gate(3.0, 0.0) == 0.0
    np.testing.assert_allclose(fused.silu_gate(2.0, math.log(3.0)), 2.0 * math.log(3.0) * 0.75,
                               rtol=1e-15)
    # large positive gates pass the output through times g
    np.testing.assert_allclose(fused.silu_gate(1.5, 40.0), 1.5 * 40.0, rtol=1e-15)


def test_prologue_applies_each_transform_only_when_asked():
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=(1, 4, 2, 8)), rng.normal(size=(1, 4, 2, 8))
    beta, la = rng.normal(size=(1, 4, 2)), rng.normal(size=(1, 4, 2))
    q0, k0, b0, l0 = fused.prologue(q, k, beta, la)
    assert np.array_equal(q0, q) and np.array_equal(b0, beta) and np.array_equal(l0, la)
    q1, k1, b1, l1 = fused.prologue(q, k, beta, la, qk_l2norm=True, beta_sigmoid=True,
                                    decay="softplus")
    np.testing.assert_allclose(np.linalg.norm(q1, axis=-1), 1.0, atol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(k1, axis=-1), 1.0, atol=1e-6)
    np.testing.assert_allclose(b1, 1.0 / (1.0 + np.exp(-beta)), rtol=1e-15)
    np.testing.assert_allclose(l1, -np.log1p(np.exp(la)), rtol=1e-13)
