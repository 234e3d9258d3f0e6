"""Pins of the oracle's steering projection (QuarkStar README, "Steering":
an FFN output m becomes m - scale * d * (d . m)) against hand-worked values,
closed forms of projections and reflections, and where in the layer it acts."""
import numpy as np
import pytest

import synth
from oracle import moe as om


def test_hand_worked_2d():
    # d = (0.6, 0.8) is a unit vector, m = (1, 2): d . m = 0.6 + 1.6 = 2.2
    d = np.array([0.6, 0.8])
    m = np.array([[1.0, 2.0]])
    assert np.allclose(om.steer(m, d, 1.0), [[1 - 1.32, 2 - 1.76]], atol=1e-15)    # (-0.32, 0.24)
    assert np.allclose(om.steer(m, d, 0.5), [[1 - 0.66, 2 - 0.88]], atol=1e-15)    # (0.34, 1.12)
    assert np.allclose(om.steer(m, d, -1.0), [[1 + 1.32, 2 + 1.76]], atol=1e-15)   # (2.32, 3.76)


def _unit(rng, n):
    v = rng.standard_normal(n)
    return v / np.linalg.norm(v)


@pytest.mark.parametrize("scale", [1.0, 0.8, 0.25, -0.5, 2.0])
def test_component_along_d_scales_by_one_minus_s(scale):
    """For a unit d: d . m' = (1 - s) (d . m), and the part of m orthogonal to
    d is untouched."""
    rng = np.random.default_rng(3)
    d = _unit(rng, 64)
    m = rng.standard_normal((5, 64))
    got = om.steer(m, d, scale)
    assert np.allclose(got @ d, (1 - scale) * (m @ d), rtol=1e-12, atol=1e-12)
    orth = np.eye(64) - np.outer(d, d)
    assert np.allclose(got @ orth, m @ orth, rtol=1e-12, atol=1e-12)


def test_scale_one_is_an_idempotent_projection():
    rng = np.random.default_rng(4)
    d = _unit(rng, 32)
    m = rng.standard_normal((3, 32))
    once = om.steer(m, d, 1.0)
    assert np.allclose(once @ d, 0.0, atol=1e-13)
    assert np.allclose(om.steer(once, d, 1.0), once, atol=1e-13)


def test_scale_two_is_the_householder_reflection():
    """s = 2 with a unit d is the reflection I - 2 d d^T: it keeps norms and
    is its own inverse; numpy's QR of the same reflector gives it back."""
    rng = np.random.default_rng(5)
    d = _unit(rng, 16)
    m = rng.standard_normal((4, 16))
    r = om.steer(m, d, 2.0)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(m, axis=1), rtol=1e-12)
    assert np.allclose(om.steer(r, d, 2.0), m, atol=1e-12)
    refl = np.eye(16) - 2.0 * np.outer(d, d)
    q, _ = np.linalg.qr(refl)
    assert np.allclose(np.abs(q @ q.T), np.eye(16), atol=1e-12)   # the reflector is orthogonal
    assert np.allclose(r, m @ refl.T, atol=1e-12)


def test_zero_scale_and_zero_direction_are_identity():
    rng = np.random.default_rng(6)
    m = rng.standard_normal((2, 8))
    assert np.array_equal(om.steer(m, _unit(rng, 8), 0.0), m)
    assert np.array_equal(om.steer(m, np.zeros(8), 1.0), m)


def test_steering_acts_on_the_moe_output_before_the_residual():
    """With scale 1 and a unit d, the layer's contribution y - x (routed
    experts plus shared expert) has no component along d; the input x keeps
    its own.  Steering after the residual add would fail this."""
    wl = synth.Workload("steer", 30, 512, 16, 2, 256, 128, "cb2", "q2k", 1, (1,))
    cb = synth.codebook()
    layer = om.Layer(wl, synth.layer_weights(wl, 0), cb)
    x = synth.tokens(wl, 3)
    d = _unit(np.random.default_rng(7), wl.hidden)
    for prenorm in (False, True):
        plain = om.moe_layer(layer, x, residual=True, prenorm=prenorm)
        st = om.moe_layer(layer, x, residual=True, prenorm=prenorm, steering=(d, 1.0))
        y = st["y"].astype(np.float64)
        delta = y - x.astype(np.float64)
        m = plain["y"].astype(np.float64) - x.astype(np.float64)
        # y is rounded to fp32 once: |(delta . d)| <= 2^-24 ||y|| per row (unit d)
        bound = 2.0 ** -24 * np.linalg.norm(y, axis=1)
        assert np.all(np.abs(delta @ d) <= bound)
        assert np.all(np.abs(m @ d) > 100 * bound)               # the unsteered output has one
        assert np.array_equal(st["ids"], plain["ids"])          # routing is not affected
        assert abs(float(x[0].astype(np.float64) @ d)) > 1e-3    # x itself has a component


def test_stack_uses_each_layers_own_direction():
    wl = synth.Workload("steer3", 31, 512, 16, 2, 256, 0, "q2k", "q2k", 3, (1,))
    cb = synth.codebook()
    layers = [om.Layer(wl, synth.layer_weights(wl, l), cb) for l in range(3)]
    rng = np.random.default_rng(8)
    dirs = np.stack([_unit(rng, wl.hidden) for _ in range(3)])
    x = synth.tokens(wl, 2)
    _, per = om.moe_stack(layers, x, prenorm=True, steering=(dirs, 1.0))
    cur = x.astype(np.float64)
    for l in range(3):
        y = per[l]["y"].astype(np.float64)
        delta = y - cur
        bound = 2.0 ** -24 * np.linalg.norm(y, axis=1)            # fp32 rounding of y
        assert np.all(np.abs(delta @ dirs[l]) <= bound)
        assert np.all(np.abs(delta @ dirs[(l + 1) % 3]) > 100 * bound)   # not along another layer's d
        cur = y
