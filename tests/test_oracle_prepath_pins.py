"""Pins for the pre-path oracle (``oracle.prepath``): textbook values and
identities of softplus, the logistic function and the Euclidean norm."""
import math

import numpy as np

from oracle import prepath


def test_softplus_and_sigmoid_values():
    assert prepath.neg_softplus(np.array([0.0]))[0] == -math.log(2.0)
    assert prepath.sigmoid(np.array([0.0]))[0] == 0.5
    # large arguments: softplus(x) -> x, softplus(-x) -> e^-x; no overflow
    x = np.array([800.0, -800.0, 40.0])
    assert np.isfinite(prepath.neg_softplus(x)).all()
    assert prepath.neg_softplus(x)[0] == -800.0
    assert abs(prepath.neg_softplus(np.array([-40.0]))[0] + math.exp(-40.0)) < 1e-30
    assert prepath.sigmoid(x)[0] == 1.0 and prepath.sigmoid(x)[1] == 0.0


def test_identities():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(1000) * 6
    s = prepath.sigmoid(x)
    assert np.allclose(s + prepath.sigmoid(-x), 1.0, atol=1e-15)
    # the decay exp(-softplus(x)) is the logistic function of -x
    assert np.allclose(np.exp(prepath.neg_softplus(x)), prepath.sigmoid(-x), rtol=1e-14, atol=1e-300)
    # derivative of softplus is the logistic function (central differences)
    h = 1e-6
    d = -(prepath.neg_softplus(x + h) - prepath.neg_softplus(x - h)) / (2 * h)
    assert np.allclose(d, s, atol=1e-8)


def test_l2_normalize():
    v = prepath.l2_normalize(np.array([[3.0, 4.0], [0.0, 0.0], [0.0, -2.0]]))
    assert np.array_equal(v, np.array([[0.6, 0.8], [0.0, 0.0], [0.0, -1.0]]))
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, 3, 128))
    y = prepath.l2_normalize(x)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-14)
    # parallel to the input, same orientation
    cos = np.sum(x * y, axis=-1) / np.linalg.norm(x, axis=-1)
    assert np.allclose(cos, 1.0, atol=1e-14)
