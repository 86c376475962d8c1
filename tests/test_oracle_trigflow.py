"""Pins for the oracle's TrigFlow <-> rectified-flow coefficients.

Printed values from the pages (tests/golden/trigflow_rf_times.json), closed
forms at t = pi/4, central differences of the coefficients and of the TrigFlow
path, and the reconstruction identities the page derives.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import trigflow as tf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "trigflow_rf_times.json")


def _theta(x):
    return math.atan(80.0) if x == "arctan(80)" else float(x)


def test_printed_rectified_flow_times():
    g = json.load(open(GOLDEN))
    theta = np.array([_theta(x) for x in g["theta"]])
    got = tf.rf_time(theta)
    half_ulp = 0.5 * 10 ** -g["printed_decimals"]
    np.testing.assert_allclose(got, g["t_rf_printed"], rtol=0, atol=half_ulp + 1e-12)
    # the page: the first time also equals sigma / (sigma + 1)
    s = g["sigma_max"]
    assert abs(got[0] - s / (s + 1)) < 1e-14
    # c_noise is the same time times the scaling factor
    np.testing.assert_allclose(tf.coefficients(theta)[3], 1000.0 * got, rtol=1e-15)


def test_closed_forms_at_quarter_pi():
    c_skip, c_out, c_in, c_noise = tf.coefficients(math.pi / 4)
    assert abs(c_skip - 1 / math.sqrt(2)) < 1e-15
    assert abs(c_in - 1 / math.sqrt(2)) < 1e-15
    assert abs(c_out + 0.5) < 1e-15
    assert abs(c_noise - 500.0) < 1e-12


@pytest.mark.parametrize("t", [0.05, 0.4, math.pi / 4, 1.2, 1.56])
def test_derivatives_match_central_differences(t):
    h = 1e-4
    d_cf = tf.coefficient_derivatives(t)
    for i in range(4):
        f = lambda x: tf.coefficients(x)[i]
        d1 = (f(t + h) - f(t - h)) / (2 * h)
        d2 = (f(t + h / 2) - f(t - h / 2)) / h
        fd = (4 * d2 - d1) / 3
        assert abs(d_cf[i] - fd) < 1e-8 * max(1.0, abs(fd)), i


@pytest.mark.parametrize("t", [0.1, 0.7, 1.3])
def test_edm_wrapper_recovers_clean_sample(t):
    # x_rf = c_in x_t, the rectified-flow velocity eps - x0, and
    # c_skip x_t + c_out (eps - x0) gives back x0 (section 时间步转换)
    rng = np.random.default_rng(0)
    x0, eps = rng.standard_normal((2, 50))
    xt = tf.trig_path(x0, eps, t)
    c_skip, c_out, c_in, _ = tf.coefficients(t)
    t_rf = tf.rf_time(t)
    x_rf = (1 - t_rf) * x0 + t_rf * eps
    np.testing.assert_allclose(c_in * xt, x_rf, atol=1e-14)
    np.testing.assert_allclose(c_skip * xt + c_out * (eps - x0), x0, atol=1e-14)
    # and the TrigFlow-space prediction from the exact x0 is the path velocity
    np.testing.assert_allclose(tf.f_pred(xt, x0, t), tf.trig_velocity(x0, eps, t), atol=1e-13)


@pytest.mark.parametrize("t", [0.2, 1.0])
def test_trig_velocity_is_path_derivative(t):
    rng = np.random.default_rng(1)
    x0, eps = rng.standard_normal((2, 20))
    h = 1e-4
    fd = (tf.trig_path(x0, eps, t + h) - tf.trig_path(x0, eps, t - h)) / (2 * h)
    np.testing.assert_allclose(tf.trig_velocity(x0, eps, t), fd, atol=1e-8)


@pytest.mark.parametrize("h", [1e-4, 0.1, 0.5])
def test_trig_path_shift_identity(h):
    # the page's finite-difference identity F(t-h) = cos h F(t) - sin h dF/dt,
    # exact for the TrigFlow velocity F = -sin t x0 + cos t eps
    rng = np.random.default_rng(2)
    x0, eps = rng.standard_normal((2, 20))
    t = 0.9
    F = lambda s: tf.trig_velocity(x0, eps, s)
    dF = -math.cos(t) * x0 - math.sin(t) * eps
    np.testing.assert_allclose(F(t - h), math.cos(h) * F(t) - math.sin(h) * dF, atol=1e-13)
