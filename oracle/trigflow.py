"""TrigFlow <-> rectified-flow coefficients, in float64.

TEST INFRASTRUCTURE (the oracle): never imported by the library.

Page "带分数正则的一致性蒸馏" (gitcode.csdn.net), section 时间步转换: a teacher
trained on the rectified-flow schedule x = (1 - t_rf) x0 + t_rf eps is used at
TrigFlow time t (x_t = cos t x0 + sin t eps, sigma_data = 1) by matching the
noise-to-signal ratio, t_rf / (1 - t_rf) = tan t.  That gives

  c_noise(t) = sin t / (sin t + cos t)    (= t_rf; the code multiplies it by a
                                           time scaling factor, 1000)
  c_in(t)    = 1 / (sin t + cos t)
  c_skip(t)  = 1 / (sin t + cos t)
  c_out(t)   = -sin t / (sin t + cos t)

and the TrigFlow-space prediction F = (cos t x_t - x0_pred) / sin t.  The same
section evaluates everything in float64.  The TrigFlow path's velocity
dx_t/dt = -sin t x0 + cos t eps is the tangent the distillation step feeds to
the network (sections 一致性模型 and 蒸馏代码).

Derivatives below are the closed forms of d/dt of the expressions above.
"""

import numpy as np

__all__ = [
    "coefficients",
    "coefficient_derivatives",
    "rf_time",
    "trig_path",
    "trig_velocity",
    "f_pred",
    "T_SCALING",
]

T_SCALING = 1000.0  # the code's rectified_flow_t_scaling_factor


def coefficients(t, t_scaling=T_SCALING):
    """(c_skip, c_out, c_in, c_noise) at TrigFlow time t (float64)."""
    t = np.asarray(t, dtype=np.float64)
    s, c = np.sin(t), np.cos(t)
    den = s + c
    c_skip = 1.0 / den
    c_out = -s / den
    c_in = 1.0 / den
    c_noise = (s / den) * t_scaling
    return c_skip, c_out, c_in, c_noise


def coefficient_derivatives(t, t_scaling=T_SCALING):
    """d/dt of (c_skip, c_out, c_in, c_noise)."""
    t = np.asarray(t, dtype=np.float64)
    s, c = np.sin(t), np.cos(t)
    den2 = (s + c) ** 2
    d_skip = (s - c) / den2
    d_out = -1.0 / den2
    d_in = (s - c) / den2
    d_noise = t_scaling / den2
    return d_skip, d_out, d_in, d_noise


def rf_time(t):
    """Rectified-flow time matched to TrigFlow time t (c_noise without the
    scaling factor)."""
    t = np.asarray(t, dtype=np.float64)
    return np.sin(t) / (np.sin(t) + np.cos(t))


def trig_path(x0, eps, t):
    """x_t = cos t x0 + sin t eps."""
    return np.cos(t) * np.asarray(x0, np.float64) + np.sin(t) * np.asarray(eps, np.float64)


def trig_velocity(x0, eps, t):
    """dx_t/dt = -sin t x0 + cos t eps."""
    return -np.sin(t) * np.asarray(x0, np.float64) + np.cos(t) * np.asarray(eps, np.float64)


def f_pred(x_t, x0_pred, t):
    """TrigFlow-space prediction (cos t x_t - x0_pred) / sin t."""
    return (np.cos(t) * np.asarray(x_t, np.float64) - np.asarray(x0_pred, np.float64)) / np.sin(t)
