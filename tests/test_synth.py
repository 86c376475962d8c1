"""Checks of the seeded input generator (shapes, determinism, recipes)."""

import math

import numpy as np
import torch

from oracle import trigflow as tf
from synth import WORKLOADS, Workload, make_inputs, sample_rows, to_float64
from synth import workloads as wl


def test_named_workloads():
    assert [w.name for w in WORKLOADS.values()] == [
        "tiny_fp32", "image_dit_4096", "t2i_prefix_4352", "video_dit_32760",
        "long_video_65520"]
    w = WORKLOADS["long_video_65520"]
    m = w.mask
    assert m["frames"] * m["tokens_per_frame"] == w.N == 65520
    assert WORKLOADS["video_dit_32760"].N == 21 * 30 * 52
    assert WORKLOADS["image_dit_4096"].flops == 12 * 2 * 24 * 4096 ** 2 * 128


def test_deterministic_and_seed_dependent():
    w = Workload("t", 1, 3, 40, 16, "bf16", 5, tangent_scale=0.1)
    a, b = make_inputs(w), make_inputs(w)
    c = make_inputs(w, seed=6)
    for n in ("q", "k", "v", "dq", "dk", "dv"):
        assert a[n].dtype == torch.bfloat16 and a[n].shape == (1, 3, 40, 16)
        assert torch.equal(a[n], b[n])
        assert not torch.equal(a[n], c[n])
    assert float(to_float64(a["dq"]).std()) < 0.2


def test_rms_normalised_rows():
    w = Workload("t", 1, 2, 64, 32, "fp32", 3, rms_qk=True)
    x = make_inputs(w)
    for n in ("q", "k"):
        rms = np.sqrt(np.mean(to_float64(x[n]) ** 2, axis=-1))
        np.testing.assert_allclose(rms, 1.0, atol=1e-5)


def test_trigflow_tangent_recipe():
    w = Workload("t", 1, 2, 12, 8, "fp32", 9, tangents="trigflow")
    x = make_inputs(w)
    t = x["trigflow_t"]
    assert 0.0 <= t <= math.pi / 2
    for h in range(2):
        x0 = wl._rng(9, wl._ID["x0"], 0, h).standard_normal((12, 8))
        eps = wl._rng(9, wl._ID["eps"], 0, h).standard_normal((12, 8))
        # the tangent source is the TrigFlow path's time derivative
        dx = tf.trig_velocity(x0, eps, t)
        for n in ("q", "k", "v"):
            wm = wl._rng(9, wl._ID["w" + n]).standard_normal((8, 8)) / math.sqrt(8)
            np.testing.assert_allclose(to_float64(x["d" + n])[0, h], dx @ wm,
                                       rtol=1e-6, atol=1e-6)


def test_sample_rows():
    r = sample_rows(1000, every=100, block=128, tokens_per_frame=300)
    assert r[0] == 0 and r[-1] == 999
    assert np.all(np.diff(r) > 0)
    assert {127, 128, 255, 299, 300, 599, 600, 899, 900}.issubset(set(r.tolist()))
    assert set(range(896, 1000)).issubset(set(r.tolist()))
