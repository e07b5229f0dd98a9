"""Pins for the K-smoothing gate oracle (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

from oracle import k_smooth_mean, key_sample

RNG = np.random.default_rng(7754)


def _arr(x):
    return np.array([[float(v) if v != "inf" else math.inf for v in row] for row in x])


def test_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "gate_worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 5
    for c in cases:
        r = k_smooth_mean(np.array(c["k"]), key_stride=c["key_stride"], max_keys=c["max_keys"], tau=c["tau"])
        np.testing.assert_allclose(r["mu"], np.array(c["mu"]), rtol=0, atol=1e-15, err_msg=c["name"])
        np.testing.assert_allclose(r["var"], np.array(c["var"]), rtol=0, atol=1e-15, err_msg=c["name"])
        np.testing.assert_array_equal(r["ratio"], _arr(c["ratio"]), err_msg=c["name"])
        np.testing.assert_array_equal(r["open"], np.array(c["open"]), err_msg=c["name"])
        np.testing.assert_array_equal(r["mean"], np.array(c["mean"]), err_msg=c["name"])


def test_key_sample_rule():
    assert list(key_sample(10, 1)) == list(range(10))
    assert list(key_sample(10, 3)) == [0, 3, 6, 9]
    assert list(key_sample(9, 3)) == [0, 3, 6]
    assert list(key_sample(10, 3, max_keys=2)) == [0, 3]
    assert list(key_sample(10, 20)) == [0]
    assert list(key_sample(0, 4)) == []
    with pytest.raises(ValueError):
        key_sample(5, 0)


def test_constant_channels():
    const = np.array([0.5, -2.0, 0.0, 7.25])
    k = np.broadcast_to(const, (2, 13, 3, 4)).copy()
    r = k_smooth_mean(k, tau=0.25)
    np.testing.assert_array_equal(r["mu"], np.broadcast_to(const, (2, 3, 4)))
    np.testing.assert_array_equal(r["var"], 0.0)
    assert r["open"].all() and np.isinf(r["ratio"]).all()
    r0 = k_smooth_mean(np.zeros((1, 5, 2, 4)), tau=0.25)
    assert not r0["open"].any() and (r0["ratio"] == 0).all()


def test_paired_keys_have_zero_mean_and_closed_gate():
    half = RNG.standard_normal((2, 8, 3, 16)) * 5.0 + 3.0
    k = np.empty((2, 16, 3, 16))
    k[:, 0::2] = half
    k[:, 1::2] = -half
    r = k_smooth_mean(k, tau=0.25)
    np.testing.assert_allclose(r["mu"], 0.0, atol=1e-15)
    assert not r["open"].any()
    assert (r["mean"] == 0.0).all()


@pytest.mark.parametrize("stride,max_keys", [(1, 0), (3, 0), (4, 5), (7, 1), (50, 0)])
def test_brute_force_python(stride, max_keys):
    b, sk, hk, d = 2, 29, 2, 3
    k = RNG.standard_normal((b, sk, hk, d)) + RNG.standard_normal((1, 1, hk, d)) * 2.0
    tau = 0.25
    r = k_smooth_mean(k, key_stride=stride, max_keys=max_keys, tau=tau)
    keys = list(range(0, sk, stride))
    if max_keys:
        keys = keys[:max_keys]
    for bb in range(b):
        for g in range(hk):
            mus, vars_ = [], []
            for c in range(d):
                xs = [float(k[bb, j, g, c]) for j in keys]
                mu = math.fsum(xs) / len(xs)
                var = math.fsum((x - mu) ** 2 for x in xs) / len(xs)
                mus.append(mu)
                vars_.append(var)
                assert abs(r["mu"][bb, g, c] - mu) < 1e-13
                assert abs(r["var"][bb, g, c] - var) < 1e-12
            num, den = math.fsum(m * m for m in mus), math.fsum(vars_)
            ratio = math.sqrt(num / den) if den > 0 else (math.inf if num > 0 else 0.0)
            assert r["ratio"][bb, g] == ratio or abs(r["ratio"][bb, g] - ratio) < 1e-12
            assert bool(r["open"][bb, g]) == (ratio > tau)
            want = mus if ratio > tau else [0.0] * d
            np.testing.assert_array_equal(r["mean"][bb, g], np.where(r["open"][bb, g], r["mu"][bb, g], 0.0))
            np.testing.assert_allclose(r["mean"][bb, g], want, atol=1e-13)


def test_shift_and_scale_behaviour():
    # The statistic is invariant to scaling K by a constant, and shifting every channel by
    # a large constant opens the gate.
    k = RNG.standard_normal((1, 64, 2, 8))
    r1 = k_smooth_mean(k)
    r2 = k_smooth_mean(k * 8.0)
    np.testing.assert_allclose(r2["ratio"], r1["ratio"], rtol=1e-12)
    r3 = k_smooth_mean(k + 10.0)
    assert r3["open"].all()


def test_empty_sample():
    r = k_smooth_mean(np.zeros((1, 0, 2, 4)))
    assert r["T"] == 0 and not r["open"].any()
    assert (r["mean"] == 0).all()
