"""Pins of the MXFP8 oracle (CPU only): hand-derived blocks, the E4M3 table by brute force,
torch's float8_e4m3fn cast, power-of-two invariance, and lossless inputs."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _golden():
    with open(os.path.join(ROOT, "tests", "golden", "mx_worked_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_worked_examples(case):
    x = np.zeros(32, dtype=np.float32)
    x[: len(case["x"])] = np.asarray(case["x"], dtype=np.float32)
    codes, exps, values = mx.mx_quantize(x)
    assert exps.shape == (1,) and int(exps[0]) == case["exp_byte"]
    n = len(case["codes"])
    assert [int(c) for c in codes[:n]] == [int(c, 16) for c in case["codes"]]
    assert list(values[:n]) == case["values"]
    assert np.array_equal(mx.mx_dequantize(codes, exps), values)


def _e4m3_table():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    keep = ~np.isnan(vals)
    return codes[keep], vals[keep]


def test_codes_are_the_nearest_e4m3_values_by_brute_force():
    # every element's code is the table entry nearest to x / 2^E (ties to the even mantissa),
    # the largest finite one past 448
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((6, 64)) * np.exp(rng.uniform(-6, 6, (6, 1)))).astype(np.float32)
    codes, exps, _ = mx.mx_quantize(x)
    tcodes, tvals = _e4m3_table()
    for r in range(x.shape[0]):
        for blk in range(2):
            e = int(exps[r, blk]) - 127
            for i in range(32):
                y = float(x[r, blk * 32 + i]) / 2.0 ** e
                y = max(min(y, 448.0), -448.0)
                dist = np.abs(tvals - y)
                best = np.flatnonzero(dist == dist.min())
                if len(best) > 1:   # a tie: the even mantissa (code bit 0 clear) wins
                    best = [b for b in best if tcodes[b] & 1 == 0 and np.signbit(tvals[b]) == (y < 0)]
                got = codes[r, blk * 32 + i]
                assert oracle.e4m3_decode(got) == tvals[best[0]], (r, blk, i, y)


def test_codes_match_torch_float8_cast():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((40, 128)) * 5).astype(np.float32)
    codes, exps, _ = mx.mx_quantize(x)
    e = np.repeat(exps.astype(np.int64) - 127, 32, axis=1)
    y = (x.astype(np.float64) / np.ldexp(1.0, e)).astype(np.float32)
    inside = np.abs(y) <= 448
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[inside], ref[inside])
    assert inside.mean() > 0.9
    # outside 448 the codes saturate
    assert np.all(np.abs(oracle.e4m3_decode(codes[~inside])) == 448)


def test_shared_exponent_puts_the_block_max_in_the_top_binade():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((50, 32)) * np.exp(rng.uniform(-20, 20, (50, 1)))).astype(np.float32)
    _, exps, _ = mx.mx_quantize(x)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    y = amax / np.ldexp(1.0, exps[:, 0].astype(np.int64) - 127)
    assert np.all((y >= 256) & (y < 512))


@pytest.mark.parametrize("k", [-30, -1, 1, 17])
def test_power_of_two_scaling_moves_only_the_exponent(k):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((8, 96)) * 3).astype(np.float32)
    c0, e0, v0 = mx.mx_quantize(x)
    c1, e1, v1 = mx.mx_quantize((x * np.float32(2.0 ** k)).astype(np.float32))
    assert np.array_equal(c0, c1)
    assert np.array_equal(e1.astype(np.int64), e0.astype(np.int64) + k)
    assert np.array_equal(v1, v0 * 2.0 ** k)


def test_blocks_run_along_the_last_axis():
    x = np.ones((2, 64), dtype=np.float32)
    x[0, 40] = 100.0                     # second block of row 0 only
    _, exps, values = mx.mx_quantize(x)
    assert exps[0, 0] == 119 and exps[1, 0] == 119 and exps[1, 1] == 119
    assert exps[0, 1] == 127 + 6 - 8     # floor(log2 100) = 6
    assert values[0, 0] == 1.0 and values[0, 33] == 1.0


def test_relative_error_bound_of_unsaturated_normals():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((64, 128)) * 2).astype(np.float32)
    codes, exps, values = mx.mx_quantize(x)
    e = np.repeat(exps.astype(np.int64) - 127, 32, axis=1)
    y = np.abs(x.astype(np.float64)) / np.ldexp(1.0, e)
    sel = (y >= 2.0 ** -6) & (y <= 448)
    rel = np.abs(values[sel] - x[sel]) / np.abs(x[sel])
    assert rel.max() <= 2.0 ** -4      # half an ulp of a 3-bit mantissa


def test_attention_on_lossless_inputs_equals_plain_attention():
    # elements that are E4M3 values times 2^k, with a block max in [256, 448] * 2^k, quantise
    # without loss: the MXFP8 attention then equals the plain one
    rng = np.random.default_rng(10)
    tcodes, tvals = _e4m3_table()
    finite = tvals[np.abs(tvals) <= 448]

    def lossless(shape):
        v = rng.choice(finite, size=shape)
        blocks = v.reshape(shape[:-1] + (shape[-1] // 32, 32))
        blocks[..., 0] = rng.choice([256.0, 320.0, 448.0, -384.0], size=blocks.shape[:-1])
        k = rng.integers(-14, -6, size=blocks.shape[:-1] + (1,))
        return (blocks * np.ldexp(1.0, k)).reshape(shape).astype(np.float32)

    q, k, v = lossless((1, 20, 2, 64)), lossless((1, 24, 1, 64)), lossless((1, 24, 1, 64))
    assert np.array_equal(mx.mx_quantize(q)[2], q.astype(np.float64))
    for causal in (False, True):
        o, lse, _ = mx.mxfp8_attention_forward(q, k, v, scale=0.125, causal=causal)
        o_ref, lse_ref = oracle.attention_forward(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                                  scale=0.125, causal=causal)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)


def test_k_mean_is_subtracted_before_quantising():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 8, 2, 32)).astype(np.float32)
    k = (rng.standard_normal((1, 8, 1, 32)) + 5).astype(np.float32)
    v = rng.standard_normal((1, 8, 1, 32)).astype(np.float32)
    mu = np.full((1, 1, 32), 5.0, dtype=np.float32)
    _, _, quant = mx.mxfp8_attention_forward(q, k, v, mu=mu, scale=0.2, causal=False)
    codes, exps = quant["k"]
    ref_codes, ref_exps, _ = mx.mx_quantize((k - np.float32(5.0)).astype(np.float32))
    assert np.array_equal(codes, ref_codes) and np.array_equal(exps, ref_exps)
