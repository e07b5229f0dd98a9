"""Pins for the E4M3 quantiser and the FP8 attention oracle (CPU only)."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import (E4M3_MAX, attention_forward, e4m3_decode, e4m3_encode, e4m3_round,
                    fp8_attention_forward, quantize_blocks)

RNG = np.random.default_rng(5335)


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_ocp_code_table(golden_dir):
    with open(os.path.join(golden_dir, "e4m3_ocp_codes.json")) as f:
        g = json.load(f)
    for c in g["codes"]:
        code = int(c["code"], 16)
        assert e4m3_decode(np.uint8(code)) == c["value"], c
        assert int(e4m3_encode(np.float64(c["value"]))) == code, c
    for c in g["nan_codes"]:
        assert np.isnan(e4m3_decode(np.uint8(int(c, 16))))
    for c in g["rounding"]["cases"]:
        assert e4m3_round(np.float64(c["x"])) == c["rounded"], c


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    np.testing.assert_array_equal(ours[ok], theirs[ok])
    np.testing.assert_array_equal(np.signbit(ours[ok]), np.signbit(theirs[ok]))


def test_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_round_matches_torch_cast_in_range():
    # torch's float -> float8_e4m3fn cast rounds to nearest even but does not saturate
    # (|x| >= 464 becomes NaN), so compare only inside the finite range.
    grid = np.unique(np.abs(e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = (grid[:-1] + grid[1:]) / 2.0                     # exact ties
    xs = [grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
          np.abs(RNG.standard_normal(200000)) * 60.0,
          np.exp(RNG.uniform(np.log(1e-5), np.log(463.0), 200000)),
          RNG.uniform(0, 2.0 ** -6, 50000)]
    x = np.concatenate(xs).astype(np.float32)
    x = x[np.abs(x) < 464.0]
    x = np.concatenate([x, -x])
    np.testing.assert_array_equal(e4m3_round(x), _torch_e4m3(x))


def test_saturation():
    x = np.array([464.0, 480.0, 1e4, 3.4e38, -470.0, -1e30])
    np.testing.assert_array_equal(e4m3_round(x), np.copysign(E4M3_MAX, x))


def test_block_scale_and_amax_code():
    x = (RNG.standard_normal((2, 300, 3, 16)) * 4.0).astype(np.float32)
    codes, scales, values = quantize_blocks(x)
    assert scales.shape == (2, 3, 3)
    for b in range(2):
        for h in range(3):
            for blk in range(3):
                xb = x[b, blk * 128:(blk + 1) * 128, h, :]
                amax = np.float32(np.abs(xb).max())
                assert scales[b, h, blk] == np.float32(amax / np.float32(448.0))
                i = np.unravel_index(np.argmax(np.abs(xb)), xb.shape)
                cb = codes[b, blk * 128:(blk + 1) * 128, h, :]
                assert e4m3_decode(cb[i]) == np.copysign(448.0, xb[i])
    # dequantised values are within half an E4M3 step (relative 2^-4) of the input
    rel = np.abs(values - x) / np.maximum(np.abs(x), 1e-30)
    big = np.abs(x) >= np.repeat(scales.transpose(0, 2, 1), 128, axis=1)[:, :300, :, None] * 2.0 ** -6
    assert rel[big].max() <= 2.0 ** -4 + 1e-12


def test_zero_block_has_unit_scale():
    x = np.zeros((1, 130, 1, 8), dtype=np.float32)
    x[0, 128:, 0, :] = 3.0
    codes, scales, values = quantize_blocks(x)
    assert scales[0, 0, 0] == 1.0 and (codes[0, :128] == 0).all()
    assert scales[0, 0, 1] == np.float32(3.0 / 448.0)


def test_blocks_are_independent():
    x = (RNG.standard_normal((1, 384, 2, 8))).astype(np.float32)
    c0, s0, _ = quantize_blocks(x)
    y = x.copy()
    y[0, 130, 1, 3] = 1000.0          # only block 1 of head 1 changes
    c1, s1, _ = quantize_blocks(y)
    mask = np.ones_like(c0, dtype=bool)
    mask[0, 128:256, 1, :] = False
    np.testing.assert_array_equal(c0[mask], c1[mask])
    assert s1[0, 1, 1] != s0[0, 1, 1]
    np.testing.assert_array_equal(np.delete(s0.ravel(), 4), np.delete(s1.ravel(), 4))   # [0, 1, 1] of [1, 2, 3]


def _on_grid_tensor(shape, exp_shift):
    """Values on the E4M3 grid times 2^exp_shift, with each 128-token block's amax = 448 * 2^exp_shift."""
    codes = RNG.integers(0, 0x7F, size=shape).astype(np.uint8)
    codes |= (RNG.integers(0, 2, size=shape).astype(np.uint8) << 7)
    vals = e4m3_decode(codes)
    b, s, h, d = shape
    for blk in range(0, s, 128):
        vals[:, blk, :, 0] = 448.0                    # pin every block's amax
    return (vals * 2.0 ** exp_shift).astype(np.float32)


def test_quantising_scaled_grid_values_is_identity():
    x = _on_grid_tensor((1, 256, 2, 8), -5)
    codes, scales, values = quantize_blocks(x)
    np.testing.assert_array_equal(scales, np.float32(2.0 ** -5))
    np.testing.assert_array_equal(values, x.astype(np.float64))


def test_fp8_attention_equals_plain_attention_on_grid_inputs():
    # Inputs already on power-of-two-scaled E4M3 grids quantise without error, so the FP8
    # oracle must reproduce the plain attention exactly.  K carries a per-channel offset mu
    # that is subtracted exactly (small dyadic numbers), exercising the smoothing step.
    q = _on_grid_tensor((1, 256, 2, 16), -6)
    kc = _on_grid_tensor((1, 256, 2, 16), -6)
    v = _on_grid_tensor((1, 256, 2, 16), -4)
    mu = (RNG.integers(-8, 9, size=(1, 2, 16)) * 0.25).astype(np.float32)
    k = (kc + mu[:, None, :, :]).astype(np.float32)
    assert np.array_equal((k - mu[:, None]).astype(np.float32), kc)   # the shift is exact
    for causal in (False, True):
        o8, l8, quant = fp8_attention_forward(q, k, v, mu=mu, scale=0.25, causal=causal)
        o, lse = attention_forward(q, kc, v, scale=0.25, causal=causal)
        np.testing.assert_array_equal(o8, o)
        np.testing.assert_array_equal(l8, lse)
        # and the smoothing only shifts LSE relative to attention on the unsmoothed K
        o_raw, l_raw = attention_forward(q, k, v, scale=0.25, causal=causal)
        np.testing.assert_allclose(o8, o_raw, atol=1e-12)
        shift = 0.25 * np.einsum("bih,bh->bi", q[:, :, 0, :].astype(np.float64), mu[:, 0, :].astype(np.float64))
        np.testing.assert_allclose(l_raw[:, 0, :] - l8[:, 0, :], shift, atol=1e-12)


def test_smoothing_reduces_quantisation_error():
    # A K with a large per-channel bias (the workload the gate targets) loses more accuracy
    # to block quantisation without smoothing than with it.
    b, s, h, d = 1, 256, 2, 32
    q = RNG.standard_normal((b, s, h, d)).astype(np.float32)
    v = RNG.standard_normal((b, s, h, d)).astype(np.float32)
    bias = (RNG.standard_normal((1, 1, h, d)) * 3.0).astype(np.float32)
    k = (RNG.standard_normal((b, s, h, d)) + bias).astype(np.float32)
    mu = k.astype(np.float64).mean(axis=1).astype(np.float32)
    exact, _ = attention_forward(q, k, v, scale=d ** -0.5, causal=False)
    o_s, _, _ = fp8_attention_forward(q, k, v, mu=mu, scale=d ** -0.5, causal=False)
    o_n, _, _ = fp8_attention_forward(q, k, v, mu=None, scale=d ** -0.5, causal=False)
    err = lambda o: np.linalg.norm(o - exact) / np.linalg.norm(exact)
    assert err(o_s) < err(o_n)
    assert err(o_s) < 0.1
