"""Pins of the sliding-window / sink oracle (CPU only): hand-derived examples, brute force,
torch's scaled_dot_product_attention with a band mask and an extra sink column, special cases."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import window as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RNG = np.random.default_rng(31)


def _golden():
    with open(os.path.join(ROOT, "tests", "golden", "window_sink_worked_examples.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
def test_worked_examples(case):
    g = _golden()
    sinks = None if case["sink"] is None else np.array([case["sink"]])
    o, lse = W.attention_window_sink(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), scale=1.0,
                                     causal=case["causal"], window_left=case["window_left"],
                                     window_right=case["window_right"], sinks=sinks)
    np.testing.assert_allclose(o[0, :, 0, 0], case["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], case["lse"], rtol=0, atol=1e-14)


def _brute(q, k, v, scale, causal, left, right, sinks):
    """Pure-Python loops over rows, keys and channels."""
    b, sq, hq, dq = q.shape
    _, sk, hk, dv = v.shape
    o = np.zeros((b, sq, hq, dv))
    lse = np.full((b, hq, sq), -math.inf)
    for bb in range(b):
        for h in range(hq):
            g = h // (hq // hk)
            for i in range(sq):
                logits = []
                for j in range(sk):
                    if causal and j > i:
                        continue
                    if left >= 0 and j < i - left:
                        continue
                    if right >= 0 and j > i + right:
                        continue
                    logits.append((j, scale * sum(float(q[bb, i, h, c]) * float(k[bb, j, g, c]) for c in range(dq))))
                sink = -math.inf if sinks is None else float(sinks[h])
                m = max([x for _, x in logits] + [sink])
                if m == -math.inf:
                    continue
                den = sum(math.exp(x - m) for _, x in logits) + math.exp(sink - m)
                for c in range(dv):
                    o[bb, i, h, c] = sum(math.exp(x - m) * float(v[bb, j, g, c]) for j, x in logits) / den
                lse[bb, h, i] = m + math.log(den)
    return o, lse


@pytest.mark.parametrize("causal,left,right,sink", [(True, 3, -1, False), (True, 0, -1, True), (False, 2, 1, True),
                                                    (False, -1, 0, False), (False, 4, -1, True), (True, 20, -1, True)])
def test_brute_force(causal, left, right, sink):
    q = RNG.standard_normal((2, 9, 4, 3))
    k = RNG.standard_normal((2, 11, 2, 3))
    v = RNG.standard_normal((2, 11, 2, 2))
    sinks = RNG.standard_normal(4) if sink else None
    o, lse = W.attention_window_sink(q, k, v, scale=0.7, causal=causal, window_left=left, window_right=right,
                                     sinks=sinks)
    o_b, lse_b = _brute(q, k, v, 0.7, causal, left, right, sinks)
    np.testing.assert_allclose(o, o_b, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,left,right", [(True, 5, -1), (False, 3, 2), (True, -1, -1), (False, 0, 6)])
def test_torch_sdpa_with_band_mask_and_sink_column(causal, left, right):
    # the sink is one more key with k = 0, v = 0 and an additive mask bias equal to the sink logit
    q = RNG.standard_normal((1, 13, 4, 8))
    k = RNG.standard_normal((1, 13, 2, 8))
    v = RNG.standard_normal((1, 13, 2, 5))
    sinks = RNG.standard_normal(4) * 2
    o, lse = W.attention_window_sink(q, k, v, scale=0.4, causal=causal, window_left=left, window_right=right,
                                     sinks=sinks)
    vis = W.visible_mask(range(13), 13, causal=causal, window_left=left, window_right=right)
    kk = np.repeat(k, 2, axis=2)
    vv = np.repeat(v, 2, axis=2)
    kk = np.concatenate([kk, np.zeros((1, 1, 4, 8))], axis=1)
    vv = np.concatenate([vv, np.zeros((1, 1, 4, 5))], axis=1)
    bias = np.where(vis, 0.0, -np.inf)[None, None].repeat(4, axis=1)                 # [1, 4, 13, 13]
    bias = np.concatenate([bias, np.broadcast_to(sinks[None, :, None, None], (1, 4, 13, 1))], axis=3)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(kk), t(vv), attn_mask=torch.from_numpy(bias),
                                                           scale=0.4).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    s = 0.4 * np.einsum("bihc,bjhc->bhij", q, kk[:, :13])
    logits = np.concatenate([np.where(vis, s, -np.inf), np.broadcast_to(sinks[None, :, None, None], (1, 4, 13, 1))],
                            axis=3)
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(logits), dim=3).numpy(), rtol=0, atol=1e-12)


def test_unbounded_window_without_sink_is_plain_attention():
    q, k, v = RNG.standard_normal((2, 7, 6, 4)), RNG.standard_normal((2, 9, 3, 4)), RNG.standard_normal((2, 9, 3, 3))
    for causal in (False, True):
        for left, right in ((-1, -1), (100, 100)):
            o, lse = W.attention_window_sink(q, k, v, scale=0.3, causal=causal, window_left=left, window_right=right)
            o_r, lse_r = oracle.attention_forward(q, k, v, scale=0.3, causal=causal)
            np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse, lse_r, rtol=0, atol=1e-14)


def test_sink_limits():
    q, k, v = RNG.standard_normal((1, 5, 2, 4)), RNG.standard_normal((1, 5, 2, 4)), RNG.standard_normal((1, 5, 2, 3))
    o0, l0 = W.attention_window_sink(q, k, v, scale=0.5, causal=True)
    o1, l1 = W.attention_window_sink(q, k, v, scale=0.5, causal=True, sinks=np.array([-np.inf, -np.inf]))
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)
    o2, l2 = W.attention_window_sink(q, k, v, scale=0.5, causal=True, sinks=np.array([60.0, 60.0]))
    assert np.abs(o2).max() < 1e-20 and np.allclose(l2, 60.0, rtol=0, atol=1e-20)
    # a sink scales every row's output by l / (l + e^sink) and adds to LSE accordingly
    sinks = np.array([0.3, -1.2])
    o3, l3 = W.attention_window_sink(q, k, v, scale=0.5, causal=True, sinks=sinks)
    frac = np.exp(l0 - np.logaddexp(l0, sinks[None, :, None]))                     # l / (l + e^sink)
    np.testing.assert_allclose(o3, o0 * frac.transpose(0, 2, 1)[..., None], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l3, np.logaddexp(l0, sinks[None, :, None]), rtol=0, atol=1e-14)


def test_rows_without_keys():
    # sk = 0: O = 0, LSE = sink (or -inf); a left window that excludes everything cannot happen
    # with the causal diagonal, but a right window on a short key range can
    q, v = RNG.standard_normal((1, 4, 1, 2)), RNG.standard_normal((1, 0, 1, 2))
    o, lse = W.attention_window_sink(q, np.zeros((1, 0, 1, 2)), v, scale=1.0, causal=False, sinks=np.array([0.5]))
    assert np.all(o == 0) and np.all(lse == 0.5)
    k = RNG.standard_normal((1, 2, 1, 2))
    o, lse = W.attention_window_sink(q, k, RNG.standard_normal((1, 2, 1, 2)), scale=1.0, causal=False,
                                     window_left=0, window_right=0)
    assert np.all(o[0, 2:] == 0) and np.all(np.isneginf(lse[0, 0, 2:]))


def test_visible_pairs():
    assert W.visible_pairs(10, 10, causal=True) == 55
    assert W.visible_pairs(10, 10, causal=True, window_left=2) == 1 + 2 + 3 * 8
    assert W.visible_pairs(6, 6, causal=False, window_left=1, window_right=1) == 2 + 3 * 4 + 2


def test_packed_sequences_without_window_are_plain_varlen():
    lens_q, lens_k = [5, 1, 9, 0], [7, 3, 9, 2]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lens_q)]), np.concatenate([[0], np.cumsum(lens_k)])
    q = RNG.standard_normal((sum(lens_q), 4, 6))
    k = RNG.standard_normal((sum(lens_k), 2, 6))
    v = RNG.standard_normal((sum(lens_k), 2, 3))
    for causal in (False, True):
        o, lse = W.attention_varlen_window_sink(q, k, v, cu_q, cu_k, scale=0.4, causal=causal)
        o_r, lse_r = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale=0.4, causal=causal)
        np.testing.assert_array_equal(o, o_r)
        np.testing.assert_array_equal(lse, lse_r)


def test_packed_sequences_match_each_sequence_alone():
    # positions restart in every sequence: sequence 1 alone, as a dense batch of one, gives the
    # same rows as its slice of the packed call
    lens = [6, 11, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = RNG.standard_normal((sum(lens), 2, 5))
    k = RNG.standard_normal((sum(lens), 1, 5))
    v = RNG.standard_normal((sum(lens), 1, 4))
    sinks = np.array([0.7, -0.2])
    o, lse = W.attention_varlen_window_sink(q, k, v, cu, cu, scale=0.5, causal=True, window_left=2, sinks=sinks)
    a, e = cu[1], cu[2]
    o1, l1 = W.attention_window_sink(q[None, a:e], k[None, a:e], v[None, a:e], scale=0.5, causal=True,
                                     window_left=2, sinks=sinks)
    np.testing.assert_array_equal(o[a:e], o1[0])
    np.testing.assert_array_equal(lse[:, a:e], l1[0])
    # a window of 2 in the packed axis would reach into sequence 0; per sequence it cannot
    assert not np.allclose(o[a], W.attention_window_sink(q[None], k[None], v[None], scale=0.5, causal=True,
                                                         window_left=2, sinks=sinks)[0][0, a])
