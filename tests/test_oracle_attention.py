"""Pins for the float64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: hand-derived
worked examples, closed forms, invariances of the definition, a pure-Python
three-pass softmax, and torch's CPU scaled_dot_product_attention in float64.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention_forward

RNG = np.random.default_rng(20261202)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# ---------------------------------------------------------------- worked examples

def test_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "attention_worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 5
    for c in cases:
        o, lse = attention_forward(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                   scale=c["scale"], causal=c["causal"])
        np.testing.assert_allclose(o, np.array(c["o"]), rtol=0, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-12, err_msg=c["name"])


# ---------------------------------------------------------------- brute force

def _python_attention(q, k, v, scale, causal):
    """Textbook three-pass softmax attention in pure Python (no numpy arithmetic)."""
    b, sq, hq, dqk = q.shape
    _, sk, hk, dv = v.shape
    grp = hq // hk
    o = [[[[0.0] * dv for _ in range(hq)] for _ in range(sq)] for _ in range(b)]
    lse = [[[0.0] * sq for _ in range(hq)] for _ in range(b)]
    for bb in range(b):
        for h in range(hq):
            g = h // grp
            for i in range(sq):
                keys = [j for j in range(sk) if (not causal or j <= i)]
                s = [scale * math.fsum(float(q[bb, i, h, c]) * float(k[bb, j, g, c]) for c in range(dqk))
                     for j in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for c in range(dv):
                    o[bb][i][h][c] = math.fsum(e[t] * float(v[bb, keys[t], g, c]) for t in range(len(keys))) / tot
                lse[bb][h][i] = m + math.log(tot)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", [(3, 3), (4, 2)])
def test_brute_force_python(causal, dims):
    dqk, dv = dims
    q, k, v = _rand(2, 5, 4, dqk), _rand(2, 5, 2, dqk), _rand(2, 5, 2, dv)
    scale = 0.7
    o, lse = attention_forward(q, k, v, scale=scale, causal=causal)
    o_ref, lse_ref = _python_attention(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- library routine

def _torch_sdpa(q, k, v, scale, causal):
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)   # [b, h, s, d]
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    gqa = qt.shape[1] != kt.shape[1]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=causal, scale=scale, enable_gqa=gqa)
    return out.permute(0, 2, 1, 3).numpy()


def test_torch_sdpa_conventions_match_the_readings():
    # torch's CPU math path: causal mask is top-left (tril of ones(sq, sk)) and GQA repeats
    # each kv head over consecutive query heads.  Check both on a one-hot probe before using
    # it as a pin for the oracle.
    sq, sk = 3, 5
    q = np.zeros((1, sq, 1, 1))
    k = np.zeros((1, sk, 1, 1))
    v = np.eye(sk).reshape(1, sk, 1, sk)
    p = _torch_sdpa(q, k, v, 1.0, True)[0, :, 0, :]      # rows are the softmax weights
    for i in range(sq):
        np.testing.assert_allclose(p[i, : i + 1], 1.0 / (i + 1), atol=1e-15)
        np.testing.assert_allclose(p[i, i + 1:], 0.0, atol=0)
    v2 = np.zeros((1, 2, 2, 1))
    v2[:, :, 1, :] = 1.0                                   # kv head g holds the value g
    out = _torch_sdpa(np.zeros((1, 2, 4, 1)), np.zeros((1, 2, 2, 1)), v2, 1.0, False)
    np.testing.assert_allclose(out[0, 0, :, 0], [0.0, 0.0, 1.0, 1.0])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    dict(b=2, sq=17, sk=17, hq=6, hk=2, dqk=8, dv=8),
    dict(b=1, sq=9, sk=23, hq=4, hk=4, dqk=12, dv=4),
    dict(b=1, sq=31, sk=7, hq=3, hk=1, dqk=5, dv=6),
])
def test_matches_torch_sdpa_float64(causal, shape):
    s = shape
    q = _rand(s["b"], s["sq"], s["hq"], s["dqk"])
    k = _rand(s["b"], s["sk"], s["hk"], s["dqk"])
    v = _rand(s["b"], s["sk"], s["hk"], s["dv"])
    scale = 1.0 / math.sqrt(s["dqk"])
    o, _ = attention_forward(q, k, v, scale=scale, causal=causal)
    np.testing.assert_allclose(o, _torch_sdpa(q, k, v, scale, causal), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def test_causal_row_zero_is_v0():
    q, k, v = _rand(2, 9, 4, 8), _rand(2, 9, 2, 8), _rand(2, 9, 2, 5)
    scale = 0.3
    o, lse = attention_forward(q, k, v, scale=scale, causal=True)
    for h in range(4):
        g = h // 2
        np.testing.assert_array_equal(o[:, 0, h, :], v[:, 0, g, :])
        s00 = scale * np.array([math.fsum(q[b, 0, h, c] * k[b, 0, g, c] for c in range(8)) for b in range(2)])
        np.testing.assert_allclose(lse[:, h, 0], s00, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_averages_v(causal):
    sq = sk = 11
    q = np.zeros((1, sq, 2, 4))
    k, v = _rand(1, sk, 1, 4), _rand(1, sk, 1, 3)
    o, lse = attention_forward(q, k, v, scale=1.0, causal=causal)
    for i in range(sq):
        n = i + 1 if causal else sk
        want = np.array([math.fsum(v[0, j, 0, c] for j in range(n)) / n for c in range(3)])
        for h in range(2):
            np.testing.assert_allclose(o[0, i, h], want, rtol=0, atol=1e-14)
            assert abs(lse[0, h, i] - math.log(n)) < 1e-14


def test_dominant_score_selects_one_value_row():
    # One key's score exceeds all others by > 1000: its weight is 1 to double precision.
    sk = 6
    q = np.zeros((1, 1, 1, sk))
    q[0, 0, 0, 4] = 2000.0
    k = np.eye(sk).reshape(1, sk, 1, sk)
    v = _rand(1, sk, 1, 3)
    o, lse = attention_forward(q, k, v, scale=1.0, causal=False)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 4, 0])
    assert lse[0, 0, 0] == 2000.0


def test_softmax_rows_sum_to_one_and_match_lse():
    # With V = identity over keys, O's rows are the softmax weights themselves.
    sq = sk = 8
    q, k = _rand(1, sq, 1, 4), _rand(1, sk, 1, 4)
    v = np.eye(sk).reshape(1, sk, 1, sk)
    scale = 0.9
    for causal in (False, True):
        p, lse = attention_forward(q, k, v, scale=scale, causal=causal)
        p = p[0, :, 0, :]
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert (p >= 0).all()
        for i in range(sq):
            for j in range(sk):
                if causal and j > i:
                    assert p[i, j] == 0.0
                else:
                    s_ij = scale * math.fsum(q[0, i, 0, c] * k[0, j, 0, c] for c in range(4))
                    assert abs((s_ij - math.log(p[i, j])) - lse[0, 0, i]) < 1e-12


# ---------------------------------------------------------------- invariances

@pytest.mark.parametrize("causal", [False, True])
def test_k_mean_shift_leaves_output_unchanged(causal):
    q, k, v = _rand(2, 10, 4, 6), _rand(2, 10, 2, 6), _rand(2, 10, 2, 5)
    mu = _rand(2, 2, 6, scale=3.0)
    scale = 0.4
    o0, lse0 = attention_forward(q, k, v, scale=scale, causal=causal)
    o1, lse1 = attention_forward(q, k + mu[:, None, :, :], v, scale=scale, causal=causal)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    for h in range(4):
        shift = scale * np.einsum("bic,bc->bi", q[:, :, h, :], mu[:, h // 2, :])
        np.testing.assert_allclose(lse1[:, h, :] - lse0[:, h, :], shift, rtol=0, atol=1e-12)


def test_gqa_equals_repeated_mha():
    q, k, v = _rand(1, 7, 6, 4), _rand(1, 7, 2, 4), _rand(1, 7, 2, 3)
    for causal in (False, True):
        o_g, l_g = attention_forward(q, k, v, scale=0.5, causal=causal)
        o_m, l_m = attention_forward(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2),
                                     scale=0.5, causal=causal)
        np.testing.assert_array_equal(o_g, o_m)
        np.testing.assert_array_equal(l_g, l_m)


def test_non_causal_key_permutation_invariance():
    q, k, v = _rand(1, 5, 2, 4), _rand(1, 9, 2, 4), _rand(1, 9, 2, 3)
    perm = RNG.permutation(9)
    o0, l0 = attention_forward(q, k, v, scale=0.8, causal=False)
    o1, l1 = attention_forward(q, k[:, perm], v[:, perm], scale=0.8, causal=False)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-13)


def test_linear_in_v():
    q, k = _rand(1, 6, 2, 4), _rand(1, 6, 2, 4)
    v1, v2 = _rand(1, 6, 2, 3), _rand(1, 6, 2, 3)
    for causal in (False, True):
        o1, _ = attention_forward(q, k, v1, scale=1.0, causal=causal)
        o2, _ = attention_forward(q, k, v2, scale=1.0, causal=causal)
        o12, _ = attention_forward(q, k, 2.0 * v1 + v2, scale=1.0, causal=causal)
        np.testing.assert_allclose(o12, 2.0 * o1 + o2, rtol=0, atol=1e-13)


def test_selected_rows_heads_batches_match_full():
    q, k, v = _rand(3, 12, 4, 5), _rand(3, 12, 2, 5), _rand(3, 12, 2, 4)
    o, lse = attention_forward(q, k, v, scale=0.6, causal=True)
    rows, heads, batches = [0, 5, 11], [3, 1], [2, 0]
    os_, ls_ = attention_forward(q, k, v, scale=0.6, causal=True, rows=rows, heads=heads, batches=batches)
    np.testing.assert_array_equal(os_, o[np.ix_(batches, rows, heads)])
    np.testing.assert_array_equal(ls_, lse[np.ix_(batches, heads, rows)])


# ---------------------------------------------------------------- degenerate sizes

def test_no_keys_gives_zero_output_and_minus_inf_lse():
    q = _rand(1, 3, 2, 4)
    o, lse = attention_forward(q, np.zeros((1, 0, 2, 4)), np.zeros((1, 0, 2, 3)), scale=1.0, causal=False)
    assert o.shape == (1, 3, 2, 3) and (o == 0).all()
    assert np.isneginf(lse).all()


def test_no_queries():
    o, lse = attention_forward(np.zeros((1, 0, 2, 4)), _rand(1, 5, 2, 4), _rand(1, 5, 2, 3),
                               scale=1.0, causal=True)
    assert o.shape == (1, 0, 2, 3) and lse.shape == (1, 2, 0)


def test_single_key():
    q, k, v = _rand(1, 4, 1, 3), _rand(1, 1, 1, 3), _rand(1, 1, 1, 2)
    o, _ = attention_forward(q, k, v, scale=1.0, causal=False)
    np.testing.assert_array_equal(o[0, :, 0, :], np.repeat(v[0, :, 0, :], 4, axis=0))
