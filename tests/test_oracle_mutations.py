"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies an oracle source file, plants one plausible mistake (a dropped
term, a wrong index or sign, a transposed operand, an off-by-one), loads the
copy as a throwaway module and runs a compact version of the pins against it.
At least one pin must reject every mutant; the unmutated source must pass all
of them.  Nothing here touches the real oracle modules.
"""

import json
import math
import os
import types

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RNG = np.random.default_rng(99)


def _load(fname, old=None, new=None, extra=None):
    path = os.path.join(ROOT, "oracle", fname)
    src = open(path).read()
    if old is not None:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new, 1)
    src = src.replace("from .attention import attention_forward", "")
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__.update(extra or {})
    exec(compile(src, path, "exec"), mod.__dict__)
    return mod


def _golden(name):
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- attention pins

def _attention_pins_pass(mod):
    f = mod.attention_forward
    try:
        for c in _golden("attention_worked_examples.json")["cases"]:
            o, lse = f(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]), scale=c["scale"], causal=c["causal"])
            if not (np.allclose(o, c["o"], atol=1e-12, rtol=0) and np.allclose(lse, c["lse"], atol=1e-12, rtol=0)):
                return False
        for causal in (False, True):
            q, k, v = RNG.standard_normal((1, 9, 4, 5)), RNG.standard_normal((1, 9, 2, 5)), RNG.standard_normal((1, 9, 2, 3))
            o, _ = f(q, k, v, scale=0.5, causal=causal)
            t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
            ref = torch.nn.functional.scaled_dot_product_attention(
                t(q), t(k), t(v), is_causal=causal, scale=0.5, enable_gqa=True).permute(0, 2, 1, 3).numpy()
            if not np.allclose(o, ref, atol=1e-12, rtol=0):
                return False
            o0, lse0 = f(np.zeros((1, 7, 1, 5)), k[:, :7, :1], v[:, :7, :1], scale=1.0, causal=causal)
            n = np.arange(1, 8) if causal else np.full(7, 7)
            if not np.allclose(lse0[0, 0], np.log(n), atol=1e-14, rtol=0):
                return False
    except Exception:
        return False
    return True


ATTENTION_MUTANTS = [
    ("gqa_modulo", "g = h // group", "g = h % hk"),
    ("dropped_scale", "s = scale * (qh @ kg.T)", "s = (qh @ kg.T)"),
    ("causal_off_by_one", "key_idx[None, :] <= rows_arr[:, None]", "key_idx[None, :] < rows_arr[:, None] + 0 * 1"),
    ("causal_transposed", "key_idx[None, :] <= rows_arr[:, None]", "key_idx[None, :] >= rows_arr[:, None]"),
    ("lse_drops_max", "m_safe + np.log(", "0.0 + np.log("),
    ("sum_wrong_axis", "l = p.sum(axis=1)", "l = p.sum(axis=0)"),
    ("transposed_pv", "out = (p @ vg)", "out = (p.T @ vg)"),
    ("sign_of_max", "p = np.exp(s - m_safe[:, None])", "p = np.exp(s + m_safe[:, None])"),
]


def test_attention_source_passes_pins():
    assert _attention_pins_pass(_load("attention.py"))


@pytest.mark.parametrize("name,old,new", ATTENTION_MUTANTS, ids=[m[0] for m in ATTENTION_MUTANTS])
def test_attention_mutant_is_caught(name, old, new):
    assert not _attention_pins_pass(_load("attention.py", old, new))


# ---------------------------------------------------------------- gate pins

def _gate_pins_pass(mod):
    try:
        for c in _golden("gate_worked_examples.json")["cases"]:
            r = mod.k_smooth_mean(np.array(c["k"]), key_stride=c["key_stride"], max_keys=c["max_keys"], tau=c["tau"])
            ratio = np.array([[math.inf if x == "inf" else float(x) for x in row] for row in c["ratio"]])
            if not (np.allclose(r["mu"], c["mu"], atol=1e-15) and np.allclose(r["var"], c["var"], atol=1e-15)
                    and np.array_equal(r["ratio"], ratio) and np.array_equal(r["open"], c["open"])
                    and np.array_equal(r["mean"], c["mean"])):
                return False
        if list(mod.key_sample(10, 3)) != [0, 3, 6, 9]:
            return False
    except Exception:
        return False
    return True


GATE_MUTANTS = [
    ("uncentred_variance", "((x - mu[:, None, :, :]) ** 2)", "(x ** 2)"),
    ("threshold_inclusive", "gate_open = ratio > tau", "gate_open = ratio >= tau"),
    ("sample_count_floor", "count = (sk + key_stride - 1) // key_stride", "count = sk // key_stride"),
    ("closed_keeps_mean", "mean = np.where(gate_open[:, :, None], mu, 0.0)", "mean = mu"),
    ("ratio_not_rooted", "ratio[bi, g] = math.sqrt(num[bi, g] / den[bi, g])", "ratio[bi, g] = num[bi, g] / den[bi, g]"),
]


def test_gate_source_passes_pins():
    assert _gate_pins_pass(_load("gate.py"))


@pytest.mark.parametrize("name,old,new", GATE_MUTANTS, ids=[m[0] for m in GATE_MUTANTS])
def test_gate_mutant_is_caught(name, old, new):
    assert not _gate_pins_pass(_load("gate.py", old, new))


# ---------------------------------------------------------------- fp8 pins

def _fp8_pins_pass(mod):
    try:
        g = _golden("e4m3_ocp_codes.json")
        for c in g["codes"]:
            if mod.e4m3_decode(np.uint8(int(c["code"], 16))) != c["value"]:
                return False
            if int(mod.e4m3_encode(np.float64(c["value"]))) != int(c["code"], 16):
                return False
        for c in g["rounding"]["cases"]:
            if mod.e4m3_round(np.float64(c["x"])) != c["rounded"]:
                return False
        x = (RNG.standard_normal(20000) * 30).astype(np.float32)
        x = x[np.abs(x) < 464]
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        if not np.array_equal(mod.e4m3_round(x), ref):
            return False
        xb = (RNG.standard_normal((1, 200, 1, 8)) * 3).astype(np.float32)
        codes, scales, _ = mod.quantize_blocks(xb)
        if scales.shape != (1, 1, 2) or scales[0, 0, 0] != np.float32(np.abs(xb[0, :128]).max() / np.float32(448)):
            return False
        k = np.ones((1, 4, 1, 2), dtype=np.float32) * 3.0
        mu = np.full((1, 1, 2), 1.0, dtype=np.float32)
        if not np.array_equal(mod.smooth_k(k, mu), np.full((1, 4, 1, 2), 2.0, dtype=np.float32)):
            return False
    except Exception:
        return False
    return True


def _fp8_extra():
    from oracle.attention import attention_forward
    return {"attention_forward": attention_forward}


FP8_MUTANTS = [
    ("truncate_not_round", "r = np.rint(mag / quantum) * quantum", "r = np.floor(mag / quantum) * quantum"),
    ("no_subnormals", "e = np.maximum(e, E4M3_MIN_NORMAL_EXP)", "e = e"),
    ("fnuz_max", "E4M3_MAX = 448.0", "E4M3_MAX = 240.0"),
    ("smoothing_sign", "(k32 - mu32[:, None, :, :])", "(k32 + mu32[:, None, :, :])"),
    ("block_64", "BLOCK_TOKENS = 128", "BLOCK_TOKENS = 64"),
    ("bias_8", "E4M3_BIAS = 7", "E4M3_BIAS = 8"),
]


def test_fp8_source_passes_pins():
    assert _fp8_pins_pass(_load("fp8.py", extra=_fp8_extra()))


@pytest.mark.parametrize("name,old,new", FP8_MUTANTS, ids=[m[0] for m in FP8_MUTANTS])
def test_fp8_mutant_is_caught(name, old, new):
    assert not _fp8_pins_pass(_load("fp8.py", old, new, extra=_fp8_extra()))


# ---------------------------------------------------------------- MXFP8 pins

def _mx_pins_pass(mod):
    try:
        for c in _golden("mx_worked_examples.json")["cases"]:
            x = np.zeros(32, dtype=np.float32)
            x[: len(c["x"])] = np.asarray(c["x"], dtype=np.float32)
            codes, exps, values = mod.mx_quantize(x)
            n = len(c["codes"])
            if exps.shape != (1,) or int(exps[0]) != c["exp_byte"]:
                return False
            if [int(v) for v in codes[:n]] != [int(v, 16) for v in c["codes"]] or list(values[:n]) != c["values"]:
                return False
        x = (RNG.standard_normal((4, 64)) * 3).astype(np.float32)
        c0, e0, _ = mod.mx_quantize(x)
        c1, e1, _ = mod.mx_quantize((x * np.float32(8.0)).astype(np.float32))
        if not (np.array_equal(c0, c1) and np.array_equal(e1.astype(int), e0.astype(int) + 3)):
            return False
        y = np.abs(x.astype(np.float64)).reshape(4, 2, 32).max(axis=2) / np.ldexp(1.0, e0.astype(int) - 127)
        if not np.all((y >= 256) & (y < 512)):
            return False
    except Exception:
        return False
    return True


def _mx_extra():
    from oracle.attention import attention_forward
    from oracle.fp8 import e4m3_decode, e4m3_encode, e4m3_round, smooth_k
    return {"attention_forward": attention_forward, "e4m3_decode": e4m3_decode, "e4m3_encode": e4m3_encode,
            "e4m3_round": e4m3_round, "smooth_k": smooth_k}


MX_ANCHOR = "from .fp8 import e4m3_decode, e4m3_encode, e4m3_round, smooth_k"

MX_MUTANTS = [
    ("emax_7", "E4M3_EMAX = 8", "E4M3_EMAX = 7"),
    ("ceil_log2", "shared = (e2.astype(np.int64) - 1) - E4M3_EMAX", "shared = e2.astype(np.int64) - E4M3_EMAX"),
    ("bias_128", "E8M0_BIAS = 127", "E8M0_BIAS = 128"),
    ("block_16", "MX_BLOCK = 32", "MX_BLOCK = 16"),
    ("zero_block_byte", "exps = np.where(amax > 0, shared + E8M0_BIAS, 0).astype(np.uint8)",
     "exps = (shared + E8M0_BIAS).astype(np.uint8)"),
    ("scale_multiplied", "q = e4m3_round(blocks / scale)", "q = e4m3_round(blocks * scale)"),
]


def _load_mx(old=None, new=None):
    path = os.path.join(ROOT, "oracle", "mx.py")
    src = open(path).read().replace(MX_ANCHOR, "")
    if old is not None:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new, 1)
    src = src.replace("from .attention import attention_forward", "")
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__.update(_mx_extra())
    exec(compile(src, path, "exec"), mod.__dict__)
    return mod


def test_mx_source_passes_pins():
    assert _mx_pins_pass(_load_mx())


@pytest.mark.parametrize("name,old,new", MX_MUTANTS, ids=[m[0] for m in MX_MUTANTS])
def test_mx_mutant_is_caught(name, old, new):
    assert not _mx_pins_pass(_load_mx(old, new))


# ---------------------------------------------------------------- window / sink pins

def _window_pins_pass(mod):
    import test_oracle_window as tw
    try:
        g = _golden("window_sink_worked_examples.json")
        for c in g["cases"]:
            sinks = None if c["sink"] is None else np.array([c["sink"]])
            o, lse = mod.attention_window_sink(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), scale=1.0,
                                               causal=c["causal"], window_left=c["window_left"],
                                               window_right=c["window_right"], sinks=sinks)
            if not (np.allclose(o[0, :, 0, 0], c["o"], rtol=0, atol=1e-13)
                    and np.allclose(lse[0, 0], c["lse"], rtol=0, atol=1e-13)):
                return False
        for causal, left, right in ((True, 3, -1), (False, 2, 1)):
            q, k, v = RNG.standard_normal((1, 7, 4, 3)), RNG.standard_normal((1, 9, 2, 3)), RNG.standard_normal((1, 9, 2, 2))
            sinks = RNG.standard_normal(4)
            o, lse = mod.attention_window_sink(q, k, v, scale=0.7, causal=causal, window_left=left, window_right=right,
                                               sinks=sinks)
            o_b, lse_b = tw._brute(q, k, v, 0.7, causal, left, right, sinks)
            if not (np.allclose(o, o_b, rtol=0, atol=1e-12) and np.allclose(lse, lse_b, rtol=0, atol=1e-12)):
                return False
        o, lse = mod.attention_window_sink(np.ones((1, 2, 1, 2)), np.zeros((1, 0, 1, 2)), np.zeros((1, 0, 1, 2)),
                                           scale=1.0, causal=False, sinks=np.array([0.5]))
        if not (np.all(o == 0) and np.all(lse == 0.5)):
            return False
    except Exception:
        return False
    return True


WINDOW_MUTANTS = [
    ("left_off_by_one", "vis &= j >= i - window_left", "vis &= j > i - window_left"),
    ("right_off_by_one", "vis &= j <= i + window_right", "vis &= j <= i + window_right + 1"),
    ("sink_not_in_denominator", "denom = p.sum(axis=1) + np.exp(sink - m_safe)", "denom = p.sum(axis=1)"),
    ("sink_scaled", "sink = -np.inf if sinks is None else float(sinks[h])",
     "sink = -np.inf if sinks is None else float(sinks[h]) * scale"),
    ("sink_per_kv_head", "sink = -np.inf if sinks is None else float(sinks[h])",
     "sink = -np.inf if sinks is None else float(sinks[g])"),
    ("sink_not_in_max", "m = np.maximum(s.max(axis=1, initial=-np.inf), sink)", "m = s.max(axis=1, initial=-np.inf)"),
]


def test_window_source_passes_pins():
    assert _window_pins_pass(_load("window.py"))


@pytest.mark.parametrize("name,old,new", WINDOW_MUTANTS, ids=[m[0] for m in WINDOW_MUTANTS])
def test_window_mutant_is_caught(name, old, new):
    assert not _window_pins_pass(_load("window.py", old, new))
