"""The Python binding refuses tensors that do not match the call's sizes, and the library reads
its debug-synchronisation switch (CPU only: every case is refused before any GPU call)."""

import os
import subprocess
import sys

import pytest
import torch

import head_attention_forward_flash_amd as mha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BF = torch.bfloat16


def _bshd(b, s, h, d, dtype=BF):
    return torch.zeros((b, s, h, d), dtype=dtype)


def _qkv(b=1, sq=8, sk=8, hq=4, hk=2, dqk=64, dv=64):
    return _bshd(b, sq, hq, dqk), _bshd(b, sk, hk, dqk), _bshd(b, sk, hk, dv)


@pytest.mark.parametrize("mutate,needle", [
    (lambda q, k, v: (q, k, _bshd(1, 7, 2, 64), None), "v: expected shape (1, 8, 2, 64)"),
    (lambda q, k, v: (q, k, _bshd(1, 8, 1, 64), None), "v: expected shape (1, 8, 2, 64)"),
    (lambda q, k, v: (q, _bshd(2, 8, 2, 64), v, None), "k: batch 2 differs"),
    (lambda q, k, v: (q, _bshd(1, 8, 2, 32), v, None), "k: expected shape (1, 8, 2, 64)"),
    (lambda q, k, v: (q, k, v.float(), None), "v must be torch.bfloat16"),
    (lambda q, k, v: (q.half(), k, v, None), "q must be torch.bfloat16"),
    (lambda q, k, v: (q, k, v, _bshd(1, 8, 4, 32)), "out: expected shape (1, 8, 4, 64)"),
    (lambda q, k, v: (q, k, v, _bshd(1, 7, 4, 64)), "out: expected shape (1, 8, 4, 64)"),
    (lambda q, k, v: (q, k, v, _bshd(1, 8, 4, 64, torch.float32)), "out must be torch.bfloat16"),
    (lambda q, k, v: (q[0], k, v, None), "q: expected a 4-d tensor"),
    (lambda q, k, v: (q, k, v, None), "ROCm device"),
])
def test_bf16_binding_refusals(mutate, needle):
    q, k, v, out = mutate(*_qkv())
    with pytest.raises(ValueError, match=None) as e:
        mha.mha_fwd_bf16(q, k, v, out=out)
    assert needle in str(e.value), str(e.value)


def test_window_sink_refuses_wrong_sinks():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="sinks: expected shape"):
        mha.mha_fwd_bf16_window_sink(q, k, v, sinks=torch.zeros(3))
    with pytest.raises(ValueError, match="sinks must be torch.float32"):
        mha.mha_fwd_bf16_window_sink(q, k, v, sinks=torch.zeros(4, dtype=torch.float64))


def test_varlen_binding_refusals():
    q, k, v = torch.zeros((16, 4, 64), dtype=BF), torch.zeros((12, 2, 64), dtype=BF), torch.zeros((12, 2, 64), dtype=BF)
    cu = torch.tensor([0, 8, 16], dtype=torch.int32)
    cuk = torch.tensor([0, 6, 12], dtype=torch.int32)
    with pytest.raises(ValueError, match=r"v: expected shape \(12, 2, 64\)"):
        mha.mha_fwd_bf16_varlen(q, k, torch.zeros((11, 2, 64), dtype=BF), cu, cuk, 8, 6)
    with pytest.raises(ValueError, match=r"out: expected shape \(16, 4, 64\)"):
        mha.mha_fwd_bf16_varlen(q, k, v, cu, cuk, 8, 6, out=torch.zeros((15, 4, 64), dtype=BF))
    with pytest.raises(ValueError, match="cu_seqlens_q must be torch.int32"):
        mha.mha_fwd_bf16_varlen(q, k, v, cu.long(), cuk, 8, 6)
    with pytest.raises(ValueError, match="b \\+ 1 offsets"):
        mha.mha_fwd_bf16_varlen(q, k, v, cu, cuk[:2], 8, 6)
    with pytest.raises(ValueError, match="ROCm device"):
        mha.mha_fwd_bf16_varlen(q, k, v, cu, cuk, 8, 6)


def test_gate_binding_refusals():
    k = _bshd(1, 300, 2, 128)
    with pytest.raises(ValueError, match="k must be torch.bfloat16"):
        mha.k_smooth_mean(k.float())
    need = mha.k_smooth_mean_workspace_bytes(1, 2, 300, 128)
    with pytest.raises(ValueError, match=f"the call needs {need}"):
        mha.k_smooth_mean(k, workspace=torch.zeros(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="contiguous 1-d uint8"):
        mha.k_smooth_mean(k, workspace=torch.zeros(need, dtype=torch.float32))
    with pytest.raises(ValueError, match="ROCm device"):
        mha.k_smooth_mean(k, workspace=torch.zeros(need, dtype=torch.uint8))


@pytest.mark.parametrize("entry", ["mha_fwd_fp8", "mha_fwd_mxfp8"])
def test_quantised_binding_refusals(entry):
    fwd = getattr(mha, entry)
    q, k, v = _qkv(dqk=128, dv=128)
    with pytest.raises(ValueError, match="head dim 64 differs"):
        fwd(q, k, _bshd(1, 8, 2, 64))
    with pytest.raises(ValueError, match=r"k_mean: expected shape \(1, 2, 128\)"):
        fwd(q, k, v, k_mean=torch.zeros((1, 2, 64)))
    with pytest.raises(ValueError, match="k_mean must be torch.float32"):
        fwd(q, k, v, k_mean=torch.zeros((1, 2, 128), dtype=torch.float64))
    with pytest.raises(ValueError, match="the call needs"):
        fwd(q, k, v, workspace=torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="ROCm device"):
        fwd(q, k, v)


def _debug_flag(value):
    env = dict(os.environ)
    env.pop("MHA_DEBUG_SYNC", None)
    if value is not None:
        env["MHA_DEBUG_SYNC"] = value
    code = "import head_attention_forward_flash_amd as m; print(m.load_library().mha_debug_sync_enabled())"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return int(r.stdout.strip().splitlines()[-1])


def test_debug_sync_switch_is_read():
    assert _debug_flag(None) == 0
    assert _debug_flag("0") == 0
    assert _debug_flag("") == 0
    assert _debug_flag("1") == 1
    assert _debug_flag("yes") == 1
