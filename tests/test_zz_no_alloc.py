"""k_smooth_mean_noalloc (the gate on the library's per-GPU scratch) against k_smooth_mean with a
caller workspace, through the C ABI: bit-identical results on two calls in a row, the second on
a smaller input, and a refusal above the scratch's 4 MiB (needs an MI355X)."""

import ctypes

import pytest
import torch

import head_attention_forward_flash_amd as mha
import workloads
from parity import require_gpu

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 4 << 20


def _k(b, sk, hk, d, seed, bias=3.0):
    k = workloads.make_random((b, sk, hk, d), seed, dtype=torch.float32)
    k = k + workloads.make_random((1, 1, hk, d), seed + 1, dtype=torch.float32) * bias
    return k.to(torch.bfloat16)


def _strides(t):
    return mha.Strides(t.stride(0), t.stride(1), t.stride(2))


def _with_workspace(lib, k, key_stride, max_keys, stream):
    b, sk, hk, d = k.shape
    need = lib.k_smooth_mean_workspace_bytes(b, hk, sk, d, key_stride, max_keys)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=k.device)
    mean = torch.empty((b, hk, d), dtype=torch.float32, device=k.device)
    gate = torch.empty((b, hk), dtype=torch.int32, device=k.device)
    st = lib.k_smooth_mean(k.data_ptr(), _strides(k), b, hk, sk, d, key_stride, max_keys, ctypes.c_float(0.25),
                           mean.data_ptr(), gate.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    assert st == 0, lib.mha_last_error().decode()
    return mean, gate


def _noalloc(lib, k, key_stride, max_keys, stream, mean, gate):
    b, sk, hk, d = k.shape
    return lib.k_smooth_mean_noalloc(k.data_ptr(), _strides(k), b, hk, sk, d, key_stride, max_keys,
                                     ctypes.c_float(0.25), mean.data_ptr(), gate.data_ptr(), stream)


def test_noalloc_matches_workspace_call_twice():
    dev = require_gpu()
    lib = mha.load_library()
    stream = torch.cuda.current_stream(dev).cuda_stream
    cases = [
        # (b, sk, hk, d, key_stride, max_keys): the full c5 gate, then a smaller, strided one whose
        # moments cover fewer chunks (the scratch then still holds the first call's tail)
        (1, 4096, 16, 128, 1, 0),
        (2, 700, 3, 64, 3, 0),
    ]
    for i, (b, sk, hk, d, ks, mk) in enumerate(cases):
        k = _k(b, sk, hk, d, 9100 + i).to(dev)
        ref_mean, ref_gate = _with_workspace(lib, k, ks, mk, stream)
        mean = torch.full((b, hk, d), float("nan"), dtype=torch.float32, device=dev)
        gate = torch.full((b, hk), -7, dtype=torch.int32, device=dev)
        st = _noalloc(lib, k, ks, mk, stream, mean, gate)
        assert st == 0, lib.mha_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(mean, ref_mean), f"case {i}: mean differs"
        assert torch.equal(gate, ref_gate), f"case {i}: gate differs"


def test_noalloc_head_sliced_view():
    # a head-sliced view of a packed K, as in the gate's own tests
    dev = require_gpu()
    lib = mha.load_library()
    stream = torch.cuda.current_stream(dev).cuda_stream
    packed = _k(1, 1000, 6, 128, 9200).to(dev)
    k = packed[:, :, 2:5]
    ref_mean, ref_gate = _with_workspace(lib, k, 1, 0, stream)
    mean = torch.empty((1, 3, 128), dtype=torch.float32, device=dev)
    gate = torch.empty((1, 3), dtype=torch.int32, device=dev)
    assert _noalloc(lib, k, 1, 0, stream, mean, gate) == 0, lib.mha_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(mean, ref_mean) and torch.equal(gate, ref_gate)


def test_noalloc_refuses_above_scratch():
    dev = require_gpu()
    lib = mha.load_library()
    stream = torch.cuda.current_stream(dev).cuda_stream
    # b * hk * chunks * 2 * d * 4 bytes: 64 kv heads x 80 chunks x 2 x 128 x 4 = 5 MiB > 4 MiB
    b, sk, hk, d = 1, 80 * 256, 64, 128
    assert lib.k_smooth_mean_workspace_bytes(b, hk, sk, d, 1, 0) > SCRATCH_BYTES
    k = torch.zeros((b, sk, hk, d), dtype=torch.bfloat16, device=dev)
    mean = torch.empty((b, hk, d), dtype=torch.float32, device=dev)
    gate = torch.empty((b, hk), dtype=torch.int32, device=dev)
    st = _noalloc(lib, k, 1, 0, stream, mean, gate)
    assert st == 6 and "scratch" in lib.mha_last_error().decode()
    # capped by max_keys the same K fits
    assert _noalloc(lib, k, 1, 4096, stream, mean, gate) == 0, lib.mha_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(mean == 0) and torch.all(gate == 0)
