"""Python binding of libmha, the gfx950 fused attention forward library.

Thin ctypes marshalling over the C ABI in include/mha.h: every step of the
computation runs in the library's HIP kernels.  PyTorch supplies device memory
and the current stream only.  There is no fallback: if libmha.so is missing or
the tensors are not on a ROCm device the calls raise.

Entry points (same names as the C ABI):
    mha_fwd_bf16(q, k, v, causal=False, softmax_scale=None, out=None, lse=True, n_split=None, workspace=None)
    mha_fwd_bf16_split_plan(b, hq, hk, sq, sk, d_qk, d_v, causal) -> n_split
    mha_fwd_bf16_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal=False, ...)
    k_smooth_mean(k, key_stride=1, max_keys=0, tau=0.25)
    mha_fwd_fp8(q, k, v, k_mean=None, causal=False, softmax_scale=None, out=None, lse=True)
Tensors are BSHD views (varlen: THD, sequences packed along the token axis) with a
contiguous channel dimension.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmha.so")

MHA_OK = 0
STATUS_NAMES = {
    0: "MHA_OK", 1: "MHA_ERR_NULL", 2: "MHA_ERR_SHAPE", 3: "MHA_ERR_UNSUPPORTED", 4: "MHA_ERR_LAYOUT",
    5: "MHA_ERR_OVERFLOW", 6: "MHA_ERR_WORKSPACE", 7: "MHA_ERR_HIP", 8: "MHA_ERR_VALUE",
}

# Every symbol include/mha.h declares.
EXPORTED_SYMBOLS = (
    "mha_fwd_bf16", "mha_fwd_bf16_varlen", "mha_fwd_bf16_window_sink", "mha_fwd_bf16_varlen_window_sink",
    "k_smooth_mean_workspace_bytes", "k_smooth_mean", "mha_fwd_fp8_workspace_bytes",
    "mha_fp8_workspace_layout", "mha_fwd_fp8", "mha_fwd_mxfp8_workspace_bytes", "mha_mxfp8_workspace_layout",
    "mha_fwd_mxfp8", "mha_status_string", "mha_last_error", "mha_debug_sync_enabled", "k_smooth_mean_noalloc",
    "mha_fwd_bf16_split", "mha_fwd_bf16_split_workspace_bytes", "mha_fwd_bf16_split_plan",
)


class MhaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("s", ctypes.c_int64), ("h", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmha.so and declare the C signatures (no GPU call happens here)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m head_attention_forward_flash_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.mha_fwd_bf16.restype = i32
    lib.mha_fwd_bf16.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides, vp,
                                 i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.mha_fwd_bf16_split.restype = i32
    lib.mha_fwd_bf16_split.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides, vp,
                                       i32, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp, sz, vp]
    lib.mha_fwd_bf16_split_workspace_bytes.restype = sz
    lib.mha_fwd_bf16_split_workspace_bytes.argtypes = [i32] * 6
    lib.mha_fwd_bf16_split_plan.restype = i32
    lib.mha_fwd_bf16_split_plan.argtypes = [i32] * 8 + [ctypes.POINTER(i32)]
    lib.mha_fwd_bf16_varlen.restype = i32
    lib.mha_fwd_bf16_varlen.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides, vp, vp, vp,
                                        i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.mha_fwd_bf16_window_sink.restype = i32
    lib.mha_fwd_bf16_window_sink.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides, vp,
                                             i32, i32, i32, i32, i32, i32, i32, f32, i32, i32, i32, vp, vp]
    lib.mha_fwd_bf16_varlen_window_sink.restype = i32
    lib.mha_fwd_bf16_varlen_window_sink.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides, vp, vp, vp,
                                                    i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, i32, i32,
                                                    vp, vp]
    lib.k_smooth_mean_workspace_bytes.restype = sz
    lib.k_smooth_mean_workspace_bytes.argtypes = [i32] * 6
    lib.k_smooth_mean.restype = i32
    lib.k_smooth_mean.argtypes = [vp, Strides, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, sz, vp]
    lib.k_smooth_mean_noalloc.restype = i32
    lib.k_smooth_mean_noalloc.argtypes = [vp, Strides, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp]
    lib.mha_fwd_fp8_workspace_bytes.restype = sz
    lib.mha_fwd_fp8_workspace_bytes.argtypes = [i32] * 6
    lib.mha_fp8_workspace_layout.restype = i32
    lib.mha_fp8_workspace_layout.argtypes = [i32] * 6 + [ctypes.POINTER(sz)]
    lib.mha_fwd_fp8.restype = i32
    lib.mha_fwd_fp8.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, vp, Strides, vp,
                                i32, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.mha_fwd_mxfp8_workspace_bytes.restype = sz
    lib.mha_fwd_mxfp8_workspace_bytes.argtypes = [i32] * 6
    lib.mha_mxfp8_workspace_layout.restype = i32
    lib.mha_mxfp8_workspace_layout.argtypes = [i32] * 6 + [ctypes.POINTER(sz)]
    lib.mha_fwd_mxfp8.restype = i32
    lib.mha_fwd_mxfp8.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, vp, Strides, vp,
                                  i32, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.mha_status_string.restype = ctypes.c_char_p
    lib.mha_status_string.argtypes = [i32]
    lib.mha_last_error.restype = ctypes.c_char_p
    lib.mha_last_error.argtypes = []
    lib.mha_debug_sync_enabled.restype = i32
    lib.mha_debug_sync_enabled.argtypes = []
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != MHA_OK:
        msg = load_library().mha_last_error().decode()
        raise MhaError(status, msg)


def _torch():
    import torch
    return torch


def _bshd_strides(t) -> Strides:
    if t.dim() != 4:
        raise ValueError(f"expected a 4-d BSHD tensor, got shape {tuple(t.shape)}")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError("the channel dimension must be contiguous (stride 1)")
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _require_device(*tensors):
    for t in tensors:
        if t is not None and t.device.type != "cuda":
            raise ValueError("tensors must live on a ROCm device (torch 'cuda' device)")


def _dims(name, t, ndim):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected a {ndim}-d tensor, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _expect(name, t, shape, dtype, device):
    """Refuse a tensor whose shape, dtype or device does not match what the call was sized from:
    the library trusts the sizes it is given, so a short buffer would be read or written past
    its end."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")


def _expect_workspace(name, ws, need, device):
    torch = _torch()
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 1-d uint8 tensor")
    if ws.device != device:
        raise ValueError(f"{name} is on {ws.device}, the other tensors on {device}")
    if ws.numel() < need:
        raise ValueError(f"{name} holds {ws.numel()} bytes, the call needs {need}")


def _attn_shapes(q, k, v, out, ndim):
    """Sizes of an attention call, every tensor checked against them (BSHD: ndim 4, THD: 3)."""
    torch = _torch()
    qs, ks, vs = _dims("q", q, ndim), _dims("k", k, ndim), _dims("v", v, ndim)
    d_qk, d_v = qs[-1], vs[-1]
    lead_q, lead_k = qs[:-2], ks[:-2]       # (b, sq) or (total_q,); (b, sk) or (total_k,)
    hq, hk = qs[-2], ks[-2]
    if ndim == 4 and ks[0] != qs[0]:
        raise ValueError(f"k: batch {ks[0]} differs from q's {qs[0]}")
    _expect("q", q, qs, torch.bfloat16, q.device)
    _expect("k", k, lead_k + (hk, d_qk), torch.bfloat16, q.device)
    _expect("v", v, lead_k + (hk, d_v), torch.bfloat16, q.device)
    if out is not None:
        _expect("out", out, lead_q + (hq, d_v), torch.bfloat16, q.device)
    return qs, ks, d_v


def mha_fwd_bf16_split_workspace_bytes(b: int, hq: int, sq: int, d_qk: int, d_v: int, n_split: int) -> int:
    """Workspace bytes of mha_fwd_bf16 with n_split key ranges (0 for n_split <= 1)."""
    return int(load_library().mha_fwd_bf16_split_workspace_bytes(b, hq, sq, d_qk, d_v, n_split))


def mha_fwd_bf16_split_plan(b: int, hq: int, hk: int, sq: int, sk: int, d_qk: int, d_v: int,
                            causal: bool = False) -> int:
    """Key ranges per query block that balance this shape's grid on the current device (1: none)."""
    n = ctypes.c_int(1)
    _check(load_library().mha_fwd_bf16_split_plan(b, hq, hk, sq, sk, d_qk, d_v, int(bool(causal)), ctypes.byref(n)))
    return n.value


def mha_fwd_bf16(q, k, v, causal: bool = False, softmax_scale: Optional[float] = None, out=None,
                 lse: bool = True, n_split: Optional[int] = None, workspace=None):
    """Fused attention forward in bf16. Returns (o, lse) with lse [b, hq, sq] fp32 (or None).

    n_split: key ranges per query block (mha_fwd_bf16_split); None asks the library for the
    split that balances the grid on q's device.  A split needs a workspace: `workspace`
    (contiguous uint8 on q's device) or one allocated here."""
    torch = _torch()
    lib = load_library()
    (b, sq, hq, d_qk), (_, sk, hk, _), d_v = _attn_shapes(q, k, v, out, 4)
    _require_device(q)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_qk)
    if out is None:
        out = torch.empty((b, sq, hq, d_v), dtype=torch.bfloat16, device=q.device)
    lse_t = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device) if lse else None
    if n_split is None:
        with torch.cuda.device(q.device):
            n_split = mha_fwd_bf16_split_plan(b, hq, hk, sq, sk, d_qk, d_v, causal)
    if n_split == 1:
        _check(lib.mha_fwd_bf16(_ptr(q), _bshd_strides(q), _ptr(k), _bshd_strides(k), _ptr(v), _bshd_strides(v),
                                _ptr(out), _bshd_strides(out), _ptr(lse_t), b, hq, hk, sq, sk, d_qk, d_v,
                                float(softmax_scale), int(bool(causal)), _stream(q.device)))
        return out, lse_t
    need = mha_fwd_bf16_split_workspace_bytes(b, hq, sq, d_qk, d_v, int(n_split))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _expect_workspace("workspace", workspace, need, q.device)
    _check(lib.mha_fwd_bf16_split(_ptr(q), _bshd_strides(q), _ptr(k), _bshd_strides(k), _ptr(v), _bshd_strides(v),
                                  _ptr(out), _bshd_strides(out), _ptr(lse_t), b, hq, hk, sq, sk, d_qk, d_v,
                                  float(softmax_scale), int(bool(causal)), int(n_split), _ptr(workspace),
                                  workspace.numel(), _stream(q.device)))
    return out, lse_t


def mha_fwd_bf16_window_sink(q, k, v, causal: bool = False, window_left: int = -1, window_right: int = -1,
                             sinks=None, softmax_scale: Optional[float] = None, out=None, lse: bool = True):
    """mha_fwd_bf16 with a sliding window (-1 = unbounded side) and per-head sink logits
    (fp32 [hq] on the device, or None). Returns (o, lse)."""
    torch = _torch()
    lib = load_library()
    (b, sq, hq, d_qk), (_, sk, hk, _), d_v = _attn_shapes(q, k, v, out, 4)
    if sinks is not None:
        _expect("sinks", sinks, (hq,), torch.float32, q.device)
        if not sinks.is_contiguous():
            raise ValueError("sinks must be contiguous")
    _require_device(q)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_qk)
    if out is None:
        out = torch.empty((b, sq, hq, d_v), dtype=torch.bfloat16, device=q.device)
    lse_t = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device) if lse else None
    _check(lib.mha_fwd_bf16_window_sink(_ptr(q), _bshd_strides(q), _ptr(k), _bshd_strides(k), _ptr(v),
                                        _bshd_strides(v), _ptr(out), _bshd_strides(out), _ptr(lse_t), b, hq, hk, sq,
                                        sk, d_qk, d_v, float(softmax_scale), int(bool(causal)), int(window_left),
                                        int(window_right), _ptr(sinks), _stream(q.device)))
    return out, lse_t


def _thd_strides(t) -> Strides:
    if t.dim() != 3:
        raise ValueError(f"expected a 3-d THD tensor [tokens, heads, d], got shape {tuple(t.shape)}")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError("the channel dimension must be contiguous (stride 1)")
    return Strides(0, t.stride(0), t.stride(1))


def mha_fwd_bf16_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                        causal: bool = False, softmax_scale: Optional[float] = None, out=None, lse: bool = True,
                        window_left: int = -1, window_right: int = -1, sinks=None):
    """Attention forward over packed sequences. q [total_q, hq, d_qk], k/v [total_k, hk, d],
    cu_seqlens_* int32 [b + 1] on the device. Returns (o [total_q, hq, d_v], lse [hq, total_q] fp32 or None).
    A window (-1 = unbounded side) or per-head sinks (fp32 [hq] on the device) select
    mha_fwd_bf16_varlen_window_sink."""
    torch = _torch()
    lib = load_library()
    (total_q, hq, d_qk), (total_k, hk, _), d_v = _attn_shapes(q, k, v, out, 3)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _expect(name, t, (_dims(name, t, 1)[0],), torch.int32, q.device)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if sinks is not None:
        _expect("sinks", sinks, (hq,), torch.float32, q.device)
        if not sinks.is_contiguous():
            raise ValueError("sinks must be contiguous")
    b = cu_seqlens_q.numel() - 1
    if b < 0 or cu_seqlens_k.numel() != b + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold b + 1 offsets")
    _require_device(q)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_qk)
    if out is None:
        out = torch.empty((total_q, hq, d_v), dtype=torch.bfloat16, device=q.device)
    lse_t = torch.empty((hq, total_q), dtype=torch.float32, device=q.device) if lse else None
    args = [_ptr(q), _thd_strides(q), _ptr(k), _thd_strides(k), _ptr(v), _thd_strides(v), _ptr(out),
            _thd_strides(out), _ptr(lse_t), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), b, hq, hk, total_q, total_k,
            int(max_seqlen_q), int(max_seqlen_k), d_qk, d_v, float(softmax_scale), int(bool(causal))]
    if window_left == -1 and window_right == -1 and sinks is None:
        _check(lib.mha_fwd_bf16_varlen(*args, _stream(q.device)))
    else:
        _check(lib.mha_fwd_bf16_varlen_window_sink(*args, int(window_left), int(window_right), _ptr(sinks),
                                                   _stream(q.device)))
    return out, lse_t


def k_smooth_mean_workspace_bytes(b, hk, sk, d, key_stride=1, max_keys=0) -> int:
    return int(load_library().k_smooth_mean_workspace_bytes(b, hk, sk, d, key_stride, max_keys))


def k_smooth_mean(k, key_stride: int = 1, max_keys: int = 0, tau: float = 0.25, workspace=None):
    """K-smoothing gate. Returns (mean [b, hk, d] fp32, gate [b, hk] int32)."""
    torch = _torch()
    lib = load_library()
    ks = _dims("k", k, 4)
    _expect("k", k, ks, torch.bfloat16, k.device)
    b, sk, hk, d = ks
    need = k_smooth_mean_workspace_bytes(b, hk, sk, d, key_stride, max_keys)
    if workspace is not None:
        _expect_workspace("workspace", workspace, need, k.device)
    _require_device(k)
    mean = torch.empty((b, hk, d), dtype=torch.float32, device=k.device)
    gate = torch.empty((b, hk), dtype=torch.int32, device=k.device)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=k.device)
    _check(lib.k_smooth_mean(_ptr(k), _bshd_strides(k), b, hk, sk, d, key_stride, max_keys, float(tau),
                             _ptr(mean), _ptr(gate), _ptr(workspace), workspace.numel(), _stream(k.device)))
    return mean, gate


def k_smooth_mean_noalloc(k, key_stride: int = 1, max_keys: int = 0, tau: float = 0.25, mean=None, gate=None):
    """k_smooth_mean on the library's per-GPU scratch (no workspace; nothing allocated when
    `mean` and `gate` are given). Returns (mean [b, hk, d] fp32, gate [b, hk] int32)."""
    torch = _torch()
    lib = load_library()
    ks = _dims("k", k, 4)
    _expect("k", k, ks, torch.bfloat16, k.device)
    b, sk, hk, d = ks
    for name, t, shape, dt in (("mean", mean, (b, hk, d), torch.float32), ("gate", gate, (b, hk), torch.int32)):
        if t is not None:
            _expect(name, t, shape, dt, k.device)
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
    _require_device(k)
    if mean is None:
        mean = torch.empty((b, hk, d), dtype=torch.float32, device=k.device)
    if gate is None:
        gate = torch.empty((b, hk), dtype=torch.int32, device=k.device)
    _check(lib.k_smooth_mean_noalloc(_ptr(k), _bshd_strides(k), b, hk, sk, d, key_stride, max_keys, float(tau),
                                     _ptr(mean), _ptr(gate), _stream(k.device)))
    return mean, gate


def mha_fwd_fp8_workspace_bytes(b, hq, hk, sq, sk, d) -> int:
    return int(load_library().mha_fwd_fp8_workspace_bytes(b, hq, hk, sq, sk, d))


def mha_fp8_workspace_layout(b, hq, hk, sq, sk, d):
    """Byte offsets of (q codes, k codes, v values as bf16, q scales, k scales, v scales) in the fp8 workspace."""
    lib = load_library()
    arr = (ctypes.c_size_t * 6)()
    _check(lib.mha_fp8_workspace_layout(b, hq, hk, sq, sk, d, arr))
    return [int(x) for x in arr]


def _fwd_quantised(entry, need_fn, q, k, v, k_mean, causal, softmax_scale, out, lse, workspace):
    torch = _torch()
    (b, sq, hq, d), (_, sk, hk, _), d_v = _attn_shapes(q, k, v, out, 4)
    if d_v != d:
        raise ValueError(f"v: head dim {d_v} differs from q/k's {d} (the quantised call has one head dim)")
    if k_mean is not None:
        _expect("k_mean", k_mean, (b, hk, d), torch.float32, q.device)
        if not k_mean.is_contiguous():
            raise ValueError("k_mean must be contiguous")
    need = need_fn(b, hq, hk, sq, sk, d)
    if workspace is not None:
        _expect_workspace("workspace", workspace, need, q.device)
    _require_device(q)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((b, sq, hq, d), dtype=torch.bfloat16, device=q.device)
    lse_t = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device) if lse else None
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(entry(_ptr(q), _bshd_strides(q), _ptr(k), _bshd_strides(k), _ptr(v), _bshd_strides(v),
                 _ptr(k_mean), _ptr(out), _bshd_strides(out), _ptr(lse_t), b, hq, hk, sq, sk, d,
                 float(softmax_scale), int(bool(causal)), _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out, lse_t, workspace


def mha_fwd_fp8(q, k, v, k_mean=None, causal: bool = False, softmax_scale: Optional[float] = None, out=None,
                lse: bool = True, workspace=None):
    """K-smoothed FP8 attention forward. Returns (o, lse, workspace)."""
    return _fwd_quantised(load_library().mha_fwd_fp8, mha_fwd_fp8_workspace_bytes, q, k, v, k_mean, causal,
                          softmax_scale, out, lse, workspace)


def mha_fwd_mxfp8_workspace_bytes(b, hq, hk, sq, sk, d) -> int:
    return int(load_library().mha_fwd_mxfp8_workspace_bytes(b, hq, hk, sq, sk, d))


def mha_mxfp8_workspace_layout(b, hq, hk, sq, sk, d):
    """Byte offsets of (q codes, k codes, v values as bf16, q exponents, k exponents) in the MXFP8 workspace."""
    lib = load_library()
    arr = (ctypes.c_size_t * 5)()
    _check(lib.mha_mxfp8_workspace_layout(b, hq, hk, sq, sk, d, arr))
    return [int(x) for x in arr]


def mha_fwd_mxfp8(q, k, v, k_mean=None, causal: bool = False, softmax_scale: Optional[float] = None, out=None,
                  lse: bool = True, workspace=None):
    """K-smoothed MXFP8 attention forward (E8M0 exponent per 32 channels). Returns (o, lse, workspace)."""
    return _fwd_quantised(load_library().mha_fwd_mxfp8, mha_fwd_mxfp8_workspace_bytes, q, k, v, k_mean, causal,
                          softmax_scale, out, lse, workspace)
