"""The C-ABI library loads, exports every declared symbol, and refuses bad arguments.

CPU only: validation happens on the host before any HIP call, so no GPU is
touched.  Pointers passed here are fake non-null addresses that no call ever
dereferences (every case is refused before a launch).
"""

import ctypes
import os
import re

import pytest

import head_attention_forward_flash_amd as mha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
S = mha.Strides
FAKE = 0x10000      # 64 KiB-aligned fake device address, never dereferenced


@pytest.fixture(scope="module")
def lib():
    # The refusal cases pass fake device addresses: a case that wrongly passed validation would
    # launch on them.  Where a GPU is visible these tests do not run at all (counting devices
    # does not initialise one).
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("fake-pointer ABI tests run only where no GPU is visible")
    return mha.load_library()


def _header_symbols():
    src = open(os.path.join(ROOT, "include", "mha.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_exports_every_header_symbol(lib):
    syms = _header_symbols()
    assert set(syms) == set(mha.EXPORTED_SYMBOLS), syms
    for s in syms:
        assert hasattr(lib, s), s


def test_status_strings(lib):
    for code, name in mha.STATUS_NAMES.items():
        assert lib.mha_status_string(code).decode() == name


def _bshd(s, h, d):
    return S(s * h * d, h * d, d)


def _bf16(lib, **kw):
    a = dict(q=FAKE, qs=_bshd(128, 2, 64), k=FAKE, ks=_bshd(128, 2, 64), v=FAKE, vs=_bshd(128, 2, 64),
             o=FAKE, os=_bshd(128, 2, 64), lse=None, b=1, hq=2, hk=2, sq=128, sk=128, dqk=64, dv=64,
             scale=0.125, causal=0)
    a.update(kw)
    st = lib.mha_fwd_bf16(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["os"], a["lse"],
                          a["b"], a["hq"], a["hk"], a["sq"], a["sk"], a["dqk"], a["dv"], a["scale"], a["causal"],
                          None)
    return st, lib.mha_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), 1, "q is NULL"),
    (dict(o=None), 1, "o is NULL"),
    (dict(hq=3), 2, "multiple of hk"),
    (dict(b=-1), 2, "b, sq, sk"),
    (dict(hk=0), 2, "hq, hk"),
    (dict(dqk=96, dv=96), 3, "not built"),
    (dict(dqk=192, dv=192), 3, "not built"),
    (dict(q=FAKE + 2), 4, "q: pointer must be 16-byte aligned"),
    (dict(ks=S(128 * 2 * 64, 2 * 64 + 4, 64)), 4, "k: strides must be multiples"),
    (dict(vs=S(-1, 128, 64)), 4, "v: strides must be non-negative"),
    (dict(lse=FAKE + 2), 4, "lse must be 4-byte aligned"),
    (dict(qs=S(0, 1 << 24, 64), sq=128), 5, "q: one (batch, head) slice"),
    (dict(ks=S(128 * 2 * 64, 32, 64)), 4, "k: rows overlap"),
    (dict(scale=float("inf")), 8, "softmax_scale"),
    (dict(causal=2), 8, "causal"),
])
def test_bf16_refusals(lib, kw, status, needle):
    st, msg = _bf16(lib, **kw)
    assert st == status, (st, msg)
    assert needle in msg, msg


def test_bf16_empty_problem_is_a_noop(lib):
    # sq == 0 and b == 0 are accepted and launch nothing (no GPU needed)
    assert _bf16(lib, sq=0)[0] == 0
    assert _bf16(lib, b=0)[0] == 0


def _split(lib, **kw):
    a = dict(q=FAKE, qs=_bshd(1000, 2, 128), k=FAKE, ks=_bshd(1000, 2, 128), v=FAKE, vs=_bshd(1000, 2, 128),
             o=FAKE, os=_bshd(1000, 2, 128), lse=None, b=1, hq=2, hk=2, sq=1000, sk=1000, dqk=128, dv=128,
             scale=0.088, causal=0, n=3, ws=FAKE, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = lib.mha_fwd_bf16_split_workspace_bytes(a["b"], a["hq"], a["sq"], a["dqk"], a["dv"], max(a["n"], 2))
    st = lib.mha_fwd_bf16_split(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["os"], a["lse"],
                                a["b"], a["hq"], a["hk"], a["sq"], a["sk"], a["dqk"], a["dv"], a["scale"],
                                a["causal"], a["n"], a["ws"], a["wsb"], None)
    return st, lib.mha_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    # causal, 300 rows: 3 blocks, the pairs (2, 0) of 5 + 2 key tiles and (1, 1) of 4
    (dict(causal=1, n=5, sq=300, sk=300, qs=_bshd(300, 2, 128), ks=_bshd(300, 2, 128), vs=_bshd(300, 2, 128),
          os=_bshd(300, 2, 128)), 8, "n_split = 5 exceeds the 4 key tiles of 64 that the shortest pair"),
    (dict(n=0), 8, "n_split = 0"),
    (dict(n=17), 8, "n_split = 17"),
    (dict(n=4, sk=150, ks=_bshd(150, 2, 128), vs=_bshd(150, 2, 128)), 8, "exceeds the 3 key tiles"),
    (dict(causal=1, n=3, sq=100, sk=100, qs=_bshd(100, 2, 128), ks=_bshd(100, 2, 128), vs=_bshd(100, 2, 128),
          os=_bshd(100, 2, 128)), 8, "exceeds the 2 key tiles of 64 that the shortest pair"),
    (dict(ws=None), 6, "ws is NULL"),
    (dict(ws=FAKE + 16), 6, "256-byte aligned"),
    (dict(wsb=4096), 6, "ws_bytes = 4096"),
    (dict(hq=3), 2, "multiple of hk"),
    (dict(q=FAKE + 2), 4, "q: pointer must be 16-byte aligned"),
])
def test_split_refusals(lib, kw, status, needle):
    st, msg = _split(lib, **kw)
    assert st == status, (st, msg)
    assert needle in msg, msg


def test_split_workspace_bytes(lib):
    # two block slots per pair of 128-row query blocks; per slot, range, wave and lane an fp32
    # (max, sum) pair; per slot, range and row d_v fp32 partial outputs; regions 256-byte aligned
    ws = lib.mha_fwd_bf16_split_workspace_bytes
    slots = 2 * 5 * 8    # b 2, hq 5, 1000 rows: 8 blocks, 4 pairs
    r256 = lambda x: (x + 255) // 256 * 256
    assert ws(2, 5, 1000, 128, 128, 3) == r256(slots * 3 * 4 * 64 * 8) + slots * 3 * 128 * 128 * 4
    # an odd block count rounds up to whole pairs: 900 rows are 8 blocks too, 1100 rows 9 -> 10
    assert ws(2, 5, 1100, 128, 128, 3) == r256(2 * 5 * 10 * 3 * 4 * 64 * 8) + 2 * 5 * 10 * 3 * 128 * 128 * 4
    # d_qk 192: 256-row blocks of 8 waves (1000 rows: 4 blocks, 2 pairs)
    assert ws(1, 2, 1000, 192, 128, 2) == r256(8 * 2 * 8 * 64 * 8) + 8 * 2 * 256 * 128 * 4
    assert ws(1, 2, 1000, 128, 128, 1) == 0 and ws(1, 2, 1000, 128, 128, 17) == 0
    assert ws(1, 2, 1000, 96, 96, 2) == 0


def test_split_plan_refusals(lib):
    n = ctypes.c_int(7)
    assert lib.mha_fwd_bf16_split_plan(1, 3, 2, 100, 100, 128, 128, 0, ctypes.byref(n)) == 2 and n.value == 1
    assert lib.mha_fwd_bf16_split_plan(1, 2, 2, 100, 100, 96, 96, 0, ctypes.byref(n)) == 3
    assert lib.mha_fwd_bf16_split_plan(1, 2, 2, 100, 100, 128, 128, 0, None) == 1


def _varlen(lib, **kw):
    a = dict(q=FAKE, qs=S(0, 2 * 64, 64), k=FAKE, ks=S(0, 2 * 64, 64), v=FAKE, vs=S(0, 2 * 64, 64),
             o=FAKE, os=S(0, 2 * 64, 64), lse=None, cuq=FAKE, cuk=FAKE, b=3, hq=2, hk=2, tq=300, tk=300,
             mq=128, mk=128, dqk=64, dv=64, scale=0.125, causal=1)
    a.update(kw)
    st = lib.mha_fwd_bf16_varlen(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["os"], a["lse"],
                                 a["cuq"], a["cuk"], a["b"], a["hq"], a["hk"], a["tq"], a["tk"], a["mq"], a["mk"],
                                 a["dqk"], a["dv"], a["scale"], a["causal"], None)
    return st, lib.mha_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(cuq=None), 1, "cu_seqlens"),
    (dict(cuk=None), 1, "cu_seqlens"),
    (dict(cuq=FAKE + 2), 4, "cu_seqlens arrays must be 4-byte aligned"),
    (dict(tq=-1), 2, "total_q"),
    (dict(mk=-5), 2, "max_seqlen"),
    (dict(q=None), 1, "q is NULL"),
    (dict(hq=3), 2, "multiple of hk"),
    (dict(dqk=96, dv=96), 3, "not built"),
    (dict(ks=S(0, 32, 16)), 4, "k: rows overlap"),
    (dict(qs=S(0, 1 << 24, 64), tq=300), 5, "q: one (batch, head) slice"),
    (dict(causal=3), 8, "causal"),
])
def test_varlen_refusals(lib, kw, status, needle):
    st, msg = _varlen(lib, **kw)
    assert st == status, (st, msg)
    assert needle in msg, msg


def test_varlen_empty_problem_is_a_noop(lib):
    assert _varlen(lib, b=0, cuq=None, cuk=None)[0] == 0
    assert _varlen(lib, tq=0, q=None, o=None)[0] == 0
    assert _varlen(lib, mq=0)[0] == 0


def test_gate_refusals_and_workspace(lib):
    need = lib.k_smooth_mean_workspace_bytes(2, 3, 1000, 128, 1, 0)
    assert need >= 2 * 3 * 4 * 2 * 128 * 4 and need % 256 == 0
    assert lib.k_smooth_mean_workspace_bytes(2, 3, 1000, 128, 0, 0) == 0

    def call(**kw):
        a = dict(k=FAKE, ks=_bshd(1000, 3, 128), b=2, hk=3, sk=1000, d=128, stride=1, maxk=0, tau=0.25,
                 mean=FAKE, gate=None, ws=FAKE, wsb=need)
        a.update(kw)
        st = lib.k_smooth_mean(a["k"], a["ks"], a["b"], a["hk"], a["sk"], a["d"], a["stride"], a["maxk"],
                               a["tau"], a["mean"], a["gate"], a["ws"], a["wsb"], None)
        return st, lib.mha_last_error().decode()

    assert call(k=None) == (1, "k is NULL")
    assert call(mean=None)[0] == 1
    assert call(d=96)[0] == 3
    assert call(stride=0)[0] == 8
    assert call(maxk=-1)[0] == 8
    assert call(tau=float("nan"))[0] == 8
    assert call(ws=None)[0] == 6
    assert call(ws=FAKE + 128)[0] == 6
    assert call(wsb=need - 1)[0] == 6
    assert call(k=FAKE + 1)[0] == 4
    assert call(b=0)[0] == 0


def test_fp8_refusals_and_layout(lib):
    off = mha.mha_fp8_workspace_layout(1, 16, 16, 4096, 4096, 128)
    assert off[0] == 0 and all(o % 256 == 0 for o in off)
    assert off[1] - off[0] >= 16 * 4096 * 128 and off[3] - off[2] >= 16 * 4096 * 128
    need = lib.mha_fwd_fp8_workspace_bytes(1, 16, 16, 4096, 4096, 128)
    assert need >= off[5] + 16 * 32 * 4

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, mean=None, o=FAKE, lse=None, b=1, hq=2, hk=2, sq=256, sk=256, d=128,
                 scale=0.088, causal=0, ws=FAKE, wsb=lib.mha_fwd_fp8_workspace_bytes(1, 2, 2, 256, 256, 128))
        a.update(kw)
        st_ = _bshd(256, 2, 128)
        st = lib.mha_fwd_fp8(a["q"], st_, a["k"], st_, a["v"], st_, a["mean"], a["o"], st_, a["lse"], a["b"],
                             a["hq"], a["hk"], a["sq"], a["sk"], a["d"], a["scale"], a["causal"], a["ws"],
                             a["wsb"], None)
        return st, lib.mha_last_error().decode()

    assert call(d=96)[0] == 3
    assert call(v=None)[0] == 1
    assert call(ws=None)[0] == 6
    assert call(wsb=1024)[0] == 6
    assert call(mean=FAKE + 2)[0] == 4
    assert call(hq=3)[0] == 2


def test_mxfp8_refusals_and_layout(lib):
    off = mha.mha_mxfp8_workspace_layout(1, 16, 16, 4096, 4096, 128)
    assert len(off) == 5 and off[0] == 0 and all(o % 256 == 0 for o in off)
    assert off[1] - off[0] >= 16 * 4096 * 128 and off[2] - off[1] >= 16 * 4096 * 128
    assert off[3] - off[2] >= 16 * 4096 * 128 * 2 and off[4] - off[3] >= 16 * 4096 * 4
    need = lib.mha_fwd_mxfp8_workspace_bytes(1, 16, 16, 4096, 4096, 128)
    assert need >= off[4] + 16 * 4096 * 4
    with pytest.raises(mha.MhaError):
        mha.mha_mxfp8_workspace_layout(1, 16, 16, 4096, 4096, 100)   # d not a multiple of 32

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, mean=None, o=FAKE, lse=None, b=1, hq=2, hk=2, sq=256, sk=256, d=128,
                 scale=0.088, causal=0, ws=FAKE, wsb=lib.mha_fwd_mxfp8_workspace_bytes(1, 2, 2, 256, 256, 128))
        a.update(kw)
        st_ = _bshd(256, 2, 128)
        st = lib.mha_fwd_mxfp8(a["q"], st_, a["k"], st_, a["v"], st_, a["mean"], a["o"], st_, a["lse"], a["b"],
                               a["hq"], a["hk"], a["sq"], a["sk"], a["d"], a["scale"], a["causal"], a["ws"],
                               a["wsb"], None)
        return st, lib.mha_last_error().decode()

    assert call(d=96)[0] == 3 and "mxfp8" in call(d=96)[1]
    assert call(v=None)[0] == 1
    assert call(ws=None)[0] == 6
    assert call(ws=FAKE + 64)[0] == 6
    # the fp8 workspace is smaller than the mxfp8 one: refused
    assert call(wsb=lib.mha_fwd_fp8_workspace_bytes(1, 2, 2, 256, 256, 128))[0] == 6
    assert call(mean=FAKE + 2)[0] == 4
    assert call(hq=3)[0] == 2
    assert call(scale=float("nan"))[0] != 0
    assert call(b=0)[0] == 0 and call(sq=0)[0] == 0


def _window_sink(lib, **kw):
    a = dict(q=FAKE, qs=_bshd(128, 2, 64), k=FAKE, ks=_bshd(128, 2, 64), v=FAKE, vs=_bshd(128, 2, 64),
             o=FAKE, os=_bshd(128, 2, 64), lse=None, b=1, hq=2, hk=2, sq=128, sk=128, dqk=64, dv=64,
             scale=0.125, causal=1, left=127, right=-1, sinks=None)
    a.update(kw)
    st = lib.mha_fwd_bf16_window_sink(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["os"], a["lse"],
                                      a["b"], a["hq"], a["hk"], a["sq"], a["sk"], a["dqk"], a["dv"], a["scale"],
                                      a["causal"], a["left"], a["right"], a["sinks"], None)
    return st, lib.mha_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(left=-2), 8, "window_left = -2"),
    (dict(right=-5, causal=0), 8, "each must be >= -1"),
    (dict(sinks=FAKE + 2), 4, "sinks must be 4-byte aligned"),
    (dict(q=None), 1, "q is NULL"),
    (dict(dqk=16, dv=16), 3, "(32,32)"),
    (dict(causal=3), 8, "causal"),
])
def test_window_sink_refusals(lib, kw, status, needle):
    st, msg = _window_sink(lib, **kw)
    assert st == status, (st, msg)
    assert needle in msg, msg


def test_window_sink_and_d32_empty_problems_are_noops(lib):
    assert _window_sink(lib, b=0)[0] == 0
    assert _window_sink(lib, sq=0, sinks=FAKE)[0] == 0
    assert _bf16(lib, b=0, dqk=32, dv=32, qs=_bshd(128, 2, 32), ks=_bshd(128, 2, 32), vs=_bshd(128, 2, 32),
                 os=_bshd(128, 2, 32))[0] == 0
