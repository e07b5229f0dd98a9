"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module only draws random numbers and names shapes. It holds none of the
attention, gate or quantisation arithmetic: the HIP library and the CPU oracle
each implement those on their own, and both receive the same input bits from
here.

Shapes follow the attention-forward workloads the pages time (the Triton MHA
forward retune page, "Test Plan" smoke commands and "Profile 1"/"Profile 2";
the mha_v4 K-smoothing gate page, "Performance" table).  The pages' own shape
lists (model_shapes.json and friends) are not available, so these seeded
N(0, 1) tensors stand in for them.

Recipe: a CPU ``torch.Generator`` seeded per workload draws float32 ``randn``
in BSHD order Q, then K, then V (then, for the FP8 workload, a per-head,
per-channel K bias ~ N(0, 3^2) of shape [h, d]); each tensor is rounded to
bfloat16 (round-to-nearest-even).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    b: int
    hq: int
    hk: int
    sq: int
    sk: int
    d_qk: int
    d_v: int
    causal: bool
    seed: int
    fp8: bool = False
    k_bias_std: float = 0.0  # per-(head, channel) K bias, FP8 smoothing workload only
    mx: bool = False         # quantised with the MXFP8 recipe (fp8 must be set too)
    window_left: int = -1    # sliding window (-1 = unbounded side)
    window_right: int = -1
    sink_std: float = 0.0    # per-query-head sink logits ~ N(0, sink_std^2) when > 0
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    def flops(self) -> float:
        """Algorithmic attention FLOPs: 2*(d_qk + d_v) per visible (query, key) pair and head:
        2*b*hq*sq*sk*(d_qk + d_v), halved when causal; with a window, the pairs it keeps."""
        if self.window_left < 0 and self.window_right < 0:
            f = 2.0 * self.b * self.hq * self.sq * self.sk * (self.d_qk + self.d_v)
            return f / 2.0 if self.causal else f
        i = torch.arange(self.sq, dtype=torch.int64)
        lo = (i - self.window_left).clamp(min=0) if self.window_left >= 0 else torch.zeros_like(i)
        hi = i if self.causal else (i + self.window_right if self.window_right >= 0 else torch.full_like(i, self.sk - 1))
        pairs = int((hi.clamp(max=self.sk - 1) - lo + 1).clamp(min=0).sum())
        return 2.0 * self.b * self.hq * pairs * (self.d_qk + self.d_v)


WORKLOADS = {
    "tiny_d64": Workload(
        "tiny_d64", b=1, hq=2, hk=2, sq=128, sk=128, d_qk=64, d_v=64, causal=False, seed=101,
        description="b1 hq2 hk2 128^2 d64 non-causal bf16"),
    "gqa_d64_causal": Workload(
        "gqa_d64_causal", b=8, hq=48, hk=8, sq=2048, sk=2048, d_qk=64, d_v=64, causal=True, seed=102,
        description="b8 hq48 hk8 2048^2 d64 causal bf16"),
    "gqa_d128_causal": Workload(
        "gqa_d128_causal", b=1, hq=32, hk=8, sq=4096, sk=4096, d_qk=128, d_v=128, causal=True, seed=103,
        description="b1 hq32 hk8 4096^2 d128 causal bf16"),
    "mla_d192_d128_causal": Workload(
        "mla_d192_d128_causal", b=1, hq=128, hk=128, sq=8192, sk=8192, d_qk=192, d_v=128, causal=True,
        seed=104, description="b1 hq128 hk128 8192^2 dqk192 dv128 causal bf16"),
    "fp8_ksmooth_d128": Workload(
        "fp8_ksmooth_d128", b=1, hq=16, hk=16, sq=4096, sk=4096, d_qk=128, d_v=128, causal=False,
        seed=105, fp8=True, k_bias_std=3.0,
        description="b1 h16 4096^2 d128 non-causal, bf16 in, K smoothed, e4m3 compute, bf16 out"),
    # Further shapes the pages time: the MLA shape without the causal mask and the d128
    # hq128/hk8 8192^2 causal shape (the retune page's fixed-shape table; its batch is not
    # printed, b = 1 here), one GPU's share of the MLA shape under 8-way head sharding, and
    # the long-context FP8 call (the gate page's Performance table; causality not printed,
    # non-causal here as for the h16 shape).
    "mla_d192_d128_noncausal": Workload(
        "mla_d192_d128_noncausal", b=1, hq=128, hk=128, sq=8192, sk=8192, d_qk=192, d_v=128, causal=False,
        seed=106, description="b1 hq128 hk128 8192^2 dqk192 dv128 non-causal bf16"),
    "gqa_d128_8192_causal": Workload(
        "gqa_d128_8192_causal", b=1, hq=128, hk=8, sq=8192, sk=8192, d_qk=128, d_v=128, causal=True,
        seed=107, description="b1 hq128 hk8 8192^2 d128 causal bf16"),
    "mla_d192_d128_tp8_causal": Workload(
        "mla_d192_d128_tp8_causal", b=1, hq=16, hk=16, sq=8192, sk=8192, d_qk=192, d_v=128, causal=True,
        seed=108, description="b1 hq16 hk16 8192^2 dqk192 dv128 causal bf16 (one rank of 8-way head sharding)"),
    # The retune page's two real-model d128 regressions ("The 8 remaining regressions" table):
    # 8192^2 d128 non-causal ("dense(c0)") with per-rank HQ/HK of 8/1 and 5/1 at TP8, i.e. one
    # GPU's share of 8-way head sharding of models with 64/8 and 40/8 query/kv heads (batch not
    # printed, b = 1 here)
    "gqa8_d128_tp8_noncausal": Workload(
        "gqa8_d128_tp8_noncausal", b=1, hq=8, hk=1, sq=8192, sk=8192, d_qk=128, d_v=128, causal=False,
        seed=115, description="b1 hq8 hk1 8192^2 d128 non-causal bf16 (one rank of 8-way head sharding)"),
    "gqa5_d128_tp8_noncausal": Workload(
        "gqa5_d128_tp8_noncausal", b=1, hq=5, hk=1, sq=8192, sk=8192, d_qk=128, d_v=128, causal=False,
        seed=116, description="b1 hq5 hk1 8192^2 d128 non-causal bf16 (one rank of 8-way head sharding)"),
    # The same ranks' causal prefill: hq8/hk1 makes 256 causal pairs of query blocks, one
    # workgroup per CU; hq5/hk1 makes 160, which the key-range split spreads over the device
    "gqa8_d128_tp8_causal": Workload(
        "gqa8_d128_tp8_causal", b=1, hq=8, hk=1, sq=8192, sk=8192, d_qk=128, d_v=128, causal=True,
        seed=117, description="b1 hq8 hk1 8192^2 d128 causal bf16 (one rank of 8-way head sharding)"),
    "gqa5_d128_tp8_causal": Workload(
        "gqa5_d128_tp8_causal", b=1, hq=5, hk=1, sq=8192, sk=8192, d_qk=128, d_v=128, causal=True,
        seed=118, description="b1 hq5 hk1 8192^2 d128 causal bf16 (one rank of 8-way head sharding)"),
    "fp8_long_h5": Workload(
        "fp8_long_h5", b=1, hq=5, hk=5, sq=65536, sk=65536, d_qk=128, d_v=128, causal=False,
        seed=109, fp8=True, k_bias_std=3.0,
        description="b1 h5 65536^2 d128 non-causal, bf16 in, K smoothed, e4m3 compute, bf16 out"),
    "mxfp8_ksmooth_d128": Workload(
        "mxfp8_ksmooth_d128", b=1, hq=16, hk=16, sq=4096, sk=4096, d_qk=128, d_v=128, causal=False,
        seed=111, fp8=True, k_bias_std=3.0, mx=True,
        description="b1 h16 4096^2 d128 non-causal, bf16 in, K smoothed, MXFP8 (E8M0 per 32 channels), bf16 out"),
    # GPT-OSS-like layers (64 query heads, 8 kv heads, head dim 64): the sliding-window layer
    # (128-token causal window) and the full causal layer, both with per-head sinks
    "gptoss_swa_sink_d64": Workload(
        "gptoss_swa_sink_d64", b=1, hq=64, hk=8, sq=8192, sk=8192, d_qk=64, d_v=64, causal=True, seed=112,
        window_left=127, sink_std=1.0,
        description="b1 hq64 hk8 8192^2 d64 causal, 128-token sliding window, per-head sinks, bf16"),
    "gptoss_sink_d64": Workload(
        "gptoss_sink_d64", b=1, hq=64, hk=8, sq=8192, sk=8192, d_qk=64, d_v=64, causal=True, seed=113,
        sink_std=1.0, description="b1 hq64 hk8 8192^2 d64 causal, per-head sinks, bf16"),
    # the small-head "vd32" shape family (2048^2, 16/16 heads, head dim 32)
    "vd32_noncausal": Workload(
        "vd32_noncausal", b=1, hq=16, hk=16, sq=2048, sk=2048, d_qk=32, d_v=32, causal=False, seed=114,
        description="b1 hq16 hk16 2048^2 d32 non-causal bf16"),
}


def _randn(gen: torch.Generator, shape) -> torch.Tensor:
    """float32 N(0,1) drawn in row-major order, then rounded to bfloat16."""
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def make_qkv(w: Workload, seed: Optional[int] = None, k_bias_std: Optional[float] = None):
    """Return (q, k, v) bfloat16 CPU tensors in BSHD layout for workload ``w``.

    ``k_bias_std`` overrides the workload's K bias (0 gives plain N(0,1) K).
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    q = _randn(gen, (w.b, w.sq, w.hq, w.d_qk))
    k32 = torch.randn((w.b, w.sk, w.hk, w.d_qk), generator=gen, dtype=torch.float32)
    v = _randn(gen, (w.b, w.sk, w.hk, w.d_v))
    std = w.k_bias_std if k_bias_std is None else k_bias_std
    if std != 0.0:
        bias = torch.randn((w.hk, w.d_qk), generator=gen, dtype=torch.float32) * std
        k32 = k32 + bias.view(1, 1, w.hk, w.d_qk)
    k = k32.to(torch.bfloat16)
    return q, k, v


def make_sinks(w: Workload) -> Optional[torch.Tensor]:
    """Seeded float32 [hq] sink logits of workload ``w`` (None when it has none)."""
    if w.sink_std <= 0.0:
        return None
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed + 1000)
    return torch.randn((w.hq,), generator=gen, dtype=torch.float32) * w.sink_std


def make_random(shape, seed: int, dtype=torch.bfloat16, std: float = 1.0, mean: float = 0.0) -> torch.Tensor:
    """A seeded N(mean, std^2) tensor of ``shape`` (drawn in float32, then cast)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = torch.randn(shape, generator=gen, dtype=torch.float32) * std + mean
    return x.to(dtype)


def sample_indices(n: int, count: int, seed: int, include=()) -> list:
    """A sorted, seeded subset of range(n) of about ``count`` items, plus ``include``."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    count = min(count, n)
    picked = set(int(i) for i in torch.randperm(n, generator=gen)[:count])
    picked.update(int(i) % n for i in include if n > 0)
    return sorted(picked)


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """Packed sequences (THD) of seeded lengths; FLOPs are summed per sequence."""
    name: str
    n_seq: int
    min_len: int
    max_len: int
    hq: int
    hk: int
    d_qk: int
    d_v: int
    causal: bool
    seed: int
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    def lengths(self):
        gen = torch.Generator(device="cpu")
        gen.manual_seed(self.seed)
        return [int(x) for x in torch.randint(self.min_len, self.max_len + 1, (self.n_seq,), generator=gen)]

    def flops(self) -> float:
        f = sum(2.0 * self.hq * n * n * (self.d_qk + self.d_v) for n in self.lengths())
        return f / 2.0 if self.causal else f

    def make_qkv(self):
        total = sum(self.lengths())
        q = make_random((total, self.hq, self.d_qk), self.seed + 1)
        k = make_random((total, self.hk, self.d_qk), self.seed + 2)
        v = make_random((total, self.hk, self.d_v), self.seed + 3)
        return q, k, v


# Packed-sequence prefill: 32 sequences of 512..8192 tokens, Llama-like GQA heads.
VARLEN_WORKLOADS = {
    "varlen_gqa_d128_causal": VarlenWorkload(
        "varlen_gqa_d128_causal", n_seq=32, min_len=512, max_len=8192, hq=32, hk=8, d_qk=128, d_v=128,
        causal=True, seed=110,
        description="32 packed sequences of 512..8192 tokens, hq32 hk8 d128 causal bf16"),
}
