"""CPU reference ("oracle") for the attention forward path. TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy code that states what the GPU library computes, so
the tests can check the library element by element.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library (``head_attention_forward_flash_amd``) never does, and
the oracle imports nothing from the library.  The two share no code: the only
common module is ``workloads.py``, which draws seeded random inputs and holds
none of the arithmetic.

Sources (web pages; cited by title and section):
  * "Tune MHA config & small-head pipeline pathology" (ROCm aiter PR 4414):
    the fused MHA forward pass and its shape families (Motivation, Technical
    Details, Test Plan, Profile 1 and Profile 2).
  * "[HIP] Mha v4: run the K-smoothing gate as one HIP call" (ROCm aiter
    PR 7754): the per-head K mean and its gate (Summary, PR-specific
    question, commit message).
  * "MHA v4: fixes, refactor, new kernel, perf tweaks" (ROCm aiter PR 5335):
    the BF16/FP8 recipe of mha_v4 (Motivation, Kernels list) and its MX
    descales (review comments).
  * OCP Microscaling Formats (MX) v1.0: the MXFP8 block format that the pages
    name but do not define.

Modules:
  attention  - softmax(scale * Q K^T + causal mask) V with GQA, and the
               per-row log-sum-exp (plain definition); the same over packed
               sequences of different lengths (varlen).
  gate       - K-smoothing gate: strided key sample, per-channel moments,
               gate decision, mean output (the algorithm's steps).
  fp8        - OCP E4M3 rounding, per-128-token-block scaling, and attention
               on the dequantised, smoothed tensors (the algorithm's steps).
  mx         - MXFP8: E4M3 elements with one E8M0 exponent per 32 channels,
               and attention on the dequantised, smoothed tensors.
  window     - sliding-window attention with per-head sink logits (plain
               definition).

Every function is pinned by a ``-m "not gpu"`` test against facts fixed
outside this package: closed forms, hand-derived examples under
``tests/golden/``, library routines (torch's CPU scaled_dot_product_attention,
torch's float8_e4m3fn cast, numpy's mean/var) and brute force.
"""

from .attention import attention_forward, attention_varlen  # noqa: F401
from .gate import k_smooth_mean, key_sample  # noqa: F401
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_round,
    e4m3_encode,
    e4m3_decode,
    quantize_blocks,
    fp8_attention_forward,
)
from .mx import mx_quantize, mx_dequantize, mxfp8_attention_forward  # noqa: F401
from .window import attention_window_sink, attention_varlen_window_sink, visible_mask, visible_pairs  # noqa: F401
