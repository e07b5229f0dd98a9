"""K-smoothing gate oracle (float64).  Test infrastructure only.

Source: "[HIP] Mha v4: run the K-smoothing gate as one HIP call" (ROCm aiter
PR 7754).  Summary: every quantised mha_v4 call evaluates a gate on a per-head
K mean.  Commit message: the statistic is taken over a strided sample of the
key axis ("mean/sum reductions over the strided key axis"), as per-(batch*head)
moments followed by a per-head fold and a threshold ("same definition, same
threshold").  Changed op tests: both gate outcomes, partial and strided
samples.

The pages never write the statistic down.  The reading taken here:

  1. sample keys j_t = t * key_stride, t = 0..T-1,
     T = ceil(sk / key_stride), capped at max_keys when max_keys > 0;
  2. per (b, kv head, channel c): mu_c = mean_t K[b, j_t, g, c] and
     var_c = mean_t (K[b, j_t, g, c] - mu_c)^2;
  3. r = sqrt(sum_c mu_c^2 / sum_c var_c)  (r = +inf when the variance sum is 0
     and the mean sum is not, r = 0 when both are 0);
  4. the gate is open iff r > tau; the returned mean is mu where open and
     exactly 0 where closed.

The moments are taken in float64 from K widened exactly; T = 0 (sk == 0)
gives mu = 0, var = 0, r = 0, closed.
"""

from __future__ import annotations

import math

import numpy as np


def key_sample(sk: int, key_stride: int, max_keys: int = 0) -> np.ndarray:
    """Indices of the sampled keys: 0, key_stride, 2*key_stride, ... (at most max_keys if > 0)."""
    if key_stride < 1:
        raise ValueError("key_stride must be >= 1")
    count = (sk + key_stride - 1) // key_stride if sk > 0 else 0
    if max_keys > 0:
        count = min(count, max_keys)
    return np.arange(count, dtype=np.int64) * key_stride


def k_smooth_mean(k, *, key_stride: int = 1, max_keys: int = 0, tau: float = 0.25):
    """Gate statistics for K of layout [b, sk, hk, d].

    Returns a dict with float64 arrays ``mu`` [b, hk, d], ``var`` [b, hk, d],
    ``ratio`` [b, hk], boolean ``open`` [b, hk], ``mean`` [b, hk, d] (mu where
    open, zeros where closed) and the sample size ``T``.
    """
    k = np.asarray(k)
    b, sk, hk, d = k.shape
    idx = key_sample(sk, key_stride, max_keys)
    t = len(idx)
    mu = np.zeros((b, hk, d), dtype=np.float64)
    var = np.zeros((b, hk, d), dtype=np.float64)
    if t > 0:
        x = k[:, idx, :, :].astype(np.float64)          # [b, T, hk, d]
        mu = x.mean(axis=1)                               # [b, hk, d]
        var = ((x - mu[:, None, :, :]) ** 2).mean(axis=1)
    num = (mu ** 2).sum(axis=2)                           # [b, hk]
    den = var.sum(axis=2)
    ratio = np.zeros((b, hk), dtype=np.float64)
    for bi in range(b):
        for g in range(hk):
            if den[bi, g] > 0.0:
                ratio[bi, g] = math.sqrt(num[bi, g] / den[bi, g])
            else:
                ratio[bi, g] = math.inf if num[bi, g] > 0.0 else 0.0
    gate_open = ratio > tau
    mean = np.where(gate_open[:, :, None], mu, 0.0)
    return {"mu": mu, "var": var, "ratio": ratio, "open": gate_open, "mean": mean, "T": t}
