"""Sliding-window attention with attention sinks (float64).  Test infrastructure only.

Source: "Tune MHA config & small-head pipeline pathology" (ROCm aiter PR 4414),
Test Result section: the tuned shape set includes the model_shapes.json MHA
entries of GPT-OSS, tagged "sink+sliding-window".  The page names the two
features but not their definition; the readings taken here are those of the
public GPT-OSS attention layer:

  * window: query i sees key j iff  j >= i - window_left  (window_left >= 0)
    and  j <= i + window_right  (window_right >= 0), on top of the causal rule;
    -1 leaves that side unbounded (GPT-OSS's 128-token window is
    window_left = 127 with causal masking);
  * sink: one logit per query head, in the units of the scaled scores, that
    joins every row's softmax normaliser without contributing a value row:

        m   = max(max_{j in J_i} s_j, sink_h)
        O_i = sum_{j in J_i} exp(s_j - m) V_j / (sum_{j in J_i} exp(s_j - m) + exp(sink_h - m))
        LSE = m + ln(sum_{j in J_i} exp(s_j - m) + exp(sink_h - m))

    A row without visible keys gets O = 0 and LSE = sink_h (-inf without a sink).

Everything else (GQA mapping, top-left causal rule, scale) is as in
``attention.attention_forward``.
"""

from __future__ import annotations

import numpy as np


def visible_mask(rows, sk, *, causal, window_left=-1, window_right=-1):
    """Boolean [len(rows), sk]: which keys each query row sees."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(sk, dtype=np.int64)[None, :]
    vis = np.ones((i.shape[0], sk), dtype=bool)
    if causal:
        vis &= j <= i
    if window_left >= 0:
        vis &= j >= i - window_left
    if window_right >= 0:
        vis &= j <= i + window_right
    return vis


def visible_pairs(sq, sk, *, causal, window_left=-1, window_right=-1):
    """Number of visible (query, key) pairs of one head: the unit of the algorithmic FLOP count."""
    return int(visible_mask(range(sq), sk, causal=causal, window_left=window_left,
                            window_right=window_right).sum())


def attention_window_sink(q, k, v, *, scale, causal, window_left=-1, window_right=-1, sinks=None,
                          heads=None, rows=None, batches=None):
    """Attention forward with a sliding window and per-head sink logits, float64.

    q [b, sq, hq, d_qk], k [b, sk, hk, d_qk], v [b, sk, hk, d_v] (BSHD); sinks [hq] or None.
    Returns (o [nb, nrows, nheads, d_v], lse [nb, nheads, nrows]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    b, sq, hq, _ = q.shape
    _, sk, hk, _ = k.shape
    d_v = v.shape[3]
    group = hq // hk
    heads = list(range(hq)) if heads is None else list(heads)
    rows = list(range(sq)) if rows is None else list(rows)
    batches = list(range(b)) if batches is None else list(batches)
    rows_arr = np.asarray(rows, dtype=np.int64)
    vis = visible_mask(rows_arr, sk, causal=causal, window_left=window_left, window_right=window_right)
    o = np.zeros((len(batches), len(rows), len(heads), d_v), dtype=np.float64)
    lse = np.full((len(batches), len(heads), len(rows)), -np.inf, dtype=np.float64)
    for bi, bb in enumerate(batches):
        for hi, h in enumerate(heads):
            g = h // group
            s = scale * (q[bb, rows_arr, h, :].astype(np.float64) @ k[bb, :, g, :].astype(np.float64).T)
            s = np.where(vis, s, -np.inf)                                       # [nrows, sk]
            sink = -np.inf if sinks is None else float(sinks[h])
            m = np.maximum(s.max(axis=1, initial=-np.inf), sink)               # [nrows]
            alive = np.isfinite(m)
            m_safe = np.where(alive, m, 0.0)
            p = np.exp(s - m_safe[:, None])
            denom = p.sum(axis=1) + np.exp(sink - m_safe)
            out = (p @ v[bb, :, g, :].astype(np.float64)) / np.where(alive, denom, 1.0)[:, None]
            out[~alive] = 0.0
            o[bi, :, hi, :] = out
            lse[bi, hi, :] = np.where(alive, m_safe + np.log(np.where(alive, denom, 1.0)), -np.inf)
    return o, lse


def attention_varlen_window_sink(q, k, v, cu_q, cu_k, *, scale, causal, window_left=-1, window_right=-1,
                                 sinks=None, heads=None, rows=None):
    """``attention_window_sink`` over packed sequences (THD tensors, b + 1 offsets per axis): each
    sequence attends to its own keys, window positions counted inside the sequence.

    Returns (o [nrows, nheads, d_v], lse [nheads, nrows]), both float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    total_q, hq, _ = q.shape
    d_v = v.shape[2]
    heads = list(range(hq)) if heads is None else list(heads)
    rows = list(range(total_q)) if rows is None else list(rows)
    o = np.zeros((len(rows), len(heads), d_v), dtype=np.float64)
    lse = np.full((len(heads), len(rows)), -np.inf, dtype=np.float64)
    for i in range(len(cu_q) - 1):
        qa, qe, ka, ke = cu_q[i], cu_q[i + 1], cu_k[i], cu_k[i + 1]
        sel = [n for n, r in enumerate(rows) if qa <= r < qe]
        if not sel:
            continue
        oi, li = attention_window_sink(q[None, qa:qe], k[None, ka:ke], v[None, ka:ke], scale=scale, causal=causal,
                                       window_left=window_left, window_right=window_right, sinks=sinks,
                                       heads=heads, rows=[rows[n] - qa for n in sel])
        o[sel] = oi[0]
        lse[:, sel] = li[0]
    return o, lse
