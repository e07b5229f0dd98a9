"""Attention forward oracle (float64).  Test infrastructure only.

Computes, for every batch b, query head h and query row i,

    kv head        g   = h // (hq // hk)                       (grouped-query mapping)
    visible keys   J_i = {0..sk-1}, or {j <= i} when causal     (top-left causal mask)
    scores         s_j = scale * sum_c Q[b,i,h,c] * K[b,j,g,c]  for j in J_i
    O[b,i,h,:]     = sum_j exp(s_j - m) V[b,j,g,:] / sum_j exp(s_j - m),  m = max_j s_j
    LSE[b,h,i]     = m + ln(sum_j exp(s_j - m))                 (natural log)

This is the "forward pass" of the fused MHA kernel whose configs are tuned on
"Tune MHA config & small-head pipeline pathology" (Motivation: causal "c1"
and non-causal "c0" shapes; Test Plan: GQA 48:8 and head-dim 64 shapes, the
dqk=192 / dv=128 MLA-prefill "PE" shapes).  The pages print no formula; the
readings taken where they are silent are: consecutive GQA grouping, top-left
causal alignment, natural-log LSE of layout [b, hq, sq].  A row with no
visible key (only possible when sk == 0) gets O = 0 and LSE = -inf.

Inputs are arrays of any floating dtype (bfloat16 tensors are widened to
float32 by the caller, which is exact); everything here runs in float64.
"""

from __future__ import annotations

import numpy as np


def attention_forward(q, k, v, *, scale, causal, heads=None, rows=None, batches=None):
    """Plain attention forward in float64.

    q: [b, sq, hq, d_qk], k: [b, sk, hk, d_qk], v: [b, sk, hk, d_v] (BSHD).
    heads / rows / batches: optional index lists that restrict which outputs
    are computed (each selected output is computed exactly as defined above;
    selecting rows does not change any other row's value).

    Returns (o, lse): o [nb, nrows, nheads, d_v] float64 and
    lse [nb, nheads, nrows] float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    b, sq, hq, d_qk = q.shape
    bk, sk, hk, d_qk2 = k.shape
    bv, sk2, hk2, d_v = v.shape
    if not (b == bk == bv and sk == sk2 and hk == hk2 and d_qk == d_qk2):
        raise ValueError("inconsistent q/k/v shapes")
    if hk == 0 or hq % hk != 0:
        raise ValueError("hq must be a multiple of hk")
    group = hq // hk
    heads = list(range(hq)) if heads is None else list(heads)
    rows = list(range(sq)) if rows is None else list(rows)
    batches = list(range(b)) if batches is None else list(batches)
    rows_arr = np.asarray(rows, dtype=np.int64)

    o = np.zeros((len(batches), len(rows), len(heads), d_v), dtype=np.float64)
    lse = np.full((len(batches), len(heads), len(rows)), -np.inf, dtype=np.float64)
    if len(rows) == 0 or sk == 0:
        return o, lse

    key_idx = np.arange(sk, dtype=np.int64)
    visible = np.ones((len(rows), sk), dtype=bool)
    if causal:
        visible = key_idx[None, :] <= rows_arr[:, None]

    for bi, bb in enumerate(batches):
        for hi, h in enumerate(heads):
            g = h // group
            qh = q[bb, rows_arr, h, :].astype(np.float64)        # [nrows, d_qk]
            kg = k[bb, :, g, :].astype(np.float64)               # [sk, d_qk]
            vg = v[bb, :, g, :].astype(np.float64)               # [sk, d_v]
            s = scale * (qh @ kg.T)                              # [nrows, sk]
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1)                                    # [nrows]
            has_key = np.isfinite(m)
            m_safe = np.where(has_key, m, 0.0)
            p = np.exp(s - m_safe[:, None])                      # exp(-inf) = 0 on masked keys
            l = p.sum(axis=1)
            out = (p @ vg) / np.where(has_key, l, 1.0)[:, None]
            out[~has_key] = 0.0
            o[bi, :, hi, :] = out
            with np.errstate(divide="ignore"):
                lse[bi, hi, :] = np.where(has_key, m_safe + np.log(np.where(has_key, l, 1.0)), -np.inf)
    return o, lse


def attention_varlen(q, k, v, cu_q, cu_k, *, scale, causal, heads=None, rows=None):
    """Attention forward over packed sequences (the "varlen" layout), float64.

    q: [total_q, hq, d_qk], k: [total_k, hk, d_qk], v: [total_k, hk, d_v] (THD);
    cu_q, cu_k: b + 1 offsets; sequence i owns query tokens cu_q[i]..cu_q[i+1]-1
    and key tokens cu_k[i]..cu_k[i+1]-1, and its rows attend to its own keys only,
    exactly as ``attention_forward`` on that sequence alone (top-left causal
    mask in the sequence's own positions).  heads / rows: optional index lists
    (rows index the packed token axis).

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
        local = [rows[n] - qa for n in sel]
        oi, li = attention_forward(q[None, qa:qe], k[None, ka:ke], v[None, ka:ke], scale=scale,
                                   causal=causal, heads=heads, rows=local)
        o[sel] = oi[0]
        lse[:, sel] = li[0]
    return o, lse
