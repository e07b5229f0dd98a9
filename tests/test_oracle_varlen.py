"""Pins of the packed-sequence (varlen) oracle against an independent formulation.

The oracle runs each sequence on its own.  The pin instead runs ONE float64 attention over
the whole packed token axis with torch's CPU scaled_dot_product_attention and an explicit
boolean mask that allows exactly the (query, key) pairs of the same sequence (and, when
causal, key position <= query position inside that sequence).  A dropped offset, a key
range taken from the query offsets, a mask that is causal in packed rather than local
positions, or a wrong GQA group all make the two disagree.
"""

import numpy as np
import pytest
import torch

from oracle import attention_forward, attention_varlen


def _packed(lens_q, lens_k, hq, hk, dqk, dv, seed):
    g = torch.Generator().manual_seed(seed)
    tq, tk = sum(lens_q), sum(lens_k)
    q = torch.randn((tq, hq, dqk), generator=g, dtype=torch.float64)
    k = torch.randn((tk, hk, dqk), generator=g, dtype=torch.float64)
    v = torch.randn((tk, hk, dv), generator=g, dtype=torch.float64)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(int)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(int)
    return q, k, v, cu_q, cu_k


def _masked_sdpa(q, k, v, cu_q, cu_k, scale, causal):
    tq, hq, _ = q.shape
    tk, hk, _ = k.shape
    allow = torch.zeros((tq, tk), dtype=torch.bool)
    for i in range(len(cu_q) - 1):
        qa, qe, ka, ke = cu_q[i], cu_q[i + 1], cu_k[i], cu_k[i + 1]
        blk = torch.ones((qe - qa, ke - ka), dtype=torch.bool)
        if causal:
            blk = torch.tril(blk)
        allow[qa:qe, ka:ke] = blk
    kk = k.repeat_interleave(hq // hk, dim=1)
    vv = v.repeat_interleave(hq // hk, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2)[None], kk.permute(1, 0, 2)[None], vv.permute(1, 0, 2)[None],
        attn_mask=allow, scale=scale)[0].permute(1, 0, 2)
    s = torch.einsum("qhd,khd->hqk", q, kk) * scale
    s = s.masked_fill(~allow[None], float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy(), allow.any(dim=1).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", [
    ([5, 1, 17, 9], [5, 1, 17, 9], 4, 2),      # equal lengths, GQA 2:1
    ([7, 12, 3], [11, 4, 20], 3, 1),           # sq != sk per sequence, GQA 3:1
    ([16, 16], [16, 16], 2, 2),
])
def test_varlen_oracle_matches_block_diagonal_mask(case, causal):
    lens_q, lens_k, hq, hk = case
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, hq, hk, 8, 6, 41 + len(lens_q))
    scale = 0.37
    o, lse = attention_varlen(q.numpy(), k.numpy(), v.numpy(), cu_q, cu_k, scale=scale, causal=causal)
    o_ref, lse_ref, has = _masked_sdpa(q, k, v, cu_q, cu_k, scale, causal)
    np.testing.assert_allclose(o[has], o_ref[has], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse[:, has], lse_ref[:, has], rtol=1e-11, atol=1e-12)


def test_varlen_empty_key_ranges_and_sampling():
    # sequence 1 has no keys: its rows are O = 0, LSE = -inf; a zero-length query range is skipped
    q, k, v, cu_q, cu_k = _packed([4, 3, 0, 5], [6, 0, 2, 5], 2, 1, 8, 8, 77)
    o, lse = attention_varlen(q.numpy(), k.numpy(), v.numpy(), cu_q, cu_k, scale=0.5, causal=False)
    assert np.all(o[4:7] == 0) and np.all(np.isneginf(lse[:, 4:7]))
    o_ref, lse_ref, has = _masked_sdpa(q, k, v, cu_q, cu_k, 0.5, False)
    np.testing.assert_allclose(o[has], o_ref[has], rtol=1e-11, atol=1e-12)
    # sampled rows and heads equal the full result's entries (up to BLAS summation order)
    rows, heads = [11, 0, 5, 8], [1]
    os_, ls_ = attention_varlen(q.numpy(), k.numpy(), v.numpy(), cu_q, cu_k, scale=0.5, causal=False,
                                heads=heads, rows=rows)
    np.testing.assert_allclose(os_, o[rows][:, heads], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ls_, lse[heads][:, rows], rtol=1e-13, atol=1e-14)


def test_varlen_single_sequence_is_dense():
    q, k, v, cu_q, cu_k = _packed([37], [37], 4, 2, 8, 8, 5)
    o, lse = attention_varlen(q.numpy(), k.numpy(), v.numpy(), cu_q, cu_k, scale=0.3, causal=True)
    od, ld = attention_forward(q.numpy()[None], k.numpy()[None], v.numpy()[None], scale=0.3, causal=True)
    np.testing.assert_array_equal(o, od[0])
    np.testing.assert_array_equal(lse, ld[0])
