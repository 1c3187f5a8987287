"""Pins for the sparse-MLA oracle: torch's scaled_dot_product_attention in
float64 with a boolean mask equal to the selected set (dense masked attention,
a library routine), the full-cache case, scipy's logsumexp, and closed forms
(one slot, equal scores, permutation invariance, the value = first 512)."""

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle.sparse_mla import sparse_mla
from oracle.quant import Bf16Cache


class _F64Cache:
    def __init__(self, rows):
        self.rows_ = np.asarray(rows, np.float64)

    def rows(self, s):
        return self.rows_[np.asarray(s, np.int64)]


def _rand(T=3, H=4, S=300, seed=0):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(T, H, 576)), rng.normal(size=(S, 576)), rng


def test_against_sdpa_with_selected_set_mask():
    q, kv, rng = _rand()
    T, H, _ = q.shape
    S = kv.shape[0]
    idx = np.full((T, 64), -1, np.int64)
    for t in range(T):
        idx[t, :40 + t] = rng.choice(S, size=40 + t, replace=False)
    scale = 1 / np.sqrt(192)
    o, lse = sparse_mla(q, _F64Cache(kv), idx, scale)
    mask = np.zeros((T, 1, 1, S), bool)
    for t in range(T):
        mask[t, 0, 0, idx[t][idx[t] >= 0]] = True
    qt = torch.from_numpy(q).unsqueeze(2)                        # [T, H, 1, 576]
    k = torch.from_numpy(kv).expand(T, 1, S, 576).expand(T, H, S, 576)
    v = torch.from_numpy(kv[:, :512]).expand(T, H, S, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, k, v, attn_mask=torch.from_numpy(mask).expand(T, H, 1, S), scale=scale)
    np.testing.assert_allclose(o, ref[:, :, 0].numpy(), rtol=1e-10, atol=1e-12)
    s = scale * np.einsum("thd,sd->ths", q, kv)
    s = np.where(mask[:, 0], s, -np.inf)
    np.testing.assert_allclose(lse, logsumexp(s, axis=-1), rtol=1e-12)


def test_short_rows_equal_full_dense_attention():
    # L <= topk: the selection is every position, i.e. plain attention over
    # the request's whole cache
    q, kv, _ = _rand(T=1, H=2, S=100, seed=1)
    idx = np.arange(128)[None, :].copy()
    idx[0, 100:] = -1
    o, _ = sparse_mla(q, _F64Cache(kv), idx, 0.1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None], torch.from_numpy(kv)[None, None],
        torch.from_numpy(kv[:, :512])[None, None], scale=0.1)
    np.testing.assert_allclose(o, ref[:, :, 0].numpy(), rtol=1e-10, atol=1e-12)


def test_single_slot_and_equal_scores():
    q, kv, _ = _rand(T=2, H=3, S=50, seed=2)
    idx = np.full((2, 8), -1)
    idx[0, 0] = 17
    o, lse = sparse_mla(q, _F64Cache(kv), idx, 0.3)
    np.testing.assert_array_equal(o[0], np.broadcast_to(kv[17, :512], (3, 512)))
    np.testing.assert_allclose(lse[0], 0.3 * q[0] @ kv[17], rtol=1e-14)
    assert (o[1] == 0).all() and np.isneginf(lse[1]).all()      # empty row
    # q = 0: all scores equal -> mean of the selected values, lse = log n
    idx2 = np.array([[3, 9, 11, -1, 40]])
    o2, lse2 = sparse_mla(np.zeros((1, 2, 576)), _F64Cache(kv), idx2, 1.0)
    np.testing.assert_allclose(o2[0, 0], kv[[3, 9, 11, 40], :512].mean(0), rtol=1e-13)
    np.testing.assert_allclose(lse2, np.log(4), rtol=1e-14)


def test_permutation_invariance_and_seqlen_prefix():
    q, kv, rng = _rand(T=1, H=2, S=80, seed=3)
    sel = rng.choice(80, 30, replace=False)
    idx = np.concatenate([sel, -np.ones(10, int)])[None]
    o1, l1 = sparse_mla(q, _F64Cache(kv), idx, 0.2)
    o2, l2 = sparse_mla(q, _F64Cache(kv), idx[:, rng.permutation(40)], 0.2)
    np.testing.assert_allclose(o1, o2, rtol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)
    # nsa_cache_seqlens limits the row to its first entries
    o3, _ = sparse_mla(q, _F64Cache(kv), idx, 0.2, nsa_cache_seqlens=[5])
    o4, _ = sparse_mla(q, _F64Cache(kv), idx[:, :5], 0.2)
    np.testing.assert_array_equal(o3, o4)


def test_bf16_cache_rows():
    x = torch.randn(10, 576, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    c = Bf16Cache(bits)
    np.testing.assert_array_equal(c.rows([3, 7]), x[[3, 7]].to(torch.float64).numpy())
