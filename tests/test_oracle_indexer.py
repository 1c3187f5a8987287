"""Pins for the indexer oracle. The scoring formula is a reading (the pages do
not show the indexer); these pin the oracle's implementation of it with
closed forms built so that a wrong page/offset, a misplaced ReLU, a dropped
scale or weight, or a transposed operand each give a different value."""

import numpy as np

from oracle import indexer as I
from oracle.formats import e4m3_encode_rne_sat


def _pack_fp32_pages(keys, scales):
    n = keys.shape[0]
    kb = keys.astype("<f4").reshape(n, -1).view(np.uint8)
    sb = scales.astype("<f4").reshape(n, -1).view(np.uint8)
    return np.concatenate([kb, sb], axis=1)


def test_page_decode_layout_fp8():
    # one page: key codes row-major [64, 8], then 64 fp32 scales
    di = 8
    codes = np.zeros((1, 64 * di), np.uint8)
    codes[0, 5 * di + 3] = 0x38          # token 5, dim 3 = 1.0
    codes[0, 63 * di + 7] = 0x7E         # token 63, dim 7 = 448
    sc = np.arange(64, dtype="<f4").reshape(1, 64)
    raw = np.concatenate([codes, sc.view(np.uint8)], axis=1)
    assert raw.shape[1] == I.index_page_bytes(di, I.KIND_FP8)
    keys, scales = I.decode_index_pages(raw, di, I.KIND_FP8)
    assert keys[0, 5, 3] == 1.0 and keys[0, 63, 7] == 448.0
    assert keys.sum() == 449.0
    np.testing.assert_array_equal(scales[0], np.arange(64))


def _onehot_setup(L, hit, di=4, seed=0):
    """Single head, w = 1, q = e_2; the key at logical position ``hit`` is
    e_2 and every other key is e_0. Pages are in a shuffled physical order."""
    rng = np.random.default_rng(seed)
    npages = (L + 63) // 64
    phys = rng.permutation(npages + 2)[:npages]           # logical -> physical
    keys = np.zeros((npages + 2, 64, di))
    keys[:, :, 0] = 1.0
    scales = rng.uniform(0.5, 2.0, (npages + 2, 64))
    p, o = phys[hit // 64], hit % 64
    keys[p, o, 0] = 0.0
    keys[p, o, 2] = 1.0
    q = np.zeros((1, 1, di))
    q[0, 0, 2] = 1.0
    return q, keys, scales, phys[None, :], (p, o)


def test_onehot_closed_form_through_shuffled_pages():
    L, hit = 200, 131
    q, keys, scales, rpt, (p, o) = _onehot_setup(L, hit)
    out = I.indexer_logits(q, np.ones((1, 1)), keys, scales, rpt, [0], [L], 256)
    expect = np.zeros(L)
    expect[hit] = scales[p, o]
    np.testing.assert_array_equal(out[0, :L], expect)
    assert np.isneginf(out[0, L:]).all()


def test_relu_is_per_head_before_weighting():
    # two heads with dots +2 and +3 (weights 1, -1) -> 2 - 3 = -1;
    # negative dots are cut per head: dots -2 and +3 with weights (1, 1) -> 3
    di = 2
    keys = np.zeros((1, 64, di))
    keys[0, :, 0] = 1.0
    scales = np.ones((1, 64))
    q = np.array([[[2.0, 0.0], [3.0, 0.0]]])
    out = I.indexer_logits(q, np.array([[1.0, -1.0]]), keys, scales,
                           np.zeros((1, 1), int), [0], [10], 10)
    np.testing.assert_array_equal(out[0], -1.0)
    q2 = np.array([[[-2.0, 0.0], [3.0, 0.0]]])
    out2 = I.indexer_logits(q2, np.array([[1.0, 1.0]]), keys, scales,
                            np.zeros((1, 1), int), [0], [10], 10)
    np.testing.assert_array_equal(out2[0], 3.0)


def test_all_negative_dots_give_exact_zero_row():
    rng = np.random.default_rng(3)
    di, hi = 16, 8
    keys = np.abs(rng.normal(size=(3, 64, di)))
    scales = rng.uniform(0.5, 1.5, (3, 64))
    q = -np.abs(rng.normal(size=(1, hi, di)))
    out = I.indexer_logits(q, rng.uniform(size=(1, hi)), keys, scales,
                           np.array([[2, 0, 1]]), [0], [150], 192)
    assert (out[0, :150] == 0.0).all()


def test_scale_and_weight_linearity_and_head_sum():
    rng = np.random.default_rng(4)
    di, hi, L = 8, 5, 100
    keys = rng.normal(size=(2, 64, di))
    scales = rng.uniform(0.5, 1.5, (2, 64))
    q = rng.normal(size=(1, hi, di))
    w = rng.uniform(size=(1, hi))
    rpt = np.array([[1, 0]])
    base = I.indexer_logits(q, w, keys, scales, rpt, [0], [L], L)
    # doubling every key scale doubles the logits
    dbl = I.indexer_logits(q, w, keys, 2 * scales, rpt, [0], [L], L)
    np.testing.assert_allclose(dbl, 2 * base, rtol=0, atol=0)
    # the logit is the sum over heads of single-head logits
    per_head = sum(I.indexer_logits(q[:, h:h + 1], w[:, h:h + 1], keys, scales,
                                    rpt, [0], [L], L) for h in range(hi))
    np.testing.assert_allclose(per_head, base, rtol=1e-12, atol=1e-12)


def test_rows_share_request_tables_and_lengths_clip():
    # rows 0 and 1 belong to request 1; row 2 to request 0; lengths differ
    rng = np.random.default_rng(5)
    di = 4
    keys = rng.normal(size=(6, 64, di))
    scales = rng.uniform(0.5, 1.5, (6, 64))
    q = rng.normal(size=(3, 2, di))
    w = rng.uniform(size=(3, 2))
    rpt = np.array([[0, 1, 2], [5, 4, 3]])
    out = I.indexer_logits(q, w, keys, scales, rpt, [1, 1, 0], [70, 500, 130],
                           150)
    assert np.isneginf(out[0, 70:]).all() and np.isfinite(out[0, :70]).all()
    assert np.isfinite(out[1]).all()               # clipped to max_seqlen_k
    # row 1 position 65 reads physical page 4, offset 1
    k = keys[4, 1]
    expect = scales[4, 1] * (w[1] @ np.maximum(q[1] @ k, 0))
    assert abs(out[1, 65] - expect) < 1e-12


def test_fp8_codes_decode_into_logits():
    # fp8 page built from exact values; logits equal the fp32-page result
    rng = np.random.default_rng(6)
    di = 8
    vals = rng.choice([-2.0, -0.5, 0.0, 0.25, 1.0, 3.0], size=(1, 64, di))
    codes = e4m3_encode_rne_sat(vals).reshape(1, -1)
    sc = rng.uniform(0.5, 1.5, (1, 64)).astype("<f4")
    raw8 = np.concatenate([codes, sc.view(np.uint8)], axis=1)
    raw32 = _pack_fp32_pages(vals, sc)
    k8, s8 = I.decode_index_pages(raw8, di, I.KIND_FP8)
    k32, s32 = I.decode_index_pages(raw32, di, I.KIND_FP32)
    np.testing.assert_array_equal(k8, k32)
    np.testing.assert_array_equal(s8, s32)
