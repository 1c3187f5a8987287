"""GPU parity: nsa_topk_transform (exact selection on oracle-made logits;
acceptance on the GPU's own logits) and nsa_sparse_mla_decode / _extend
(against the oracle given identical indices)."""

import numpy as np
import pytest
import torch

import oracle
from helpers import (DEV, need_gpu, note, check_topk_row, check_attention,
                     CacheFromRows, host_key_hist)

pytestmark = pytest.mark.gpu


def _topk_rows(rng, lengths, width, kind):
    x = np.full((len(lengths), width), np.nan, np.float32)   # unwritten tail
    for t, L in enumerate(lengths):
        if kind == "normal":
            x[t, :L] = rng.normal(size=L) * 20 + 40
        elif kind == "ties":
            x[t, :L] = rng.integers(0, 7, size=L).astype(np.float32)
        elif kind == "const":
            x[t, :L] = 3.0
        elif kind == "special":
            v = rng.normal(size=L).astype(np.float32)
            v[rng.random(L) < 0.05] = -np.inf
            v[rng.random(L) < 0.05] = np.nan
            v[rng.random(L) < 0.01] = np.inf
            v[rng.random(L) < 0.1] = -0.0
            x[t, :L] = v
        elif kind == "neg_inf_heavy":   # threshold in the -inf / NaN bins
            v = rng.normal(size=L).astype(np.float32)
            r = rng.random(L)
            v[r < 0.97] = -np.inf
            v[r < 0.02] = np.nan
            x[t, :L] = v
        elif kind == "pos_inf_heavy":   # threshold in the +inf bin
            v = rng.normal(size=L).astype(np.float32)
            v[rng.random(L) < 0.3] = np.inf
            x[t, :L] = v
    return x


KINDS = ["normal", "ties", "const", "special", "neg_inf_heavy", "pos_inf_heavy"]
# row lengths around the edges of the select: rows of at most topk, the
# 16384-position histogram chunks, 1..3 positions past the last vector; the
# "short" set keeps the row width (max_seqlen_k) within 65536 positions and
# is repeated to 516 rows (the select's short-row variant, used for batches of
# at least 512 such rows); repeated rows must equal their first copy
LENGTHS = {
    "long": lambda k: [0, 1, k - 1, k, k + 1, 3 * k + 5, 20000, 131072 - 3,
                       16384, 16385, 32768 + 11],
    "short": lambda k: [0, 1, k - 1, k, k + 1, 3 * k + 5, 20000, 65536 - 131,
                        16384, 16385, 32768 + 11, 65536 - 192],
}
SHORT_ROWS = 516


def _tile_rows(x, lengths, span):
    if span != "short":
        return x, lengths
    reps = -(-SHORT_ROWS // len(lengths))
    return np.tile(x, (reps, 1))[:SHORT_ROWS], (lengths * reps)[:SHORT_ROWS]


def _check_repeats(got, n0):
    for t in range(n0, len(got)):
        np.testing.assert_array_equal(got[t], got[t % n0], err_msg=f"repeated row {t}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("topk", [256, 2048, 8192])
@pytest.mark.parametrize("pad", [6, 67])   # odd row stride: scalar loads; else vector
@pytest.mark.parametrize("span", ["long", "short"])
def test_topk_exact_on_given_logits(kind, topk, pad, span):
    nsa = need_gpu()
    note(f"topk exact {kind} topk={topk} pad={pad} {span}")
    rng = np.random.default_rng(topk)
    lengths = LENGTHS[span](topk)
    n0 = len(lengths)
    width = max(lengths) + pad
    x = _topk_rows(rng, lengths, width, kind)
    xt, lt = _tile_rows(x, lengths, span)
    lg = torch.as_tensor(xt, device=DEV)
    ln = torch.as_tensor(lt, dtype=torch.int32, device=DEV)
    got = nsa.nsa_topk_transform(lg, ln, topk, width).cpu().numpy()
    _check_repeats(got, n0)
    for t, L in enumerate(lengths):
        sel = got[t]
        check_topk_row(sel, L, topk, what=f"row {t}")
        # both sides break ties by position and rank NaN lowest: equal sets
        want = oracle.topk.topk_row(x[t].astype(np.float64), L, topk)
        want = np.sort(want[want >= 0])
        np.testing.assert_array_equal(sel[:len(want)], want, err_msg=f"row {t} L={L}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("pad", [6, 67])
@pytest.mark.parametrize("span,split", [("long", True), ("long", False), ("short", True)])
def test_topk_with_histogram_exact_on_given_logits(kind, pad, span, split):
    # the select that takes the indexer's row histograms (here the histogram
    # of the same logits, computed on the host from its definition): each
    # row equals the oracle's set, and the histogram is left zero. "long"
    # rows run both the split select (rows over 16384 positions classified
    # by many blocks, through a workspace) and the one-block-per-row select
    nsa = need_gpu()
    topk = 2048
    note(f"topk with histogram {kind} pad={pad} {span} split={split}")
    rng = np.random.default_rng(7)
    lengths = LENGTHS[span](topk)
    n0 = len(lengths)
    width = max(lengths) + pad
    x = _topk_rows(rng, lengths, width, kind)
    kh_host = np.stack([host_key_hist(x[t], L) for t, L in enumerate(lengths)])
    xt, lt = _tile_rows(x, lengths, span)
    kh_host, _ = _tile_rows(kh_host, lengths, span)
    kh = torch.as_tensor(kh_host.astype(np.uint32).view(np.int32), device=DEV)
    lg = torch.as_tensor(xt, device=DEV)
    ln = torch.as_tensor(lt, dtype=torch.int32, device=DEV)
    got = nsa.nsa_topk_transform(lg, ln, topk, width, key_hist=kh,
                                 split=split).cpu().numpy()
    assert int(kh.abs().sum()) == 0
    _check_repeats(got, n0)
    for t, L in enumerate(lengths):
        sel = got[t]
        check_topk_row(sel, L, topk, what=f"row {t}")
        want = oracle.topk.topk_row(x[t].astype(np.float64), L, topk)
        want = np.sort(want[want >= 0])
        np.testing.assert_array_equal(sel[:len(want)], want, err_msg=f"row {t} L={L}")


@pytest.mark.parametrize("pad", [0, 67])   # vector loads; odd stride: scalar loads
def test_topk_split_select_matches_one_block_select(pad):
    # rows around the 16384-position segments of the split select (1..3
    # positions past a segment's or the row's last whole vector, rows of at
    # most topk, one row whose histogram does not add up to its length: the
    # multi-pass select), mapped through a page table: the split select and
    # the one-block-per-row select give identical slots, equal to the
    # oracle's, also on later calls over a workspace that still holds the
    # previous call's bitmaps (and starts as garbage). The third call packs
    # 3000 keys of one threshold bin ([5, 5.5), many equal) into the first
    # segment of every row: a crowded bin, resolved among ties by position
    nsa = need_gpu()
    topk = 2048
    note(f"topk split vs one-block pad={pad}")
    rng = np.random.default_rng(11 + pad)
    lengths = [0, 2048, 2049, 16383, 16384, 16385, 16387, 32769, 49151, 65535,
               100002, 131071, 131072]
    T = len(lengths)
    width = max(lengths) + pad
    ncol = -(-width // 64)
    table_h = rng.permutation(3 * ncol)[:2 * ncol].reshape(2, ncol)
    table = torch.as_tensor(table_h, dtype=torch.int32, device=DEV)
    t2r_h = [t % 2 for t in range(T)]
    t2r = torch.as_tensor(t2r_h, dtype=torch.int32, device=DEV)
    ln = torch.as_tensor(lengths, dtype=torch.int32, device=DEV)
    need = nsa.topk_hist_workspace_size(T, width, topk)
    assert need > 0
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
    for call in range(3):
        x = _topk_rows(rng, lengths, width, ["normal", "special", "normal"][call])
        if call == 2:
            for t, L in enumerate(lengths):
                if L > 3100:
                    x[t, :L] = np.clip(rng.normal(size=L) * 0.5, -3.9, 3.9)
                    c = 5.0 + rng.integers(0, 400, size=3000) / 800.0
                    x[t, 100:3100] = c.astype(np.float32)
        kh_host = np.stack([host_key_hist(x[t], L) for t, L in enumerate(lengths)])
        kh_host[7, 4000] += 1                     # row 7: counts do not add up
        lg = torch.as_tensor(x, device=DEV)
        outs = []
        for split in (True, False):
            kh = torch.as_tensor(kh_host.astype(np.uint32).view(np.int32), device=DEV)
            outs.append(nsa.nsa_topk_transform(
                lg, ln, topk, width, table=table, token_to_req=t2r, key_hist=kh,
                workspace=ws if split else None, split=split).cpu().numpy())
            assert int(kh.abs().sum()) == 0
        np.testing.assert_array_equal(outs[0], outs[1], err_msg=f"call {call}")
        want = np.full((T, topk), -1, np.int64)
        for t, L in enumerate(lengths):
            w = oracle.topk.topk_row(x[t].astype(np.float64), L, topk)
            w = np.sort(w[w >= 0])
            want[t, :len(w)] = w
        want = oracle.transform.transform_compact(want, table_h, t2r_h)
        np.testing.assert_array_equal(outs[0], want, err_msg=f"call {call}")


def test_topk_without_logits_when_rows_fit():
    # every row holds at most topk positions (max_seqlen_k <= topk): no
    # logits are needed; each row keeps all its positions in order, mapped
    # through the page table, then -1 (with and without a histogram)
    nsa = need_gpu()
    topk, width = 256, 200
    lengths = [0, 1, 63, 64, 65, 199, 200]
    ln = torch.as_tensor(lengths, dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(3)
    table = torch.as_tensor(rng.permutation(64)[:2 * 4].reshape(2, 4), dtype=torch.int32,
                            device=DEV)
    t2r = torch.as_tensor([i % 2 for i in range(len(lengths))], dtype=torch.int32,
                          device=DEV)
    logical = nsa.nsa_topk_transform(None, ln, topk, width).cpu().numpy()
    slots = nsa.nsa_topk_transform(None, ln, topk, width, table=table,
                                   token_to_req=t2r).cpu().numpy()
    kh = nsa.new_key_hist(len(lengths), DEV)
    kh[:, 7] = 5                                   # any content: cleared, unused
    slots_h = nsa.nsa_topk_transform(None, ln, topk, width, table=table,
                                     token_to_req=t2r, key_hist=kh).cpu().numpy()
    assert int(kh.abs().sum()) == 0
    tab = table.cpu().numpy()
    for t, L in enumerate(lengths):
        want = np.full(topk, -1, np.int64)
        want[:L] = np.arange(L)
        np.testing.assert_array_equal(logical[t], want)
        want_s = np.where(want >= 0, tab[t % 2][np.maximum(want, 0) // 64] * 64 + want % 64, -1)
        np.testing.assert_array_equal(slots[t], want_s)
        np.testing.assert_array_equal(slots_h[t], want_s)


def test_topk_fused_table_and_strides():
    nsa = need_gpu()
    rng = np.random.default_rng(1)
    lengths = [5000, 100, 7000]
    width = 7040
    x = _topk_rows(rng, lengths, width, "normal")
    big = torch.zeros(3, width + 64, device=DEV)
    big[:, :width] = torch.as_tensor(x, device=DEV)
    lg = big[:, :width]                                    # row stride > width
    ln = torch.as_tensor(lengths, dtype=torch.int32, device=DEV)
    table = torch.as_tensor(rng.permutation(500)[:2 * 110].reshape(2, 110),
                            dtype=torch.int32, device=DEV)
    t2r = torch.tensor([1, 0, 1], dtype=torch.int32, device=DEV)
    logical = nsa.nsa_topk_transform(lg, ln, 2048, width).cpu().numpy()
    slots = nsa.nsa_topk_transform(lg, ln, 2048, width, table=table,
                                   token_to_req=t2r).cpu().numpy()
    want = oracle.transform.transform_compact(logical, table.cpu().numpy(), [1, 0, 1])
    np.testing.assert_array_equal(slots, want)


def _random_case(rng, T, H, topk, num_slots, kind, frac_pad=0.1):
    q = torch.randn(T, H, 576, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30))))
    q = q.to(torch.bfloat16)
    kv = torch.randn(num_slots, 576, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    bits = kv.view(torch.int16).numpy().view(np.uint16)
    if kind == "fp8":
        raw = oracle.quant.quantize_k_cache(bits)
        cache_dev = torch.as_tensor(raw, device=DEV)
        vals = oracle.quant.dequantize_rows(raw)
    else:
        cache_dev = kv.to(DEV)
        vals = oracle.formats.bf16_bits_to_f64(bits)
    idx = np.full((T, topk), -1, np.int64)
    for t in range(T):
        n = int(topk * (1 - frac_pad * rng.random()))
        idx[t, :n] = rng.choice(num_slots, size=n, replace=False)
        if t % 3 == 1:
            rng.shuffle(idx[t])       # -1 interleaved
    return q, cache_dev, vals, idx


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("T,H,topk", [(1, 16, 2048), (3, 128, 2048), (5, 64, 256),
                                      (2, 32, 100), (40, 16, 64), (4, 48, 512),
                                      # 64-head blocks: many splits, an odd last
                                      # step of a split, > 2048 slots per row
                                      (2, 128, 300), (200, 64, 96), (1, 64, 4096),
                                      # the other head counts the entry points
                                      # take, and the largest topk (8192)
                                      (3, 80, 160), (2, 96, 8192), (2, 112, 1000),
                                      (1, 128, 8192)])
def test_sparse_mla_decode(kind, T, H, topk):
    nsa = need_gpu()
    note(f"sparse_mla {kind} T={T} H={H} topk={topk}")
    rng = np.random.default_rng(T * 1000 + H + topk)
    q, cache, vals, idx = _random_case(rng, T, H, topk, max(6000, topk + 1000), kind)
    kvd = nsa.KV_FP8_656 if kind == "fp8" else nsa.KV_BF16_576
    out, lse = nsa.nsa_sparse_mla_decode(q.to(DEV), cache, kvd,
                                         torch.as_tensor(idx, dtype=torch.int32, device=DEV),
                                         0.0721)
    o_ref, lse_ref = oracle.sparse_mla.sparse_mla(q.to(torch.float64).numpy(),
                                                  CacheFromRows(dict(enumerate(vals))),
                                                  idx, 0.0721)
    check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, kind)


def test_sparse_mla_seqlens_invalid_slots_and_empty_rows():
    nsa = need_gpu()
    rng = np.random.default_rng(3)
    T, H, topk, S = 6, 16, 512, 3000
    q, cache, vals, idx = _random_case(rng, T, H, topk, S, "bf16", frac_pad=0.0)
    idx[1, :] = -1                      # empty row
    idx[2, 7] = S + 5                   # out of range: ignored
    idx[2, 9] = -7
    idx[3, 1:] = -1                     # one slot
    seqlens = np.array([topk, topk, topk, topk, 33, 0], np.int32)
    out, lse = nsa.nsa_sparse_mla_decode(
        q.to(DEV), cache, nsa.KV_BF16_576,
        torch.as_tensor(idx, dtype=torch.int32, device=DEV), 0.1,
        nsa_cache_seqlens=torch.as_tensor(seqlens, device=DEV))
    clean = np.where((idx >= 0) & (idx < S), idx, -1)
    o_ref, lse_ref = oracle.sparse_mla.sparse_mla(q.to(torch.float64).numpy(),
                                                  CacheFromRows(dict(enumerate(vals))),
                                                  clean, 0.1, nsa_cache_seqlens=seqlens)
    o = out.float().cpu().numpy()
    check_attention(o, lse.cpu().numpy(), o_ref, lse_ref, "bf16")
    assert (o[1] == 0).all() and (o[5] == 0).all()
    assert np.isneginf(lse.cpu().numpy()[[1, 5]]).all()
    np.testing.assert_allclose(o[3], np.broadcast_to(vals[idx[3, 0], :512], (H, 512)),
                               rtol=1e-2, atol=1e-2)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_sparse_mla_extend_entry(kind):
    nsa = need_gpu()
    note(f"sparse_mla extend {kind}")
    rng = np.random.default_rng(11)
    T, H, topk = 300, 16, 256
    q, cache, vals, idx = _random_case(rng, T, H, topk, 4000, kind)
    kvd = nsa.KV_FP8_656 if kind == "fp8" else nsa.KV_BF16_576
    idx_d = torch.as_tensor(idx, dtype=torch.int32, device=DEV)
    out, lse = nsa.nsa_sparse_mla_extend(q.to(DEV), cache, kvd, idx_d, 0.05)
    rows = [0, 1, 150, 299]
    o_ref, lse_ref = oracle.sparse_mla.sparse_mla(q[rows].to(torch.float64).numpy(),
                                                  CacheFromRows(dict(enumerate(vals))),
                                                  idx[rows], 0.05)
    check_attention(out.float().cpu().numpy()[rows], lse.cpu().numpy()[rows],
                    o_ref, lse_ref, kind)
    # the decode entry computes the same function
    out2, _ = nsa.nsa_sparse_mla_decode(q.to(DEV), cache, kvd, idx_d, 0.05)
    check_attention(out2.float().cpu().numpy()[rows], None, o_ref, lse_ref, kind)


def test_sparse_mla_strided_q_and_determinism():
    nsa = need_gpu()
    rng = np.random.default_rng(5)
    T, H, topk = 4, 128, 2048
    q, cache, vals, idx = _random_case(rng, T, H, topk, 5000, "bf16")
    qbig = torch.zeros(T, H, 640, dtype=torch.bfloat16)
    qbig[:, :, :576] = q
    qd = qbig.to(DEV)[:, :, :576]
    idx_d = torch.as_tensor(idx, dtype=torch.int32, device=DEV)
    a, la = nsa.nsa_sparse_mla_decode(qd, cache, nsa.KV_BF16_576, idx_d, 0.07)
    b, lb = nsa.nsa_sparse_mla_decode(q.to(DEV), cache, nsa.KV_BF16_576, idx_d, 0.07)
    assert torch.equal(a, b) and torch.equal(la, lb)
    o_ref, lse_ref = oracle.sparse_mla.sparse_mla(q.to(torch.float64).numpy(),
                                                  CacheFromRows(dict(enumerate(vals))),
                                                  idx, 0.07)
    check_attention(a.float().cpu().numpy(), la.cpu().numpy(), o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("H,T", [(64, 2), (128, 2), (128, 130)])
def test_sparse_mla_score_jump_reruns_exactly(H, T):
    """Scores of a later step far above the first step's (exp2 of the scaled
    difference, about 332, overflows fp32): the 64-head fp8 kernel, alone
    (H = 64) or as two head blocks (H = 128), and the 128-head kernel (more
    than 128 rows) must still match the oracle (they run the split or row
    again with the true maximum)."""
    nsa = need_gpu()
    topk = 64
    q = torch.ones(T, H, 576, dtype=torch.bfloat16)
    kv = torch.zeros(64, 576, dtype=torch.bfloat16)
    kv[32:] = 0.1                                    # second step: q.k = 57.6
    bits = kv.view(torch.int16).numpy().view(np.uint16)
    raw = oracle.quant.quantize_k_cache(bits)
    vals = oracle.quant.dequantize_rows(raw)
    idx = np.tile(np.arange(64), (T, 1))
    idx[1::2] = idx[1::2, ::-1]                      # large scores first
    out, lse = nsa.nsa_sparse_mla_decode(q.to(DEV), torch.as_tensor(raw, device=DEV),
                                         nsa.KV_FP8_656,
                                         torch.as_tensor(idx, dtype=torch.int32, device=DEV),
                                         4.0)
    o_ref, lse_ref = oracle.sparse_mla.sparse_mla(q.to(torch.float64).numpy(),
                                                  CacheFromRows(dict(enumerate(vals))),
                                                  idx, 4.0)
    check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "fp8")


@pytest.mark.parametrize("T,topk", [(5, 2048), (3, 100), (128, 160), (64, 2048),
                                    # more than 128 rows: one 128-head block per row
                                    (129, 2048), (200, 300), (256, 256), (300, 64),
                                    # one and two 32-slot steps per block (the
                                    # prologue alone, one loop iteration)
                                    (160, 24), (140, 40)])
def test_sparse_mla_128_heads_fp8_edges_and_determinism(T, topk):
    """128 heads over an fp8 cache, the 128-head kernel: up to 128 rows
    split over KV (2 splits at 128 rows, 4 at 64, 16 at 5; merged from bf16
    partials), above 128 rows one block per row; a tiny topk (3 rows, 100
    slots) takes the 64-head kernel. Index rows with nsa_cache_seqlens cuts,
    an empty row, a one-slot row and out-of-range slots; two calls on one
    workspace give bit-identical results (splits are merged in split
    order)."""
    nsa = need_gpu()
    rng = np.random.default_rng(T + topk)
    H, S = 128, 4000
    q, cache, vals, idx = _random_case(rng, T, H, topk, S, "fp8", frac_pad=0.2)
    idx[0, :] = -1                                   # empty row
    idx[1, 1:] = -1                                  # one slot (row 1 is shuffled
    idx[1, 0] = 17                                   # by _random_case: set it)
    idx[2, 3] = S + 11                               # out of range: ignored
    seqlens = np.full(T, topk, np.int32)
    seqlens[2] = min(topk, 70)
    if T > 4:
        seqlens[4] = 0
    idx_d = torch.as_tensor(idx, dtype=torch.int32, device=DEV)
    sl_d = torch.as_tensor(seqlens, device=DEV)
    ws = torch.empty(max(nsa.sparse_mla_workspace_size(T, H, topk), 16),
                     dtype=torch.uint8, device=DEV)
    nsa.nsa_check_device_errors()
    a, la = nsa.nsa_sparse_mla_decode(q.to(DEV), cache, nsa.KV_FP8_656, idx_d, 0.0721,
                                      nsa_cache_seqlens=sl_d, workspace=ws)
    b, lb = nsa.nsa_sparse_mla_decode(q.to(DEV), cache, nsa.KV_FP8_656, idx_d, 0.0721,
                                      nsa_cache_seqlens=sl_d, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert nsa.nsa_check_device_errors() == nsa.DEVERR_SLOT
    clean = np.where((idx >= 0) & (idx < S), idx, -1)
    o_ref, lse_ref = oracle.sparse_mla.sparse_mla(q.to(torch.float64).numpy(),
                                                  CacheFromRows(dict(enumerate(vals))),
                                                  clean, 0.0721, nsa_cache_seqlens=seqlens)
    o = a.float().cpu().numpy()
    check_attention(o, la.cpu().numpy(), o_ref, lse_ref, "fp8", what=f"128 heads T={T}")
    assert (o[0] == 0).all() and np.isneginf(la.cpu().numpy()[0]).all()
    np.testing.assert_allclose(o[1], np.broadcast_to(vals[idx[1, 0], :512], (H, 512)),
                               rtol=1e-2, atol=1e-2)
