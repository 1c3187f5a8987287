"""Device-side id checks: ids the host cannot see (request indices, page ids,
slots, pool rows, top-k indices past a table) are treated as absent by the
kernels and recorded in the device error word that nsa_check_device_errors()
returns -- the capacity check of "dsa_backend.py (sglang main)",
init_forward_metadata (extend branch), made a device-side flag. Every case
here stays inside the buffers: the kernels mask the bad ids before any
access. Also: the binding's shape checks, and the extend metadata's rows past
sum(extend_lens)."""

import numpy as np
import pytest
import torch

import workloads as W
import oracle
from helpers import DEV, need_gpu, note, to_dev, gpu_metadata, oracle_metadata

pytestmark = pytest.mark.gpu


def _small(nsa, name="decode_b32", **kw):
    w = to_dev(W.make_workload(name, **kw))
    nsa.nsa_check_device_errors()     # start from a clear word
    return w


def test_clean_step_records_nothing():
    nsa = need_gpu()
    w = _small(nsa, bs=3, seqlen_range=(2500, 5000))
    md = gpu_metadata(nsa, w)
    kh = nsa.new_key_hist(w.num_rows, DEV)
    lg = nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                                md["real_page_table"], md["token_to_req"],
                                md["seqlens_expanded"], w.max_seqlen_k, key_hist=kh)
    slots = nsa.nsa_topk_transform(lg, md["seqlens_expanded"], w.topk, w.max_seqlen_k,
                                   table=md["real_page_table"],
                                   token_to_req=md["token_to_req"], key_hist=kh)
    nsa.nsa_sparse_mla_decode(w.q, w.kv_bf16, nsa.KV_BF16_576, slots, w.sm_scale,
                              md["nsa_cache_seqlens"])
    assert nsa.nsa_check_device_errors() == 0
    assert nsa.nsa_check_device_errors() == 0      # and reading clears


@pytest.mark.parametrize("hint", [1, 4])
def test_bad_request_index_gives_empty_rows(hint):
    nsa = need_gpu()
    w = _small(nsa, "verify", bs=3, seqlen_range=(2500, 5000))
    md = gpu_metadata(nsa, w)
    T = w.num_rows
    t2r = md["token_to_req"].clone()
    t2r[1] = w.bs + 5                  # past the table
    t2r[6] = -3
    kh = nsa.new_key_hist(T, DEV)
    lg = torch.full((T, nsa.logits_row_stride(w.max_seqlen_k)), 7.0, device=DEV)
    nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache, md["real_page_table"],
                           t2r, md["seqlens_expanded"], w.max_seqlen_k, logits=lg,
                           key_hist=kh, rows_per_request=hint)
    torch.cuda.synchronize()
    assert nsa.nsa_check_device_errors() == nsa.DEVERR_REQUEST
    # those rows are left unwritten, the others are scored as usual
    assert bool((lg[1] == 7.0).all()) and bool((lg[6] == 7.0).all())
    assert int(kh[1].sum()) == 0 and int(kh[6].sum()) == 0
    ref = nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                                 md["real_page_table"], md["token_to_req"],
                                 md["seqlens_expanded"], w.max_seqlen_k)
    L = md["seqlens_expanded"].cpu().numpy()
    for t in (0, 2, 5, 7):
        assert torch.equal(lg[t, :L[t]], ref[t, :L[t]])
    # the fused top-k writes no slot for them
    slots = nsa.nsa_topk_transform(lg, md["seqlens_expanded"], w.topk, w.max_seqlen_k,
                                   table=md["real_page_table"], token_to_req=t2r,
                                   key_hist=kh)
    sl = slots.cpu().numpy()
    assert (sl[1] == -1).all() and (sl[6] == -1).all()
    assert (sl[0, :min(int(L[0]), w.topk)] >= 0).all()
    assert nsa.nsa_check_device_errors() == nsa.DEVERR_REQUEST
    assert int(kh.abs().sum()) == 0
    # the page transform too
    logical = nsa.nsa_topk_transform(ref, md["seqlens_expanded"], w.topk, w.max_seqlen_k)
    mapped = nsa.nsa_page_table_transform(logical, t2r,
                                          real_page_table=md["real_page_table"]).cpu().numpy()
    assert (mapped[1] == -1).all() and (mapped[6] == -1).all()
    assert nsa.nsa_check_device_errors() == nsa.DEVERR_REQUEST


def test_bad_page_id_and_index_past_table():
    nsa = need_gpu()
    w = _small(nsa, bs=2, seqlen_range=(3000, 3000))
    md = gpu_metadata(nsa, w)
    rpt = md["real_page_table"].clone()
    rpt[0, 3] = w.num_pages + 1
    lg = nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache, rpt,
                                md["token_to_req"], md["seqlens_expanded"],
                                w.max_seqlen_k).cpu().numpy()
    assert np.isneginf(lg[0, 192:256]).all() and np.isfinite(lg[0, :192]).all()
    assert nsa.nsa_check_device_errors() == nsa.DEVERR_PAGE_ID
    # a logical index past the compact table's width maps to -1
    idx = torch.tensor([[0, 64 * rpt.shape[1] + 5, -1, 70]], dtype=torch.int32, device=DEV)
    out = nsa.nsa_page_table_transform(idx, md["token_to_req"][:1],
                                       real_page_table=md["real_page_table"]).cpu().numpy()
    want = md["real_page_table"][0].cpu().numpy()
    assert out[0, 1] == -1 and out[0, 2] == -1
    assert out[0, 0] == want[0] * 64 and out[0, 3] == want[1] * 64 + 6
    assert nsa.nsa_check_device_errors() == nsa.DEVERR_INDEX


@pytest.mark.parametrize("kv,heads", [("bf16", 16), ("fp8", 128)])
def test_bad_slots_count_as_unused(kv, heads):
    nsa = need_gpu()
    w = _small(nsa, "decode_b128" if kv == "fp8" else "decode_b32", bs=2,
               seqlen_range=(3000, 4000))
    md = gpu_metadata(nsa, w)
    slots = nsa.nsa_topk_transform(
        nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                               md["real_page_table"], md["token_to_req"],
                               md["seqlens_expanded"], w.max_seqlen_k),
        md["seqlens_expanded"], w.topk, w.max_seqlen_k,
        table=md["real_page_table"], token_to_req=md["token_to_req"])
    cache = nsa.nsa_quantize_k_cache(w.kv_bf16) if kv == "fp8" else w.kv_bf16
    kvd = nsa.KV_FP8_656 if kv == "fp8" else nsa.KV_BF16_576
    bad = slots.clone()
    bad[0, 5] = cache.shape[0] + 3
    bad[1, 100] = -9
    clean = slots.clone()
    clean[0, 5] = -1
    clean[1, 100] = -1
    nsa.nsa_check_device_errors()
    o1, l1 = nsa.nsa_sparse_mla_decode(w.q, cache, kvd, bad, w.sm_scale)
    torch.cuda.synchronize()
    assert nsa.nsa_check_device_errors() == nsa.DEVERR_SLOT
    o2, l2 = nsa.nsa_sparse_mla_decode(w.q, cache, kvd, clean, w.sm_scale)
    torch.cuda.synchronize()
    assert nsa.nsa_check_device_errors() == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert w.heads == heads


def test_bad_pool_row_and_cache_loc():
    nsa = need_gpu()
    w = _small(nsa, bs=3, seqlen_range=(500, 900))
    rpi = w.req_pool_indices.clone()
    rpi[2] = w.req_to_token.shape[0] + 4
    md = nsa.nsa_build_metadata(w.mode, w.seq_lens, w.req_to_token, rpi, w.topk,
                                w.max_seqlen_k, w.num_rows, want_page_table_1=True)
    torch.cuda.synchronize()
    assert nsa.nsa_check_device_errors() == nsa.DEVERR_POOL_ROW
    rpt = md["real_page_table"].cpu().numpy()
    assert (rpt[2] == -1).all() and (md["page_table_1"][2] == -1).all()
    ref = oracle_metadata(w)
    n0 = (int(ref["cache_seqlens"][0]) + 63) // 64
    np.testing.assert_array_equal(rpt[0, :n0], ref["real_page_table"][0, :n0])
    # quantize-on-write skips (and flags) a destination outside the cache
    cache = nsa.nsa_quantize_k_cache(w.kv_bf16[:256].contiguous())
    before = cache.clone()
    rows = w.kv_bf16[:2].contiguous()
    loc = torch.tensor([7, 256 + 1], dtype=torch.int32, device=DEV)
    nsa.nsa_set_mla_kv_buffer(rows[:, :512], rows[:, 512:], loc, cache, nsa.KV_FP8_656)
    torch.cuda.synchronize()
    assert nsa.nsa_check_device_errors() == nsa.DEVERR_SLOT
    want = oracle.quant.quantize_k_cache(rows[:1].view(torch.int16).cpu().numpy().view(np.uint16))
    np.testing.assert_array_equal(cache[7].cpu().numpy(), want[0])
    keep = torch.ones(256, dtype=torch.bool)
    keep[7] = False
    assert torch.equal(cache[keep.to(DEV)], before[keep.to(DEV)])


@pytest.mark.parametrize("mode", [W.MODE_EXTEND, W.MODE_DRAFT_EXTEND])
def test_extend_rows_past_the_sum_are_empty(mode):
    # a host bound T above sum(extend_lens): the extra rows are empty rows of
    # request 0, and the indexer / top-k / attention treat them as such
    nsa = need_gpu()
    if mode == W.MODE_EXTEND:
        w = _small(nsa, "extend", bs=2, extend_lens=[30, 70], prefix_lens=[100, 2500])
    else:
        w = _small(nsa, "draft_extend", bs=3, seqlen_range=(100, 3000))
    T = w.num_rows + 9
    md = nsa.nsa_build_metadata(w.mode, w.seq_lens, w.req_to_token, w.req_pool_indices,
                                w.topk, w.max_seqlen_k, T, extend_lens=w.extend_lens,
                                draft_token_num=w.draft)
    ref = oracle_metadata(w)
    n = w.num_rows
    se = md["seqlens_expanded"].cpu().numpy()
    np.testing.assert_array_equal(se[:n], ref["seqlens_expanded"])
    assert (se[n:] == 0).all()
    assert (md["nsa_cache_seqlens"][n:] == 0).all() and (md["token_to_req"][n:] == 0).all()
    cuk = md["nsa_cu_seqlens_k"].cpu().numpy()
    np.testing.assert_array_equal(cuk[:n + 1], ref["nsa_cu_seqlens_k"])
    assert (cuk[n + 1:] == cuk[n]).all()
    np.testing.assert_array_equal(md["nsa_cu_seqlens_q"].cpu().numpy(), np.arange(T + 1))
    q_idx = torch.cat([w.q_idx, w.q_idx[:9]])
    wts = torch.cat([w.idx_weights, w.idx_weights[:9]])
    lg = nsa.nsa_indexer_logits(q_idx, wts, w.index_cache, md["real_page_table"],
                                md["token_to_req"], md["seqlens_expanded"], w.max_seqlen_k)
    slots = nsa.nsa_topk_transform(lg, md["seqlens_expanded"], w.topk, w.max_seqlen_k,
                                   table=md["real_page_table"],
                                   token_to_req=md["token_to_req"]).cpu().numpy()
    assert (slots[n:] == -1).all()
    assert nsa.nsa_check_device_errors() == 0
    note(f"extend tail rows: T={T}, sum={n}")


def test_binding_rejects_misshaped_tensors():
    nsa = need_gpu()
    w = to_dev(W.make_workload("decode_b32", bs=2, seqlen_range=(500, 900)))
    md = gpu_metadata(nsa, w)
    T = w.num_rows
    args = (w.q_idx, w.idx_weights, w.index_cache, md["real_page_table"],
            md["token_to_req"], md["seqlens_expanded"], w.max_seqlen_k)
    with pytest.raises(ValueError):          # logits with too few rows
        nsa.nsa_indexer_logits(*args, logits=torch.empty(T - 1, 2048, device=DEV))
    with pytest.raises(ValueError):          # weights of the wrong shape
        nsa.nsa_indexer_logits(w.q_idx, w.idx_weights[:, :32].contiguous(), *args[2:])
    with pytest.raises(ValueError):          # too few page-table columns
        nsa.nsa_indexer_logits(*args[:3], md["real_page_table"][:, :2].contiguous(),
                               *args[4:])
    lg = nsa.nsa_indexer_logits(*args)
    with pytest.raises(ValueError):          # top-k output too small
        nsa.nsa_topk_transform(lg, md["seqlens_expanded"], w.topk, w.max_seqlen_k,
                               out=torch.empty(T, w.topk - 1, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):          # token_to_req shorter than the rows
        nsa.nsa_topk_transform(lg, md["seqlens_expanded"], w.topk, w.max_seqlen_k,
                               table=md["real_page_table"], token_to_req=md["token_to_req"][:1])
    idx = torch.full((T, w.topk), -1, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):          # index rows fewer than q rows
        nsa.nsa_sparse_mla_decode(w.q, w.kv_bf16, nsa.KV_BF16_576, idx[:1], w.sm_scale)
    with pytest.raises(ValueError):          # seqlens shorter than the rows
        nsa.nsa_sparse_mla_decode(w.q, w.kv_bf16, nsa.KV_BF16_576, idx, w.sm_scale,
                                  nsa_cache_seqlens=md["nsa_cache_seqlens"][:1])
    with pytest.raises(ValueError):          # out of the wrong shape
        nsa.nsa_sparse_mla_decode(w.q, w.kv_bf16, nsa.KV_BF16_576, idx, w.sm_scale,
                                  out=torch.empty(T, w.heads, 256, dtype=torch.bfloat16,
                                                  device=DEV))
    with pytest.raises(ValueError):          # lse of the wrong shape
        nsa.nsa_sparse_mla_decode(w.q, w.kv_bf16, nsa.KV_BF16_576, idx, w.sm_scale,
                                  lse=torch.empty(T, 1, device=DEV))
