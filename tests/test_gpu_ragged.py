"""GPU parity of the RAGGED extend route ("dsa_backend.py (sglang main)",
extend branch of init_forward_metadata, _cal_indexer_k_start_end,
forward_extend RAGGED, dequantize_k_cache_paged; get_valid_kv_indices): each
entry point bit for bit against the oracle, then the whole route on an extend
batch with an fp8 cache -- its shifted positions must reach exactly the slots
of the paged route, and its attention over the flattened bf16 rows must match
the oracle."""

import numpy as np
import pytest
import torch

import workloads as W
import oracle
from helpers import (DEV, need_gpu, note, to_dev, oracle_metadata, gpu_metadata,
                     idx_dtype, check_attention, CacheFromRows)

pytestmark = pytest.mark.gpu


def _ragged_ref(w, ref):
    h = W.host_inputs(w)
    return oracle.ragged.ragged_metadata(ref["cache_seqlens"], ref["seqlens_expanded"],
                                         ref["token_to_req"], h["req_to_token"],
                                         h["req_pool_indices"])


@pytest.mark.parametrize("case", [
    dict(name="extend"),
    dict(name="extend", bs=2, extend_lens=[3, 2], prefix_lens=[7, 2]),
    dict(name="draft_extend", bs=5, seqlen_range=(100, 3000)),
])
def test_ragged_metadata_bit_exact(case):
    nsa = need_gpu()
    case = dict(case)
    name = case.pop("name")
    note(f"ragged metadata {name} {case}")
    w = to_dev(W.make_workload(name, parts=(), **case))
    md = gpu_metadata(nsa, w)
    ref = oracle_metadata(w)
    want = _ragged_ref(w, ref)
    total_k = int(ref["cache_seqlens"].sum())
    got = nsa.nsa_ragged_extend_metadata(md, w.max_seqlen_k, total_k)
    for k in ("ks", "ke", "topk_indices_offset", "page_table_1_flattened"):
        np.testing.assert_array_equal(got[k].cpu().numpy(), want[k], err_msg=k)
    # a short flattened buffer: positions past its end are not written
    cut = nsa.nsa_ragged_extend_metadata(md, w.max_seqlen_k, total_k // 2)
    np.testing.assert_array_equal(cut["page_table_1_flattened"].cpu().numpy(),
                                  want["page_table_1_flattened"][:total_k // 2])


def test_ragged_index_transform_and_in_place():
    nsa = need_gpu()
    g = torch.Generator().manual_seed(1)
    idx = torch.randint(0, 5000, (37, 300), generator=g, dtype=torch.int32)
    idx[torch.rand(37, 300, generator=g) < 0.3] = -1
    off = torch.randint(0, 1 << 20, (37,), generator=g, dtype=torch.int32)
    want = oracle.ragged.ragged_index_transform(idx.numpy(), off.numpy())
    got = nsa.nsa_ragged_index_transform(idx.to(DEV), off.to(DEV)).cpu().numpy()
    np.testing.assert_array_equal(got, want)
    d = idx.to(DEV)
    nsa.nsa_ragged_index_transform(d, off.to(DEV), out=d)
    np.testing.assert_array_equal(d.cpu().numpy(), want)


def test_dequantize_k_cache_paged_bit_exact():
    nsa = need_gpu()
    g = torch.Generator().manual_seed(2)
    x = torch.randn(700, 576, generator=g)
    x[5:] *= torch.exp(torch.randn(695, 1, generator=g) * 4)     # subnormal codes too
    xb = x.to(torch.bfloat16)
    cache = nsa.nsa_quantize_k_cache(xb.to(DEV))
    slots = torch.randint(0, 700, (1000,), generator=g, dtype=torch.int32)
    slots[[0, 9, 500]] = torch.tensor([-1, 700, -5], dtype=torch.int32)
    got = nsa.nsa_dequantize_k_cache_paged(cache, slots.to(DEV))
    want = oracle.ragged.dequantize_k_cache_paged(cache.cpu().numpy(), slots.numpy())
    np.testing.assert_array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), want)
    # strided output rows
    big = torch.zeros(1000, 640, dtype=torch.bfloat16, device=DEV)
    nsa.nsa_dequantize_k_cache_paged(cache, slots.to(DEV), out=big[:, :576])
    np.testing.assert_array_equal(
        big[:, :576].contiguous().view(torch.int16).cpu().numpy().view(np.uint16), want)
    assert int(big[:, 576:].abs().sum()) == 0


@pytest.mark.parametrize("T,K,p", [(300, 2048, 0.3), (5, 7, 0.5), (1, 1, 1.0), (2000, 64, 0.0)])
def test_valid_kv_indices_bit_exact(T, K, p):
    nsa = need_gpu()
    g = torch.Generator().manual_seed(T + K)
    idx = torch.randint(0, 1 << 24, (T, K), generator=g, dtype=torch.int32)
    idx[torch.rand(T, K, generator=g) < p] = -1
    ip, flat = nsa.nsa_valid_kv_indices(idx.to(DEV))
    want_ip, want_flat = oracle.ragged.valid_kv_indices(idx.numpy())
    np.testing.assert_array_equal(ip.cpu().numpy(), want_ip)
    n = int(want_ip[-1])
    np.testing.assert_array_equal(flat[:n].cpu().numpy(), want_flat)
    # a short capacity keeps the row pointers and the leading entries
    cap = n // 3
    ip2, flat2 = nsa.nsa_valid_kv_indices(idx.to(DEV), capacity=cap)
    np.testing.assert_array_equal(ip2.cpu().numpy(), want_ip)
    np.testing.assert_array_equal(flat2.cpu().numpy(), want_flat[:cap])


def test_valid_kv_indices_empty():
    nsa = need_gpu()
    ip, flat = nsa.nsa_valid_kv_indices(torch.zeros(0, 16, dtype=torch.int32, device=DEV))
    assert ip.cpu().tolist() == [0] and flat.numel() == 0


@pytest.mark.parametrize("case", [
    dict(bs=2, extend_lens=[40, 300], prefix_lens=[100, 2600], kv="fp8"),
    dict(kv="fp8"),
])
def test_ragged_route_end_to_end(case):
    nsa = need_gpu()
    note(f"ragged route {case}")
    w = to_dev(W.make_workload("extend", **case))
    md = gpu_metadata(nsa, w)
    ref = oracle_metadata(w)
    logits = nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                                    md["real_page_table"], md["token_to_req"],
                                    md["seqlens_expanded"], w.max_seqlen_k,
                                    dtype=idx_dtype(nsa, w))
    logical = nsa.nsa_topk_transform(logits, md["seqlens_expanded"], w.topk,
                                     w.max_seqlen_k)
    paged = nsa.nsa_topk_transform(logits, md["seqlens_expanded"], w.topk,
                                   w.max_seqlen_k, table=md["real_page_table"],
                                   token_to_req=md["token_to_req"])
    cache = nsa.nsa_quantize_k_cache(w.kv_bf16)
    total_k = int(ref["cache_seqlens"].sum())
    rg = nsa.nsa_ragged_extend_metadata(md, w.max_seqlen_k, total_k)
    glob = nsa.nsa_ragged_index_transform(logical, rg["topk_indices_offset"])
    flat = rg["page_table_1_flattened"]
    # the RAGGED positions name exactly the slots the paged route selects
    g = glob.long()
    via_flat = torch.where(g >= 0, flat[g.clamp(min=0)], torch.full_like(glob, -1))
    assert torch.equal(via_flat, paged)
    flat_kv = nsa.nsa_dequantize_k_cache_paged(cache, flat)
    out, lse = nsa.nsa_sparse_mla_extend(w.q, flat_kv, nsa.KV_BF16_576, glob,
                                         w.sm_scale, md["nsa_cache_seqlens"])
    torch.cuda.synchronize()
    T = w.num_rows
    rows = sorted({0, T // 3, T // 2, T - 1})
    gi = glob.cpu().numpy()[rows]
    used = np.unique(gi[gi >= 0])
    bits = oracle.ragged.dequantize_k_cache_paged(
        cache.cpu().numpy(), flat.cpu().numpy()[used])
    kv = CacheFromRows({int(u): oracle.formats.bf16_bits_to_f64(bits[i])
                        for i, u in enumerate(used)})
    q64 = w.q[torch.as_tensor(rows, device=DEV)].to(torch.float64).cpu().numpy()
    o_ref, lse_ref = oracle.sparse_mla.sparse_mla(
        q64, kv, gi, w.sm_scale, nsa_cache_seqlens=ref["nsa_cache_seqlens"][rows])
    ri = torch.as_tensor(rows, device=DEV)
    check_attention(out[ri].float().cpu().numpy(), lse[ri].cpu().numpy(), o_ref,
                    lse_ref, "bf16", what="ragged route")
