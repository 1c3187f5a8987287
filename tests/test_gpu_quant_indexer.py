"""GPU parity: nsa_quantize_k_cache (bit-exact) and nsa_indexer_logits
(within the fp32-summation tolerance) against the oracle."""

import numpy as np
import pytest
import torch

import workloads as W
import oracle
from helpers import (DEV, need_gpu, note, to_dev, oracle_metadata, gpu_metadata,
                     idx_dtype, oracle_logits_and_bounds, check_logits, full_workload)

pytestmark = pytest.mark.gpu


def _special_rows(n, seed=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, 576, generator=g)
    x[0] = 0.0                                   # all-zero row
    x[1, :128] = -0.0                            # negative zeros block
    x[2] *= 1e-30                                # tiny values (subnormal codes)
    x[3, 5] = 1e4                                # one dominant value per block
    x[4] = torch.linspace(-3, 3, 576)
    x[5, 130] = 7.0
    x[6:] *= torch.exp(torch.randn(n - 6, 1, generator=g) * 4)   # magnitude spread
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("n", [1, 7, 4096])
def test_quantize_bit_exact(n):
    nsa = need_gpu()
    note(f"quantize n={n}")
    x = _special_rows(max(n, 7))[:n]
    got = nsa.nsa_quantize_k_cache(x.to(DEV)).cpu().numpy()
    want = oracle.quant.quantize_k_cache(x.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(got, want)


def test_quantize_strided_rows():
    nsa = need_gpu()
    x = _special_rows(64, seed=3)
    big = torch.zeros(64, 640, dtype=torch.bfloat16)
    big[:, :576] = x
    got = nsa.nsa_quantize_k_cache(big.to(DEV)[:, :576]).cpu().numpy()
    want = oracle.quant.quantize_k_cache(x.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("fp8", [True, False])
def test_set_mla_kv_buffer_matches_oracle(fp8):
    # quantize-on-write: k / k_rope are column slices of one [n, 576] tensor
    # (strided rows); destinations are distinct, some out of range
    nsa = need_gpu()
    note(f"set_mla_kv_buffer fp8={fp8}")
    n, slots = 300, 5000
    x = _special_rows(n, seed=11)
    g = torch.Generator().manual_seed(4)
    loc = torch.randperm(slots, generator=g)[:n].to(torch.int32)
    loc[[3, 100]] = -1
    loc[7] = slots + 5
    xd = x.to(DEV)
    if fp8:
        init = torch.randint(0, 256, (slots, 656), generator=g, dtype=torch.uint8)
        kvd = nsa.KV_FP8_656
    else:
        init = torch.randn(slots, 576, generator=g).to(torch.bfloat16)
        kvd = nsa.KV_BF16_576
    cache = init.to(DEV)
    nsa.nsa_set_mla_kv_buffer(xd[:, :512], xd[:, 512:], loc.to(DEV), cache, kvd)
    got = cache.cpu()
    bits = x.view(torch.int16).numpy().view(np.uint16)
    init_np = init.numpy() if fp8 else init.view(torch.int16).numpy().view(np.uint16)
    want = oracle.quant.set_mla_kv_buffer(init_np, bits[:, :512], bits[:, 512:],
                                          loc.numpy(), fp8=fp8)
    got_np = got.numpy() if fp8 else got.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got_np, want)
    if fp8:   # the same bytes as converting the rows with nsa_quantize_k_cache
        conv = nsa.nsa_quantize_k_cache(xd).cpu()
        ok = (loc >= 0) & (loc < slots)
        np.testing.assert_array_equal(got[loc[ok].long()].numpy(), conv[ok].numpy())
    # n == 0 is a no-op
    nsa.nsa_set_mla_kv_buffer(xd[:0, :512], xd[:0, 512:],
                              torch.zeros(0, dtype=torch.int32, device=DEV), cache, kvd)
    torch.cuda.synchronize()
    assert torch.equal(cache.cpu(), got)


def test_quantize_full_cache_sampled():
    nsa = need_gpu()
    w = full_workload("decode_b128")
    note(f"quantize full decode_b128 cache: {w.kv_bf16.shape[0]} slots")
    q8 = nsa.nsa_quantize_k_cache(w.kv_bf16)
    rng = np.random.default_rng(0)
    rows = np.concatenate([[0, w.kv_bf16.shape[0] - 1],
                           rng.integers(0, w.kv_bf16.shape[0], 2000)])
    ri = torch.as_tensor(rows, device=DEV)
    want = oracle.quant.quantize_k_cache(
        w.kv_bf16[ri].view(torch.int16).cpu().numpy().view(np.uint16))
    np.testing.assert_array_equal(q8[ri].cpu().numpy(), want)


def _indexer_case(nsa, w, rows=None):
    md = gpu_metadata(nsa, w)
    ref = oracle_metadata(w)
    logits = nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                                    md["real_page_table"], md["token_to_req"],
                                    md["seqlens_expanded"], w.max_seqlen_k,
                                    dtype=idx_dtype(nsa, w))
    torch.cuda.synchronize()
    rows = list(range(w.num_rows)) if rows is None else rows
    want, bounds = oracle_logits_and_bounds(w, ref, rows)
    worst = (0.0, 0.0)
    for t in rows:
        L = int(ref["seqlens_expanded"][t])
        e, ratio = check_logits(logits[t].cpu().numpy(), want[t], L,
                                what=f"{w.name} row {t}", abs_sum=bounds[t])
        worst = (max(worst[0], e), max(worst[1], ratio))
    note(f"  max logit error {worst[0]:.3e} = {worst[1]:.2f} x 2^-24 A")
    return logits


@pytest.mark.parametrize("case", [
    dict(name="tiny"),
    dict(name="decode_b32", bs=4, seqlen_range=(1, 3000)),
    dict(name="decode_b32", bs=3, seqlen_range=(2047, 2049)),
    dict(name="verify", bs=3, seqlen_range=(100, 4000)),
    dict(name="extend", bs=2, extend_lens=[3, 40], prefix_lens=[5, 2100]),
    dict(name="tiny", seq_lens=[1, 65], idx_heads=3, idx_dim=12),
])
def test_indexer_small(case):
    nsa = need_gpu()
    case = dict(case)
    name = case.pop("name")
    note(f"indexer {name} {case}")
    w = to_dev(W.make_workload(name, parts=("indexer",), **case))
    _indexer_case(nsa, w)


def test_indexer_invalid_pages_give_neg_inf():
    nsa = need_gpu()
    w = to_dev(W.make_workload("decode_b32", parts=("indexer",), bs=2,
                               seqlen_range=(300, 300)))
    md = gpu_metadata(nsa, w)
    rpt = md["real_page_table"].clone()
    rpt[0, 1] = -5
    rpt[1, 2] = w.num_pages + 10
    logits = nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache, rpt,
                                    md["token_to_req"], md["seqlens_expanded"],
                                    w.max_seqlen_k).cpu().numpy()
    assert np.isneginf(logits[0, 64:128]).all() and np.isfinite(logits[0, :64]).all()
    assert np.isneginf(logits[1, 128:192]).all() and np.isfinite(logits[1, 192:300]).all()
    assert nsa.nsa_check_device_errors() & nsa.DEVERR_PAGE_ID


@pytest.mark.parametrize("name", ["decode_b128", "verify"])
def test_indexer_full_size_sampled_rows(name):
    # the plain entry point (no histogram, one-row schedule) at full size;
    # the benchmark's fused launch is checked on every row in test_gpu_pipeline
    nsa = need_gpu()
    w = full_workload(name)
    note(f"indexer full {name}: T={w.num_rows} max_L={w.max_seqlen_k}")
    ref = oracle_metadata(w)
    L = ref["seqlens_expanded"]
    rows = sorted({int(np.argmax(L)), int(np.argmin(L)), w.num_rows - 1} |
                  set(range(0, w.num_rows, max(1, w.num_rows // 16))))
    _indexer_case(nsa, w, rows=rows)
