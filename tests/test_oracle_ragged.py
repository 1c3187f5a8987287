"""Pins for the RAGGED extend oracle: the pages' worked key-window example,
the RAGGED route reaching exactly the slots of the paged route, paged
dequantization against torch's fp8 and bf16 casts, and CSR lists against
plain loops."""

import json
import os

import numpy as np
import torch

from oracle import metadata as M, ragged as R, transform as X, quant as Q


def _alloc(seq_lens, page=64, seed=0):
    rng = np.random.default_rng(seed)
    npages = [(int(n) + page - 1) // page for n in seq_lens]
    perm = rng.permutation(sum(npages) + 3)
    rtt = np.zeros((len(seq_lens) + 1, (max(npages) + 1) * page), np.int64)
    rpi = rng.permutation(len(seq_lens) + 1)[:len(seq_lens)]
    p0 = 0
    for r, n in enumerate(npages):
        rtt[rpi[r], :n * page] = (perm[p0:p0 + n, None] * page + np.arange(page)).reshape(-1)
        p0 += n
    return rtt, rpi


def test_worked_key_windows(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "extend_k_start_end.json")))
    rtt, rpi = _alloc(g["seq_lens"])
    md = M.build_metadata(M.MODE_EXTEND, g["seq_lens"], rtt, rpi, topk=2048,
                          extend_lens=g["extend_seq_lens"])
    rg = R.ragged_metadata(md["cache_seqlens"], md["seqlens_expanded"],
                           md["token_to_req"], rtt, rpi)
    np.testing.assert_array_equal(rg["ks"], g["ks"])
    np.testing.assert_array_equal(rg["ke"], g["ke"])
    np.testing.assert_array_equal(rg["topk_indices_offset"], g["ks"])
    # the flattened table lists request 0's 10 slots, then request 1's 4
    want = np.concatenate([rtt[rpi[0], :10], rtt[rpi[1], :4]])
    np.testing.assert_array_equal(rg["page_table_1_flattened"], want)


def test_ragged_route_reaches_the_paged_slots():
    seq_lens, ext = [300, 1000, 77], [20, 5, 77]
    rtt, rpi = _alloc(seq_lens, seed=3)
    md = M.build_metadata(M.MODE_EXTEND, seq_lens, rtt, rpi, topk=64, extend_lens=ext)
    rg = R.ragged_metadata(md["cache_seqlens"], md["seqlens_expanded"],
                           md["token_to_req"], rtt, rpi)
    rng = np.random.default_rng(1)
    T = len(md["token_to_req"])
    idx = np.full((T, 64), -1, np.int64)
    for t in range(T):
        L = int(md["seqlens_expanded"][t])
        k = min(L, 64)
        idx[t, :k] = rng.choice(L, size=k, replace=False)
    glob = R.ragged_index_transform(idx, rg["topk_indices_offset"])
    assert ((glob == -1) == (idx == -1)).all()
    flat = rg["page_table_1_flattened"]
    via_ragged = np.where(glob >= 0, flat[np.maximum(glob, 0)], -1)
    via_paged = X.transform_compact(idx, md["real_page_table"], md["token_to_req"])
    np.testing.assert_array_equal(via_ragged, via_paged)
    # every shifted position stays inside its token's window [ks, ke)
    v = glob >= 0
    assert (glob[v] >= np.repeat(rg["ks"], 64).reshape(T, 64)[v]).all()
    assert (glob[v] < np.repeat(rg["ke"], 64).reshape(T, 64)[v]).all()


def test_dequantize_paged_against_torch_casts():
    g = torch.Generator().manual_seed(2)
    x = (torch.randn(40, 576, generator=g) * torch.exp(torch.randn(40, 1, generator=g) * 3))
    xb = x.to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    cache = Q.quantize_k_cache(bits)
    slots = np.array([5, -1, 39, 0, 40, 5, 17])
    got = R.dequantize_k_cache_paged(cache, slots)
    # torch: fp8 codes -> fp32 (its own e4m3fn decoder), times the scale in
    # fp32, then torch's bf16 cast (round to nearest even)
    codes = torch.from_numpy(cache[:, :512].copy()).view(torch.float8_e4m3fn).to(torch.float32)
    scales = torch.from_numpy(cache[:, 512:528].copy().view("<f4").copy())
    prod = codes * scales.repeat_interleave(128, dim=1)
    want_nope = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for i, s in enumerate(slots):
        if 0 <= s < 40:
            np.testing.assert_array_equal(got[i, :512], want_nope[s])
            np.testing.assert_array_equal(got[i, 512:], bits[s, 512:])
        else:
            assert (got[i] == 0).all()


def test_valid_kv_indices_against_loops():
    rng = np.random.default_rng(4)
    idx = rng.integers(0, 1000, (9, 13))
    idx[rng.random((9, 13)) < 0.4] = -1
    idx[3] = -1                                  # an empty row
    indptr, flat = R.valid_kv_indices(idx)
    ip, fl = [0], []
    for row in idx:
        for v in row:
            if v != -1:
                fl.append(v)
        ip.append(len(fl))
    np.testing.assert_array_equal(indptr, ip)
    np.testing.assert_array_equal(flat, fl)
    # valid-first rows (as the top-k writes them): row pointers are the
    # cumulative clipped lengths
    L = np.array([0, 5, 13, 20, 1])
    vf = np.full((5, 13), -1)
    for t, n in enumerate(np.minimum(L, 13)):
        vf[t, :n] = np.arange(n)
    np.testing.assert_array_equal(R.valid_kv_indices(vf)[0],
                                  M.compute_cu_seqlens(np.minimum(L, 13)))
