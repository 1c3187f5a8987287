"""Pins for the metadata oracle: the pages' worked extend example, the field
invariants the pages state, causality properties of each mode, and the
draft-extend modes against the modes they reduce to."""

import json
import os

import numpy as np
import pytest

from oracle import metadata as M


def _alloc(seq_lens, page=64, seed=0, extra_rows=2):
    """Page-aligned random-order allocation (independent of the oracle)."""
    rng = np.random.default_rng(seed)
    npages = [(int(n) + page - 1) // page for n in seq_lens]
    perm = rng.permutation(sum(npages) + 5)
    width = (max(npages) + 1) * page
    rows = len(seq_lens) + extra_rows
    rtt = np.zeros((rows, width), np.int64)
    rpi = rng.permutation(rows)[:len(seq_lens)]
    p0 = 0
    for r, n in enumerate(npages):
        pages = perm[p0:p0 + n]
        p0 += n
        rtt[rpi[r], :n * page] = (pages[:, None] * page + np.arange(page)).reshape(-1)
    return rtt, rpi


def test_worked_extend_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "extend_k_start_end.json")))
    seq_lens, ext = g["seq_lens"], g["extend_seq_lens"]
    rtt, rpi = _alloc(seq_lens)
    md = M.build_metadata(M.MODE_EXTEND, seq_lens, rtt, rpi, topk=2048,
                          extend_lens=ext)
    ks, ke = np.array(g["ks"]), np.array(g["ke"])
    np.testing.assert_array_equal(md["seqlens_expanded"], ke - ks)
    np.testing.assert_array_equal(md["token_to_req"], [0, 0, 0, 1, 1])
    oks, oke, otb = M.indexer_k_start_end(seq_lens, ext)
    np.testing.assert_array_equal(oks, ks)
    np.testing.assert_array_equal(oke, ke)
    np.testing.assert_array_equal(otb, [0, 0, 0, 1, 1])
    # both requests have a prefix, so cu_seqlens_q is the cumsum of extend lens
    np.testing.assert_array_equal(md["cu_seqlens_q"], [0, 3, 5])
    np.testing.assert_array_equal(md["cu_seqlens_k"], [0, 10, 14])


def _check_field_invariants(md, topk):
    # NSAMetadata field comments: clipped to topk; arange; cumsum of clipped
    se, nc = md["seqlens_expanded"], md["nsa_cache_seqlens"]
    np.testing.assert_array_equal(nc, np.where(se < topk, se, topk))
    np.testing.assert_array_equal(md["nsa_cu_seqlens_q"],
                                  np.arange(len(md["nsa_cu_seqlens_k"])))
    np.testing.assert_array_equal(np.diff(md["nsa_cu_seqlens_k"]), nc)
    assert md["nsa_cu_seqlens_k"][0] == 0
    np.testing.assert_array_equal(np.diff(md["cu_seqlens_k"]), md["cache_seqlens"])
    assert len(md["token_to_req"]) == len(se)


def _check_tables(md, rtt, rpi, page=64):
    """Compact table == every 64th wide entry // 64, and wide == slice."""
    pt1, rpt = md["page_table_1"], md["real_page_table"]
    msk = md["max_seqlen_k"]
    for r in range(len(rpi)):
        np.testing.assert_array_equal(pt1[r], rtt[rpi[r], :msk])
        for p in range((msk + page - 1) // page):
            assert rpt[r, p] == rtt[rpi[r], p * page] // page
    # brute force: every valid token is reached through the compact table
    for r in range(len(rpi)):
        L = md["cache_seqlens"][r]
        s = np.arange(L)
        np.testing.assert_array_equal(rpt[r, s // page] * page + s % page,
                                      rtt[rpi[r], s])


def test_decode_invariants():
    seq_lens = [300, 700, 64, 1]
    rtt, rpi = _alloc(seq_lens)
    md = M.build_metadata(M.MODE_DECODE, seq_lens, rtt, rpi, topk=256)
    np.testing.assert_array_equal(md["cache_seqlens"], seq_lens)
    np.testing.assert_array_equal(md["seqlens_expanded"], seq_lens)
    np.testing.assert_array_equal(md["cu_seqlens_q"], np.arange(5))
    np.testing.assert_array_equal(md["nsa_cache_seqlens"], [256, 256, 64, 1])
    np.testing.assert_array_equal(md["token_to_req"], [0, 1, 2, 3])
    assert md["max_seqlen_q"] == 1 and md["max_seqlen_k"] == 700
    _check_field_invariants(md, 256)
    _check_tables(md, rtt, rpi)


def test_target_verify_causality():
    seq_lens, D = [5, 130, 64], 3
    rtt, rpi = _alloc([n + D for n in seq_lens])
    md = M.build_metadata(M.MODE_TARGET_VERIFY, seq_lens, rtt, rpi, topk=66,
                          draft_token_num=D)
    np.testing.assert_array_equal(md["cache_seqlens"], np.array(seq_lens) + D)
    np.testing.assert_array_equal(md["cu_seqlens_q"], np.arange(len(seq_lens) * D + 1))
    se = md["seqlens_expanded"].reshape(len(seq_lens), D)
    # draft token j sees the prefix plus drafts 0..j; the last one sees all
    np.testing.assert_array_equal(se[:, 0], np.array(seq_lens) + 1)
    np.testing.assert_array_equal(se[:, -1], md["cache_seqlens"])
    assert (np.diff(se, axis=1) == 1).all()
    np.testing.assert_array_equal(md["token_to_req"], np.repeat(np.arange(3), D))
    _check_field_invariants(md, 66)
    _check_tables(md, rtt, rpi)


def test_draft_extend_hand_example():
    # draft-extend v1 ("dsa_backend.py (sglang main)", init_forward_metadata,
    # draft-extend branch): seq_lens count the new tokens; request 0 accepted
    # 2 drafts (extends by 3), request 1 none (extends by 1); every token is
    # its own query row and sees its prefix plus itself
    seq_lens, ext = [10, 7], [3, 1]
    rtt, rpi = _alloc(seq_lens)
    md = M.build_metadata(M.MODE_DRAFT_EXTEND, seq_lens, rtt, rpi, topk=9,
                          extend_lens=ext)
    np.testing.assert_array_equal(md["cache_seqlens"], [10, 7])
    np.testing.assert_array_equal(md["seqlens_expanded"], [8, 9, 10, 7])
    np.testing.assert_array_equal(md["nsa_cache_seqlens"], [8, 9, 9, 7])
    np.testing.assert_array_equal(md["cu_seqlens_q"], [0, 1, 2, 3, 4])
    np.testing.assert_array_equal(md["token_to_req"], [0, 0, 0, 1])
    assert md["max_seqlen_q"] == 1
    _check_field_invariants(md, 9)
    _check_tables(md, rtt, rpi)


def test_draft_extend_v2_is_verify_with_drafts_in_seq_lens():
    # v2 extends every request by the draft count with seq_lens already
    # holding the drafts; target-verify adds them itself: same forward
    seq_lens, D = [5, 130, 64, 1000], 4
    rtt, rpi = _alloc([n + D for n in seq_lens])
    ver = M.build_metadata(M.MODE_TARGET_VERIFY, seq_lens, rtt, rpi, topk=100,
                           draft_token_num=D)
    v2 = M.build_metadata(M.MODE_DRAFT_EXTEND_V2, [n + D for n in seq_lens], rtt,
                          rpi, topk=100, draft_token_num=D)
    for k in ver:
        np.testing.assert_array_equal(np.asarray(v2[k]), np.asarray(ver[k]), err_msg=k)
    _check_field_invariants(v2, 100)


def test_draft_extend_v1_reduces_to_v2_and_to_extend():
    seq_lens, D = [40, 300, 77], 3
    rtt, rpi = _alloc(seq_lens)
    v1 = M.build_metadata(M.MODE_DRAFT_EXTEND, seq_lens, rtt, rpi, topk=64,
                          extend_lens=[D] * 3)
    v2 = M.build_metadata(M.MODE_DRAFT_EXTEND_V2, seq_lens, rtt, rpi, topk=64,
                          draft_token_num=D)
    for k in v2:
        np.testing.assert_array_equal(np.asarray(v1[k]), np.asarray(v2[k]), err_msg=k)
    # with variable lengths, the rows are those of a chunked extend of the
    # same tokens; only the query offsets differ (one row per token)
    ext = [1, 3, 2]
    d1 = M.build_metadata(M.MODE_DRAFT_EXTEND, seq_lens, rtt, rpi, topk=64,
                          extend_lens=ext)
    ex = M.build_metadata(M.MODE_EXTEND, seq_lens, rtt, rpi, topk=64,
                          extend_lens=ext)
    for k in ("cache_seqlens", "cu_seqlens_k", "seqlens_expanded",
              "nsa_cache_seqlens", "nsa_cu_seqlens_k", "nsa_cu_seqlens_q",
              "real_page_table", "token_to_req"):
        np.testing.assert_array_equal(d1[k], ex[k], err_msg=k)
    np.testing.assert_array_equal(d1["cu_seqlens_q"], np.arange(sum(ext) + 1))
    np.testing.assert_array_equal(ex["cu_seqlens_q"], [0, 1, 4, 6])
    _check_field_invariants(d1, 64)


@pytest.mark.parametrize("prefix", [[0, 0], [7, 0], [100, 33]])
def test_extend_causality(prefix):
    ext = [5, 70]
    seq_lens = [p + e for p, e in zip(prefix, ext)]
    rtt, rpi = _alloc(seq_lens)
    md = M.build_metadata(M.MODE_EXTEND, seq_lens, rtt, rpi, topk=64,
                          extend_lens=ext)
    se = md["seqlens_expanded"]
    assert len(se) == sum(ext)
    # token j of request r sees its prefix plus extend tokens 0..j
    k = 0
    for r in range(2):
        for j in range(ext[r]):
            assert se[k] == prefix[r] + j + 1
            k += 1
    # cu_seqlens_q is the cumsum of extend lengths (equal to cu_seqlens_k
    # when no request has a prefix)
    np.testing.assert_array_equal(md["cu_seqlens_q"], [0, ext[0], sum(ext)])
    _check_field_invariants(md, 64)
    _check_tables(md, rtt, rpi)


def test_wide_table_explicit_bound():
    seq_lens = [100, 10]
    rtt, rpi = _alloc(seq_lens)
    md = M.build_metadata(M.MODE_DECODE, seq_lens, rtt, rpi, topk=8,
                          max_seqlen_k=130)
    assert md["page_table_1"].shape == (2, 130)
    assert md["real_page_table"].shape == (2, 3)
