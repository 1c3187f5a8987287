"""GPU parity of the whole path -- metadata, indexer, top-k (+ fused page
transform), sparse MLA -- in the launch configuration the benchmark times.
Small workloads are checked on every row. Full-size workloads: every row of
the decode batch of 128 (in four slices), and rows spread over the requests
of the other workloads, which the oracle computes one by one (metadata is
checked in full). No kernel may record a device error on valid inputs."""

import numpy as np
import pytest
import torch

import workloads as W
import oracle
from helpers import (DEV, need_gpu, note, to_dev, oracle_metadata, gpu_metadata,
                     idx_dtype, full_workload, host_key_hist, check_path_rows,
                     spread_rows)

pytestmark = pytest.mark.gpu


def run_path(nsa, w, fused=True, hist=False):
    nsa.nsa_check_device_errors()          # clear what earlier tests left
    md = gpu_metadata(nsa, w)
    kh = nsa.new_key_hist(w.num_rows, DEV) if hist else None
    logits = nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                                    md["real_page_table"], md["token_to_req"],
                                    md["seqlens_expanded"], w.max_seqlen_k,
                                    dtype=idx_dtype(nsa, w), key_hist=kh,
                                    rows_per_request=w.rows_per_request)
    if hist:
        # the benchmark's launch: the fused top-k with the page table consumes
        # the indexer's histogram; the logical positions come after it
        slots = nsa.nsa_topk_transform(logits, md["seqlens_expanded"], w.topk,
                                       w.max_seqlen_k, table=md["real_page_table"],
                                       token_to_req=md["token_to_req"], key_hist=kh)
        assert int(kh.abs().sum()) == 0, "the top-k clears the histogram it used"
        logical = nsa.nsa_topk_transform(logits, md["seqlens_expanded"], w.topk,
                                         w.max_seqlen_k)
    else:
        logical = nsa.nsa_topk_transform(logits, md["seqlens_expanded"], w.topk,
                                         w.max_seqlen_k)
        if fused:
            slots = nsa.nsa_topk_transform(logits, md["seqlens_expanded"], w.topk,
                                           w.max_seqlen_k, table=md["real_page_table"],
                                           token_to_req=md["token_to_req"])
        else:
            slots = nsa.nsa_page_table_transform(logical, md["token_to_req"],
                                                 real_page_table=md["real_page_table"])
    if w.kv_kind == "fp8":
        cache = nsa.nsa_quantize_k_cache(w.kv_bf16)
        kvd = nsa.KV_FP8_656
    else:
        cache, kvd = w.kv_bf16, nsa.KV_BF16_576
    entry = nsa.nsa_sparse_mla_extend if w.mode == W.MODE_EXTEND else nsa.nsa_sparse_mla_decode
    out, lse = entry(w.q, cache, kvd, slots, w.sm_scale, md["nsa_cache_seqlens"])
    torch.cuda.synchronize()
    assert nsa.nsa_check_device_errors() == 0, "a kernel flagged valid inputs"
    return md, logits, logical, slots, cache, out, lse


@pytest.mark.parametrize("case", [
    dict(name="tiny"),
    dict(name="decode_b32", bs=3, seqlen_range=(1000, 5000)),
    dict(name="decode_b128", bs=2, seqlen_range=(2000, 9000)),
    dict(name="verify", bs=2, seqlen_range=(100, 3000)),
    dict(name="extend", bs=2, extend_lens=[30, 70], prefix_lens=[100, 2500]),
    dict(name="draft_extend", bs=3, seqlen_range=(100, 3000)),
    dict(name="draft_extend_v2", bs=2, seqlen_range=(100, 3000)),
])
@pytest.mark.parametrize("fused,hist", [(True, False), (False, False), (True, True)])
def test_pipeline_small(case, fused, hist):
    nsa = need_gpu()
    case = dict(case)
    name = case.pop("name")
    if hist and name == "tiny":
        pytest.skip("the fused histogram is an fp8-indexer feature")
    note(f"pipeline {name} {case} fused={fused} hist={hist}")
    w = to_dev(W.make_workload(name, **case))
    res = run_path(nsa, w, fused=fused, hist=hist)
    err, ratio = check_path_rows(w, *res, rows=list(range(w.num_rows)))
    note(f"  max logit error {err:.3e} = {ratio:.2f} x 2^-24 A")


_FULL = {}


def _full_run(nsa, name):
    # the full-size step in the benchmark's launch configuration (fused
    # histogram, row-group hint of the workload), run once per workload
    if name not in _FULL:
        _FULL.clear()                      # one full-size workload held at a time
        w = full_workload(name)
        _FULL[name] = (w, run_path(nsa, w, hist=w.idx_kind == "fp8"))
    return _FULL[name]


@pytest.mark.parametrize("part", range(4))
def test_pipeline_full_size_decode_b128_every_row(part):
    nsa = need_gpu()
    w, res = _full_run(nsa, "decode_b128")
    rows = list(range(part * 32, (part + 1) * 32))
    note(f"pipeline full decode_b128 rows {rows[0]}..{rows[-1]}")
    err, ratio = check_path_rows(w, *res, rows=rows, check_cache=part == 0)
    note(f"  max logit error {err:.3e} = {ratio:.2f} x 2^-24 A")


@pytest.mark.parametrize("name", ["decode_b32", "verify", "extend", "draft_extend",
                                  "draft_extend_v2"])
def test_pipeline_full_size_spread_rows(name):
    nsa = need_gpu()
    w, res = _full_run(nsa, name)
    rows = spread_rows(w, 32)
    note(f"pipeline full {name}: T={w.num_rows} max_L={w.max_seqlen_k}, {len(rows)} rows")
    err, ratio = check_path_rows(w, *res, rows=rows)
    note(f"  max logit error {err:.3e} = {ratio:.2f} x 2^-24 A")


@pytest.mark.parametrize("name,grouped", [("decode_b32", False), ("verify", False),
                                          ("verify", True), ("extend", True),
                                          ("decode_b128", False)])
def test_fused_histogram_exact_and_topk_identical(name, grouped):
    # grouped: the rows-per-request hint of the workload, which scores a
    # request's rows four at a time (verify: its 4 drafts; extend).
    # decode_b128 (128 rows of up to 131072 positions) runs the split select
    # (mark and finish kernels) with the binding's workspace; the others run
    # one block per row
    nsa = need_gpu()
    w = full_workload(name)
    note(f"fused histogram {name}: T={w.num_rows} grouped={grouped} split top-k="
         f"{nsa.topk_hist_workspace_size(w.num_rows, w.max_seqlen_k, w.topk) > 0}")
    md = gpu_metadata(nsa, w)
    kh = nsa.new_key_hist(w.num_rows, DEV)
    logits = nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                                    md["real_page_table"], md["token_to_req"],
                                    md["seqlens_expanded"], w.max_seqlen_k,
                                    dtype=idx_dtype(nsa, w), key_hist=kh,
                                    rows_per_request=w.rows_per_request if grouped else 1)
    torch.cuda.synchronize()
    L = md["seqlens_expanded"].cpu().numpy()
    hist = kh.cpu().numpy().view(np.uint32)
    for t in sorted({0, int(np.argmax(L)), int(np.argmin(L)), w.num_rows - 1}):
        n = min(int(L[t]), w.max_seqlen_k)
        np.testing.assert_array_equal(hist[t], host_key_hist(logits[t].cpu().numpy(), n),
                                      err_msg=f"{name} row {t}")
    assert (hist.sum(axis=1) == np.minimum(L, w.max_seqlen_k)).all()
    args = (logits, md["seqlens_expanded"], w.topk, w.max_seqlen_k)
    kw = dict(table=md["real_page_table"], token_to_req=md["token_to_req"])
    plain = nsa.nsa_topk_transform(*args, **kw)
    fused = nsa.nsa_topk_transform(*args, key_hist=kh, **kw)
    torch.cuda.synchronize()
    assert torch.equal(plain, fused)
    assert int(kh.abs().sum()) == 0
    # a histogram that does not match the logits (here: all zero) takes the
    # exact multi-pass path and still gives the same selection
    again = nsa.nsa_topk_transform(*args, key_hist=kh, **kw)
    torch.cuda.synchronize()
    assert torch.equal(plain, again)


@pytest.mark.parametrize("name,overrides", [
    ("verify", dict(bs=6, seqlen_range=(3000, 40000))),
    ("draft_extend_v2", dict(bs=5, seqlen_range=(3000, 40000))),
    ("decode_b32", dict(bs=7)),
    # groups of 4 rows that straddle requests (extend lens not multiples of 4)
    ("extend", dict(bs=3, extend_lens=[5, 130, 63], prefix_lens=[100, 3000, 777])),
    ("draft_extend", dict(bs=9, seqlen_range=(100, 9000))),
    # full size: the one-row schedule (hint 1) ends with short tail blocks
    ("decode_b128", {}),
])
def test_indexer_row_groups_change_nothing(name, overrides):
    # the row-group hint changes the schedule (XCD-adjacent blocks for 2 or
    # 3, four rows per block sharing their key pages for 4 and more), never
    # the result: logits, unwritten positions and histogram counts are
    # identical for every hint, including ones that do not match the layout
    nsa = need_gpu()
    w = W.make_workload(name, device=DEV, parts=("indexer",), **overrides)
    md = gpu_metadata(nsa, w)
    outs = []
    for g in (1, 2, 3, 4, 8, max(w.draft, 1)):
        kh = nsa.new_key_hist(w.num_rows, DEV)
        lg = torch.full((w.num_rows, nsa.logits_row_stride(w.max_seqlen_k)), 7.0,
                        device=DEV)
        nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                               md["real_page_table"], md["token_to_req"],
                               md["seqlens_expanded"], w.max_seqlen_k, logits=lg,
                               key_hist=kh, rows_per_request=g)
        torch.cuda.synchronize()
        outs.append((lg.cpu(), kh.cpu()))
    for lg, kh in outs[1:]:
        assert torch.equal(lg, outs[0][0]) and torch.equal(kh, outs[0][1])
    # the entry point without a histogram (and without a hint) writes the
    # same logits
    lg = torch.full((w.num_rows, nsa.logits_row_stride(w.max_seqlen_k)), 7.0, device=DEV)
    nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                           md["real_page_table"], md["token_to_req"],
                           md["seqlens_expanded"], w.max_seqlen_k, logits=lg)
    torch.cuda.synchronize()
    assert torch.equal(lg.cpu(), outs[0][0])


def test_indexer_row_groups_with_unordered_rows():
    # rows whose requests are not consecutive (a caller-built token_to_req):
    # groups of four then mix requests and are scored row by row; the result
    # equals the one-row schedule's bit for bit
    nsa = need_gpu()
    w = W.make_workload("verify", device=DEV, parts=("indexer",), bs=6,
                        seqlen_range=(200, 20000))
    md = gpu_metadata(nsa, w)
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(w.num_rows, generator=g).to(DEV)
    t2r = md["token_to_req"][perm].contiguous()
    lens = md["seqlens_expanded"][perm].contiguous()
    lens[3] = 0                                   # an empty row
    outs = []
    for hint in (1, 4):
        kh = nsa.new_key_hist(w.num_rows, DEV)
        lg = torch.full((w.num_rows, nsa.logits_row_stride(w.max_seqlen_k)), 7.0,
                        device=DEV)
        nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                               md["real_page_table"], t2r, lens, w.max_seqlen_k,
                               logits=lg, key_hist=kh, rows_per_request=hint)
        torch.cuda.synchronize()
        outs.append((lg.cpu(), kh.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert int(outs[1][1][3].sum()) == 0 and bool((outs[1][0][3] == 7.0).all())
