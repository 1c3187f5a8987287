"""GPU parity, bit-exact: nsa_build_metadata and nsa_page_table_transform
against the oracle, on every workload at full size and on edge cases."""

import numpy as np
import pytest
import torch

import workloads as W
import oracle
from helpers import DEV, need_gpu, note, to_dev, oracle_metadata, gpu_metadata

pytestmark = pytest.mark.gpu

FIELDS = ["cache_seqlens", "cu_seqlens_k", "cu_seqlens_q", "seqlens_expanded",
          "nsa_cache_seqlens", "nsa_cu_seqlens_k", "nsa_cu_seqlens_q",
          "token_to_req", "real_page_table"]


def _compare(md, ref, wide=False):
    for f in FIELDS + (["page_table_1"] if wide else []):
        got = md[f].cpu().numpy()
        want = np.asarray(ref[f])
        if f == "real_page_table":
            got = got[:, :want.shape[1]]
        assert got.shape == want.shape, (f, got.shape, want.shape)
        np.testing.assert_array_equal(got, want, err_msg=f)


@pytest.mark.parametrize("name", ["tiny", "decode_b32", "decode_b128", "extend", "verify",
                                  "draft_extend", "draft_extend_v2"])
def test_metadata_full_configs(name):
    nsa = need_gpu()
    note(f"metadata {name}")
    w = to_dev(W.make_workload(name, parts=()))
    md = gpu_metadata(nsa, w, want_page_table_1=(name != "decode_b128"))
    _compare(md, oracle_metadata(w), wide=(name != "decode_b128"))


@pytest.mark.parametrize("case", [
    dict(name="decode_b32", bs=1, seqlen_range=(1, 1)),
    dict(name="decode_b32", bs=3, seqlen_range=(64, 64)),
    dict(name="decode_b32", bs=5, seqlen_range=(1, 200), topk=100),
    dict(name="verify", bs=3, draft=1, seqlen_range=(1, 70)),
    dict(name="verify", bs=4, draft=7, seqlen_range=(60, 130), topk=64),
    dict(name="extend", bs=2, extend_lens=[5, 64], prefix_lens=[0, 0]),
    dict(name="extend", bs=3, extend_lens=[1, 300, 2], prefix_lens=[0, 65, 2047]),
    dict(name="decode_b32", bs=300, seqlen_range=(1, 3000)),
])
def test_metadata_edge_cases(case):
    nsa = need_gpu()
    case = dict(case)
    name = case.pop("name")
    note(f"metadata edge {name} {case}")
    w = to_dev(W.make_workload(name, parts=(), **case))
    md = gpu_metadata(nsa, w, want_page_table_1=True)
    _compare(md, oracle_metadata(w), wide=True)


def test_metadata_empty_batch():
    nsa = need_gpu()
    z = torch.zeros(0, dtype=torch.int32, device=DEV)
    rtt = torch.zeros(1, 64, dtype=torch.int32, device=DEV)
    md = nsa.nsa_build_metadata(nsa.MODE_DECODE, z, rtt, z, 2048, 0, 0)
    torch.cuda.synchronize()
    assert md["cu_seqlens_k"].cpu().tolist() == [0]
    assert md["nsa_cu_seqlens_k"].cpu().tolist() == [0]


@pytest.mark.parametrize("name,bs", [("decode_b32", 6), ("extend", 3), ("verify", 5)])
def test_page_table_transform_both_forms(name, bs):
    nsa = need_gpu()
    note(f"transform {name}")
    w = to_dev(W.make_workload(name, parts=(), bs=bs))
    md = gpu_metadata(nsa, w, want_page_table_1=True)
    ref = oracle_metadata(w)
    rng = np.random.default_rng(7)
    K = 2048
    T = w.num_rows
    idx = np.full((T, K), -1, np.int64)
    for t in range(T):
        L = int(ref["seqlens_expanded"][t])
        m = min(L, K) - rng.integers(0, 3)
        idx[t, :max(m, 0)] = rng.choice(L, size=max(m, 0), replace=False)
        rng.shuffle(idx[t])          # -1 anywhere in the row
    idx[0, :5] = [-1, 0, L - 1 if (L := int(ref["seqlens_expanded"][0])) else 0, -1, 1]
    want = oracle.transform.transform_wide(idx, ref["page_table_1"], ref["token_to_req"])
    want_c = oracle.transform.transform_compact(idx, ref["real_page_table"],
                                                ref["token_to_req"])
    np.testing.assert_array_equal(want, want_c)
    idx_d = torch.as_tensor(idx, dtype=torch.int32, device=DEV)
    got_w = nsa.nsa_page_table_transform(idx_d, md["token_to_req"],
                                         page_table_1=md["page_table_1"])
    got_c = nsa.nsa_page_table_transform(idx_d, md["token_to_req"],
                                         real_page_table=md["real_page_table"])
    np.testing.assert_array_equal(got_w.cpu().numpy(), want)
    np.testing.assert_array_equal(got_c.cpu().numpy(), want)


def test_page_table_transform_out_of_width_and_strided():
    nsa = need_gpu()
    rpt = torch.arange(12, dtype=torch.int32, device=DEV).reshape(2, 6)[:, :4]  # strided
    t2r = torch.tensor([1, 0, 1], dtype=torch.int32, device=DEV)
    idx = torch.tensor([[0, 63, 64, 255, 256, -1, 1000, 5]] * 3, dtype=torch.int32,
                       device=DEV)
    got = nsa.nsa_page_table_transform(idx, t2r, real_page_table=rpt).cpu().numpy()
    r = rpt.cpu().numpy()
    for t, req in enumerate([1, 0, 1]):
        exp = [r[req, 0] * 64, r[req, 0] * 64 + 63, r[req, 1] * 64, r[req, 3] * 64 + 63,
               -1, -1, -1, r[req, 0] * 64 + 5]
        assert got[t].tolist() == exp
