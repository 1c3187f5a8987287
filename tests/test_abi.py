"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/nsa.h declares, and rejects bad arguments with status
codes before launching anything."""

import ctypes
import os
import re

import pytest

from sparse_attention_decode_indexer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

N = None  # NULL


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "nsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nsa_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_decode_indexer_amd.build import build_library
        build_library()
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of date"


def test_version_and_empty_error(lib):
    assert lib.nsa_version() >= 100
    assert isinstance(lib.nsa_last_error(), bytes)


def _err(lib):
    return lib.nsa_last_error().decode()


def test_metadata_rejects_bad_arguments(lib):
    out = [ctypes.c_void_p(16)] * 8
    # unknown mode
    assert lib.nsa_build_metadata(7, 1, 0, 8, 64, 16, N, 16, 64, 4, 16, 64, 1,
                                  *out, 1, 16, N, 0, N) == -1
    assert "mode" in _err(lib)
    # page size
    assert lib.nsa_build_metadata(0, 1, 0, 8, 32, 16, N, 16, 64, 4, 16, 64, 1,
                                  *out, 1, 16, N, 0, N) == -2
    # decode needs num_q_rows == bs
    assert lib.nsa_build_metadata(0, 2, 0, 8, 64, 16, N, 16, 64, 4, 16, 64, 3,
                                  *out, 1, 16, N, 0, N) == -1
    # verify needs bs * draft rows
    assert lib.nsa_build_metadata(2, 2, 3, 8, 64, 16, N, 16, 64, 4, 16, 64, 5,
                                  *out, 1, 16, N, 0, N) == -1
    # extend needs extend_lens
    assert lib.nsa_build_metadata(1, 2, 0, 8, 64, 16, N, 16, 64, 4, 16, 64, 5,
                                  *out, 1, 16, N, 0, N) == -1
    # real_page_table stride too small for max_seqlen_k = 200 (needs 4)
    assert lib.nsa_build_metadata(0, 1, 0, 8, 64, 16, N, 16, 256, 4, 16, 200, 1,
                                  *out, 3, 16, N, 0, N) == -1
    assert "rpt_stride" in _err(lib)


def test_indexer_rejects_bad_arguments(lib):
    p = ctypes.c_void_p(256)
    # fp8 path supports only 64 heads x 128 dims
    assert lib.nsa_indexer_logits(p, 2, p, p, 2, 10, p, 4, 4, p, p, 4, 32, 128, 64,
                                  200, p, 256, N) == -2
    # mismatched dtypes
    assert lib.nsa_indexer_logits(p, 2, p, p, 0, 10, p, 4, 4, p, p, 4, 64, 128, 64,
                                  200, p, 256, N) == -2
    # logits stride below max_seqlen_k
    assert lib.nsa_indexer_logits(p, 2, p, p, 2, 10, p, 4, 4, p, p, 4, 64, 128, 64,
                                  200, p, 100, N) == -1
    # misaligned q
    assert lib.nsa_indexer_logits(ctypes.c_void_p(257), 2, p, p, 2, 10, p, 4, 4, p,
                                  p, 4, 64, 128, 64, 200, p, 256, N) == -1
    # the fp8 path reads page 0 in place of an absent page: an empty cache
    # is rejected (also with the row-group hint)
    assert lib.nsa_indexer_logits(p, 2, p, p, 2, 0, p, 4, 4, p, p, 4, 64, 128, 64,
                                  200, p, 256, N) == -1
    assert "num_pages" in _err(lib)
    assert lib.nsa_indexer_logits_hist(p, 2, p, p, 2, 0, p, 4, 4, p, p, 4, 64, 128, 64,
                                       200, p, 256, p, 4, N) == -1


def test_topk_and_transform_reject_bad_arguments(lib):
    p = ctypes.c_void_p(256)
    assert lib.nsa_topk_transform(p, 100, p, 4, 0, 100, N, 0, 4, N, 64, p, 16, N, 0,
                                  N) == -1                      # topk 0
    assert lib.nsa_topk_transform(p, 100, p, 4, 16, 100, p, 1, 4, p, 64, p, 16, N, 0,
                                  N) == -1                      # table stride
    assert lib.nsa_topk_transform(p, 100, p, 4, 16, 100, N, 0, 4, N, 64, p, 8, N, 0,
                                  N) == -1                      # out stride
    # exactly one table
    assert lib.nsa_page_table_transform(p, 8, 2, 8, p, 8, 8, p, 8, 8, 4, 64, p, p, 8,
                                        N) == -1
    assert lib.nsa_page_table_transform(p, 8, 2, 8, N, 0, 0, N, 0, 0, 4, 64, p, p, 8,
                                        N) == -1
    # zero rows is a no-op
    assert lib.nsa_topk_transform(N, 0, N, 0, 8, 0, N, 0, 4, N, 64, N, 8, N, 0, N) == 0
    ws = ctypes.c_size_t(99)
    assert lib.nsa_topk_workspace_size(4, 100, 16, ctypes.byref(ws)) == 0


def test_sparse_mla_rejects_bad_arguments(lib):
    p = ctypes.c_void_p(256)
    args = lambda **kw: dict(dict(q=p, ts=128 * 576, hs=576, kv=p, kvd=0, ns=1000,  # noqa: E731
                                  idx=p, istr=2048, sl=N, T=2, H=128, topk=2048,
                                  dqk=576, dv=512, sc=0.1, out=p, lse=N, ws=p,
                                  wsb=1 << 30, st=N), **kw)
    call = lambda a: lib.nsa_sparse_mla_decode(*a.values())  # noqa: E731
    assert call(args(H=24)) == -2              # not a multiple of 16
    assert call(args(H=144, ts=144 * 576)) == -2
    assert call(args(dqk=512)) == -2
    assert call(args(kvd=5)) == -2
    assert call(args(istr=1024)) == -1         # index stride < topk
    assert call(args(q=ctypes.c_void_p(258))) == -1
    assert call(args(hs=570)) == -1
    assert call(args(ws=N, wsb=0)) == -3       # decode plan needs a workspace
    assert "workspace" in _err(lib)
    size = ctypes.c_size_t(0)
    assert lib.nsa_sparse_mla_workspace_size(2, 128, 2048, 512, ctypes.byref(size)) == 0
    assert size.value > 0
    assert lib.nsa_sparse_mla_workspace_size(2, 100, 2048, 512, ctypes.byref(size)) == -1


def test_quantize_rejects_bad_arguments(lib):
    p = ctypes.c_void_p(256)
    assert lib.nsa_quantize_k_cache(p, 10, 500, p, N) == -1      # stride < 576
    assert lib.nsa_quantize_k_cache(ctypes.c_void_p(8), 10, 576, p, N) == -1
    assert lib.nsa_quantize_k_cache(N, 0, 576, N, N) == 0


def test_set_mla_kv_buffer_rejects_bad_arguments(lib):
    p, loc = ctypes.c_void_p(256), ctypes.c_void_p(512)
    ok = dict(k_nope=p, nope_stride=576, k_rope=ctypes.c_void_p(256 + 1024),
              rope_stride=576, cache_loc=loc, n=4, kv_cache=p,
              kv_dtype=1, num_slots=100, stream=N)
    f = lib.nsa_set_mla_kv_buffer
    call = lambda **kw: f(*{**ok, **kw}.values())
    assert call(n=0) == 0 and call(num_slots=0) == 0                # no-ops
    assert call(kv_dtype=7) == -2
    assert call(n=-1) == -1
    assert call(k_nope=N) == -1
    assert call(nope_stride=500) == -1                                # < 512
    assert call(nope_stride=580) == -1                                # not a multiple of 8
    assert call(k_nope=ctypes.c_void_p(264)) == -1                   # 8-byte aligned
    assert call(rope_stride=60) == -1
    assert call(k_rope=ctypes.c_void_p(257)) == -1                   # odd address
    # a bf16 cache copies rope with 16-byte moves
    assert call(kv_dtype=0, k_rope=ctypes.c_void_p(258)) == -1
    assert call(kv_dtype=0, rope_stride=580) == -1
    assert call(kv_cache=ctypes.c_void_p(8)) == -1
    assert "nsa_set_mla_kv_buffer" in lib.nsa_last_error().decode()


def test_binding_refuses_cpu_tensors():
    import torch
    import sparse_attention_decode_indexer_amd as nsa
    with pytest.raises(ValueError):
        nsa.nsa_quantize_k_cache(torch.zeros(4, 576, dtype=torch.bfloat16))


def test_fused_histogram_entry_points_validate(lib):
    P = ctypes.c_void_p
    # null key_hist
    assert lib.nsa_indexer_logits_hist(P(16), 2, P(16), P(16), 2, 10, P(16), 4, 4, P(16),
                                       P(16), 1, 64, 128, 64, 256, P(16), 256, N, 1, N) == -1
    assert "key_hist" in _err(lib)
    # the histogram needs the fp8 path
    assert lib.nsa_indexer_logits_hist(P(16), 0, P(16), P(16), 0, 10, P(16), 4, 4, P(16),
                                       P(16), 1, 4, 64, 64, 256, P(16), 256, P(16), 1, N) == -2
    # misaligned key_hist for the top-k
    assert lib.nsa_topk_transform_hist(P(16), 256, P(16), 1, 64, 256, N, 0, 4, N, 64,
                                       P(18), P(16), 64, N, 0, N) == -1
    assert "aligned" in _err(lib)
    # the split select's workspace: sized per row when rows exceed one
    # 16384-position segment, else 0; a given workspace too small is refused
    ws = ctypes.c_size_t(99)
    assert lib.nsa_topk_hist_workspace_size(4, 16384, 2048, ctypes.byref(ws)) == 0
    assert ws.value == 0
    assert lib.nsa_topk_hist_workspace_size(4, 16385, 2048, ctypes.byref(ws)) == 0
    assert ws.value == 4 * (16 + 2 * 516) * 4
    assert lib.nsa_topk_hist_workspace_size(4, 262145, 2048, ctypes.byref(ws)) == 0
    assert ws.value == 0
    assert lib.nsa_topk_hist_workspace_size(128, 65536, 2048, ctypes.byref(ws)) == 0
    assert ws.value == 128 * (16 + 2 * 2048) * 4
    assert lib.nsa_topk_hist_workspace_size(129, 65536, 2048, ctypes.byref(ws)) == 0
    assert ws.value == 0            # more rows: one block per row fills the GPU
    assert lib.nsa_topk_hist_workspace_size(-1, 65536, 2048, ctypes.byref(ws)) == -1
    assert lib.nsa_topk_transform_hist(P(16), 131072, P(16), 4, 2048, 131072, N, 0, 4, N,
                                       64, P(16), P(16), 2048, P(16), 4096, N) == -3
    assert lib.nsa_topk_transform_hist(P(16), 131072, P(16), 4, 2048, 131072, N, 0, 4, N,
                                       64, P(16), P(16), 2048, P(20), 1 << 22, N) == -1
    assert "aligned" in _err(lib)


def test_ragged_entry_points_validate(lib):
    p = ctypes.c_void_p(256)
    # metadata: nothing to do for empty inputs; null per-row outputs refused
    assert lib.nsa_ragged_extend_metadata(N, N, 0, N, N, 0, N, 0, 0, N, N, N, N, 0, N) == 0
    assert lib.nsa_ragged_extend_metadata(p, p, 2, p, p, 5, p, 4, 100, N, p, N, N, 0, N) == -1
    assert lib.nsa_ragged_extend_metadata(p, p, -1, p, p, 5, p, 4, 100, p, p, N, N, 0, N) == -1
    # flattened table: row stride below ceil(max_seqlen_k / 64)
    assert lib.nsa_ragged_extend_metadata(p, p, 2, p, p, 0, p, 1, 100, N, N, N, p, 10, N) == -1
    # index transform
    assert lib.nsa_ragged_index_transform(N, 0, 0, 8, N, N, 0, N) == 0
    assert lib.nsa_ragged_index_transform(p, 4, 3, 8, p, p, 8, N) == -1      # stride < topk
    assert lib.nsa_ragged_index_transform(p, 8, 3, 8, N, p, 8, N) == -1      # null offset
    # paged dequantization
    assert lib.nsa_dequantize_k_cache_paged(p, 10, p, 0, p, 576, N) == 0
    assert lib.nsa_dequantize_k_cache_paged(p, 10, p, 4, p, 570, N) == -1   # stride < 576
    assert lib.nsa_dequantize_k_cache_paged(p, 10, p, 4, p, 580, N) == -1   # not a multiple of 8
    assert lib.nsa_dequantize_k_cache_paged(p, 10, p, 4, ctypes.c_void_p(8), 576, N) == -1
    assert lib.nsa_dequantize_k_cache_paged(p, 10, N, 4, p, 576, N) == -1
    # CSR lists
    assert lib.nsa_valid_kv_indices(p, 8, 2, 8, N, p, 16, N) == -1           # null indptr
    assert lib.nsa_valid_kv_indices(p, 4, 2, 8, p, p, 16, N) == -1           # stride < topk
    assert lib.nsa_valid_kv_indices(p, 8, 2, 8, p, N, 16, N) == -1           # null kv_indices
    assert lib.nsa_valid_kv_indices(p, 8, -2, 8, p, p, 16, N) == -1
    assert "nsa_valid_kv_indices" in lib.nsa_last_error().decode()


def test_empty_batches_launch_nothing(lib):
    # no query rows (T = 0) or no slots: every compute entry point returns OK
    # before it touches a pointer, so NULL buffers are accepted
    P = ctypes.c_void_p
    f = ctypes.c_float
    assert lib.nsa_indexer_logits(N, 2, N, N, 2, 10, N, 4, 4, N, N, 0, 64, 128, 64,
                                  256, N, 256, N) == 0
    assert lib.nsa_indexer_logits_hist(N, 2, N, N, 2, 10, N, 4, 4, N, N, 0, 64, 128, 64,
                                       256, N, 256, N, 1, N) == 0
    assert lib.nsa_topk_transform(N, 0, N, 0, 64, 256, N, 0, 4, N, 64, N, 64, N, 0, N) == 0
    assert lib.nsa_topk_transform_hist(N, 0, N, 0, 64, 256, N, 0, 4, N, 64, N, N, 64, N,
                                       0, N) == 0
    assert lib.nsa_page_table_transform(N, 64, 0, 64, N, 0, 0, P(16), 4, 4, 4, 64, N, N,
                                        64, N) == 0
    for entry in (lib.nsa_sparse_mla_decode, lib.nsa_sparse_mla_extend):
        assert entry(N, 0, 576, N, 0, 0, N, 64, N, 0, 16, 64, 576, 512, f(0.1),
                     N, N, N, 0, N) == 0
    assert lib.nsa_quantize_k_cache(N, 0, 576, N, N) == 0
    assert _err(lib) == ""
