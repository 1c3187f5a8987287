"""The allocation-free sparse MLA entry point (nsa_sparse_mla_decode_noalloc,
workspace in the library's static device array) against nsa_sparse_mla_decode
with a caller-owned workspace: the same plan and kernels, so the outputs must
be bit-identical. Two calls in a row share the static array; the second has
fewer rows, so stale contents of the first call must not leak into it."""

import ctypes

import pytest
import torch

import workloads as W
from helpers import DEV, need_gpu, note

pytestmark = pytest.mark.gpu


def _noalloc(nsa, q, cache, kvd, idx, sm_scale, seqlens, out, lse):
    T, H, dqk = q.shape
    nsa.call("nsa_sparse_mla_decode_noalloc",
             ctypes.c_void_p(q.data_ptr()), q.stride(0), q.stride(1),
             ctypes.c_void_p(cache.data_ptr()), kvd, cache.shape[0],
             ctypes.c_void_p(idx.data_ptr()), idx.stride(0),
             ctypes.c_void_p(seqlens.data_ptr() if seqlens is not None else 0),
             T, H, idx.shape[1], dqk, nsa.D_V, ctypes.c_float(sm_scale),
             ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _slots(nsa, w):
    md = nsa.nsa_build_metadata(w.mode, w.seq_lens, w.req_to_token, w.req_pool_indices,
                                w.topk, w.max_seqlen_k, w.num_rows,
                                draft_token_num=w.draft)
    lg = nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                                md["real_page_table"], md["token_to_req"],
                                md["seqlens_expanded"], w.max_seqlen_k)
    slots = nsa.nsa_topk_transform(lg, md["seqlens_expanded"], w.topk, w.max_seqlen_k,
                                   table=md["real_page_table"],
                                   token_to_req=md["token_to_req"])
    return slots, md["nsa_cache_seqlens"]


@pytest.mark.parametrize("name,big,small", [
    ("decode_b32", 24, 5),        # 16 heads, bf16 cache: the narrow kernel, KV splits
    ("decode_b128", 6, 2),        # 128 heads, fp8 cache: the 128-head kernel, KV splits
])
def test_noalloc_matches_caller_workspace_twice(name, big, small):
    nsa = need_gpu()
    w = W.make_workload(name, device=DEV, bs=big, seqlen_range=(3000, 9000))
    fp8 = w.kv_kind == "fp8"
    cache = nsa.nsa_quantize_k_cache(w.kv_bf16) if fp8 else w.kv_bf16
    kvd = nsa.KV_FP8_656 if fp8 else nsa.KV_BF16_576
    slots, seqlens = _slots(nsa, w)
    for T in (big, small):
        q, idx, sl = w.q[:T].contiguous(), slots[:T].contiguous(), seqlens[:T].contiguous()
        note(f"noalloc {name}: T={T} H={w.heads} kv={w.kv_kind}")
        need = nsa.sparse_mla_workspace_size(T, w.heads, w.topk)
        assert need > 0, "the shape must use a workspace"
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        ref_o, ref_l = nsa.nsa_sparse_mla_decode(q, cache, kvd, idx, w.sm_scale, sl,
                                                 workspace=ws)
        out = torch.full((T, w.heads, 512), 5.0, dtype=torch.bfloat16, device=DEV)
        lse = torch.full((T, w.heads), 9.0, dtype=torch.float32, device=DEV)
        _noalloc(nsa, q, cache, kvd, idx, w.sm_scale, sl, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"{name} T={T}: out differs"
        assert torch.equal(lse, ref_l), f"{name} T={T}: lse differs"
