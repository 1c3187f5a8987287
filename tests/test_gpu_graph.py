"""The per-layer step captured as one HIP graph: metadata into static,
caller-owned buffers, the indexer with the fused top-k histogram, the top-k
with the page transform, sparse MLA. Every replay must equal the eager step
bit for bit, also after the request lengths are refreshed in place between
replays (no host sync, no re-capture) -- the graph-capturable metadata of
"nsa_backend.py (EngineX-Hygon sglang fork)", init_forward_metadata_replay_
cuda_graph, and "dsa_backend.py (sglang main)", the static metadata buffers
updated in place. Eager work and synchronisations run between the replays.
Every replay, the refreshed ones included, is also checked against the
oracle on rows spread over the requests: metadata bit-exact, logits, the
top-k acceptance, slots and attention."""

import pytest
import torch

import workloads as W
from helpers import DEV, need_gpu, note, idx_dtype, check_path_rows, spread_rows

pytestmark = pytest.mark.gpu


def make_step(nsa, w, hint=1):
    T = w.num_rows
    md = nsa.new_metadata_buffers(w.mode, w.bs, T, w.max_seqlen_k, DEV)
    logits = torch.empty(T, nsa.logits_row_stride(w.max_seqlen_k),
                         dtype=torch.float32, device=DEV)
    kh = nsa.new_key_hist(T, DEV)
    # the split top-k's bitmaps (batches of at most 128 rows longer than one
    # 16384-position segment: the reduced verify cases below)
    tk_ws = torch.empty(max(nsa.topk_hist_workspace_size(T, w.max_seqlen_k, w.topk), 16),
                        dtype=torch.uint8, device=DEV)
    slots = torch.empty(T, w.topk, dtype=torch.int32, device=DEV)
    if w.kv_kind == "fp8":
        cache, kvd = nsa.nsa_quantize_k_cache(w.kv_bf16), nsa.KV_FP8_656
    else:
        cache, kvd = w.kv_bf16, nsa.KV_BF16_576
    out = torch.empty(T, w.heads, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(T, w.heads, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(nsa.sparse_mla_workspace_size(T, w.heads, w.topk), 16),
                     dtype=torch.uint8, device=DEV)
    attn = (nsa.nsa_sparse_mla_extend if w.mode == W.MODE_EXTEND
            else nsa.nsa_sparse_mla_decode)

    def step():
        nsa.nsa_build_metadata(w.mode, w.seq_lens, w.req_to_token,
                               w.req_pool_indices, w.topk, w.max_seqlen_k, T,
                               extend_lens=w.extend_lens,
                               draft_token_num=w.draft, out=md)
        nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                               md["real_page_table"], md["token_to_req"],
                               md["seqlens_expanded"], w.max_seqlen_k,
                               logits=logits, dtype=idx_dtype(nsa, w), key_hist=kh,
                               rows_per_request=hint)
        nsa.nsa_topk_transform(logits, md["seqlens_expanded"], w.topk,
                               w.max_seqlen_k, table=md["real_page_table"],
                               token_to_req=md["token_to_req"], out=slots,
                               key_hist=kh, workspace=tk_ws)
        attn(w.q, cache, kvd, slots, w.sm_scale, md["nsa_cache_seqlens"],
             out=out, lse=lse, workspace=ws)

    def snapshot():
        return dict(seqlens_expanded=md["seqlens_expanded"].clone(),
                    nsa_cache_seqlens=md["nsa_cache_seqlens"].clone(),
                    slots=slots.clone(), out=out.clone(), lse=lse.clone(),
                    key_hist_sum=int(kh.sum()))

    def scribble():   # eager work between replays; outputs must be rewritten
        slots.fill_(-7)
        out.fill_(3.0)
        lse.fill_(-1.0)

    def against_oracle(what):
        rows = spread_rows(w, 12)
        err, _ = check_path_rows(w, md, logits, None, slots, cache, out, lse, rows,
                                 check_cache=False)
        note(f"  {what}: {len(rows)} rows match the oracle (max logit error {err:.2e})")

    return step, snapshot, scribble, against_oracle


def assert_same(got, want, what):
    for k in want:
        if isinstance(want[k], torch.Tensor):
            assert torch.equal(got[k], want[k]), f"{what}: {k} differs from eager"
        else:
            assert got[k] == want[k], f"{what}: {k} {got[k]} != {want[k]}"


@pytest.mark.parametrize("name,overrides,hint", [
    ("decode_b32", {}, 1),
    ("verify", dict(bs=8, seqlen_range=(16384, 32768)), 1),
    # the verify launch of the benchmark: four rows per indexer block
    ("verify", dict(bs=8, seqlen_range=(16384, 32768)), 4),
])
def test_step_graph_replays_match_eager_and_oracle(name, overrides, hint):
    nsa = need_gpu()
    w = W.make_workload(name, device=DEV, **overrides)
    note(f"graph: {name} T={w.num_rows} H={w.heads} kv={w.kv_kind} hint={hint} "
         f"split top-k={nsa.topk_hist_workspace_size(w.num_rows, w.max_seqlen_k, w.topk) > 0}")
    step, snapshot, scribble, against_oracle = make_step(nsa, w, hint)
    step()
    torch.cuda.synchronize()
    ref = snapshot()
    assert ref["key_hist_sum"] == 0
    against_oracle("eager step")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        scribble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(snapshot(), ref, f"{name} replay {rep}")
        against_oracle(f"replay {rep}")
        step()                      # eager step between replays
        torch.cuda.synchronize()

    # refresh the request lengths in place: shorter contexts, same pages
    gen = torch.Generator(device="cpu").manual_seed(7)
    cut = torch.randint(1, 4000, (w.bs,), generator=gen).to(DEV, torch.int32)
    w.seq_lens.copy_(torch.clamp(w.seq_lens - cut, min=1))
    step()
    torch.cuda.synchronize()
    ref2 = snapshot()
    assert not torch.equal(ref2["seqlens_expanded"], ref["seqlens_expanded"])
    against_oracle("eager step after the refresh")
    for rep in range(2):
        scribble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(snapshot(), ref2, f"{name} refreshed replay {rep}")
        against_oracle(f"refreshed replay {rep}")
