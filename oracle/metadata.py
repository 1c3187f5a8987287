"""Per-forward metadata of the sparse attention step (oracle, test infrastructure).

Follows the metadata construction on the pages:

* "nsa_backend.py (EngineX-Hygon sglang fork)", ``NSAMetadata`` (field
  meanings), ``compute_cu_seqlens``, ``_transform_table_1_to_real`` and
  ``NativeSparseAttnBackend.init_forward_metadata`` (decode and extend
  branches).
* "dsa_backend.py (sglang main)", ``DeepseekSparseAttnBackend.
  init_forward_metadata`` (decode, target-verify and extend branches) and
  ``_cal_indexer_k_start_end`` (the per-token batch index).
* "nsa_backend.py (sglang 0.5.3rc2 -> 0.5.4 diff)", target-verify metadata.
* Draft-extend (the speculative draft model's forward): "dsa_backend.py
  (sglang main)", ``init_forward_metadata``, the draft-extend branch (v1:
  each request extends by its own accepted count + 1; v2: every request by
  the fixed number of draft tokens, ``seq_lens`` already counting them), and
  the v2 branch of ``init_forward_metadata_replay_cuda_graph``.

Readings where the pages are silent:

* ``compute_nsa_seqlens`` is not shown; the field comment says the result is
  the expanded seqlens limited to topk, read as an elementwise minimum.
* Target-verify rows: one query row per draft token (``cu_seqlens_q`` steps by
  one, ``max_seqlen_q`` is 1), as the sglang-main page builds it.
* Draft-extend rows: as on the sglang-main page, one query row per token
  (``cu_seqlens_q`` steps by one, ``max_seqlen_q`` is 1) and the cache
  lengths are ``seq_lens`` themselves (the 0.5.4 diff instead adds the draft
  count to ``seq_lens`` and steps ``cu_seqlens_q`` per request).
* ``seqlens_expand_triton`` is not shown; read as the per-request expansion
  the 0.5.4 diff writes out for draft-extend: a request with q_len rows and
  kv_len cached tokens gives rows kv_len - q_len + 1 .. kv_len.
* ``real_page_table`` keeps one row per request; query rows reach it through
  ``token_to_req`` (the pages repeat the row once per draft token instead; the
  values seen by every query row are the same).
"""

import numpy as np

MODE_DECODE = 0
MODE_EXTEND = 1
MODE_TARGET_VERIFY = 2
MODE_DRAFT_EXTEND = 3
MODE_DRAFT_EXTEND_V2 = 4


def compute_cu_seqlens(seqlens):
    """[0, cumsum(seqlens)] -- ``compute_cu_seqlens`` (pad a cumulative sum
    with a leading zero)."""
    s = np.asarray(seqlens, dtype=np.int64)
    return np.concatenate([np.zeros(1, np.int64), np.cumsum(s)])


def transform_table_1_to_real(page_table_1, page_size):
    """Token-granular table -> page-granular table: every ``page_size``-th
    column, floor-divided by ``page_size`` (``_transform_table_1_to_real``)."""
    pt = np.asarray(page_table_1, dtype=np.int64)
    if page_size == 1:
        return pt.copy()
    return pt[:, 0::page_size] // page_size


def build_metadata(mode, seq_lens, req_to_token, req_pool_indices, topk,
                   page_size=64, extend_lens=None, draft_token_num=0,
                   max_seqlen_k=None):
    """All metadata tensors of one forward pass, as int64 numpy arrays.

    Arguments follow the pages' ForwardBatch fields: ``seq_lens`` are the
    per-request KV lengths (for extend and draft-extend: including the new
    tokens; for target-verify: excluding the draft tokens), ``extend_lens``
    the per-request number of new tokens (extend and draft-extend v1),
    ``draft_token_num`` the fixed per-request count of target-verify and
    draft-extend v2, ``req_to_token`` the
    ``[pool, max_ctx]`` token -> slot table and ``req_pool_indices`` each
    request's row in it. ``max_seqlen_k`` is the host-side bound that sizes the
    tables (default: the batch maximum of the cache seqlens, as the pages
    compute it).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    rtt = np.asarray(req_to_token, dtype=np.int64)
    rpi = np.asarray(req_pool_indices, dtype=np.int64)
    bs = len(seq_lens)

    d = draft_token_num if mode == MODE_TARGET_VERIFY else 0
    cache_seqlens = seq_lens + d
    cu_seqlens_k = compute_cu_seqlens(cache_seqlens)
    if max_seqlen_k is None:
        max_seqlen_k = int(cache_seqlens.max()) if bs else 0
    page_table = rtt[rpi, :max_seqlen_k]

    if mode == MODE_DECODE:
        q_lens = np.ones(bs, np.int64)
        cu_seqlens_q = np.arange(bs + 1, dtype=np.int64)
        seqlens_expanded = cache_seqlens.copy()
        max_seqlen_q = 1
    elif mode == MODE_TARGET_VERIFY:
        q_lens = np.full(bs, d, np.int64)
        cu_seqlens_q = np.arange(bs * d + 1, dtype=np.int64)
        # every draft token of request r is a query row whose visible length
        # runs from kv_len - D + 1 up to kv_len, with kv_len = seq_len + D
        parts = [np.arange(kv - d + 1, kv + 1, dtype=np.int64)
                 for kv in cache_seqlens]
        seqlens_expanded = (np.concatenate(parts) if parts
                            else np.zeros(0, np.int64))
        max_seqlen_q = 1
    elif mode == MODE_EXTEND:
        ext = np.asarray(extend_lens, dtype=np.int64)
        q_lens = ext
        prefix_lens = seq_lens - ext
        if np.any(prefix_lens):
            cu_seqlens_q = compute_cu_seqlens(ext)
            max_seqlen_q = int(ext.max()) if bs else 1
        else:
            cu_seqlens_q = cu_seqlens_k.copy()
            max_seqlen_q = max_seqlen_k
        parts = [np.arange(kv - qo + 1, kv + 1, dtype=np.int64)
                 for qo, kv in zip(ext, seq_lens)]
        seqlens_expanded = (np.concatenate(parts) if parts
                            else np.zeros(0, np.int64))
    elif mode in (MODE_DRAFT_EXTEND, MODE_DRAFT_EXTEND_V2):
        if mode == MODE_DRAFT_EXTEND:
            q_lens = np.asarray(extend_lens, dtype=np.int64)
        else:
            q_lens = np.full(bs, draft_token_num, np.int64)
        cu_seqlens_q = np.arange(int(q_lens.sum()) + 1, dtype=np.int64)
        parts = [np.arange(kv - qo + 1, kv + 1, dtype=np.int64)
                 for qo, kv in zip(q_lens, cache_seqlens)]
        seqlens_expanded = (np.concatenate(parts) if parts
                            else np.zeros(0, np.int64))
        max_seqlen_q = 1
    else:
        raise ValueError(f"unsupported mode {mode}")

    nsa_cache_seqlens = np.minimum(seqlens_expanded, topk)
    nsa_cu_seqlens_k = compute_cu_seqlens(nsa_cache_seqlens)
    nsa_cu_seqlens_q = np.arange(len(nsa_cu_seqlens_k), dtype=np.int64)
    token_to_req = np.repeat(np.arange(bs, dtype=np.int64), q_lens)

    return dict(
        cache_seqlens=cache_seqlens,
        cu_seqlens_k=cu_seqlens_k,
        cu_seqlens_q=cu_seqlens_q,
        seqlens_expanded=seqlens_expanded,
        nsa_cache_seqlens=nsa_cache_seqlens,
        nsa_cu_seqlens_k=nsa_cu_seqlens_k,
        nsa_cu_seqlens_q=nsa_cu_seqlens_q,
        page_table_1=page_table,
        real_page_table=transform_table_1_to_real(page_table, page_size),
        token_to_req=token_to_req,
        max_seqlen_q=max_seqlen_q,
        max_seqlen_k=max_seqlen_k,
    )


def indexer_k_start_end(seq_lens, extend_lens):
    """Per-token logits windows over the concatenated keys of an extend batch
    (``_cal_indexer_k_start_end``): token j of request i gets
    ``ks = sum(seq_lens[:i])`` and ``ke = ks + (seq_len_i - ext_i + 1 + j)``.
    Returned with the per-token batch index."""
    ks, ke, tb = [], [], []
    k_off = 0
    for i, (sl, el) in enumerate(zip(seq_lens, extend_lens)):
        for j in range(el):
            ks.append(k_off)
            ke.append(k_off + sl - el + 1 + j)
            tb.append(i)
        k_off += sl
    return (np.asarray(ks, np.int64), np.asarray(ke, np.int64),
            np.asarray(tb, np.int64))
