"""Indexer logits ("paged MQA logits") -- oracle, test infrastructure.

What the pages fix: the indexer scores every cached position of a query row
against that row's query with many heads sharing one key per position ("MQA"),
reads the index-key cache through the 64-token page table
(``get_page_table_64`` / ``real_page_table``), and takes the row's visible
length from the expanded seqlens ("nsa_backend.py (EngineX-Hygon sglang
fork)", ``NSAIndexerMetadata``; "dsa_backend.py (sglang main)",
``DSAIndexerMetadata`` and ``_to_2d_context_lens``, which feeds the paged MQA
logits kernel one context length per query row).

What they leave open -- the scoring formula itself (the indexer module is not
on the pages). Reading adopted, the DeepSeek sparse-attention "lightning
indexer":

    logit[t, s] = kscale[s] * sum_h  w[t, h] * max(0, q[t, h, :] . k[s, :])

with q and k in fp8 e4m3 (fp32 for the tiny configuration, where kscale = 1),
``w`` the per-head weights (any query-side scale folded in by the caller) and
``kscale`` the per-token fp32 scale stored next to the fp8 key. Because the
pages never show it, this formula is a reading: the tests pin this oracle's
implementation of it (closed forms, brute force, page-order invariance), not
the reading. Positions s >= L_t are not scored (returned as -inf here).

Index-key cache page layout (a choice): each 64-token
page holds 64 rows of ``Di`` key elements (fp8 codes, or fp32 for the tiny
configuration) followed by 64 little-endian fp32 per-token scales.
"""

import numpy as np

from .formats import e4m3_decode, f32_bits_to_f64

KIND_FP8 = "fp8"
KIND_FP32 = "fp32"


def index_page_bytes(di, kind, page_size=64):
    elem = 1 if kind == KIND_FP8 else 4
    return page_size * di * elem + page_size * 4


def decode_index_pages(raw, di, kind, page_size=64):
    """Raw index-key cache ``[num_pages, page_bytes]`` (uint8) -> keys
    ``[num_pages, page_size, di]`` and scales ``[num_pages, page_size]``, both
    float64 (exact)."""
    raw = np.asarray(raw, dtype=np.uint8)
    n = raw.shape[0]
    if kind == KIND_FP8:
        kbytes = page_size * di
        keys = e4m3_decode(raw[:, :kbytes]).reshape(n, page_size, di)
    else:
        kbytes = page_size * di * 4
        keys = f32_bits_to_f64(raw[:, :kbytes]).reshape(n, page_size, di)
    scales = f32_bits_to_f64(raw[:, kbytes:kbytes + page_size * 4])
    return keys, scales.reshape(n, page_size)


def indexer_logits(q, w, keys, kscales, real_page_table, token_to_req,
                   seqlens_expanded, max_seqlen_k, page_size=64):
    """Logits ``[T, max_seqlen_k]`` in float64; -inf at positions >= L_t.

    q: ``[T, Hi, Di]`` float64 (decoded), w: ``[T, Hi]``, keys/kscales: the
    decoded cache (``decode_index_pages``).
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T = q.shape[0]
    out = np.full((T, max_seqlen_k), -np.inf)
    for t in range(T):
        r = int(token_to_req[t])
        L = int(min(seqlens_expanded[t], max_seqlen_k))
        if L <= 0:
            continue
        s = np.arange(L)
        pages = np.asarray(real_page_table[r], dtype=np.int64)[s // page_size]
        offs = s % page_size
        k = keys[pages, offs]          # [L, Di]: the key of every position
        ks = kscales[pages, offs]      # [L]
        dots = q[t] @ k.T              # [Hi, L]
        relu = np.maximum(dots, 0.0)
        out[t, :L] = ks * (w[t] @ relu)
    return out
