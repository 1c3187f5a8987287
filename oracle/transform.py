"""Logical position -> physical KV slot -- oracle, test infrastructure.

Follows "nsa_backend.py (EngineX-Hygon sglang fork)": ``forward_decode`` /
``forward_extend`` pass ``page_table_1`` (the token-granular slot table,
"always with page_size = 1") and the top-k indices to
``transform_index_page_table_decode/prefill``, and the fused top-k variant
returns the same physical table directly (``NSAIndexerMetadata.
topk_transform``). The transform body is not on the pages; reading: slot =
``page_table_1[request of the row, index]``, with -1 passed through.

The compact form reaches the same slot through the 64-token page table
(``real_page_table[r, p] = page_table_1[r, 64 p] // 64``, see
``_transform_table_1_to_real``): ``real_page_table[r, i // 64] * 64 + i % 64``.
The two agree whenever a request's tokens fill whole pages in order, which
is how a paged allocator with page size 64 lays them out ("dsa_backend.py
(sglang main)", ``dsa_drop_wide_page_table``: the wide table is dropped and
only the compact one kept).
"""

import numpy as np


def transform_wide(topk_indices, page_table_1, token_to_req):
    """slot[t, j] = page_table_1[req(t), idx[t, j]], or -1 where idx < 0."""
    idx = np.asarray(topk_indices, dtype=np.int64)
    pt = np.asarray(page_table_1, dtype=np.int64)
    req = np.asarray(token_to_req, dtype=np.int64)[:, None]
    safe = np.where(idx >= 0, idx, 0)
    return np.where(idx >= 0, pt[req, safe], -1)


def transform_compact(topk_indices, real_page_table, token_to_req, page_size=64):
    """slot[t, j] = real_page_table[req(t), i // 64] * 64 + i % 64, or -1."""
    idx = np.asarray(topk_indices, dtype=np.int64)
    rpt = np.asarray(real_page_table, dtype=np.int64)
    req = np.asarray(token_to_req, dtype=np.int64)[:, None]
    safe = np.where(idx >= 0, idx, 0)
    slot = rpt[req, safe // page_size] * page_size + safe % page_size
    return np.where(idx >= 0, slot, -1)
