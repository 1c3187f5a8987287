"""Length-masked top-k over indexer logits -- oracle, test infrastructure.

Follows "nsa_backend.py (EngineX-Hygon sglang fork)",
``NSAIndexerMetadata.topk_transform``: the selection gets the logits and the
expanded seqlens as ``lengths`` and returns ``topk`` indices per row; the
``nsa_cache_seqlens_int32`` field comment (its lengths are limited to topk) fixes that a row
keeps ``min(L, topk)`` positions. Unused entries are -1, the padding value the
pages use for index rows ("dsa_backend.py (sglang main)",
``_pad_topk_indices``).

Readings: output order inside the valid prefix is not fixed by the pages
(valid entries first, then -1). Ties at the threshold may be broken either
way; this oracle breaks them by ascending position so that it is
deterministic.
"""

import numpy as np


def topk_row(scores, length, topk):
    """Indices of the ``min(length, topk)`` largest ``scores[:length]``
    (score-descending, ties by ascending position), then -1 up to ``topk``."""
    n = int(length)
    out = np.full(topk, -1, dtype=np.int64)
    if n <= 0:
        return out
    if n <= topk:
        out[:n] = np.arange(n)
        return out
    s = np.asarray(scores[:n], dtype=np.float64)
    order = np.lexsort((np.arange(n), -s))  # primary: -score, then position
    out[:] = order[:topk]
    return out


def topk(logits, lengths, topk):
    """Row-wise ``topk_row``: ``[T, topk]`` int64."""
    T = len(lengths)
    return np.stack([topk_row(logits[t], lengths[t], topk) for t in range(T)]) \
        if T else np.zeros((0, topk), np.int64)


def kth_largest(scores, length, topk):
    """The score a selection must reach: the ``topk``-th largest of
    ``scores[:length]`` (or -inf when the row keeps every position)."""
    n = int(length)
    if n <= topk:
        return -np.inf
    return np.sort(np.asarray(scores[:n], np.float64))[::-1][topk - 1]
