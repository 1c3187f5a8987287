"""RAGGED extend route (oracle, test infrastructure).

"dsa_backend.py (sglang main)" has a second prefill route besides the paged
one: the indexer scores every extend token against the *concatenated* keys of
the batch, the top-k positions are shifted into that concatenation, and the
attention reads a contiguous bf16 copy of the batch's latent rows.

* ``init_forward_metadata``, extend branch: ``page_table_1_flattened`` is the
  concatenation over requests of ``page_table[i, :kv_len]`` (the physical
  slot of every cached token, request after request), and
  ``topk_indices_offset`` repeats ``cu_seqlens_k[:-1]`` once per extend token.
* ``_cal_indexer_k_start_end``: token j of request i gets the logits window
  ``[ks, ke)`` with ``ks`` = the keys of the requests before it and
  ``ke = ks + seqlens_expanded``; its batch index is i (worked example in the
  method's comment).
* ``forward_extend``, RAGGED: valid top-k positions (not -1) get the token's
  offset added; ``dequantize_k_cache_paged(kv_cache, page_table_1_flattened)``
  turns the fp8 cache rows of the flattened table into the bf16 latent rows
  the attention reads.
* The aiter decode route's ``get_valid_kv_indices``: CSR lists of the valid
  entries of an index matrix, ``kv_indptr[1:] = cumsum(count of != -1 per
  row)`` and the valid entries of every row, in order, concatenated.

Readings: the body of ``dequantize_k_cache_paged`` is
not shown; each value is read as the fp32 product of its e4m3 code and block
scale rounded to bf16 (nearest even), the rope values copied, and a slot
outside the cache giving a zero row.
"""

import numpy as np

from .formats import e4m3_decode

D_NOPE, D_ROPE, BLOCK = 512, 64, 128


def ragged_metadata(cache_seqlens, seqlens_expanded, token_to_req, req_to_token,
                    req_pool_indices):
    """ks, ke, topk_indices_offset and page_table_1_flattened of an extend
    batch, from the per-forward metadata and the token -> slot table."""
    cache_seqlens = np.asarray(cache_seqlens, np.int64)
    se = np.asarray(seqlens_expanded, np.int64)
    t2r = np.asarray(token_to_req, np.int64)
    rtt = np.asarray(req_to_token, np.int64)
    rpi = np.asarray(req_pool_indices, np.int64)
    k_start = np.concatenate([[0], np.cumsum(cache_seqlens)[:-1]]).astype(np.int64)
    ks = k_start[t2r] if len(t2r) else np.zeros(0, np.int64)
    ke = ks + se
    offset = ks.copy()
    flat = [rtt[rpi[i], :kv] for i, kv in enumerate(cache_seqlens)]
    flat = np.concatenate(flat) if flat else np.zeros(0, np.int64)
    return dict(ks=ks, ke=ke, topk_indices_offset=offset,
                page_table_1_flattened=flat)


def ragged_index_transform(topk_indices, offset):
    """Logical top-k positions -> positions in the concatenated keys:
    ``where(idx != -1, idx + offset[t], -1)``."""
    idx = np.asarray(topk_indices, np.int64)
    off = np.asarray(offset, np.int64)[:, None]
    return np.where(idx != -1, idx + off, -1)


def _f32_to_bf16_bits(x):
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def dequantize_k_cache_paged(cache, slots):
    """fp8 cache rows ``[num_slots, 656]`` gathered by ``slots`` -> bf16 bit
    patterns ``[n, 576]``: each no-rope value is the fp32 product of its e4m3
    code and its block's fp32 scale, rounded to bf16 (nearest even); the rope
    bf16 values are copied; a slot outside the cache gives zeros."""
    cache = np.ascontiguousarray(np.asarray(cache, np.uint8))
    slots = np.asarray(slots, np.int64)
    out = np.zeros((len(slots), D_NOPE + D_ROPE), np.uint16)
    ok = (slots >= 0) & (slots < cache.shape[0])
    rows = cache[slots[ok]]
    codes = e4m3_decode(rows[:, :D_NOPE]).astype(np.float32)          # exact
    scales = np.ascontiguousarray(rows[:, D_NOPE:D_NOPE + 16]).view("<f4")
    prod = codes * np.repeat(scales, BLOCK, axis=1).astype(np.float32)  # fp32 product
    out[ok, :D_NOPE] = _f32_to_bf16_bits(prod)
    out[ok, D_NOPE:] = np.ascontiguousarray(rows[:, D_NOPE + 16:]).view("<u2")
    return out


def valid_kv_indices(indices):
    """CSR lists of the entries != -1 of an index matrix ``[T, K]``:
    ``(kv_indptr [T+1], kv_indices [kv_indptr[T]])``, rows in order and the
    entries of each row in their column order."""
    idx = np.asarray(indices, np.int64)
    valid = idx != -1
    indptr = np.concatenate([[0], np.cumsum(valid.sum(axis=1))]).astype(np.int64)
    flat = idx[valid]          # row-major order: rows, then columns
    return indptr, flat
