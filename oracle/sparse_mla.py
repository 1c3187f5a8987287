"""Sparse MLA attention over the selected KV slots -- oracle, test
infrastructure.

The semantic reference on the pages is the FA3 route ("nsa_backend.py
(EngineX-Hygon sglang fork)", ``_forward_fa3``; same in "dsa_backend.py
(sglang main)"): the latent cache row is split into ``c_kv = kv[:512]`` (the
value, and the no-rope part of the key) and ``k_rope = kv[512:]``; the query
into ``q_nope`` (512) and ``q_rope`` (64); the score is
``q_rope . k_rope + q_nope . c_kv`` scaled by ``sm_scale``; the value is
``c_kv``; the key set of a row is the first ``nsa_cache_seqlens[t]`` entries of
its transformed (physical-slot) table. The FlashMLA routes take the same
inputs as one 576-wide query and key (``q_all``, ``indices``, ``sm_scale``,
``d_v = 512``) and return the output and, for the decode kernel, the
log-sum-exp.

So, per query row t and head h, with I_t the valid (non -1) selected slots:

    s_i = sm_scale * sum_{d < 576} q[t, h, d] * K_i[d]
    o[t, h, :] = sum_i softmax(s)_i * K_i[:512]
    lse[t, h] = log sum_i exp(s_i)

Readings: no logit soft-cap; an empty I_t gives o = 0 and lse = -inf; the
order of I_t does not matter.
"""

import numpy as np


def sparse_mla(q, cache, indices, sm_scale, d_v=512, nsa_cache_seqlens=None):
    """``q``: ``[T, H, 576]`` float64; ``cache``: an object with ``rows(slots)
    -> [n, 576] float64`` (see ``quant.Bf16Cache`` / ``quant.Fp8Cache``);
    ``indices``: ``[T, topk]`` physical slots, -1 = unused.
    Returns ``(o [T, H, d_v], lse [T, H])`` in float64."""
    q = np.asarray(q, dtype=np.float64)
    idx = np.asarray(indices, dtype=np.int64)
    T, H, _ = q.shape
    o = np.zeros((T, H, d_v))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        row = idx[t]
        if nsa_cache_seqlens is not None:
            row = row[:int(nsa_cache_seqlens[t])]
        sel = row[row >= 0]
        if len(sel) == 0:
            continue
        K = cache.rows(sel)                       # [n, 576]
        s = sm_scale * (q[t] @ K.T)               # [H, n]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        den = e.sum(axis=1, keepdims=True)
        o[t] = (e @ K[:, :d_v]) / den
        lse[t] = m[:, 0] + np.log(den[:, 0])
    return o, lse
