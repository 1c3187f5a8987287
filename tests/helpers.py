"""Shared pieces of the GPU parity tests: device workloads, oracle-side views
of the same inputs, and the acceptance checks with their tolerances.

Tolerances:
* metadata, page transform, fp8 cache bytes: bit-exact.
* indexer logits: |gpu - oracle| <= 1e-3 + 1e-4 * |oracle| (fp32 sums of exact
  fp8 products; the error bound is ~(128 + 64) * 2^-24 of the sum of |terms|).
* top-k: count == min(L, topk), unique, in [0, L), ascending, and every
  selected position's oracle score >= the oracle's topk-th score - 1e-3.
* attention (identical indices): per row max|o - o_ref| / max|o_ref| <= 2e-2
  (bf16 KV) or 5e-2 (fp8 KV); |lse - lse_ref| <= 1e-2.
"""

import functools

import numpy as np
import pytest
import torch

import workloads as W
import oracle

LOGIT_ATOL, LOGIT_RTOL = 1e-3, 1e-4
TOPK_SLACK = 1e-3
ATTN_TOL = {"bf16": 2e-2, "fp8": 5e-2}
LSE_ATOL = 1e-2

DEV = torch.device("cuda:0")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_indexer_amd as nsa
    nsa.load()
    return nsa


def note(msg):
    print(msg, flush=True)


def to_dev(w):
    """Moves a CPU-built workload's tensors to the GPU (in place)."""
    for k in ("seq_lens", "extend_lens", "req_to_token", "req_pool_indices",
              "q_idx", "idx_weights", "index_cache", "q", "kv_bf16"):
        v = getattr(w, k)
        if v is not None:
            setattr(w, k, v.to(DEV))
    return w


def oracle_metadata(w):
    h = {k: (v.cpu().numpy() if v is not None else None) for k, v in dict(
        seq_lens=w.seq_lens, extend_lens=w.extend_lens,
        req_to_token=w.req_to_token, req_pool_indices=w.req_pool_indices).items()}
    return oracle.metadata.build_metadata(
        w.mode, h["seq_lens"], h["req_to_token"], h["req_pool_indices"], w.topk,
        extend_lens=h["extend_lens"], draft_token_num=w.draft,
        max_seqlen_k=w.max_seqlen_k)


def gpu_metadata(nsa, w, **kw):
    return nsa.nsa_build_metadata(w.mode, w.seq_lens, w.req_to_token,
                                  w.req_pool_indices, w.topk, w.max_seqlen_k,
                                  w.num_rows, extend_lens=w.extend_lens,
                                  draft_token_num=w.draft, **kw)


def idx_dtype(nsa, w):
    return nsa.DTYPE_FP8_E4M3 if w.idx_kind == "fp8" else nsa.DTYPE_FP32


def oracle_logits_rows(w, ref_md, rows):
    """Oracle logits for a subset of rows, decoding only the pages they use."""
    out = {}
    rpt = ref_md["real_page_table"]
    for t in rows:
        r = int(ref_md["token_to_req"][t])
        L = int(min(ref_md["seqlens_expanded"][t], w.max_seqlen_k))
        npg = (L + 63) // 64
        pages = rpt[r, :npg]
        raw = w.index_cache[torch.as_tensor(pages, device=w.index_cache.device)].cpu().numpy()
        keys, ks = oracle.indexer.decode_index_pages(raw, w.idx_dim, w.idx_kind)
        q = w.q_idx[t:t + 1].cpu()
        if w.idx_kind == "fp8":
            q64 = oracle.formats.e4m3_decode(q.numpy())
        else:
            q64 = q.numpy().astype(np.float64)
        local = np.arange(npg)[None, :]
        out[t] = oracle.indexer.indexer_logits(
            q64, w.idx_weights[t:t + 1].cpu().numpy(), keys, ks, local, [0], [L],
            L)[0]
    return out


def check_logits(got_row, ref_row, L, what=""):
    g, r = got_row[:L].astype(np.float64), ref_row[:L]
    err = np.abs(g - r)
    bound = LOGIT_ATOL + LOGIT_RTOL * np.abs(r)
    bad = np.nonzero(err > bound)[0]
    assert len(bad) == 0, (f"{what}: {len(bad)} logits out of tolerance, first at "
                           f"{bad[:5]} got {g[bad[:5]]} want {r[bad[:5]]}")


def check_topk_row(sel, L, topk, ref_scores=None, what=""):
    """Acceptance of one top-k row of logical positions."""
    n = min(L, topk)
    valid, pad = sel[:n], sel[n:]
    assert (pad == -1).all(), f"{what}: entries past min(L, topk) must be -1"
    assert ((valid >= 0) & (valid < L)).all(), f"{what}: index out of [0, L)"
    assert (np.diff(valid) > 0).all(), f"{what}: not unique / not ascending"
    if ref_scores is not None and L > topk:
        kth = oracle.topk.kth_largest(ref_scores, L, topk)
        worst = ref_scores[valid].min()
        assert worst >= kth - TOPK_SLACK, f"{what}: selected {worst} < kth {kth}"


class CacheFromRows:
    """Oracle cache view over a dict slot -> float64 row."""

    def __init__(self, rows):
        self.r = rows

    def rows(self, slots):
        return np.stack([self.r[int(s)] for s in slots])


def oracle_kv_rows(w, slots):
    """float64 latent rows for the given slots, decoded by the oracle from the
    generator's bf16 cache (for fp8, quantized by the oracle first)."""
    slots = np.unique(np.asarray(slots, np.int64))
    slots = slots[slots >= 0]
    bits = w.kv_bf16[torch.as_tensor(slots, device=w.kv_bf16.device)] \
        .view(torch.int16).cpu().numpy().view(np.uint16)
    if w.kv_kind == "fp8":
        vals = oracle.quant.dequantize_rows(oracle.quant.quantize_k_cache(bits))
    else:
        vals = oracle.formats.bf16_bits_to_f64(bits)
    return CacheFromRows({int(s): vals[i] for i, s in enumerate(slots)})


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref, kind, what=""):
    tol = ATTN_TOL[kind]
    for t in range(o_ref.shape[0]):
        den = np.abs(o_ref[t]).max()
        if den == 0:
            assert np.abs(o_gpu[t]).max() == 0, f"{what} row {t}: expected zeros"
            continue
        rel = np.abs(o_gpu[t] - o_ref[t]).max() / den
        assert rel <= tol, f"{what} row {t}: rel err {rel:.3e} > {tol}"
    if lse_gpu is not None:
        fin = np.isfinite(lse_ref)
        assert (np.isfinite(lse_gpu) == fin).all(), f"{what}: lse finiteness"
        if fin.any():
            d = np.abs(lse_gpu[fin] - lse_ref[fin]).max()
            assert d <= LSE_ATOL, f"{what}: lse err {d}"


@functools.lru_cache(maxsize=1)
def full_workload(name):
    """Full-size workload generated on the GPU (cached for the session)."""
    return W.make_workload(name, device=DEV, seed=0)


def host_key_hist(logits_row, n):
    """Histogram of the top 12 bits of the order-preserving key (NaN lowest,
    -0 == +0) over positions [0, n): the definition stated in nsa.h."""
    x = np.ascontiguousarray(logits_row[:n], dtype=np.float32)
    u = x.view(np.uint32).copy()
    u[x == 0] = 0
    neg = (u & 0x80000000) != 0
    key = np.where(neg, ~u, u | 0x80000000).astype(np.uint32)
    key[np.isnan(x)] = 0
    return np.bincount(key >> 20, minlength=4096)
