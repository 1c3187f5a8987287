"""Shared pieces of the GPU parity tests: device workloads, oracle-side views
of the same inputs, and the acceptance checks with their tolerances.

Tolerances:
* metadata, page transform, fp8 cache bytes: bit-exact.
* indexer logits: |gpu - oracle| <= 256 * 2^-24 * A, with A = |kscale| *
  sum_h |w_h| * sum_d |q_hd k_d| (computed in float64 next to the oracle).
  The products of two fp8 values are exact in fp32; a sum of n fp32 terms in
  any order is within (n - 1) * 2^-24 of the sum of |terms|, and the kernels
  add 128 products per head, then 64 weighted heads, then scale once, so
  (127 + 1 + 63 + 1 + 1) * 2^-24 * A bounds the error; 256 leaves margin.
  ReLU is 1-Lipschitz, so an error before it is not amplified. Rows without
  a computed A (none in the parity tests) fall back to 1e-3 + 1e-4 |oracle|.
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

LOGIT_ATOL, LOGIT_RTOL = 1e-3, 1e-4      # fallback only (no |terms| sum given)
LOGIT_SUM_ULPS = 256                      # error bound in units of 2^-24 * A
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
    return oracle_logits_and_bounds(w, ref_md, rows)[0]


def oracle_logits_and_bounds(w, ref_md, rows):
    """(logits, A) per row: the oracle's logits and, from the same decoded
    values, A[s] = |kscale_s| * sum_h |w_h| * sum_d |q_hd k_sd|, the sum of
    absolute terms that bounds the fp32 summation error (see the module
    docstring)."""
    out, bounds = {}, {}
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
        wt = w.idx_weights[t:t + 1].cpu().numpy()
        out[t] = oracle.indexer.indexer_logits(q64, wt, keys, ks, local, [0], [L], L)[0]
        kf = np.abs(keys.reshape(-1, keys.shape[-1])[:L])           # [L, Di]
        absdots = np.abs(q64[0]) @ kf.T                              # [Hi, L]
        bounds[t] = np.abs(ks.reshape(-1)[:L]) * (np.abs(wt[0].astype(np.float64)) @ absdots)
    return out, bounds


def check_logits(got_row, ref_row, L, what="", abs_sum=None):
    """Logits of one row within tolerance; returns (max |err|, max |err| /
    (2^-24 A)) for the report (the second is None without A)."""
    g, r = got_row[:L].astype(np.float64), ref_row[:L]
    err = np.abs(g - r)
    if abs_sum is not None:
        ulps = np.asarray(abs_sum[:L]) * 2.0 ** -24
        bound = LOGIT_SUM_ULPS * ulps
    else:
        bound = LOGIT_ATOL + LOGIT_RTOL * np.abs(r)
    bad = np.nonzero(err > bound)[0]
    assert len(bad) == 0, (f"{what}: {len(bad)} logits out of tolerance, first at "
                           f"{bad[:5]} got {g[bad[:5]]} want {r[bad[:5]]}")
    if L == 0:
        return 0.0, 0.0 if abs_sum is not None else None
    ratio = None
    if abs_sum is not None:
        nz = ulps > 0
        ratio = float((err[nz] / ulps[nz]).max()) if nz.any() else 0.0
    return float(err.max()), ratio


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


def positions_from_slots(slot_row, rpt_row, L):
    """Logical positions of a row of physical slots through the request's
    compact page table (pages of one request are distinct)."""
    npg = (L + 63) // 64
    col = {int(p): c for c, p in enumerate(np.asarray(rpt_row[:npg]))}
    out = np.full(len(slot_row), -1, np.int64)
    for j, sl in enumerate(slot_row):
        if sl >= 0:
            out[j] = col[int(sl) >> 6] * 64 + (int(sl) & 63)
    return out


def check_path_rows(w, md, logits, logical, slots, cache, out, lse, rows,
                    check_cache=True):
    """The whole path on `rows` against the oracle: metadata bit-exact (every
    row), logits within the |terms| bound, the top-k acceptance (count,
    uniqueness, range, ascending order, every kept score >= the oracle's k-th
    - slack), slots == the oracle transform of the kept positions, attention
    on the GPU's own slot lists within the dtype's bar. `logical` may be None
    (fused path only): the positions are then recovered from the slots
    through the oracle's page table. Returns the largest logit error and
    error / (2^-24 A) seen."""
    ref = oracle_metadata(w)
    for f in ("seqlens_expanded", "nsa_cache_seqlens", "token_to_req", "nsa_cu_seqlens_k"):
        np.testing.assert_array_equal(md[f].cpu().numpy(), ref[f], err_msg=f)
    L_all = ref["seqlens_expanded"]
    rpt_gpu = md["real_page_table"].cpu().numpy()
    for r in range(w.bs):
        n = (int(ref["cache_seqlens"][r]) + 63) // 64
        np.testing.assert_array_equal(rpt_gpu[r, :n], ref["real_page_table"][r, :n],
                                      err_msg=f"real_page_table row {r}")
    ref_logits, bounds = oracle_logits_and_bounds(w, ref, rows)
    lg = logits.cpu().numpy() if logits.numel() < (1 << 26) else None
    sel_all = logical.cpu().numpy() if logical is not None else None
    sl_all = slots.cpu().numpy()
    worst = [0.0, 0.0]
    for t in rows:
        L = int(L_all[t])
        row = lg[t] if lg is not None else logits[t].cpu().numpy()
        e, ratio = check_logits(row, ref_logits[t], L, what=f"{w.name} logits row {t}",
                                abs_sum=bounds[t])
        worst[0] = max(worst[0], e)
        worst[1] = max(worst[1], ratio or 0.0)
        r = int(ref["token_to_req"][t])
        sel = (sel_all[t] if sel_all is not None
               else positions_from_slots(sl_all[t], ref["real_page_table"][r], L))
        check_topk_row(sel, L, w.topk, ref_scores=ref_logits[t],
                       what=f"{w.name} topk row {t}")
        want_slots = oracle.transform.transform_compact(sel[None], ref["real_page_table"],
                                                        ref["token_to_req"][t:t + 1])
        np.testing.assert_array_equal(sl_all[t], want_slots[0], err_msg=f"slots row {t}")
    # attention on the GPU's own slot lists (identical indices)
    idx = sl_all[rows]
    kvrows = oracle_kv_rows(w, idx.reshape(-1))
    if w.kv_kind == "fp8" and check_cache:
        used = np.unique(idx[idx >= 0])[:512]
        ui = torch.as_tensor(used, device=DEV)
        want = oracle.quant.quantize_k_cache(
            w.kv_bf16[ui].view(torch.int16).cpu().numpy().view(np.uint16))
        np.testing.assert_array_equal(cache[ui].cpu().numpy(), want)
    q64 = w.q[torch.as_tensor(rows, device=DEV)].to(torch.float64).cpu().numpy()
    o_ref, lse_ref = oracle.sparse_mla.sparse_mla(
        q64, kvrows, idx, w.sm_scale, nsa_cache_seqlens=ref["nsa_cache_seqlens"][rows])
    ri = torch.as_tensor(rows, device=DEV)
    check_attention(out[ri].float().cpu().numpy(), lse[ri].cpu().numpy(), o_ref,
                    lse_ref, w.kv_kind, what=w.name)
    return worst


def spread_rows(w, n):
    """About n rows spread over the batch: every request's first and last
    row where there are few requests, else evenly spaced rows, plus the
    longest and shortest row."""
    ref = oracle_metadata(w)
    L = ref["seqlens_expanded"]
    t2r = ref["token_to_req"]
    rows = {0, w.num_rows - 1, int(np.argmax(L)), int(np.argmin(L))}
    if w.bs <= n // 2:
        for r in range(w.bs):
            ts = np.nonzero(t2r == r)[0]
            if len(ts):
                rows |= {int(ts[0]), int(ts[-1]), int(ts[len(ts) // 2])}
    step = max(1, w.num_rows // n)
    rows |= set(range(0, w.num_rows, step))
    return sorted(rows)
