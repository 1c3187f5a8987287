"""MI355X (gfx950) sparse-attention decode step: Python binding of libnsa.so.

Every step of the path runs in the library's HIP kernels; this module only
marshals arguments: it checks torch tensors (device, dtype, contiguity),
allocates outputs with torch when none are given, and passes raw pointers and
the current HIP stream to the C ABI declared in include/nsa.h. There is no
fallback: if the library is missing, the calls raise.

Names follow the C entry points. Constants mirror nsa.h.
"""

import ctypes

import torch

from ._lib import NsaError, call, load  # noqa: F401

MODE_DECODE, MODE_EXTEND, MODE_TARGET_VERIFY = 0, 1, 2
MODE_DRAFT_EXTEND, MODE_DRAFT_EXTEND_V2 = 3, 4
DTYPE_FP32, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2
KV_BF16_576, KV_FP8_656 = 0, 1
PAGE_SIZE, D_QK, D_V = 64, 576, 512


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(t, name, dtype=None, ndim=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def new_metadata_buffers(mode, bs, num_q_rows, max_seqlen_k, device,
                         want_page_table_1=False):
    """Caller-owned metadata outputs for ``nsa_build_metadata(out=...)``:
    static buffers that a captured graph keeps referring to while the inputs
    (seq_lens, req_to_token, ...) are refreshed in place between replays."""
    i32 = torch.int32
    T = int(num_q_rows)
    ncols = (max_seqlen_k + PAGE_SIZE - 1) // PAGE_SIZE
    nq = bs + 1 if mode == MODE_EXTEND else T + 1
    out = dict(
        cache_seqlens=torch.empty(bs, dtype=i32, device=device),
        cu_seqlens_k=torch.empty(bs + 1, dtype=i32, device=device),
        cu_seqlens_q=torch.empty(nq, dtype=i32, device=device),
        seqlens_expanded=torch.empty(T, dtype=i32, device=device),
        nsa_cache_seqlens=torch.empty(T, dtype=i32, device=device),
        nsa_cu_seqlens_k=torch.empty(T + 1, dtype=i32, device=device),
        nsa_cu_seqlens_q=torch.empty(T + 1, dtype=i32, device=device),
        real_page_table=torch.empty(bs, max(ncols, 1), dtype=i32, device=device),
        token_to_req=torch.empty(T, dtype=i32, device=device),
    )
    if want_page_table_1:
        out["page_table_1"] = torch.empty(bs, max(max_seqlen_k, 1), dtype=i32,
                                          device=device)
    return out


def nsa_build_metadata(mode, seq_lens, req_to_token, req_pool_indices, topk,
                       max_seqlen_k, num_q_rows, extend_lens=None,
                       draft_token_num=0, page_size=PAGE_SIZE,
                       want_page_table_1=False, out=None):
    """Per-forward metadata (one kernel launch). Returns a dict of int32
    device tensors named as in nsa.h: ``out`` (from new_metadata_buffers)
    when given, else newly allocated ones."""
    i32 = torch.int32
    _check(seq_lens, "seq_lens", i32, 1)
    _check(req_to_token, "req_to_token", i32, 2)
    _check(req_pool_indices, "req_pool_indices", i32, 1)
    if extend_lens is not None:
        _check(extend_lens, "extend_lens", i32, 1)
    bs = seq_lens.numel()
    T = int(num_q_rows)
    dev = seq_lens.device
    if out is None:
        out = new_metadata_buffers(mode, bs, T, max_seqlen_k, dev,
                                   want_page_table_1)
    else:
        ncols = (max_seqlen_k + PAGE_SIZE - 1) // PAGE_SIZE
        nq = bs + 1 if mode == MODE_EXTEND else T + 1
        sizes = dict(cache_seqlens=bs, cu_seqlens_k=bs + 1, cu_seqlens_q=nq,
                     seqlens_expanded=T, nsa_cache_seqlens=T,
                     nsa_cu_seqlens_k=T + 1, nsa_cu_seqlens_q=T + 1,
                     token_to_req=T)
        for k, n in sizes.items():
            _check(out[k], k, i32, 1)
            if out[k].numel() < n:
                raise ValueError(f"out[{k!r}] needs at least {n} entries")
        tables = dict(real_page_table=max(ncols, 1))
        if want_page_table_1:
            if "page_table_1" not in out:
                raise ValueError("out has no 'page_table_1'")
            tables["page_table_1"] = max(max_seqlen_k, 1)
        for k, cols in tables.items():
            _check(out[k], k, i32, 2)
            if out[k].shape[0] < bs or out[k].shape[1] < cols:
                raise ValueError(f"out[{k!r}] must be at least [{bs}, {cols}]")
    pt1 = out.get("page_table_1") if want_page_table_1 else None
    if req_pool_indices.numel() < bs:
        raise ValueError("req_pool_indices needs an entry per request")
    if extend_lens is not None and extend_lens.numel() < bs:
        raise ValueError("extend_lens needs an entry per request")
    if bs and req_to_token.shape[1] < max_seqlen_k:
        raise ValueError("req_to_token needs max_seqlen_k columns")
    call("nsa_build_metadata", mode, bs, draft_token_num, topk, page_size,
         _ptr(seq_lens), _ptr(extend_lens), _ptr(req_to_token),
         req_to_token.stride(0), req_to_token.shape[0], _ptr(req_pool_indices),
         max_seqlen_k, T,
         _ptr(out["cache_seqlens"]), _ptr(out["cu_seqlens_k"]),
         _ptr(out["cu_seqlens_q"]), _ptr(out["seqlens_expanded"]),
         _ptr(out["nsa_cache_seqlens"]), _ptr(out["nsa_cu_seqlens_k"]),
         _ptr(out["nsa_cu_seqlens_q"]), _ptr(out["real_page_table"]),
         out["real_page_table"].stride(0), _ptr(out["token_to_req"]),
         _ptr(pt1), pt1.stride(0) if pt1 is not None else 0, _stream())
    return out


def logits_row_stride(max_seqlen_k):
    """Row stride (elements) for a logits buffer: max_seqlen_k rounded up to a
    multiple of 64 so every row starts 256-byte aligned (vector loads in
    top-k, whole-line stores in the indexer)."""
    return max(64, (max_seqlen_k + 63) // 64 * 64)


KEY_BINS = 4096


def new_key_hist(T, device):
    """A zeroed [T, 4096] key histogram (int32 storage of uint32 counts) for
    the fused indexer / top-k pair; the top-k clears it again after use."""
    return torch.zeros(T, KEY_BINS, dtype=torch.int32, device=device)


def nsa_indexer_logits(q, weights, index_cache, real_page_table, token_to_req,
                       seqlens_expanded, max_seqlen_k, logits=None,
                       dtype=DTYPE_FP8_E4M3, key_hist=None, rows_per_request=1):
    """Indexer logits [T, >= max_seqlen_k] fp32 (positions past each row's
    length are left unwritten). ``q``: [T, Hi, Di] uint8 fp8 codes (dtype
    DTYPE_FP8_E4M3) or float32 (DTYPE_FP32). With ``key_hist`` (zeroed, see
    new_key_hist) the logits' top-k histogram is counted in the same pass,
    and ``rows_per_request`` (draft_token_num for target-verify and
    draft-extend v2) lets a request's rows share their key-page reads; it
    does not change the results."""
    _check(q, "q", torch.uint8 if dtype == DTYPE_FP8_E4M3 else torch.float32, 3)
    _check(weights, "weights", torch.float32, 2)
    _check(index_cache, "index_cache", torch.uint8, 2)
    _check(real_page_table, "real_page_table", torch.int32, 2)
    _check(token_to_req, "token_to_req", torch.int32, 1)
    _check(seqlens_expanded, "seqlens_expanded", torch.int32, 1)
    T, Hi, Di = q.shape
    if tuple(weights.shape) != (T, Hi):
        raise ValueError(f"weights must be [{T}, {Hi}]")
    if token_to_req.numel() < T or seqlens_expanded.numel() < T:
        raise ValueError("token_to_req / seqlens_expanded need an entry per row")
    if real_page_table.shape[1] < (max_seqlen_k + PAGE_SIZE - 1) // PAGE_SIZE:
        raise ValueError("real_page_table needs ceil(max_seqlen_k / 64) columns")
    if logits is None:
        logits = torch.empty(T, logits_row_stride(max_seqlen_k),
                             dtype=torch.float32, device=q.device)
    _check(logits, "logits", torch.float32, 2, contiguous=False)
    if logits.shape[0] < T or logits.shape[1] < max_seqlen_k or logits.stride(1) != 1:
        raise ValueError(f"logits must be [>= {T}, >= {max_seqlen_k}] with unit column stride")
    args = (_ptr(q), dtype, _ptr(weights), _ptr(index_cache), dtype,
            index_cache.shape[0], _ptr(real_page_table), real_page_table.stride(0),
            real_page_table.shape[0], _ptr(token_to_req), _ptr(seqlens_expanded),
            T, Hi, Di, PAGE_SIZE, max_seqlen_k, _ptr(logits), logits.stride(0))
    if key_hist is None:
        call("nsa_indexer_logits", *args, _stream())
    else:
        _check(key_hist, "key_hist", torch.int32, 2)
        if key_hist.shape[0] < T or key_hist.shape[1] != KEY_BINS:
            raise ValueError("key_hist must be [>= T, 4096]")
        call("nsa_indexer_logits_hist", *args, _ptr(key_hist), int(rows_per_request),
             _stream())
    return logits


def topk_hist_workspace_size(T, max_seqlen_k, topk):
    """Bytes of the optional workspace of the top-k with key_hist (0: unused)."""
    ws = ctypes.c_size_t(0)
    call("nsa_topk_hist_workspace_size", int(T), int(max_seqlen_k), int(topk),
         ctypes.byref(ws))
    return ws.value


def nsa_topk_transform(logits, lengths, topk, max_seqlen_k, table=None,
                       token_to_req=None, out=None, key_hist=None,
                       workspace=None, split=True):
    """Top-k positions per row (ascending position order, -1 padded), or
    physical slots when ``table`` (the compact page table) is given. With
    ``key_hist`` (filled by nsa_indexer_logits on the same logits) the logits
    are read once and key_hist is cleared for reuse; long rows are then
    split over many blocks through ``workspace`` (uint8, at least
    topk_hist_workspace_size bytes; allocated here when not given), unless
    ``split`` is False."""
    _check(lengths, "lengths", torch.int32, 1)
    T = lengths.numel()
    if logits is not None:
        _check(logits, "logits", torch.float32, 2, contiguous=False)
        if logits.shape[0] < T or logits.shape[1] < max_seqlen_k or logits.stride(1) != 1:
            raise ValueError(f"logits must be [>= {T}, >= {max_seqlen_k}] with unit column stride")
    if table is not None:
        _check(table, "table", torch.int32, 2)
        _check(token_to_req, "token_to_req", torch.int32, 1)
        if token_to_req.numel() < T:
            raise ValueError("token_to_req needs an entry per row")
        if table.shape[1] < (max_seqlen_k + PAGE_SIZE - 1) // PAGE_SIZE:
            raise ValueError("table needs ceil(max_seqlen_k / 64) columns")
    if out is None:
        out = torch.empty(T, topk, dtype=torch.int32, device=lengths.device)
    _check(out, "out", torch.int32, 2, contiguous=False)
    if out.shape[0] < T or out.shape[1] < topk or out.stride(1) != 1:
        raise ValueError(f"out must be [>= {T}, >= {topk}] with unit column stride")
    trows = table.shape[0] if table is not None else 0
    if key_hist is not None:
        _check(key_hist, "key_hist", torch.int32, 2)
        if key_hist.shape[0] < T or key_hist.shape[1] != KEY_BINS:
            raise ValueError("key_hist must be [>= T, 4096]")
        need = topk_hist_workspace_size(T, max_seqlen_k, topk) if split else 0
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=lengths.device)
        if not need:
            workspace = None
        if workspace is not None:
            _check(workspace, "workspace", torch.uint8, 1)
        call("nsa_topk_transform_hist", _ptr(logits),
             logits.stride(0) if logits is not None else 0, _ptr(lengths), T, topk,
             max_seqlen_k, _ptr(table), table.stride(0) if table is not None else 0,
             trows, _ptr(token_to_req), PAGE_SIZE, _ptr(key_hist), _ptr(out),
             out.stride(0), _ptr(workspace),
             workspace.numel() if workspace is not None else 0, _stream())
        return out
    ws = ctypes.c_size_t(0)
    call("nsa_topk_workspace_size", T, max_seqlen_k, topk, ctypes.byref(ws))
    work = (torch.empty(ws.value, dtype=torch.uint8, device=lengths.device)
            if ws.value else None)
    call("nsa_topk_transform", _ptr(logits),
         logits.stride(0) if logits is not None else 0, _ptr(lengths), T, topk,
         max_seqlen_k, _ptr(table), table.stride(0) if table is not None else 0,
         trows, _ptr(token_to_req), PAGE_SIZE, _ptr(out), out.stride(0), _ptr(work),
         ws.value, _stream())
    return out


def nsa_page_table_transform(topk_indices, token_to_req, page_table_1=None,
                             real_page_table=None, out=None):
    """Logical positions -> physical slots (-1 kept). Give exactly one table."""
    _check(topk_indices, "topk_indices", torch.int32, 2, contiguous=False)
    _check(token_to_req, "token_to_req", torch.int32, 1)
    T, K = topk_indices.shape
    if token_to_req.numel() < T:
        raise ValueError("token_to_req needs an entry per row")
    if topk_indices.stride(1) != 1:
        raise ValueError("topk_indices must have unit column stride")
    if out is None:
        out = torch.empty(T, K, dtype=torch.int32, device=topk_indices.device)
    _check(out, "out", torch.int32, 2, contiguous=False)
    if out.shape[0] < T or out.shape[1] < K or out.stride(1) != 1:
        raise ValueError(f"out must be [>= {T}, >= {K}] with unit column stride")
    pt1_stride = pt1_width = rpt_stride = rpt_width = rows = 0
    for tab in (page_table_1, real_page_table):
        if tab is not None and tab.stride(1) != 1:
            raise ValueError("page tables must have unit column stride")
    if page_table_1 is not None:
        _check(page_table_1, "page_table_1", torch.int32, 2, contiguous=False)
        pt1_stride, pt1_width = page_table_1.stride(0), page_table_1.shape[1]
        rows = page_table_1.shape[0]
    if real_page_table is not None:
        _check(real_page_table, "real_page_table", torch.int32, 2, contiguous=False)
        rpt_stride, rpt_width = real_page_table.stride(0), real_page_table.shape[1]
        rows = real_page_table.shape[0]
    call("nsa_page_table_transform", _ptr(topk_indices), topk_indices.stride(0),
         T, K, _ptr(page_table_1), pt1_stride, pt1_width, _ptr(real_page_table),
         rpt_stride, rpt_width, rows, PAGE_SIZE, _ptr(token_to_req), _ptr(out),
         out.stride(0), _stream())
    return out


def sparse_mla_workspace_size(T, H, topk):
    ws = ctypes.c_size_t(0)
    call("nsa_sparse_mla_workspace_size", T, H, topk, D_V, ctypes.byref(ws))
    return ws.value


def _sparse_mla(name, q, kv_cache, kv_dtype, indices, sm_scale,
                nsa_cache_seqlens, out, lse, workspace, want_lse):
    _check(q, "q", torch.bfloat16, 3, contiguous=False)
    if q.stride(2) != 1:
        raise ValueError("q must be contiguous in its last dimension")
    T, H, dqk = q.shape
    if kv_dtype == KV_BF16_576:
        _check(kv_cache, "kv_cache", torch.bfloat16, 2)
    else:
        _check(kv_cache, "kv_cache", torch.uint8, 2)
    _check(indices, "indices", torch.int32, 2, contiguous=False)
    if nsa_cache_seqlens is not None:
        _check(nsa_cache_seqlens, "nsa_cache_seqlens", torch.int32, 1)
    topk = indices.shape[1]
    if indices.shape[0] < T or indices.stride(1) != 1:
        raise ValueError(f"indices must be [>= {T}, topk] with unit column stride")
    if nsa_cache_seqlens is not None and nsa_cache_seqlens.numel() < T:
        raise ValueError("nsa_cache_seqlens needs an entry per row")
    if out is None:
        out = torch.empty(T, H, D_V, dtype=torch.bfloat16, device=q.device)
    _check(out, "out", torch.bfloat16, 3)
    if tuple(out.shape) != (T, H, D_V):
        raise ValueError(f"out must be [{T}, {H}, {D_V}]")
    if lse is None and want_lse:
        lse = torch.empty(T, H, dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, 2)
        if tuple(lse.shape) != (T, H):
            raise ValueError(f"lse must be [{T}, {H}]")
    need = sparse_mla_workspace_size(T, H, topk)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    call(name, _ptr(q), q.stride(0), q.stride(1), _ptr(kv_cache), kv_dtype,
         kv_cache.shape[0], _ptr(indices), indices.stride(0),
         _ptr(nsa_cache_seqlens), T, H, topk, dqk, D_V, float(sm_scale),
         _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream())
    return out, lse


def nsa_sparse_mla_decode(q, kv_cache, kv_dtype, indices, sm_scale,
                          nsa_cache_seqlens=None, out=None, lse=None,
                          workspace=None, want_lse=True):
    """Sparse MLA over selected slots (decode / verify rows): returns
    (out [T, H, 512] bf16, lse [T, H] fp32 or None)."""
    return _sparse_mla("nsa_sparse_mla_decode", q, kv_cache, kv_dtype, indices,
                       sm_scale, nsa_cache_seqlens, out, lse, workspace, want_lse)


def nsa_sparse_mla_extend(q, kv_cache, kv_dtype, indices, sm_scale,
                          nsa_cache_seqlens=None, out=None, lse=None,
                          workspace=None, want_lse=True):
    """Sparse MLA for many query rows (chunked extend)."""
    return _sparse_mla("nsa_sparse_mla_extend", q, kv_cache, kv_dtype, indices,
                       sm_scale, nsa_cache_seqlens, out, lse, workspace, want_lse)


def nsa_check_device_errors():
    """Waits for the current stream and returns (then clears) the
    NSA_DEVERR_* bits the kernels recorded on this device: 0 when no kernel
    met an out-of-range id. Synchronises with the host: for tests and debug
    paths, not for captured graphs."""
    lib = load()
    st = lib.nsa_check_device_errors(_stream())
    if st < 0:
        raise NsaError("nsa_check_device_errors", st, lib.nsa_last_error().decode())
    return st


DEVERR_PAGE_ID, DEVERR_SLOT, DEVERR_REQUEST, DEVERR_POOL_ROW, DEVERR_INDEX = (
    0x1, 0x2, 0x4, 0x8, 0x10)


def nsa_quantize_k_cache(kv_bf16, out=None):
    """bf16 latent cache [slots, >=576] -> fp8 block-scaled [slots, 656] uint8."""
    _check(kv_bf16, "kv_bf16", torch.bfloat16, 2, contiguous=False)
    if kv_bf16.stride(1) != 1:
        raise ValueError("kv_bf16 rows must be contiguous")
    n = kv_bf16.shape[0]
    if out is None:
        out = torch.empty(n, 656, dtype=torch.uint8, device=kv_bf16.device)
    _check(out, "out", torch.uint8, 2)
    call("nsa_quantize_k_cache", _ptr(kv_bf16), n, kv_bf16.stride(0), _ptr(out),
         _stream())
    return out


def nsa_set_mla_kv_buffer(k_nope, k_rope, cache_loc, kv_cache, kv_dtype):
    """Write new latent rows into their cache slots, in place: row i of
    k_nope [n, >=512] / k_rope [n, >=64] (bf16, rows contiguous) goes to slot
    cache_loc[i] (int32; out-of-range entries skipped) of kv_cache
    ([slots, 656] uint8 for KV_FP8_656, quantized as nsa_quantize_k_cache
    does; [slots, 576] bf16 for KV_BF16_576). Returns kv_cache."""
    for t, name in ((k_nope, "k_nope"), (k_rope, "k_rope")):
        _check(t, name, torch.bfloat16, 2, contiguous=False)
        if t.stride(1) != 1:
            raise ValueError(f"{name} rows must be contiguous")
    _check(cache_loc, "cache_loc", torch.int32, 1)
    n = cache_loc.numel()
    if k_nope.shape[0] < n or k_rope.shape[0] < n:
        raise ValueError("k_nope / k_rope need a row per cache_loc entry")
    if kv_dtype == KV_FP8_656:
        _check(kv_cache, "kv_cache", torch.uint8, 2)
    else:
        _check(kv_cache, "kv_cache", torch.bfloat16, 2)
    call("nsa_set_mla_kv_buffer", _ptr(k_nope), k_nope.stride(0), _ptr(k_rope),
         k_rope.stride(0), _ptr(cache_loc), n, _ptr(kv_cache), kv_dtype,
         kv_cache.shape[0], _stream())
    return kv_cache


# ---- RAGGED extend route ----------------------------------------------------

def nsa_ragged_extend_metadata(md, max_seqlen_k, total_k, want_flat=True):
    """RAGGED-route metadata of an extend batch from nsa_build_metadata's
    outputs ``md``: ks / ke (each row's window in the concatenated keys),
    topk_indices_offset (= ks) and, with ``want_flat``,
    page_table_1_flattened [total_k] (every cached token's slot, request after
    request). ``total_k`` is the host-known sum of the cache lengths (the
    pages' seq_lens_sum); ``max_seqlen_k`` the bound given to
    nsa_build_metadata."""
    i32 = torch.int32
    T = md["seqlens_expanded"].numel()
    bs = md["cache_seqlens"].numel()
    dev = md["seqlens_expanded"].device
    out = dict(ks=torch.empty(T, dtype=i32, device=dev),
               ke=torch.empty(T, dtype=i32, device=dev),
               topk_indices_offset=torch.empty(T, dtype=i32, device=dev))
    flat = torch.empty(max(int(total_k), 0), dtype=i32, device=dev) if want_flat else None
    rpt = md["real_page_table"]
    call("nsa_ragged_extend_metadata", _ptr(md["cu_seqlens_k"]),
         _ptr(md["cache_seqlens"]), bs, _ptr(md["seqlens_expanded"]),
         _ptr(md["token_to_req"]), T, _ptr(rpt), rpt.stride(0), max_seqlen_k,
         _ptr(out["ks"]), _ptr(out["ke"]), _ptr(out["topk_indices_offset"]),
         _ptr(flat) if flat is not None and flat.numel() else None,
         flat.numel() if flat is not None else 0, _stream())
    if flat is not None:
        out["page_table_1_flattened"] = flat
    return out


def nsa_ragged_index_transform(topk_indices, offset, out=None):
    """Shift valid top-k positions [T, topk] by offset[T] (-1 kept)."""
    _check(topk_indices, "topk_indices", torch.int32, 2)
    _check(offset, "offset", torch.int32, 1)
    T, k = topk_indices.shape
    if out is None:
        out = torch.empty_like(topk_indices)
    _check(out, "out", torch.int32, 2)
    call("nsa_ragged_index_transform", _ptr(topk_indices), topk_indices.stride(0),
         T, k, _ptr(offset), _ptr(out), out.stride(0), _stream())
    return out


def nsa_dequantize_k_cache_paged(kv_fp8, slots, out=None):
    """bf16 latent rows [n, 576] of the fp8 cache rows ``slots`` [n]."""
    _check(kv_fp8, "kv_fp8", torch.uint8, 2)
    _check(slots, "slots", torch.int32, 1)
    n = slots.numel()
    if out is None:
        out = torch.empty(n, 576, dtype=torch.bfloat16, device=slots.device)
    _check(out, "out", torch.bfloat16, 2, contiguous=False)
    call("nsa_dequantize_k_cache_paged", _ptr(kv_fp8), kv_fp8.shape[0], _ptr(slots),
         n, _ptr(out), out.stride(0), _stream())
    return out


def nsa_valid_kv_indices(indices, capacity=None):
    """CSR lists of the entries != -1 of ``indices`` [T, topk]: (kv_indptr
    [T+1], kv_indices [capacity]); ``capacity`` defaults to T * topk."""
    _check(indices, "indices", torch.int32, 2)
    T, k = indices.shape
    cap = T * k if capacity is None else int(capacity)
    indptr = torch.empty(T + 1, dtype=torch.int32, device=indices.device)
    flat = torch.empty(max(cap, 1), dtype=torch.int32, device=indices.device)
    call("nsa_valid_kv_indices", _ptr(indices), indices.stride(0), T, k,
         _ptr(indptr), _ptr(flat), cap, _stream())
    return indptr, flat[:cap]
