"""Seeded synthetic inputs for the sparse-attention decode path.

Shared by the tests, the benchmark and the oracle checks. This module holds
input generation only -- random draws, the page allocator's layout and byte
packing of the cache formats -- and none of the method's arithmetic. The fp8
and bf16 roundings of the random draws are torch's own casts.

Workloads (shapes and distributions of the workloads described with the
sparse-attention backend pages; every value is synthetic and seed-fixed):

* ``tiny``        decode, batch 2, KV lengths [300, 700], topk 256; indexer 4
                  heads x 64 dims fp32 (N(0,1)), per-head weights U(0,1), key
                  scales 1; MLA 16 heads, latent 512 + 64 rope, values N(0,1)
                  rounded once to bf16.
* ``decode_b32``  decode, batch 32, lengths U{4096..16384}, topk 2048; indexer
                  64 x 128 fp8 e4m3 of N(0,1) * 0.5 with per-token fp32 scales
                  U(0.5, 1.5); MLA 16 heads, bf16 KV.
* ``decode_b128`` decode, batch 128, lengths U{32768..131072}, topk 2048;
                  indexer as above; MLA 128 heads, fp8 block-scaled KV.
* ``extend``      chunked extend, 4 requests, extend lengths
                  [512, 1024, 2048, 4096] on prefixes [8192, 16384, 24576,
                  32768]; MLA 16 heads, bf16 KV; indexer as above.
* ``verify``      speculative target-verify, batch 64, 4 draft tokens,
                  prefixes U{16384..131072}; MLA 128 heads, fp8 KV.
* ``draft_extend`` / ``draft_extend_v2``  the draft model's extend after a
                  verify of 4 draft tokens, batch 64, KV lengths (already
                  counting the new tokens) U{16384..131072}: v1 extends each
                  request by its accepted count + 1, drawn U{1..4}; v2 by
                  all 4. MLA 128 heads, fp8 KV (the verify configuration).

Pages of every request come from one seed-fixed random permutation of the
page pool (random physical page order); ``req_to_token[row, s] = page(s // 64)
* 64 + s % 64`` inside a request's pages and 0 beyond them.
"""

from dataclasses import dataclass, field
import math

import torch

MODE_DECODE = 0
MODE_EXTEND = 1
MODE_TARGET_VERIFY = 2
MODE_DRAFT_EXTEND = 3
MODE_DRAFT_EXTEND_V2 = 4

PAGE = 64
D_NOPE = 512
D_ROPE = 64
D_QK = D_NOPE + D_ROPE

CONFIGS = {
    "tiny": dict(mode=MODE_DECODE, bs=2, seq_lens=[300, 700], topk=256,
                 idx_heads=4, idx_dim=64, idx_kind="fp32", heads=16, kv="bf16"),
    "decode_b32": dict(mode=MODE_DECODE, bs=32, seqlen_range=(4096, 16384),
                       topk=2048, idx_heads=64, idx_dim=128, idx_kind="fp8",
                       heads=16, kv="bf16"),
    "decode_b128": dict(mode=MODE_DECODE, bs=128,
                        seqlen_range=(32768, 131072), topk=2048, idx_heads=64,
                        idx_dim=128, idx_kind="fp8", heads=128, kv="fp8"),
    "extend": dict(mode=MODE_EXTEND, bs=4, extend_lens=[512, 1024, 2048, 4096],
                   prefix_lens=[8192, 16384, 24576, 32768], topk=2048,
                   idx_heads=64, idx_dim=128, idx_kind="fp8", heads=16,
                   kv="bf16"),
    "verify": dict(mode=MODE_TARGET_VERIFY, bs=64, draft=4,
                   seqlen_range=(16384, 131072), topk=2048, idx_heads=64,
                   idx_dim=128, idx_kind="fp8", heads=128, kv="fp8"),
    "draft_extend": dict(mode=MODE_DRAFT_EXTEND, bs=64, draft=4,
                         seqlen_range=(16384, 131072), topk=2048, idx_heads=64,
                         idx_dim=128, idx_kind="fp8", heads=128, kv="fp8"),
    "draft_extend_v2": dict(mode=MODE_DRAFT_EXTEND_V2, bs=64, draft=4,
                            seqlen_range=(16384, 131072), topk=2048,
                            idx_heads=64, idx_dim=128, idx_kind="fp8",
                            heads=128, kv="fp8"),
}

SM_SCALE = 1.0 / math.sqrt(192.0)


@dataclass
class Workload:
    name: str
    mode: int
    bs: int
    topk: int
    draft: int
    idx_heads: int
    idx_dim: int
    idx_kind: str          # "fp8" or "fp32"
    heads: int
    kv_kind: str           # "bf16" or "fp8"
    sm_scale: float
    num_rows: int          # query rows T
    max_seqlen_k: int      # host bound: max cache seqlen
    num_pages: int         # page pool size
    # metadata inputs (int32)
    seq_lens: torch.Tensor = None
    extend_lens: torch.Tensor = None
    req_to_token: torch.Tensor = None
    req_pool_indices: torch.Tensor = None
    # indexer inputs
    q_idx: torch.Tensor = None        # [T, Hi, Di] uint8 fp8 codes or fp32
    idx_weights: torch.Tensor = None  # [T, Hi] fp32
    index_cache: torch.Tensor = None  # [num_pages, page_bytes] uint8
    # attention inputs
    q: torch.Tensor = None            # [T, H, 576] bf16
    kv_bf16: torch.Tensor = None      # [num_pages * 64, 576] bf16
    host: dict = field(default_factory=dict)

    @property
    def rows_per_request(self):
        """Mean query rows per request, rounded down: the indexer's hint
        for letting a request's rows share their key-page reads."""
        return max(self.num_rows // self.bs, 1) if self.bs else 1


def _randint(gen, lo, hi, n, device):
    return torch.randint(lo, hi + 1, (n,), generator=gen, device=device,
                         dtype=torch.int64)


def _fp8_codes(x):
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def make_workload(name, device="cpu", seed=0, parts=("indexer", "attention"),
                  **overrides):
    """Build one workload on ``device`` with a seeded torch generator.

    ``overrides`` replace entries of the configuration (e.g. ``bs`` or
    ``seqlen_range``) for reduced-size parity cases. ``parts`` selects the
    large inputs to draw: "indexer" (q, weights, index-key cache) and
    "attention" (MLA q and the bf16 latent cache); metadata inputs are always
    drawn first, so they do not depend on ``parts``.
    """
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    mode, bs = cfg["mode"], cfg["bs"]
    # fixed per-request token count of target-verify and draft-extend v2
    draft = (cfg.get("draft", 0)
             if mode in (MODE_TARGET_VERIFY, MODE_DRAFT_EXTEND_V2) else 0)

    if mode == MODE_EXTEND:
        ext = torch.tensor(cfg["extend_lens"][:bs], dtype=torch.int64)
        pre = torch.tensor(cfg["prefix_lens"][:bs], dtype=torch.int64)
        seq_lens = (pre + ext).to(dev)
        extend_lens = ext.to(dev)
        num_rows = int(ext.sum())
    else:
        if "seq_lens" in cfg:
            seq_lens = torch.tensor(cfg["seq_lens"][:bs], dtype=torch.int64,
                                    device=dev)
        else:
            lo, hi = cfg["seqlen_range"]
            seq_lens = _randint(gen, lo, hi, bs, dev)
        extend_lens = None
        num_rows = bs * (draft if draft else 1)
        if mode == MODE_DRAFT_EXTEND:   # accepted drafts + 1 per request
            extend_lens = _randint(gen, 1, cfg["draft"], bs, dev)
            num_rows = int(extend_lens.sum())

    # tokens held per request: target-verify adds the drafts to seq_lens,
    # the other modes count them in seq_lens already
    kv_lens = (seq_lens + (draft if mode == MODE_TARGET_VERIFY else 0)).cpu()
    pages_per_req = [(int(n) + PAGE - 1) // PAGE for n in kv_lens]
    spare = 3
    num_pages = sum(pages_per_req) + spare
    perm = torch.randperm(num_pages, generator=gen, device=dev).cpu()
    max_seqlen_k = int(kv_lens.max()) if bs else 0
    max_ctx = ((max_seqlen_k + PAGE - 1) // PAGE + 1) * PAGE
    pool_rows = bs + 2
    row_of_req = torch.randperm(pool_rows, generator=gen, device=dev).cpu()[:bs]
    rtt = torch.zeros(pool_rows, max_ctx, dtype=torch.int32)
    off = torch.arange(PAGE, dtype=torch.int32)
    p0 = 0
    for r in range(bs):
        n = pages_per_req[r]
        pages = perm[p0:p0 + n].to(torch.int32)
        p0 += n
        rtt[row_of_req[r], :n * PAGE] = (pages[:, None] * PAGE + off[None, :]).reshape(-1)

    w = Workload(name=name, mode=mode, bs=bs, topk=cfg["topk"], draft=draft,
                 idx_heads=cfg["idx_heads"], idx_dim=cfg["idx_dim"],
                 idx_kind=cfg["idx_kind"], heads=cfg["heads"],
                 kv_kind=cfg["kv"], sm_scale=SM_SCALE, num_rows=num_rows,
                 max_seqlen_k=max_seqlen_k, num_pages=num_pages)
    w.seq_lens = seq_lens.to(torch.int32)
    w.extend_lens = extend_lens.to(torch.int32) if extend_lens is not None else None
    w.req_to_token = rtt.to(dev)
    w.req_pool_indices = row_of_req.to(torch.int32).to(dev)

    T, Hi, Di = num_rows, w.idx_heads, w.idx_dim
    if "indexer" in parts:
        _draw_indexer(w, gen, dev, T, Hi, Di, num_pages)
    if "attention" in parts:
        gen_a = torch.Generator(device=dev)
        gen_a.manual_seed(seed + 1000003)
        w.q = torch.randn(T, w.heads, D_QK, generator=gen_a, device=dev).to(torch.bfloat16)
        w.kv_bf16 = _randn_bf16(num_pages * PAGE, D_QK, gen_a, dev)
    return w


def _randn_bf16(rows, cols, gen, dev, chunk=1 << 20):
    """N(0,1) rounded to bf16, drawn in row chunks (bounded fp32 temporaries)."""
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device=dev)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        out[r0:r1] = torch.randn(r1 - r0, cols, generator=gen, device=dev)
    return out


def _draw_indexer(w, gen, dev, T, Hi, Di, num_pages):
    if w.idx_kind == "fp8":
        w.q_idx = _fp8_codes(torch.randn(T, Hi, Di, generator=gen, device=dev) * 0.5)
        keys = _fp8_codes(torch.randn(num_pages, PAGE * Di, generator=gen,
                                      device=dev) * 0.5)
        kscale = torch.rand(num_pages, PAGE, generator=gen, device=dev) + 0.5
    else:
        w.q_idx = torch.randn(T, Hi, Di, generator=gen, device=dev)
        keys = torch.randn(num_pages, PAGE * Di, generator=gen, device=dev) \
            .contiguous().view(torch.uint8)
        kscale = torch.ones(num_pages, PAGE, device=dev)
    w.idx_weights = torch.rand(T, Hi, generator=gen, device=dev)
    w.index_cache = torch.cat(
        [keys.reshape(num_pages, -1),
         kscale.to(torch.float32).contiguous().view(torch.uint8).reshape(num_pages, -1)],
        dim=1).contiguous()


def host_inputs(w):
    """numpy copies of the metadata inputs (for the oracle)."""
    h = dict(seq_lens=w.seq_lens.cpu().numpy(),
             req_to_token=w.req_to_token.cpu().numpy(),
             req_pool_indices=w.req_pool_indices.cpu().numpy())
    h["extend_lens"] = (w.extend_lens.cpu().numpy()
                        if w.extend_lens is not None else None)
    return h
