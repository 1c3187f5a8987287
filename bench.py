"""Benchmark of the sparse-attention decode step on one MI355X.

A step is one pass of the whole path over one batch: metadata, indexer
logits, fused top-k + page transform, sparse MLA. The default workload is the
decode batch of 128 requests with KV lengths uniform in [32768, 131072],
topk 2048, 128 MLA heads over an fp8 block-scaled latent cache and a 64-head
x 128-dim fp8 indexer. Inputs are synthetic, seeded and resident in HBM
before timing starts.

Prints one JSON line. `value` is query rows (tokens) per second over the
timed steps; `roofline` is for the dominant kernel (the indexer), with its
algorithmic bytes (or, where its fp8 dot products take longer at peak than
its bytes, its flops) per launch divided by its average launch time,
measured with HIP events on the launch stream; `cpu_baseline` is the CPU oracle timed
on a bounded sample of rows of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0     # dense fp8 MFMA
METRIC = "query-tokens/s through indexer+topk+sparse MLA; % of HBM roofline"
PMC_FILE = os.path.join(ROOT, "profiles", "indexer_fp8_decode_b128_pmc.txt")
PMC_WORKLOAD = "decode_b128"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_b128",
                    choices=["decode_b128", "decode_b32", "verify", "extend",
                             "draft_extend", "draft_extend_v2"])
    ap.add_argument("--cpu-rows", type=int, default=40,
                    help="rows of the oracle sample (0 = skip the CPU leg)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cold", action="store_true",
                    help="also time single steps, each after writing a 1 GiB "
                         "buffer so no input is left in the 256 MB last-level "
                         "cache (cold_ms_per_step) and each without it "
                         "(single_ms_per_step); value stays the warm, "
                         "back-to-back rate")
    ap.add_argument("--graph", action="store_true",
                    help="also capture the step in one HIP graph and time "
                         "`steps` replays back to back (graph_ms_per_step); "
                         "value stays the eager rate")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (a known-size "
                         "kernel for scaling HBM counters)")
    return ap.parse_args()


def indexer_cost(lengths, t2r, hi=64, di=128):
    """Strict algorithmic bytes, flops and logit bytes of one indexer launch.
    Strict bytes: per row its q row and weights; per request the fp8 key and
    fp32 scale of every position its longest row sees, and one page-table
    entry per 64 of them (rows of one request read the same keys, which need
    to come from HBM once). The fp32 logit written per (row, position) is an
    intermediate (implementation traffic), returned apart. Flops: 2 * hi * di
    per (row, position) for the dot products."""
    longest = {}
    b = fl = lg = 0
    for L, r in zip(lengths, t2r):
        L = int(L)
        b += hi * di + hi * 4
        lg += L * 4
        fl += 2 * hi * di * L
        longest[int(r)] = max(longest.get(int(r), 0), L)
    for L in longest.values():
        b += L * (di + 4) + ((L + 63) // 64) * 4
    return b, fl, lg


def pipeline_bytes(lengths, t2r, topk, heads, kv_row_bytes, hi=64, di=128):
    """Strict algorithmic bytes of one step: the indexer's (keys once per
    request), then per row the selected latent rows, MLA q and output."""
    b, _, _ = indexer_cost(lengths, t2r, hi, di)
    for L in lengths:
        L = int(L)
        b += min(L, topk) * kv_row_bytes + heads * 576 * 2 + heads * 512 * 2 + heads * 4
    return b


def measured_hbm(dev, gib=1, reps=10):
    """HBM rate measured in this process on 1 GiB buffers (HIP events, best
    of `reps`): a device copy, reading and writing 1 GiB each, counted as
    2 GiB. GB/s. (torch's reductions read far below the memory's rate here,
    so no read-only figure is taken from them.)"""
    import torch
    n = (gib << 30) // 4
    a = torch.ones(n, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    out = {}
    for name, fn, nbytes in (("copy", lambda: b.copy_(a), 2 * n * 4),):
        for _ in range(3):
            fn()
        best = None
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        out[name] = nbytes / (best * 1e-3) / 1e9
    del a, b
    return out


def read_pmc(expected_sha):
    """HBM traffic of the indexer from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    if not os.path.exists(PMC_FILE):
        return None
    kv = {}
    for line in open(PMC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("indexer_source_sha256") != expected_sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, rows):
    """The oracle, as it stands, on `rows` query rows of the same workload:
    metadata for the batch, then per row indexer -> top-k -> transform ->
    sparse MLA. Returns rows/s, threads used and the sample description."""
    import numpy as np
    import torch
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    h = {k: getattr(w, k).cpu().numpy() if getattr(w, k) is not None else None
         for k in ("seq_lens", "extend_lens", "req_to_token", "req_pool_indices")}
    sample = list(range(0, w.num_rows, max(1, w.num_rows // rows)))[:rows]
    # inputs of the sampled rows, copied to the host before the clock starts
    md0 = oracle.metadata.build_metadata(w.mode, h["seq_lens"], h["req_to_token"],
                                         h["req_pool_indices"], w.topk,
                                         extend_lens=h["extend_lens"],
                                         draft_token_num=w.draft)
    per_row = []
    for t in sample:
        r = int(md0["token_to_req"][t])
        L = int(md0["seqlens_expanded"][t])
        pages = md0["real_page_table"][r, :(L + 63) // 64]
        raw_idx = w.index_cache[torch.as_tensor(pages, device=w.index_cache.device)].cpu().numpy()
        slots_all = md0["page_table_1"][r, :L]
        per_row.append(dict(t=t, r=r, L=L, raw_idx=raw_idx,
                            q_idx=w.q_idx[t:t + 1].cpu().numpy(),
                            wts=w.idx_weights[t:t + 1].cpu().numpy(),
                            q=w.q[t:t + 1].to(torch.float64).cpu().numpy(),
                            slots_all=slots_all))
    kv_rows = {}
    for pr in per_row:
        s = torch.as_tensor(pr["slots_all"], device=w.kv_bf16.device)
        kv_rows[pr["t"]] = w.kv_bf16[s].view(torch.int16).cpu().numpy().view(np.uint16)

    t_quant = 0.0
    t0 = time.perf_counter()
    md = oracle.metadata.build_metadata(w.mode, h["seq_lens"], h["req_to_token"],
                                        h["req_pool_indices"], w.topk,
                                        extend_lens=h["extend_lens"],
                                        draft_token_num=w.draft)
    for pr in per_row:
        keys, ks = oracle.indexer.decode_index_pages(pr["raw_idx"], w.idx_dim, w.idx_kind)
        q64 = (oracle.formats.e4m3_decode(pr["q_idx"]) if w.idx_kind == "fp8"
               else pr["q_idx"].astype(np.float64))
        npg = (pr["L"] + 63) // 64
        logits = oracle.indexer.indexer_logits(q64, pr["wts"], keys, ks,
                                               np.arange(npg)[None], [0], [pr["L"]],
                                               pr["L"])
        sel = oracle.topk.topk(logits, [pr["L"]], w.topk)
        slots = oracle.transform.transform_compact(sel, md["real_page_table"],
                                                   [pr["r"]])
        # the latent cache rows the row reads, in the cache's stored format
        pos = sel[0][sel[0] >= 0]
        bits = kv_rows[pr["t"]][pos]
        if w.kv_kind == "fp8":
            # the GPU step reads an already quantized cache: not timed
            tq = time.perf_counter()
            cache = oracle.quant.Fp8Cache(oracle.quant.quantize_k_cache(bits))
            t_quant += time.perf_counter() - tq
        else:
            cache = oracle.quant.Bf16Cache(bits)
        local = np.full_like(slots, -1)
        local[0, :len(pos)] = np.arange(len(pos))
        oracle.sparse_mla.sparse_mla(pr["q"], cache, local, w.sm_scale)
    dt = time.perf_counter() - t0 - t_quant
    return dict(value=len(per_row) / dt, unit="query-tokens/s", cores=int(cores),
                kind="oracle",
                sample=(f"{len(per_row)} of {w.num_rows} query rows of the same "
                        f"workload (rows {per_row[0]['t']}..{per_row[-1]['t']}), "
                        f"{dt:.1f} s; numpy fp64, batch metadata included, quantization "
                        f"of the cache rows read excluded"))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: one GPU per process only (asked for --gpus "
              f"{args.gpus}); decode shards over requests with no exchange, so "
              "each GPU would run this benchmark on its own share of requests",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import sparse_attention_decode_indexer_amd as nsa
    import workloads as W

    nsa.load()
    dev = torch.device("cuda:0")
    w = W.make_workload(args.workload, device=dev, seed=args.seed)
    fp8_kv = w.kv_kind == "fp8"
    cache = nsa.nsa_quantize_k_cache(w.kv_bf16) if fp8_kv else w.kv_bf16
    kvd = nsa.KV_FP8_656 if fp8_kv else nsa.KV_BF16_576
    T = w.num_rows
    idt = nsa.DTYPE_FP8_E4M3 if w.idx_kind == "fp8" else nsa.DTYPE_FP32
    ncols = (w.max_seqlen_k + 63) // 64

    # preallocated outputs (the library never allocates)
    i32 = torch.int32
    logits = torch.empty(T, nsa.logits_row_stride(w.max_seqlen_k),
                         dtype=torch.float32, device=dev)
    slots = torch.empty(T, w.topk, dtype=i32, device=dev)
    # top-k histogram counted by the indexer; the top-k clears it after use
    key_hist = nsa.new_key_hist(T, dev) if idt == nsa.DTYPE_FP8_E4M3 else None
    # bitmaps of the top-k whose long rows are spread over many blocks
    tk_ws = torch.empty(max(nsa.topk_hist_workspace_size(T, w.max_seqlen_k, w.topk), 16),
                        dtype=torch.uint8, device=dev)
    out = torch.empty(T, w.heads, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(T, w.heads, dtype=torch.float32, device=dev)
    ws = torch.empty(max(nsa.sparse_mla_workspace_size(T, w.heads, w.topk), 16),
                     dtype=torch.uint8, device=dev)
    attn = nsa.nsa_sparse_mla_extend if w.mode == W.MODE_EXTEND else nsa.nsa_sparse_mla_decode

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
          for _ in range(args.steps)]

    # caller-owned metadata outputs, refilled in place every step (what a
    # captured graph refers to)
    md_buf = nsa.new_metadata_buffers(w.mode, w.bs, T, w.max_seqlen_k, dev)

    def step(e=None):
        if e: e[0].record()
        md = nsa.nsa_build_metadata(w.mode, w.seq_lens, w.req_to_token,
                                    w.req_pool_indices, w.topk, w.max_seqlen_k, T,
                                    extend_lens=w.extend_lens, draft_token_num=w.draft,
                                    out=md_buf)
        if e: e[1].record()
        nsa.nsa_indexer_logits(w.q_idx, w.idx_weights, w.index_cache,
                               md["real_page_table"], md["token_to_req"],
                               md["seqlens_expanded"], w.max_seqlen_k,
                               logits=logits, dtype=idt, key_hist=key_hist,
                               rows_per_request=w.rows_per_request)
        if e: e[2].record()
        nsa.nsa_topk_transform(logits, md["seqlens_expanded"], w.topk,
                               w.max_seqlen_k, table=md["real_page_table"],
                               token_to_req=md["token_to_req"], out=slots,
                               key_hist=key_hist, workspace=tk_ws)
        if e: e[3].record()
        attn(w.q, cache, kvd, slots, w.sm_scale, md["nsa_cache_seqlens"],
             out=out, lse=lse, workspace=ws)
        if e: e[4].record()
        return md

    for _ in range(args.warmup):
        step()
    if args.copy_calibration:
        # an elementwise int32 -> fp32 kernel over 1 GiB: reads 1 GiB, writes 1 GiB
        src_c = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        dst_c = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c
    # the timed steps carry no per-stage events (each event adds a queue
    # packet between dependent kernels); the stage split comes from a second
    # pass of the same steps with events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        md = step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()

    stage = np.array([[ev[k][i].elapsed_time(ev[k][i + 1]) for i in range(4)]
                      for k in range(args.steps)])          # ms
    graph_ms = None
    if args.graph:
        # captured on a side stream after one warm step there (torch's
        # protocol), then `steps` replays back to back between two syncs
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - g0) * 1e3 / args.steps
    cold_ms = single_ms = None
    if args.cold:
        # each step timed alone (HIP events around it, synchronised); for the
        # cold time a 1 GiB fill outside the events first evicts the inputs
        # from the last-level cache
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

        def lone(evict):
            times = []
            for k in range(args.steps):
                if evict:
                    flush.fill_(float(k))
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                step()
                b.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b))
            return float(np.median(times))

        single_ms = lone(False)
        cold_ms = lone(True)
        del flush
    stage_ms = stage.mean(axis=0)
    ms_per_step = elapsed * 1e3 / args.steps
    se = md["seqlens_expanded"].cpu().numpy()     # visible length of every row
    t2r = md["token_to_req"].cpu().numpy()
    idx_bytes, idx_flops, idx_logit_bytes = indexer_cost(se, t2r, w.idx_heads, w.idx_dim)
    idx_ms = stage_ms[1]
    meas = measured_hbm(dev)
    # the indexer's bound: HBM for its bytes or fp8 MFMA for its dot
    # products, whichever takes longer at peak
    if idx_flops / FP8_PEAK_TFLOPS > idx_bytes / HBM_PEAK_GBPS * 1e3:
        roof = {"bound": "mfma", "achieved": idx_flops / (idx_ms * 1e-3) / 1e12,
                "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": idx_bytes / (idx_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if roof["bound"] == "hbm":
        # the same figure against this GPU's measured copy rate
        roof["measured_peak"] = meas["copy"]
        roof["frac_of_measured"] = roof["achieved"] / meas["copy"]
    pipe = pipeline_bytes(se, t2r, w.topk, w.heads, 656 if fp8_kv else 1152,
                          w.idx_heads, w.idx_dim)
    pipe_gbps = pipe / (ms_per_step * 1e-3) / 1e9
    src = open(os.path.join(ROOT, "sparse_attention_decode_indexer_amd", "csrc",
                            "indexer.hip"), "rb").read()
    # the committed counters were taken on the default decode workload
    traffic = (read_pmc(hashlib.sha256(src).hexdigest())
               if args.workload == PMC_WORKLOAD else None)
    grouped = idt == nsa.DTYPE_FP8_E4M3 and w.rows_per_request >= 4
    kernel = ("indexer_fp8_rows_kernel" if grouped else
              "indexer_fp8_kernel" if idt == nsa.DTYPE_FP8_E4M3 else "indexer_fp32_kernel")

    res = {
        "metric": METRIC,
        "value": T * args.steps / elapsed,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (indexer, KV cache) / bf16 MFMA + fp32 softmax (MLA)",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": args.workload, "batch": w.bs, "query_rows": T,
                   "max_seqlen_k": w.max_seqlen_k, "topk": w.topk,
                   "mla_heads": w.heads, "kv_cache": w.kv_kind,
                   "indexer": f"{w.idx_heads}x{w.idx_dim} {w.idx_kind}",
                   "parallelism": "single GPU"},
        "roofline": dict(kernel=kernel, **roof, traffic=traffic,
                         traffic_source=("rocprofv3 FETCH_SIZE + WRITE_SIZE of this kernel "
                                         "source, committed in profiles/"
                                         if traffic is not None else None),
                         algorithmic_bytes_per_launch=idx_bytes,
                         algorithmic_flops_per_launch=idx_flops,
                         implementation_bytes_per_launch=idx_logit_bytes),
        "pipeline": {"algorithmic_bytes_per_step": pipe, "GBps": pipe_gbps,
                     "hbm_roofline_frac": pipe_gbps / HBM_PEAK_GBPS,
                     "frac_of_measured_copy": pipe_gbps / meas["copy"]},
        "measured_hbm_GBps": {"copy": meas["copy"],
                              "nominal": HBM_PEAK_GBPS},
        "stages_ms": {"metadata": stage_ms[0], "indexer": stage_ms[1],
                      "topk_transform": stage_ms[2], "sparse_mla": stage_ms[3]},
        "cpu_baseline": None,
    }
    if cold_ms is not None:
        res["single_ms_per_step"] = single_ms
        res["cold_ms_per_step"] = cold_ms
    if graph_ms is not None:
        res["graph_ms_per_step"] = graph_ms
    if args.cpu_rows > 0:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
