"""SGA decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: decode at 128K context, 16 sequences x 131,072 cached tokens,
one query each, k = 2048, 64 heads (sga_inputs "decode_b16_n128k"). A step is
one sga_layer_fwd call over the whole batch: indexer scores -> top-k -> sparse
MLA -> gate. Inputs are generated on the GPU before timing and stay resident;
the latent and index caches are rotated over 3 copies so that a step never
finds the previous step's caches in the 256 MB Infinity Cache.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, published
MAX_GRAPH_STEPS = 48           # consecutive steps captured in one HIP graph
METRIC = "SGA decode queries/s at 128K ctx, k=2048; % of HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "index_scores_fp8_traffic.json")
# the sources the decode index kernel is compiled from
INDEX_SRCS = [os.path.join(ROOT, "sparse_top_latent_amd", "csrc", f)
              for f in ("index_scores.hip", "index_common.h", "common.h", "kernels.h")]
# the sources the cache append kernel is compiled from
APPEND_SRCS = [os.path.join(ROOT, "sparse_top_latent_amd", "csrc", f)
               for f in ("cache_append.hip", "common.h", "kernels.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(case):
    """Bytes the method must move for the batch: the index keys a sequence's
    queries scan (once per sequence: its queries can share the scan), the
    latent rows each query selects, and per-query inputs and output; and the
    index pass's share (index keys + index queries + weights)."""
    H, Dc, D, HI, DI = case.heads, case.d_latent, case.d_qk, case.idx_heads, case.idx_dim
    row = D * 2 if case.kv_dtype == "bf16" else D + D // 32
    qbytes = H * D * 2 + HI * DI + HI * 4 + H * Dc * 2 + H * Dc * (2 if case.out_dtype == "bf16" else 4)
    lens = case.kv_len.cpu().tolist()
    seqs = case.q_seq.cpu().tolist()
    pos = case.q_pos.cpu().tolist()
    scan = {}
    total = index = 0
    for b, p in zip(seqs, pos):
        n = max(0, min(p + 1, lens[b]))
        scan[b] = max(scan.get(b, 0), n)
        total += min(n, case.topk) * row + qbytes
        index += HI * DI + HI * 4
    keys = sum(scan.values()) * DI
    return total + keys, index + keys


def traffic_record(workload, name=None, srcs=None):
    """Measured HBM bytes of a kernel (by default the decode index kernel), if
    taken on the current sources and for this workload."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", name) if name else TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != index_source_sha(srcs) or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch") if name else rec


def index_source_sha(srcs=None):
    h = hashlib.sha256()
    for f in srcs or INDEX_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def stream_read_gbs(torch, sga, bufs, reps=10):
    """Read bandwidth of the library's streaming-read reference (the decode
    indexer's LDS-DMA copy pattern without the scoring) over the rotated
    buffers `bufs`, timed with HIP events on the launch stream."""
    sink = torch.empty((sga.lib().sga_stream_read_sink_words(),), dtype=torch.int32, device=bufs[0].device)
    for b in bufs:
        sga.sga_stream_read(b, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        sga.sga_stream_read(bufs[i % len(bufs)], sink)
    e1.record()
    torch.cuda.synchronize()
    nbytes = bufs[0].numel() * bufs[0].element_size() // 8192 * 8192
    return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def host_subcase(case, queries):
    """The listed queries of a device case, with only their sequences, on the host."""
    import torch
    from sga_inputs.gen import SgaCase

    seqs = sorted({int(case.q_seq[t]) for t in queries})
    starts = case.kv_start.cpu().tolist()
    lens = case.kv_len.cpu().tolist()
    remap = {b: i for i, b in enumerate(seqs)}
    rows = torch.cat([torch.arange(starts[b], starts[b] + lens[b]) for b in seqs]).to(case.kv.device)
    new_lens = [lens[b] for b in seqs]
    new_starts = [0]
    for n in new_lens[:-1]:
        new_starts.append(new_starts[-1] + n)
    qi = torch.as_tensor(queries, device=case.q.device)

    def pick(x, idx):
        return None if x is None else x.index_select(0, idx).cpu()

    return SgaCase(
        name=case.name + "-sample", heads=case.heads, d_latent=case.d_latent, d_rope=case.d_rope,
        idx_heads=case.idx_heads, idx_dim=case.idx_dim, topk=case.topk,
        softmax_scale=case.softmax_scale, q_dtype=case.q_dtype, kv_dtype=case.kv_dtype,
        idx_dtype=case.idx_dtype, gate_dtype=case.gate_dtype, out_dtype=case.out_dtype,
        lens=new_lens,
        q_seq=torch.tensor([remap[int(case.q_seq[t])] for t in queries], dtype=torch.int32),
        q_pos=case.q_pos.index_select(0, qi).cpu(),
        kv_start=torch.tensor(new_starts, dtype=torch.int64),
        kv_len=torch.tensor(new_lens, dtype=torch.int32),
        q=pick(case.q, qi), kv=pick(case.kv, rows), kv_scale=pick(case.kv_scale, rows),
        q_idx=pick(case.q_idx, qi), k_idx=pick(case.k_idx, rows), w=pick(case.w, qi),
        gate=pick(case.gate, qi))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def time_decode(args, case, prob, sga, torch, steps, warmup):
    """Time `steps` sga_layer_fwd calls over the batch, then the same steps
    eagerly with the library's per-phase HIP events.

    The timed steps are replayed from one HIP graph of up to MAX_GRAPH_STEPS
    consecutive steps (rotating over `args.copies` independent cache copies,
    which keeps each step's caches out of the 256 MB Infinity Cache, as a
    decode loop would run them back to back) plus one graph for a remainder,
    so the graph launch cost is paid once per graph. (Measured on MI355X:
    graphs of 3 to 48 steps run at 85.4 to 83.6 us per step, 12 steps and
    more within 0.3 us of each other.)"""
    dev = case.q.device
    T, H, Dc = case.num_q, case.heads, case.d_latent
    out = torch.empty((T, H, Dc), dtype=sga.out_torch_dtype(prob.c.out_dtype), device=dev)
    ws = sga.workspace(prob, sga.SGA_OP_LAYER, device=dev)
    copies = args.copies
    kvs = [case.kv] + [case.kv.clone() for _ in range(copies - 1)]
    kis = [case.k_idx] + [case.k_idx.clone() for _ in range(copies - 1)]
    scs = [case.kv_scale] + ([case.kv_scale.clone() for _ in range(copies - 1)]
                             if case.kv_scale is not None else [None] * (copies - 1))

    def step(i):
        c = i % copies
        sga.sga_layer_fwd(prob, case.q_idx, case.w, kis[c], case.q, kvs[c], scs[c], case.gate,
                          out, None, None, ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    graphs = []
    chunk = min(steps, MAX_GRAPH_STEPS - MAX_GRAPH_STEPS % copies)
    plan = [(chunk, steps // chunk)] + ([(steps % chunk, 1)] if steps % chunk else [])
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(copies):
                step(c)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for n, reps in plan:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    step(i)
            graphs.append((g, reps))
        for i in range(max(1, warmup // chunk)):
            graphs[0][0].replay()
        torch.cuda.synchronize()

    # timed regions: exactly `steps` steps each, replayed from the graphs and
    # launched eagerly (no events); the faster launch mode gives the result
    def timed(run):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def replay():
        for g, reps in graphs:
            for _ in range(reps):
                g.replay()

    def eager():
        for i in range(steps):
            step(i)

    ms_graph = timed(replay) if graphs else None
    ms_plain = timed(eager)
    use_graph = ms_graph is not None and ms_graph <= ms_plain
    ms_step = ms_graph if use_graph else ms_plain
    qps = T * 1e3 / ms_step
    del graphs

    # per-kernel durations: the same steps launched eagerly with HIP events
    # recorded by the library around each phase on the launch stream
    sga.sga_profile_enable(steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t1) * 1e3 / steps
    phase_ms, calls = sga.sga_profile_collect(4)
    sga.sga_profile_enable(0)
    phases = {n: round(v / max(calls, 1) * 1e3, 2) for n, v in
              zip(("index_us", "topk_us", "mla_us", "combine_us"), phase_ms)}
    return {"ms_step": ms_step, "qps": qps, "eager_ms": eager_ms, "phases": phases,
            "idx_ms": phase_ms[0] / max(calls, 1), "kis": kis, "graphs": use_graph,
            "ms_graph": ms_graph, "ms_plain": ms_plain,
            "launch": (f"hip-graph ({' + '.join(f'{r} x {n}' for n, r in plan)} steps)" if use_graph
                       else "eager launches")}


def cpu_baseline(case, budget_s=15.0):
    """The oracle, as it stands, on host-resident queries of the same workload.

    Queries are taken in a fixed order until about `budget_s` seconds of oracle
    time are spent; copying each query's sequence to the host is not timed."""
    from oracle import case as ocase

    T = case.num_q
    order = list(range(0, T, 2)) + list(range(1, T, 2))
    done, t_used, passes = 0, 0.0, 0
    subs = {}
    while t_used < budget_s and passes < 50:
        for t in order:
            if t_used >= budget_s:
                break
            if t not in subs:
                subs[t] = host_subcase(case, [t])
            t0 = time.perf_counter()
            ocase.run_queries(subs[t], keep_scores=False)
            t_used += time.perf_counter() - t0
            done += 1
        passes += 1
        if len(subs) * 200e6 > 8e9:  # keep at most ~8 GB of host copies around
            subs.clear()
    return {
        "value": round(done / t_used, 3),
        "unit": "queries/s",
        "cores": blas_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{done} query evaluations over the {T} queries of {case.name} through the whole path "
                   f"(exact scores, full-sort top-k, two-pass softmax MLA, gate) in float64, "
                   f"host-resident inputs, {t_used:.1f} s of oracle time"),
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_oracle_rate(case, budget_s, threads=None):
    """Oracle queries/s over whole queries of `case` (bounded by budget_s
    seconds of oracle time; at least one query), with BLAS limited to
    `threads` threads when given."""
    from oracle import case as ocase

    def run():
        done, t_used = 0, 0.0
        for t in range(case.num_q):
            sub = host_subcase(case, [t])
            t0 = time.perf_counter()
            ocase.run_queries(sub, keep_scores=False)
            t_used += time.perf_counter() - t0
            done += 1
            if t_used >= budget_s:
                break
        return done, t_used

    if threads is None:
        done, t_used = run()
        cores = blas_threads()
    else:
        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=threads):
            done, t_used = run()
        cores = threads
    return {"value": round(done / t_used, 3), "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {done} queries of {case.name} (whole path, float64), {t_used:.1f} s"}


def indexer_flops(case):
    lens = case.kv_len.cpu().tolist()
    seqs = case.q_seq.cpu().tolist()
    pos = case.q_pos.cpu().tolist()
    pairs = sum(max(0, min(p + 1, lens[b])) for b, p in zip(seqs, pos))
    return 2.0 * case.idx_heads * case.idx_dim * pairs, pairs


def time_indexer(case, prob, sga, torch, steps, warmup, copies):
    """Average milliseconds of one sga_index_scores pass over the batch (HIP
    events around `steps` passes, index caches rotated over `copies`), and the
    wall time of the timed region."""
    scores = torch.empty((case.num_q, case.max_kv_len), dtype=torch.float32, device=case.q.device)
    kis = [case.k_idx] + [case.k_idx.clone() for _ in range(copies - 1)]

    def step(i):
        sga.sga_index_scores(prob, case.q_idx, case.w, kis[i % copies], scores)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0


def indexer_only(args, case, prob, sga, torch):
    """The indexer score pass alone (the unit of the prefill target)."""
    ms, elapsed = time_indexer(case, prob, sga, torch, args.steps, args.warmup, args.copies)
    flops, pairs = indexer_flops(case)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] indexer {case.name}: {ms * 1e3:.1f} us per pass, {tflops:.0f} TFLOP/s "
        f"({tflops / FP8_PEAK_TFLOPS:.1%} of FP8 MFMA peak), {pairs} (query, key) pairs")
    print(json.dumps({
        "metric": "SGA prefill indexer score pass TFLOP/s; % of FP8 MFMA peak",
        "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": case.name, "queries": case.num_q, "ctx": case.max_kv_len,
                   "idx_heads": case.idx_heads, "idx_dim": case.idx_dim},
        "roofline": {"bound": "mfma", "kernel": "indexer score pass", "achieved": round(tflops, 1),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / FP8_PEAK_TFLOPS, 4), "flops_per_launch": flops,
                     "traffic": None},
        "cpu_baseline": None,
    }), flush=True)


def append_bytes(N, D, DI):
    """Bytes one cache append of N tokens must move: bf16 source rows and keys
    in, MXFP8 rows (values + one scale byte per 32) and FP8 keys out, and the
    int64 slot of each token."""
    return N * (2 * D + 2 * DI + D + D // 32 + DI + 8)


def cache_append_bench(args, torch, sga):
    """Cache append alone: a prefill chunk of new tokens quantised into the caches."""
    from sga_inputs import block_scaled_rows
    from sga_inputs.gen import FULL_DIMS

    dev = torch.device("cuda", 0)
    D = FULL_DIMS["d_latent"] + FULL_DIMS["d_rope"]
    DI = FULL_DIMS["idx_dim"]
    N = args.append_tokens
    rows = max(N, 131072)
    prob = sga.Problem.for_cache(num_kv_rows=rows, d_latent=FULL_DIMS["d_latent"],
                                 d_rope=FULL_DIMS["d_rope"], idx_dim=DI, kv_dtype="mxfp8",
                                 idx_dtype="fp8", device=dev)
    srcs = [(block_scaled_rows(N, D, c, "bench.kv", device=dev),
             block_scaled_rows(N, DI, c, "bench.ki", spread=2, device=dev))
            for c in range(args.copies)]
    caches = [(torch.empty((rows, D), dtype=torch.uint8, device=dev),
               torch.empty((rows, D // 32), dtype=torch.uint8, device=dev),
               torch.empty((rows, DI), dtype=torch.uint8, device=dev)) for _ in range(args.copies)]
    slots = torch.arange(rows - N, rows, dtype=torch.int64, device=dev)

    def step(i):
        c = i % args.copies
        kv, sc, ki = caches[c]
        sga.sga_cache_append(prob, srcs[c][0], srcs[c][1], slots, kv, sc, ki)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    nbytes = append_bytes(N, D, DI)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tps = N / (ms * 1e-3)
    # reference: a plain device copy moving the same bytes (half read, half written)
    a = torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)
    bs = [torch.empty_like(a) for _ in range(args.copies)]
    for b in bs:
        b.copy_(a)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        bs[i % args.copies].copy_(a)
    ev1.record()
    torch.cuda.synchronize()
    copy_gbs = nbytes / (ev0.elapsed_time(ev1) / args.steps * 1e-3) / 1e9
    del a, bs
    log(f"[bench] cache append of {N} tokens: {ms * 1e3:.1f} us per launch, {gbs:,.0f} GB/s "
        f"({gbs / HBM_PEAK_GBS:.1%} of HBM, {gbs / copy_gbs:.1%} of a plain device copy's "
        f"{copy_gbs:,.0f} GB/s), {tps:,.0f} tokens/s")
    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline_append(srcs[0], D, DI)
    print(json.dumps({
        "metric": "SGA cache append tokens/s (bf16 -> MXFP8 latent rows + FP8 index keys); % of HBM roofline",
        "value": round(tps, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16->fp8",
        "data": "synthetic",
        "config": {"workload": f"append_{N}_tokens", "tokens": N, "cache_rows": rows, "row": D,
                   "idx_dim": DI, "kv": "mxfp8", "index": "fp8", "source": "bf16",
                   "cache_copies": args.copies},
        "roofline": {"bound": "hbm", "kernel": "k_cache_append (cache append)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
                     "traffic": traffic_record(f"append_{N}_tokens", "cache_append_traffic.json",
                                               APPEND_SRCS),
                     "copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(gbs / copy_gbs, 4)},
        "cpu_baseline": base,
    }), flush=True)


FP32_PEAK_TFLOPS = 157.3  # MI355X fp32 (vector and MFMA), published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def indexer_kl_split(case, k):
    """(bf16 MFMA FLOPs, fp32 FLOPs) of one sga_indexer_kl call on the MI355X
    shapes: the attention logits (2 H D per selected row) and the index scores
    z in the forward and again in the backward (2 x 2 HI DI) run on bf16 MFMA;
    the three gradient products (d_q_idx and d_k_idx on fp32 MFMA, d_w on the
    vector ALUs; 3 x 2 HI DI) in fp32."""
    rows = case.num_q * k
    D, H, HI, DI = case.d_qk, case.heads, case.idx_heads, case.idx_dim
    return rows * (2.0 * H * D + 4.0 * HI * DI), rows * 6.0 * HI * DI


def indexer_kl_flops(case, k):
    """FLOPs of one sga_indexer_kl call: per selected (query, row) the attention
    logits of every head (2 H D), the indexer scores twice (forward and again
    in the backward, 2 x 2 HI DI) and the three gradient products (3 x 2 HI DI)."""
    D, H, HI, DI = case.d_qk, case.heads, case.idx_heads, case.idx_dim
    return case.num_q * k * (2.0 * H * D + 10.0 * HI * DI)


def indexer_kl_bench(args, case, prob, sga, torch):
    """The indexer KL loss and gradients alone (training side), after one forward."""
    dev = case.q.device
    T, H, HI, DI = case.num_q, case.heads, case.idx_heads, case.idx_dim
    out = torch.empty((T, H, case.d_latent), dtype=sga.out_torch_dtype(prob.c.out_dtype), device=dev)
    idx = torch.empty((T, case.topk), dtype=torch.int32, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = sga.workspace(prob, sga.SGA_OP_LAYER, device=dev)
    sga.sga_layer_fwd(prob, case.q_idx, case.w, case.k_idx, case.q, case.kv, case.kv_scale, case.gate,
                      out, idx, lse, ws)
    loss = torch.empty((T,), device=dev)
    d_w = torch.empty((T, HI), device=dev)
    d_q = torch.empty((T, HI, DI), device=dev)
    d_k = torch.zeros((case.num_kv_rows, DI), device=dev)
    kws = sga.workspace(prob, sga.SGA_OP_INDEXER_KL, device=dev)

    def step():
        sga.sga_indexer_kl(prob, case.q_idx, case.w, case.k_idx, case.q, case.kv, case.kv_scale, idx, lse,
                           loss, d_w, d_q, d_k, kws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = indexer_kl_flops(case, case.topk)
    tflops = flops / (ms * 1e-3) / 1e12
    # mixed-rate compute bound: each part of the work at the peak of the unit
    # it runs on (bf16 MFMA 2.5 PFLOP/s, fp32 157.3 TFLOP/s)
    f_bf16, f_fp32 = indexer_kl_split(case, case.topk)
    ideal_ms = (f_bf16 / (BF16_PEAK_TFLOPS * 1e12) + f_fp32 / (FP32_PEAK_TFLOPS * 1e12)) * 1e3
    mixed_peak = flops / (ideal_ms * 1e-3) / 1e12
    kl_roofline = {"bound": "mfma", "kernel": "indexer KL (k_kl_mass_lds, k_kl_grad, k_kl_reduce; per call)", "achieved": round(tflops, 2),
                   "peak": round(mixed_peak, 1), "unit": "TFLOP/s", "frac": round(tflops / mixed_peak, 4),
                   "flops_per_launch": flops, "bf16_mfma_flops": f_bf16, "fp32_flops": f_fp32,
                   "ideal_us": round(ideal_ms * 1e3, 2), "traffic": None}
    log(f"[bench] indexer KL {case.name}: {ms * 1e3:.1f} us per call, {tflops:.1f} TFLOP/s, "
        f"{tflops / mixed_peak:.1%} of the mixed bf16/fp32 rate ({ideal_ms * 1e3:.1f} us ideal)")
    base = None
    if not args.no_cpu_baseline:
        from oracle import case as ocase

        t1 = time.perf_counter()
        n = 0
        while n < T and time.perf_counter() - t1 < 15.0:
            ocase.kl_queries(case, [n])
            n += 1
        base = {"value": round(n / (time.perf_counter() - t1), 3), "unit": "queries/s", "cores": blas_threads(),
                "kind": "oracle", "sample": f"the first {n} queries of the workload (float64, whole KL and gradients)"}
    print(json.dumps({
        "metric": "SGA indexer KL loss + gradients, queries/s (training side)",
        "value": round(T / (ms * 1e-3), 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": case.name, "queries": T, "topk": case.topk, "heads": H, "idx_heads": HI,
                   "idx_dim": DI},
        "roofline": kl_roofline,
        "cpu_baseline": base,
    }), flush=True)


def cpu_baseline_append(src, D, DI, budget_s=10.0):
    """The oracle's cache append timed on host cores over a bounded sample of
    the same new tokens (as many leading tokens as fit the time budget)."""
    import numpy as np

    from oracle import quant

    kv_new = src[0].float().cpu().numpy().astype(np.float64)
    ki_new = src[1].float().cpu().numpy().astype(np.float64)
    rows = 4096
    kv = np.zeros((rows, D), np.uint8)
    sc = np.zeros((rows, D // 32), np.uint8)
    ki = np.zeros((rows, DI), np.uint8)
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and done < min(rows, kv_new.shape[0]):
        n = min(16, rows - done)
        quant.cache_append(kv_new[done:done + n], ki_new[done:done + n], np.arange(done, done + n),
                           kv, sc, ki, "mxfp8", "fp8")
        done += n
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {done} of the bench's new tokens (float64 Python encoder, one thread)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_b16_n128k")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other configurations measured after the headline")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--indexer-only", action="store_true",
                    help="time only sga_index_scores (reported in TFLOP/s against the FP8 MFMA peak)")
    ap.add_argument("--cache-append", action="store_true",
                    help="time only sga_cache_append of --append-tokens new tokens (bf16 -> MXFP8 + FP8)")
    ap.add_argument("--append-tokens", type=int, default=131072)
    ap.add_argument("--indexer-kl", action="store_true",
                    help="time only sga_indexer_kl (loss and gradients) after one forward of --workload")
    ap.add_argument("--page-size", type=int, default=0,
                    help="lay the caches out in pages of this many rows (seeded random page order, "
                         "block table) instead of contiguous rows")
    args = ap.parse_args()
    if args.gpus != 1:
        log(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
            "(the SGA decode path shards whole sequences per GPU with no exchange; "
            "see the design notes)")
        sys.exit(2)

    import torch

    import sparse_top_latent_amd as sga
    from sga_inputs import make_case

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.cache_append:
        return cache_append_bench(args, torch, sga)
    t0 = time.time()
    case = make_case(args.workload, device=dev)
    if args.page_size:
        from sga_inputs import paged_copy

        case = paged_copy(case, args.page_size)
    torch.cuda.synchronize()
    log(f"[bench] generated {args.workload} on the GPU in {time.time() - t0:.1f} s "
        f"({case.num_kv_rows} cached rows, {case.num_q} queries)")
    prob = sga.Problem.from_case(case)
    T, H, Dc = case.num_q, case.heads, case.d_latent
    if args.indexer_only:
        return indexer_only(args, case, prob, sga, torch)
    if args.indexer_kl:
        return indexer_kl_bench(args, case, prob, sga, torch)
    r = time_decode(args, case, prob, sga, torch, args.steps, args.warmup)
    ms_step, qps, eager_ms, phases, idx_ms, kis = (r[k] for k in ("ms_step", "qps", "eager_ms", "phases",
                                                                 "idx_ms", "kis"))
    graphs, launch, r_ms_graph, r_ms_plain = r["graphs"], r["launch"], r["ms_graph"], r["ms_plain"]
    total_bytes, index_bytes = algorithmic_bytes(case)
    achieved = index_bytes / (idx_ms * 1e-3) / 1e9
    step_gbs = total_bytes / (ms_step * 1e-3) / 1e9
    log(f"[bench] {ms_step * 1e3:.1f} us/step ({launch}; graph "
        f"{'-' if r_ms_graph is None else f'{r_ms_graph * 1e3:.1f}'}, eager {r_ms_plain * 1e3:.1f}, "
        f"eager with phase events {eager_ms * 1e3:.1f} us/step), "
        f"{qps:,.0f} queries/s, step {step_gbs:,.0f} GB/s of per-query bytes ({step_gbs / HBM_PEAK_GBS:.1%} of HBM), "
        f"phases {phases}")
    rec = traffic_record(args.workload) if not args.page_size else None
    # Several queries per sequence share the scan of its index keys. With few
    # of them (multi-query decode) the index pass stays HBM-bound; with many
    # (prefill) its FLOP per key byte pass the FP8 ridge (625 FLOP/B) and it is
    # rated in FLOP against the MFMA peak, and the selected rows, which
    # neighbouring queries share, no longer bound the step.
    flops_all, _ = indexer_flops(case)
    mfma_bound = flops_all / index_bytes > FP8_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3
    stream_gbs = None
    if not mfma_bound:
        stream_gbs = stream_read_gbs(torch, sga, kis)
        log(f"[bench] index kernel {achieved:,.0f} GB/s; the library's streaming-read reference over "
            f"{kis[0].numel() / 1e6:.0f} MB index caches {stream_gbs:,.0f} GB/s")
    del r, kis
    if mfma_bound:
        flops, _ = indexer_flops(case)
        tflops = flops / (idx_ms * 1e-3) / 1e12
        roofline = {
            "bound": "mfma", "kernel": "k_index_fp8_pf (indexer score pass)",
            "achieved": round(tflops, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / FP8_PEAK_TFLOPS, 4), "flops_per_launch": flops, "traffic": None,
        }
    else:
        roofline = {
            "bound": "hbm", "kernel": "k_index_fp8 (indexer score pass)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "bytes_per_launch": index_bytes,
            "traffic": None if rec is None else rec["hbm_bytes_per_launch"],
            "frac_of_stream_read": round(achieved / stream_gbs, 4),
        }
    if case.name == "decode_b16_n128k" and not args.page_size:
        metric = METRIC
    elif mfma_bound:
        metric = f"SGA prefill layer queries/s ({T} queries over {case.num_seqs} sequence(s)); index pass % of FP8 MFMA peak"
    else:
        metric = f"SGA decode queries/s ({case.name}, k={case.topk}); % of HBM roofline"
    result = {
        "metric": metric,
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16",
        "data": "synthetic",
        "launch": launch,
        "ms_per_step_by_launch": {"hip_graph": None if r_ms_graph is None else round(r_ms_graph, 5),
                                  "eager": round(r_ms_plain, 5),
                                  "eager_with_phase_events": round(eager_ms, 5)},
        "config": {"workload": case.name, "seqs": case.num_seqs, "queries": T,
                   "ctx": case.max_kv_len, "topk": case.topk, "heads": H, "d_latent": Dc,
                   "d_rope": case.d_rope, "idx_heads": case.idx_heads, "idx_dim": case.idx_dim,
                   "kv": case.kv_dtype, "index": case.idx_dtype, "out": case.out_dtype,
                   "cache_copies": args.copies, "page_size": args.page_size},
        "step_hbm": None if mfma_bound else {
            "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(step_gbs / HBM_PEAK_GBS, 4), "bytes_per_step": total_bytes,
            "stream_read_gbs": round(stream_gbs, 1),
            "frac_of_stream_read": round(step_gbs / stream_gbs, 4)},
        "phases_us": phases,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and not args.page_size:  # (the paged run adds no new oracle work)
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(case)
        result["cpu_baseline"]["single_thread"] = cpu_oracle_rate(case, 5.0, threads=1)
    if case.name == "decode_b16_n128k" and not args.page_size and not args.no_secondary:
        del case, prob
        torch.cuda.empty_cache()
        result["secondary"] = secondary_lines(args, sga, torch, not args.no_cpu_baseline)
    print(json.dumps(result), flush=True)


def secondary_lines(args, sga, torch, cpu):
    """The other configurations measured in the same run as the headline:
    the prefill indexer pass (FP8 MFMA target), the 32 x 32K decode batch and
    the mixed-length MXFP8 batch (each with a bounded oracle figure)."""
    from sga_inputs import make_case

    dev = torch.device("cuda", 0)
    out = {}
    case = make_case("prefill_q4096_n128k", device=dev)
    prob = sga.Problem.from_case(case)
    ms, _ = time_indexer(case, prob, sga, torch, max(5, args.steps // 4), max(2, args.warmup // 4), args.copies)
    flops, pairs = indexer_flops(case)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] secondary prefill_q4096_n128k indexer: {ms * 1e3:.1f} us per pass, {tflops:.0f} TFLOP/s "
        f"({tflops / FP8_PEAK_TFLOPS:.1%} of FP8 MFMA peak)")
    out["prefill_q4096_n128k_indexer"] = {
        "metric": "indexer score pass TFLOP/s (4,096 queries x up to 131,072 keys)", "value": round(tflops, 1),
        "unit": "TFLOP/s", "ms_per_pass": round(ms, 4),
        "roofline": {"bound": "mfma", "kernel": "k_index_fp8_pf", "achieved": round(tflops, 1),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / FP8_PEAK_TFLOPS, 4),
                     "flops_per_launch": flops}}
    del case, prob
    torch.cuda.empty_cache()
    for name in ("decode_b32_n32k", "varlen_mxfp8_b64"):
        case = make_case(name, device=dev)
        prob = sga.Problem.from_case(case)
        r = time_decode(args, case, prob, sga, torch, args.steps, args.warmup)
        total_bytes, index_bytes = algorithmic_bytes(case)
        gbs = total_bytes / (r["ms_step"] * 1e-3) / 1e9
        idx_gbs = index_bytes / (r["idx_ms"] * 1e-3) / 1e9
        log(f"[bench] secondary {name}: {r['ms_step'] * 1e3:.1f} us/step, {r['qps']:,.0f} queries/s, "
            f"{gbs / HBM_PEAK_GBS:.1%} of HBM, phases {r['phases']}")
        out[name] = {
            "metric": f"SGA decode queries/s ({name}, k={case.topk})", "value": round(r["qps"], 1),
            "unit": "queries/s", "ms_per_step": round(r["ms_step"], 5), "launch": r["launch"],
            "ms_per_step_by_launch": {"hip_graph": None if r["ms_graph"] is None else round(r["ms_graph"], 5),
                                      "eager": round(r["ms_plain"], 5)},
            "step_hbm": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": total_bytes},
            "index_hbm": {"achieved": round(idx_gbs, 1), "frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_launch": index_bytes},
            "phases_us": r["phases"],
            "cpu_baseline": cpu_oracle_rate(case, 5.0) if cpu else None}
        del case, prob, r
        torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
