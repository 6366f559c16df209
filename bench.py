#!/usr/bin/env python3
"""PagedAttention decode bench on one MI355X.

A step is one decode of the whole batch: every sequence's single query token
attends over its paged context (all layers of the workload), through the
C-ABI library -- per layer one paged_attn_decode call, i.e. the decode kernel
and the merge kernel of split sequences.  Inputs are seeded, synthetic and
resident in HBM before timing starts.  Each timed step is preceded (outside
the timed events) by a 2 GiB device READ that evicts the KV cache from the
256 MB MALL and the L2s with clean lines, so the KV bytes really come from
HBM.  (A write-based flush would leave the MALL full of dirty lines whose
write-back then competes with the timed kernel.)

Prints ONE JSON line.  `value` is decode tokens/s (each step produces one
token per sequence); `roofline` relates the algorithmic bytes of one decode
call to its measured duration (HIP events on the launch stream) against the
8 TB/s HBM peak; `traffic` is the HBM bytes per call that rocprofv3 counters
measured for this kernel source (null if the source changed since);
`hbm_read_probe_gbps` is what a plain coalesced read of the same number of
bytes achieves on this device; `cpu_baseline` is the fp64 oracle timed on the
host's cores on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload llama3_8b]

With --workload kv_write_llama3_8b (or kv_write_int8_ / kv_write_fp8_llama3_8b) it times the
KV write path instead -- one paged_kv_write call per step, storing a
16384-token prefill chunk into the paged cache -- and prints the same kind of
line for it; with --workload scores_<decode workload> (e.g. scores_llama3_8b)
it times PagedEviction's token scoring over that workload's whole cache; with
--workload prefill_llama3_8b it times chunked-prefill attention (the eight
512-token chunks of a 4096-token prompt in one call) against the bf16
matrix-core peak; with --workload compress_<decode workload> it times
PagedEviction's prefill-phase compression of that workload's cache to a
1024-token budget per sequence.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published
METRIC = ("decode attention tokens/s and achieved KV-read HBM GB/s (% of peak), "
          "Llama-3-8B shape")
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--split-tokens", type=int, default=None,
                    help="work item length in tokens (default: the workload's; 0 = balanced)")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the read-probe ceiling")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--split-decodes", action="store_true",
                    help="prefill workloads: send the one-token queries of the batch to "
                         "paged_attn_decode and only the chunks to paged_attn_prefill (two calls)")
    ap.add_argument("--key-splits", type=int, default=None,
                    help="prefill workloads: key pieces per row tile of the prefill call (default: "
                         "paged_attn_prefill_plan's; 1 = the unsplit call)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, copy this many bytes 3x with the probe copy kernel "
                         "(reference for hardware byte counters)")
    return ap.parse_args()


def event_ms(stream, fn, reps, before=None):
    """Per-rep durations (ms) of fn() between HIP events recorded on `stream`."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        if before is not None:
            before()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def copy_for_counters(args, dev, stream) -> None:
    """After timing: copy --copy-bytes bytes three times with the probe copy
    kernel, the reference that scales hardware byte counters."""
    if args.copy_bytes <= 0:
        return
    import torch

    from paged_kv_cache_393_amd import probe as P

    src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        P.copy(src, dst, stream)
    torch.cuda.synchronize()
    del src, dst


def measured_traffic(workload: str, operation: str = "decode"):
    """Bytes per call from the committed counter summary, if it was taken on
    the current source of the operation's kernels."""
    from paged_kv_cache_393_amd import rocprof_summary as R

    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    shas = ", ".join(R.source_sha256(src) for src in R.OPERATIONS[operation][1])
    if rec.get("workload") != workload or rec.get("source_sha256") != shas:
        return None
    return rec.get("bytes_per_call")


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this decode path has no multi-GPU leg: every box here has one GPU.", file=sys.stderr)
        return 2

    import torch

    from paged_kv_cache_393_amd import accounting as A
    from paged_kv_cache_393_amd import binding as B
    from paged_kv_cache_393_amd import inputs as I
    from paged_kv_cache_393_amd import probe as P

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    B.load()   # fails loudly if the HIP library is missing
    if args.workload in I.WRITE_WORKLOADS:
        return bench_write(args)
    if args.workload.startswith("scores_"):
        return bench_scores(args)
    if args.workload.startswith("compress_"):
        return bench_compress(args)
    if args.workload in I.PREFILL_WORKLOADS:
        return bench_prefill(args)
    wl = I.WORKLOADS[args.workload]
    split = wl.split_tokens if args.split_tokens is None else args.split_tokens
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    inp = I.make_inputs(wl, dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs for {wl.name} ready in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    L = wl.num_layers
    layers = [I.layer_views(inp, l) for l in range(L)]
    shape = B.shape_of(layers[0]["q"], layers[0]["k_cache"], layers[0]["block_tables"], split)
    plan_split, plan_items = B.plan(shape)
    workspace = B.alloc_workspace(shape, dev)
    outs = [torch.empty(v["q"].shape, dtype=torch.float32, device=dev) for v in layers]
    stream = torch.cuda.current_stream()

    def step():
        for v, o in zip(layers, outs):
            B.decode_views(v, out=o, split_tokens=split, workspace=workspace, stream=stream)

    flush_buf = None
    if not args.no_flush:
        flush_buf = torch.ones((2 << 30) // 4, dtype=torch.float32, device=dev)

    def evict():
        if flush_buf is not None:
            flush_buf.amax()      # a read of 2 GiB: clean eviction of MALL and L2

    for _ in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ms = event_ms(stream, step, args.steps, before=evict)
    wall = time.perf_counter() - w0
    ms_sorted = sorted(ms)
    ms_mean = statistics.fmean(ms)
    pct = lambda q: ms_sorted[min(len(ms_sorted) - 1, int(q * len(ms_sorted)))]
    print(f"[bench] {args.steps} timed steps done", file=sys.stderr, flush=True)

    ctx = inp["context_lens"].cpu().tolist()
    S = wl.num_seqs
    call_bytes = A.decode_bytes(ctx, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                wl.block_size, wl.kv_dtype)
    step_bytes = L * call_bytes
    kv_bytes = L * sum(ctx) * (A.kv_bytes_per_token(1, wl.num_kv_heads, wl.head_dim,
                                                     2 if wl.kv_dtype == "bf16" else 1)
                               + (2 * wl.num_kv_heads * 4 if wl.kv_dtype == "int8" else 0))
    flops = L * A.decode_flops(ctx, wl.num_q_heads, wl.head_dim)
    t_s = ms_mean / 1e3
    gbps = step_bytes / t_s / 1e9

    probe_gbps = None
    if not args.no_probe:
        nbytes = (call_bytes // 16) * 16
        pbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        pbuf.fill_(1)
        sink = torch.zeros(256, dtype=torch.int32, device=dev)
        pms = event_ms(stream, lambda: P.read(pbuf, sink, stream), 20, before=evict)
        probe_gbps = nbytes / (statistics.median(pms) / 1e3) / 1e9
        del pbuf

    copy_for_counters(args, dev, stream)

    record = {
        "metric": METRIC,
        "value": S / t_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_mean,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, shuffled block pool)",
        "config": {
            "workload": wl.name,
            "num_seqs": S, "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim, "block_size": wl.block_size, "layers": L,
            "context_tokens": sum(ctx), "ctx_min": min(ctx), "ctx_max": max(ctx),
            "num_blocks": inp["num_blocks"], "kv_dtype": wl.kv_dtype,
            "split_tokens": plan_split, "max_items": plan_items,
            "cache_evict_between_steps": "2 GiB read" if flush_buf is not None else None,
        },
        "kv_gbps": kv_bytes / t_s / 1e9,
        "pct_of_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
        "ms_p10": pct(0.10), "ms_median": pct(0.50), "ms_p90": pct(0.90),
        "wall_ms_per_step_incl_evict": wall / args.steps * 1e3,
        "tflops": flops / t_s / 1e12,
        "hbm_read_probe_gbps": probe_gbps,
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_attn_decode call: pa_decode_kernel + pa_merge_kernel",
            "achieved": gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "traffic": measured_traffic(wl.name),
            "algorithmic_bytes_per_call": call_bytes,
            "calls_per_step": L,
            "ms_per_call": ms_mean / L,
        },
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        record["cpu_baseline"] = cpu_baseline(wl, layers[0], outs[0], ctx, L, args.cpu_seconds)

    print(json.dumps(record), flush=True)
    return 0


def bench_write(args) -> int:
    """The KV write path on its own: one paged_kv_write(_int8 / _fp8) call per step."""
    import torch

    from paged_kv_cache_393_amd import accounting as A
    from paged_kv_cache_393_amd import binding as B
    from paged_kv_cache_393_amd import inputs as I
    from paged_kv_cache_393_amd import probe as P

    ww = I.WRITE_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = I.make_write_inputs(ww, dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print(f"[bench] inputs for {ww.name} ready", file=sys.stderr, flush=True)

    def step():
        B.kv_write_inputs(inp, stream=stream)

    flush_buf = None if args.no_flush else torch.ones((2 << 30) // 4, dtype=torch.float32,
                                                       device=dev)

    def evict():
        if flush_buf is not None:
            flush_buf.amax()

    for _ in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()
    ms = event_ms(stream, step, args.steps, before=evict)
    ms_sorted = sorted(ms)
    ms_mean = statistics.fmean(ms)
    pct = lambda q: ms_sorted[min(len(ms_sorted) - 1, int(q * len(ms_sorted)))]
    print(f"[bench] {args.steps} timed steps done", file=sys.stderr, flush=True)
    T = ww.num_tokens
    written = int((inp["slots"] >= 0).sum())
    nbytes = A.write_bytes(T, written, ww.num_kv_heads, ww.head_dim, ww.kv_dtype)
    t_s = ms_mean / 1e3
    gbps = nbytes / t_s / 1e9

    copy_gbps = None
    if not args.no_probe:
        # a plain copy moving the same number of bytes (half read, half written)
        half = (nbytes // 2 // 16) * 16
        src = torch.ones(half // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        pms = event_ms(stream, lambda: P.copy(src, dst, stream), 20, before=evict)
        copy_gbps = 2 * half / (statistics.median(pms) / 1e3) / 1e9
        del src, dst

    copy_for_counters(args, dev, stream)

    record = {
        "metric": "KV write path tokens/s and achieved HBM GB/s (% of peak), Llama-3-8B shape",
        "value": T / t_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_mean,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ww.kv_dtype,
        "data": "synthetic (seeded N(0,1) bf16 K/V rows, random distinct slots)",
        "config": {
            "workload": ww.name, "num_tokens": T, "num_kv_heads": ww.num_kv_heads,
            "head_dim": ww.head_dim, "block_size": ww.block_size, "num_blocks": ww.num_blocks,
            "kv_dtype": ww.kv_dtype, "tokens_written": written,
            "cache_evict_between_steps": "2 GiB read" if flush_buf is not None else None,
        },
        "pct_of_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
        "ms_p10": pct(0.10), "ms_median": pct(0.50), "ms_p90": pct(0.90),
        "hbm_copy_probe_gbps": copy_gbps,
        "roofline": {
            "bound": "hbm",
            "kernel": "kv_write_kernel",
            "achieved": gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "traffic": measured_traffic(ww.name, "write"),
            "algorithmic_bytes_per_call": nbytes,
            "calls_per_step": 1,
            "ms_per_call": ms_mean,
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_write(ww, inp),
    }
    print(json.dumps(record), flush=True)
    return 0


def bench_scores(args) -> int:
    """PagedEviction scoring on its own: one paged_kv_token_scores call per step
    over every token of a decode workload's cache (scores_<workload>)."""
    import torch

    from paged_kv_cache_393_amd import accounting as A
    from paged_kv_cache_393_amd import binding as B
    from paged_kv_cache_393_amd import inputs as I
    from paged_kv_cache_393_amd import probe as P

    wl = I.WORKLOADS[args.workload[len("scores_"):]]
    if wl.num_layers != 1:
        raise SystemExit("scoring bench takes a single-layer workload")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = I.make_inputs(wl, dev)
    v = I.layer_views(inp, 0)
    scores = torch.zeros(tuple(v["k_cache"].shape[:2]), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print(f"[bench] inputs for scores of {wl.name} ready", file=sys.stderr, flush=True)

    def step():
        B.token_scores(v, scores=scores, stream=stream)

    flush_buf = None if args.no_flush else torch.ones((2 << 30) // 4, dtype=torch.float32,
                                                       device=dev)

    def evict():
        if flush_buf is not None:
            flush_buf.amax()

    for _ in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()
    ms = event_ms(stream, step, args.steps, before=evict)
    ms_sorted = sorted(ms)
    ms_mean = statistics.fmean(ms)
    pct = lambda q: ms_sorted[min(len(ms_sorted) - 1, int(q * len(ms_sorted)))]
    print(f"[bench] {args.steps} timed steps done", file=sys.stderr, flush=True)
    ctx = inp["context_lens"].cpu().tolist()
    nbytes = A.score_bytes(ctx, wl.num_kv_heads, wl.head_dim, wl.block_size, wl.kv_dtype)
    t_s = ms_mean / 1e3
    gbps = nbytes / t_s / 1e9
    probe_gbps = None
    if not args.no_probe:
        nb = (nbytes // 16) * 16
        pbuf = torch.empty(nb, dtype=torch.uint8, device=dev)
        pbuf.fill_(1)
        sink = torch.zeros(256, dtype=torch.int32, device=dev)
        pms = event_ms(stream, lambda: P.read(pbuf, sink, stream), 20, before=evict)
        probe_gbps = nb / (statistics.median(pms) / 1e3) / 1e9
        del pbuf
    copy_for_counters(args, dev, stream)
    name = "scores_" + wl.name
    record = {
        "metric": "PagedEviction token-importance scoring tokens/s and achieved HBM GB/s "
                  "(% of peak), Llama-3-8B shape",
        "value": sum(ctx) / t_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_mean,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic (seeded N(0,1) K/V, shuffled block pool)",
        "config": {"workload": name, "num_seqs": wl.num_seqs, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "context_tokens": sum(ctx), "kv_dtype": wl.kv_dtype,
                   "cache_evict_between_steps": "2 GiB read" if flush_buf is not None else None},
        "pct_of_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
        "ms_p10": pct(0.10), "ms_median": pct(0.50), "ms_p90": pct(0.90),
        "hbm_read_probe_gbps": probe_gbps,
        "roofline": {
            "bound": "hbm",
            "kernel": "token_scores_kernel",
            "achieved": gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "traffic": measured_traffic(name, "scores"),
            "algorithmic_bytes_per_call": nbytes,
            "calls_per_step": 1,
            "ms_per_call": ms_mean,
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_scores(v, ctx),
    }
    print(json.dumps(record), flush=True)
    return 0


COMPRESS_BUDGET = 1024   # tokens kept per sequence (the PagedEviction section's cache budget)


def bench_compress(args) -> int:
    """PagedEviction's prefill phase on its own: one paged_kv_compress_prefill
    call per step, compressing every sequence of a decode workload's cache
    (importances from paged_kv_token_scores) to COMPRESS_BUDGET tokens.  The
    call works in place, so the cache, importances and lengths are restored
    from a pristine copy before each step, outside the timed region."""
    import torch

    from paged_kv_cache_393_amd import accounting as A
    from paged_kv_cache_393_amd import binding as B
    from paged_kv_cache_393_amd import inputs as I

    wl = I.WORKLOADS[args.workload[len("compress_"):]]
    if wl.num_layers != 1:
        raise SystemExit("compression bench takes a single-layer workload")
    budget = COMPRESS_BUDGET
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = I.make_inputs(wl, dev)
    v = I.layer_views(inp, 0)
    scores = B.token_scores(v)
    names = ["k_cache", "v_cache", "context_lens"] + (["k_scales", "v_scales"] if "k_scales" in v else [])
    pristine = {n: v[n].clone() for n in names}
    pristine_scores = scores.clone()
    ws = torch.empty(max(16, B.compress_workspace_bytes(v["k_cache"], v["block_tables"], budget)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print(f"[bench] inputs for compression of {wl.name} ready", file=sys.stderr, flush=True)

    def step():
        B.compress_prefill(v, scores, budget, workspace=ws, stream=stream)

    flush_buf = None if args.no_flush else torch.ones((2 << 30) // 4, dtype=torch.float32,
                                                       device=dev)

    def restore_and_evict():
        for n in names:
            v[n].copy_(pristine[n])
        scores.copy_(pristine_scores)
        if flush_buf is not None:
            flush_buf.amax()

    for _ in range(args.warmup):
        restore_and_evict()
        step()
    torch.cuda.synchronize()
    ms = event_ms(stream, step, args.steps, before=restore_and_evict)
    ms_sorted = sorted(ms)
    ms_mean = statistics.fmean(ms)
    pct = lambda q: ms_sorted[min(len(ms_sorted) - 1, int(q * len(ms_sorted)))]
    print(f"[bench] {args.steps} timed steps done", file=sys.stderr, flush=True)

    ctx = pristine["context_lens"].cpu().tolist()
    sc_host = pristine_scores.cpu().numpy()
    bt_host = v["block_tables"].cpu().numpy()
    bs = wl.block_size
    logical = []
    for s_, n in enumerate(ctx):
        t = list(range(n))
        logical.append(sc_host[bt_host[s_][[x // bs for x in t]], [x % bs for x in t]])
    moved = A.compress_moved_tokens(logical, budget)
    nbytes = A.compress_bytes(ctx, budget, moved, wl.num_kv_heads, wl.head_dim, bs, wl.kv_dtype)
    t_s = ms_mean / 1e3
    gbps = nbytes / t_s / 1e9
    copy_for_counters(args, dev, stream)
    name = "compress_" + wl.name
    over = [c for c in ctx if c > budget]
    record = {
        "metric": "PagedEviction prefill-phase compression context tokens/s and achieved HBM GB/s "
                  "(% of peak), Llama-3-8B shape",
        "value": sum(over) / t_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_mean,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic (seeded N(0,1) K/V, shuffled block pool; importances ||V||/||K|| of it)",
        "config": {"workload": name, "num_seqs": wl.num_seqs, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": bs, "budget": budget,
                   "context_tokens": sum(ctx), "compressed_seqs": len(over),
                   "compressed_context_tokens": sum(over), "moved_tokens": moved,
                   "kv_dtype": wl.kv_dtype,
                   "cache_evict_between_steps": "2 GiB read" if flush_buf is not None else None},
        "pct_of_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
        "ms_p10": pct(0.10), "ms_median": pct(0.50), "ms_p90": pct(0.90),
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_kv_compress_prefill call: select kernel(s) + compress_move_kernel",
            "achieved": gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "traffic": measured_traffic(name, "compress"),
            "algorithmic_bytes_per_call": nbytes,
            "calls_per_step": 1,
            "ms_per_call": ms_mean,
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_compress(
            {n: pristine[n] for n in names} | {"block_tables": v["block_tables"]}, pristine_scores,
            budget, v, scores, sum(over)),
    }
    print(json.dumps(record), flush=True)
    return 0


def cpu_baseline_compress(pristine, pristine_scores, budget, gpu_views, gpu_scores, tokens,
                          budget_s=12.0):
    """The oracle's compression of the whole workload (one thread), median of
    repeated runs on the host copy, scaled to compressed context tokens/s; and
    whether the GPU's last result is bit-identical to it."""
    import numpy as np
    import torch

    import oracle

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    host = {n: t.cpu() for n, t in pristine.items()}
    sc = pristine_scores.cpu().numpy()
    times, ref = [], None
    while sum(times) < budget_s and len(times) < 5:
        t = time.perf_counter()
        ref = oracle.compress_prefill(host, sc, budget)
        times.append(time.perf_counter() - t)
    t_med = statistics.median(times)
    raw = lambda x: x.detach().cpu().contiguous().view(torch.uint8).numpy().reshape(ref["k_cache"].shape)
    same = (np.array_equal(raw(gpu_views["k_cache"]), ref["k_cache"]) and
            np.array_equal(raw(gpu_views["v_cache"]), ref["v_cache"]) and
            np.array_equal(gpu_views["context_lens"].cpu().numpy(), ref["context_lens"]) and
            np.array_equal(gpu_scores.cpu().numpy().view(np.uint32), ref["scores"].view(np.uint32)))
    return {
        "value": tokens / t_med,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the whole workload ({tokens} context tokens of compressed sequences), one "
                  f"thread, median of {len(times)} runs of {t_med:.2f}s",
        "parity_bit_identical_vs_gpu": bool(same),
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak, published


def bench_prefill(args) -> int:
    """Chunked-prefill attention on its own: one paged_attn_prefill call per step."""
    import torch

    from paged_kv_cache_393_amd import accounting as A
    from paged_kv_cache_393_amd import binding as B
    from paged_kv_cache_393_amd import inputs as I

    pw = I.PREFILL_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    v = I.make_prefill_inputs(pw, dev)
    out = torch.empty(v["q"].shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print(f"[bench] inputs for {pw.name} ready", file=sys.stderr, flush=True)

    def key_split_of(views):
        if args.key_splits is not None:
            return args.key_splits
        return B.prefill_plan(B.prefill_shape_of(views, views["q"], views["q_offsets"],
                                                 views["max_q_len"]))

    def pf_workspace(views, ks):
        sh = B.prefill_shape_of(views, views["q"], views["q_offsets"], views["max_q_len"])
        return B.alloc_prefill_workspace(sh, ks, dev)

    key_splits = key_split_of(v)
    pf_ws = pf_workspace(v, key_splits)

    def step():
        B.prefill_views(v, v["q"], v["q_offsets"], v["max_q_len"], out=out, stream=stream,
                        key_splits=key_splits, workspace=pf_ws)

    split = None
    if args.split_decodes:
        split = split_decode_batch(pw, v, out, dev)
        key_splits = key_split_of(split["chunks"])
        pf_ws = pf_workspace(split["chunks"], key_splits)

        def step():
            B.prefill_views(split["chunks"], split["chunks"]["q"], split["chunks"]["q_offsets"],
                            split["chunks"]["max_q_len"], out=split["chunk_out"], stream=stream,
                            key_splits=key_splits, workspace=pf_ws)
            B.decode_views(split["decodes"], out=split["decode_out"], workspace=split["ws"],
                           stream=stream)

    flush_buf = None if args.no_flush else torch.ones((2 << 30) // 4, dtype=torch.float32,
                                                       device=dev)

    def evict():
        if flush_buf is not None:
            flush_buf.amax()

    for _ in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()
    ms = event_ms(stream, step, args.steps, before=evict)
    ms_sorted = sorted(ms)
    ms_mean = statistics.fmean(ms)
    pct = lambda q: ms_sorted[min(len(ms_sorted) - 1, int(q * len(ms_sorted)))]
    print(f"[bench] {args.steps} timed steps done", file=sys.stderr, flush=True)
    flops = A.prefill_flops(pw.ctx, pw.n_q, pw.num_q_heads, pw.head_dim)
    nbytes = A.prefill_bytes(pw.ctx, pw.n_q, pw.num_q_heads, pw.num_kv_heads, pw.head_dim,
                             pw.block_size, pw.kv_dtype)
    t_s = ms_mean / 1e3
    tflops = flops / t_s / 1e12
    gbps = nbytes / t_s / 1e9
    # The bound is whichever resource the batch would saturate first: a batch
    # of long chunks is matrix-core work, one chunk among many decodes mostly
    # streams the decodes' K/V.
    hbm_bound = nbytes / (HBM_PEAK_GBPS * 1e9) > flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    pf_name = "paged_attn_prefill_split" if key_splits > 1 else "paged_attn_prefill"
    pf_kernels = "pa_prefill_kernel + pa_prefill_merge_kernel" if key_splits > 1 else "pa_prefill_kernel"
    split_check = None
    if split is not None:
        # the same queries through one paged_attn_prefill call, for comparison
        whole = B.prefill_views(v, v["q"], v["q_offsets"], v["max_q_len"])
        torch.cuda.synchronize()
        split_check = split_max_diff(split, whole)
        # the batch's output, as the two calls left it, for the oracle's check
        out.index_copy_(0, split["rows_c"], split["chunk_out"])
        out.index_copy_(0, split["rows_d"], split["decode_out"])
        torch.cuda.synchronize()
    copy_for_counters(args, dev, stream)
    record = {
        "metric": "chunked-prefill attention query tokens/s and achieved bf16 matrix-core "
                  "TFLOP/s (% of peak), Llama-3-8B shape",
        "value": sum(pw.n_q) / t_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_mean,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/K/V, shuffled block pool)",
        "config": {"workload": pw.name, "kv_dtype": pw.kv_dtype, "context_lens": list(pw.ctx),
                   "query_tokens": list(pw.n_q),
                   "num_q_heads": pw.num_q_heads, "num_kv_heads": pw.num_kv_heads,
                   "head_dim": pw.head_dim, "block_size": pw.block_size,
                   "cache_evict_between_steps": "2 GiB read" if flush_buf is not None else None},
        "ms_p10": pct(0.10), "ms_median": pct(0.50), "ms_p90": pct(0.90),
        "hbm_gbps": gbps,
        "tflops": tflops,
        "calls": (f"{pf_name} (chunks) + paged_attn_decode (one-token queries)"
                  if split is not None else pf_name),
        "key_splits": key_splits,
        "split_vs_single_call_max_abs_diff": split_check,
        "roofline": {
            "bound": "hbm" if hbm_bound else "mfma",
            "kernel": (f"{pf_kernels} + pa_decode_kernel + pa_merge_kernel" if split is not None
                       else pf_kernels),
            "achieved": gbps if hbm_bound else tflops,
            "peak": HBM_PEAK_GBPS if hbm_bound else MFMA_BF16_PEAK_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": gbps / HBM_PEAK_GBPS if hbm_bound else tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": (measured_traffic(f"{pw.name}_split", "serving")
                        if split is not None and key_splits > 1
                        else None if split is not None or key_splits > 1
                        else measured_traffic(pw.name, "prefill")),
            "algorithmic_flops_per_call": flops,
            "algorithmic_bytes_per_call": nbytes,
            "calls_per_step": 1,
            "ms_per_call": ms_mean,
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_prefill(pw, v, out, flops),
    }
    print(json.dumps(record), flush=True)
    return 0


def split_decode_batch(pw, v, out, dev):
    """The batch of a prefill workload as two calls' inputs: its multi-token
    chunks (a paged_attn_prefill batch) and its one-token queries (a
    paged_attn_decode batch), views of the same cache, with their outputs and
    the decode workspace."""
    import torch

    from paged_kv_cache_393_amd import binding as B

    qo = v["q_offsets"].cpu().tolist()
    chunk_ids = [s for s, n in enumerate(pw.n_q) if n > 1]
    dec_ids = [s for s, n in enumerate(pw.n_q) if n == 1]
    if not chunk_ids or not dec_ids:
        raise SystemExit("--split-decodes needs a batch with both chunks and one-token queries")
    base = {n: v[n] for n in ("k_cache", "v_cache", "scale") if n in v}
    for n in ("k_scales", "v_scales"):
        if n in v:
            base[n] = v[n]
    ci = torch.tensor(chunk_ids, device=dev)
    di = torch.tensor(dec_ids, device=dev)
    rows_c = torch.cat([torch.arange(qo[s], qo[s + 1]) for s in chunk_ids]).to(dev)
    rows_d = torch.tensor([qo[s] for s in dec_ids], device=dev)
    nq_c = torch.tensor([0] + [pw.n_q[s] for s in chunk_ids], dtype=torch.int64)
    chunks = dict(base, q=v["q"].index_select(0, rows_c).contiguous(),
                  q_offsets=torch.cumsum(nq_c, 0).to(torch.int32).to(dev),
                  max_q_len=max(pw.n_q[s] for s in chunk_ids),
                  block_tables=v["block_tables"].index_select(0, ci).contiguous(),
                  context_lens=v["context_lens"].index_select(0, ci).contiguous())
    decodes = dict(base, q=v["q"].index_select(0, rows_d).contiguous(),
                   block_tables=v["block_tables"].index_select(0, di).contiguous(),
                   context_lens=v["context_lens"].index_select(0, di).contiguous())
    shape = B.shape_of(decodes["q"], decodes["k_cache"], decodes["block_tables"], 0)
    return {"chunks": chunks, "decodes": decodes, "rows_c": rows_c, "rows_d": rows_d,
            "chunk_out": torch.empty(chunks["q"].shape, dtype=torch.float32, device=dev),
            "decode_out": torch.empty(decodes["q"].shape, dtype=torch.float32, device=dev),
            "ws": B.alloc_workspace(shape, dev)}


def split_max_diff(split, whole) -> float:
    """Largest |difference| between the two-call outputs and one paged_attn_prefill call's."""
    a = (split["chunk_out"] - whole.index_select(0, split["rows_c"])).abs().max()
    b = (split["decode_out"] - whole.index_select(0, split["rows_d"])).abs().max()
    return float(max(a, b))


def cpu_baseline_prefill(pw, v, out, flops_total):
    """The oracle on the first (shortest) chunk of the batch, median of repeated
    runs up to about 3 s, scaled to the whole call by flop count; and its
    largest difference from the GPU output on that chunk."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_393_amd import accounting as A
    from paged_kv_cache_393_amd import inputs as I

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    sub = I.select_sequences(v, [0], pw.block_size)
    nq = pw.n_q[0]
    q0 = I.bf16_bits(v["q"][:nq].cpu())
    tail = (sub["block_tables"].numpy(), sub["context_lens"].numpy(), [0, nq], sub["scale"])
    if pw.kv_dtype == "int8":
        fn = oracle.paged_prefill_int8
        args = (q0, sub["k_cache"].numpy(), sub["v_cache"].numpy(), sub["k_scales"].numpy(),
                sub["v_scales"].numpy()) + tail
    elif pw.kv_dtype == "fp8":
        fn = oracle.paged_prefill_fp8
        codes = lambda t: t.contiguous().view(torch.uint8).numpy()
        args = (q0, codes(sub["k_cache"]), codes(sub["v_cache"])) + tail
    else:
        fn = oracle.paged_prefill_bf16
        args = (q0, I.bf16_bits(sub["k_cache"]), I.bf16_bits(sub["v_cache"])) + tail
    times, ref = [], None
    while sum(times) < 3.0 and len(times) < 25:
        t = time.perf_counter()
        ref = fn(*args)
        times.append(time.perf_counter() - t)
    t_med = statistics.median(times)
    f0 = A.prefill_flops(pw.ctx[:1], pw.n_q[:1], pw.num_q_heads, pw.head_dim)
    t_full = t_med * flops_total / f0
    return {
        "value": sum(pw.n_q) / t_full,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"chunk 0 ({nq} queries over {pw.ctx[0]} tokens), median of {len(times)} runs "
                   f"of {t_med:.3f}s, scaled to the whole call by flop count"),
        "parity_max_abs_vs_gpu": float(np.abs(out[:nq].double().cpu().numpy() - ref).max()),
    }


def cpu_baseline_scores(views, ctx, budget_s=3.0):
    """The oracle's scoring on the first sequences (about budget_s per run),
    median of repeated runs, scaled to tokens/s; and its largest relative
    difference from the GPU's scores on that sample."""
    import numpy as np

    import oracle
    from paged_kv_cache_393_amd import inputs as I

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    S = len(ctx)
    t = time.perf_counter()
    host = I.select_sequences(views, [0], views["k_cache"].shape[1])
    oracle.token_scores(host)
    per_tok = (time.perf_counter() - t) / max(1, ctx[0])
    n = max(1, min(S, int(budget_s / max(per_tok * sum(ctx) / S, 1e-12))))
    sub = I.select_sequences(views, list(range(n)), views["k_cache"].shape[1])
    times, ref = [], None
    while sum(times) < budget_s and len(times) < 25:
        t = time.perf_counter()
        ref = oracle.token_scores(sub)
        times.append(time.perf_counter() - t)
    t_med = statistics.median(times)
    tokens = sum(ctx[:n])
    return {
        "value": tokens / t_med,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the first {n} of {S} sequences ({tokens} tokens), one thread, median of "
                  f"{len(times)} runs of {t_med:.3f}s",
    }


def cpu_baseline_write(ww, inp, budget_s=3.0):
    """The oracle's write on a prefix of the workload's tokens sized to about
    budget_s per run (host copies of the same inputs; the whole workload when
    it fits), median of repeated runs scaled to all tokens, and whether the
    sampled tokens' cache rows match the GPU's bytes."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_393_amd import inputs as I

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    kb_all, vb_all = I.bf16_bits(inp["key"]), I.bf16_bits(inp["value"])
    sl_all = inp["slots"].cpu().numpy()
    shape = tuple(inp["k_cache"].shape)
    rows = lambda a: a.reshape(shape[0] * shape[1], *a.shape[2:])
    if ww.kv_dtype == "bf16":
        z = np.zeros(shape, dtype=np.uint16)
        run = lambda n: oracle.kv_write_bf16(kb_all[:n], vb_all[:n], sl_all[:n], z, z)
        got = (I.bf16_bits(inp["k_cache"]), I.bf16_bits(inp["v_cache"]))
    elif ww.kv_dtype == "fp8":
        z = np.zeros(shape, dtype=np.uint8)
        run = lambda n: oracle.kv_write_fp8(kb_all[:n], vb_all[:n], sl_all[:n], z, z)
        got = tuple(inp[k].view(torch.uint8).cpu().numpy() for k in ("k_cache", "v_cache"))
    else:
        z = np.zeros(shape, dtype=np.int8)
        zs = np.zeros(tuple(inp["k_scales"].shape), dtype=np.float32)
        run = lambda n: oracle.kv_write_int8(kb_all[:n], vb_all[:n], sl_all[:n], z, z, zs, zs)
        got = tuple(inp[k].cpu().numpy() for k in ("k_cache", "v_cache", "k_scales", "v_scales"))
    T = ww.num_tokens
    t = time.perf_counter()
    run(min(T, 256))
    per_tok = (time.perf_counter() - t) / min(T, 256)
    n = max(256, min(T, int(budget_s / max(per_tok, 1e-12))))
    times, ref = [], None
    while sum(times) < budget_s and len(times) < 25:
        t = time.perf_counter()
        ref = run(n)
        times.append(time.perf_counter() - t)
    t_med = statistics.median(times)
    written = sl_all[:n][sl_all[:n] >= 0]
    same = all(np.array_equal(rows(a)[written].view(np.uint8), rows(b)[written].view(np.uint8))
               for a, b in zip(got, ref))
    return {
        "value": n / t_med,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"the first {n} of {T} tokens, one thread, median of {len(times)} runs of "
                   f"{t_med:.3f}s (the copy of the caches into fresh arrays included), "
                   f"tokens/s of the sample"),
        "bit_identical_to_gpu_on_sample": bool(same),
    }


def cpu_baseline(wl, views0, out0, ctx, n_layers, budget_s):
    """fp64 oracle on a bounded sample of layer 0, scaled to the whole step by
    context-token count.  The sample is a prefix of the batch sized to about
    budget_s of work; small samples are timed several times (median)."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_393_amd import inputs as I

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    threads = oracle.num_threads()

    def run(ids):
        sub = I.select_sequences(views0, ids, wl.block_size)
        qb = I.bf16_bits(sub["q"])
        bt = sub["block_tables"].numpy()
        cl = sub["context_lens"].numpy()
        if sub["k_cache"].dtype == torch.float8_e4m3fn:
            args = (qb, sub["k_cache"].view(torch.uint8).numpy(),
                    sub["v_cache"].view(torch.uint8).numpy(), bt, cl, sub["scale"])
            fn = oracle.paged_decode_fp8
        elif "k_scales" in sub:
            args = (qb, sub["k_cache"].numpy(), sub["v_cache"].numpy(), sub["k_scales"].numpy(),
                    sub["v_scales"].numpy(), bt, cl, sub["scale"])
            fn = oracle.paged_decode_int8
        else:
            args = (qb, I.bf16_bits(sub["k_cache"]), I.bf16_bits(sub["v_cache"]), bt, cl,
                    sub["scale"])
            fn = oracle.paged_decode_bf16
        t = time.perf_counter()
        ref = fn(*args)
        return time.perf_counter() - t, ref, args, fn

    t1, _, _, _ = run([0])
    per_token = t1 / max(1, ctx[0])
    avg = sum(ctx) / len(ctx)
    n = max(1, min(len(ctx), int(budget_s / max(per_token * avg, 1e-9))))
    ids = list(range(n))
    t_first, ref, args, fn = run(ids)
    times = [t_first]
    while sum(times) < min(budget_s, 3.0) and len(times) < 25:
        t = time.perf_counter()
        fn(*args)
        times.append(time.perf_counter() - t)
    t_sample = statistics.median(times)
    got = out0[ids].double().cpu().numpy()
    sample_tokens = sum(ctx[i] for i in ids)
    t_full = t_sample * (sum(ctx) / sample_tokens) * n_layers
    return {
        "value": len(ctx) / t_full,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{n} of {len(ctx)} sequences of layer 0 of {n_layers} "
                   f"({sample_tokens} of {sum(ctx)} context tokens), median of {len(times)} runs "
                   f"of {t_sample:.3f}s, scaled to the full step by context-token count"),
        "parity_max_abs_vs_gpu": float(np.abs(got - ref).max()),
    }


if __name__ == "__main__":
    sys.exit(main())
