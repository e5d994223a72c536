"""Benchmark of the fused indexer -> Top-K -> sparse-attention decode step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  A step is one dsa_decode_step over one batch of the
workload (default: long-context decode, batch 4 x 131072, FP8 indexer
64 x 128, Top-2048, 128-head MQA over a 576/512 bf16 latent).  Inputs are
resident in HBM before timing starts; R independent input sets rotate so the
bytes touched per rotation exceed the 256 MB Infinity Cache several times.

value      decode tokens/s = rows * steps / timed seconds (whole GPU)
roofline   the dominant kernel, the indexer scan as the fused step launches
           it: the algorithmic bytes of its launch (index keys, queries,
           weights, block-table entries; no score matrix) over its average
           duration, from HIP events that the kernel's own dispatch stamps
           on the launch stream (dsa_decode_step_timed), against
           the 8 TB/s HBM peak; `traffic` is the counter-measured HBM bytes per
           launch from profiles/ (null when the kernel source changed since)
stages     average duration of each stage of the fused step (scan, Top-K
           selection, attention, split-key merge) from the same events, and
           the gaps between them, with
           the attention's own HBM and bf16-MFMA roofline fractions
indexer_scores_launch  the scan launched alone by dsa_indexer_scores (it
           also writes the float32 score rows), timed with HIP events
cpu_baseline  the plain C++ oracle on the host: whole rows, on one thread
           and on every affinity core
workloads  the other workload shapes (decode 32 x 32k, ragged 64 x
           U[1k, 128k] with a shuffled table, chunked prefill of 4096 rows on
           a 61440-token prefix): step time, tokens/s, HBM fraction, and for
           the prefill the fraction of the FP8 + bf16 MFMA roofline
mxfp8_indexer  the same workload with MXFP8 indexer operands (one E8M0 scale
           per 32 dims): the fused step and the indexer scan alone, timed the
           same way over their own rotating input sets (--no-mxfp8 skips it)
step_us_spread  p10 / p50 / p90 of the step time over graph replays timed one by one
stream_launch  the same steps launched one by one on the stream (graph_replay
           instead when --graph 0 times stream launches for the headline)
read_reference a library streaming read (torch.sum over 1 GiB) as a reference for HBM reads
candidate_indexer  the same workload with a candidate-restricted indexer
           (16384 candidate positions per row): the fused step and the scan
           alone, timed the same way (--no-cand skips it)
indexer_prolog  dsa_indexer_prolog for the headline's rows and for 4096 prefill
           rows (4096-wide input, 64 x 128 MXFP8 outputs): launch time, HBM
           fraction of its weight stream, bf16 MFMA fraction (--no-prolog
           skips it)
fp8_kv_cache  the same workload over an FP8 KV cache (E4M3 latent rows, one
           float32 scale per tile of 128 elements): the fused step and its
           stage times, with the attention's HBM fraction (--no-fp8-kv skips it)
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFS = 5000.0    # dense FP8 MFMA, TFLOP/s
BF16_PEAK_TFS = 2500.0   # dense bf16 MFMA, TFLOP/s
MALL_BYTES = 256 << 20
OTHER_WORKLOADS = "decode_32x32k,ragged_64_1k_128k,prefill_4096_on_61440"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--mode", default=None, help="int or gauss (default: the workload's)")
    ap.add_argument("--rotate", type=int, default=0, help="input sets (0: auto)")
    ap.add_argument("--graph", type=int, default=1,
                    help="time graph replays (1) or stream launches (0); the two run within about "
                         "1 us per step of each other, but stream launches fall behind when the "
                         "host is slowed (under a profiler)")
    ap.add_argument("--no-graph-legs", action="store_true",
                    help="with --graph 0, capture no graphs (skips step_us_spread, graph_replay)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cand", action="store_true",
                    help="skip the candidate-restricted indexer leg")
    ap.add_argument("--no-mxfp8", action="store_true",
                    help="skip the MXFP8-indexer leg (same workload, group-32 scales)")
    ap.add_argument("--no-prolog", action="store_true",
                    help="skip the indexer-prolog leg (q and head-weight projections, key norm)")
    ap.add_argument("--no-fp8-kv", action="store_true",
                    help="skip the FP8-KV-cache leg (same workload, E4M3 rows, tile-128 scales)")
    ap.add_argument("--table", default=None)
    ap.add_argument("--legs", default=OTHER_WORKLOADS,
                    help="comma-separated other workloads to time after the headline ('none')")
    ap.add_argument("--no-scan-leg", action="store_true",
                    help="skip timing the scan launched alone by dsa_indexer_scores")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain elementwise copy of MIB MiB (float32 in, float32 out) "
                         "so that hardware byte counters can be scaled against known traffic")
    return ap.parse_args()


def log(msg):
    """Progress line on stderr (the JSON result alone goes to stdout)."""
    print(f"bench.py: {msg}", file=sys.stderr, flush=True)


def step_bytes(wl, lengths):
    """Algorithmic HBM bytes of one step: every index key of every history,
    the gathered KV rows, the queries, weights, block-table entries and the
    output (no score matrix: the fused step need not materialise one)."""
    total = 0
    row_kv = kv_row_bytes(wl)
    for L in lengths:
        n = min(wl.K, L)
        total += (wl.D_I * L + row_kv * n + wl.H_I * wl.D_I + 4 * wl.H_I
                  + 2 * wl.H_q * wl.D_qk + 2 * wl.H_q * wl.D_v + 4 * ((L + 63) // 64))
    return total


def indexer_bytes(wl, lengths, mx=False, scores=False):
    """Algorithmic bytes of one indexer-scan launch: index keys, queries,
    weights and block-table entries; with MXFP8 operands also one scale byte
    per 32 dims of every key and query; with ``scores`` the float32 score
    rows that dsa_indexer_scores writes (the fused step needs none)."""
    per = wl.D_I + (wl.D_I // 32 if mx else 0)
    return sum(per * L + wl.H_I * per + 4 * wl.H_I + 4 * ((L + 63) // 64)
               + (4 * L if scores else 0) for L in lengths)


def attention_bytes(wl, lengths):
    """Algorithmic bytes of the attention stage: the gathered KV rows, the
    queries and the output (the selection it reads is a few KiB)."""
    row_kv = kv_row_bytes(wl)
    return sum(row_kv * min(wl.K, L) + 2 * wl.H_q * wl.D_qk + 2 * wl.H_q * wl.D_v
               for L in lengths)


def kv_row_bytes(wl):
    """Bytes of one gathered KV row: bf16 K (and V), or FP8 codes plus one
    float32 scale per tile of 128 elements."""
    if getattr(wl, "kv_fmt", "bf16") == "fp8":
        return wl.D_qk + 4 * ((wl.D_qk + 127) // 128)
    return 2 * (wl.D_qk if wl.latent else wl.D_qk + wl.D_v)


def step_flops(wl, lengths):
    """(FP8 indexer flops, bf16 attention flops) of one step."""
    fp8 = sum(2 * wl.H_I * wl.D_I * L for L in lengths)
    bf16 = sum(2 * wl.H_q * (wl.D_qk + wl.D_v) * min(wl.K, L) for L in lengths)
    return fp8, bf16


def recorded_traffic(workload):
    """HBM bytes per indexer-scan dispatch from the committed counter summary
    for this workload, or None when there is none or when the kernel's source
    has changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"indexer_scan_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    h = re.search(r"source_sha256: ([0-9a-f]{64})", text)
    if not m or not h:
        return None
    csrc = os.path.join(ROOT, "indexer_top_sparse_score_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read()
                   for f in ("indexer_scan.hip", "dsa_common.h"))
    return int(m.group(1)) if hashlib.sha256(src).hexdigest() == h.group(1) else None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(decode shards by request; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from indexer_top_sparse_score_amd import binding as B
    from workloads import BENCH_WORKLOAD, CONFIGS, make_batch, row_positions

    B.load()
    name = args.workload or BENCH_WORKLOAD
    wl = CONFIGS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    first = make_batch(wl, device=dev, seed=wl.seed, mode=args.mode, table=args.table)
    lengths = [first.lengths[b] if not wl.prefill_rows else p + 1
               for b, p in row_positions(first)]
    rows = first.rows
    sb = step_bytes(wl, lengths)
    rotate = args.rotate or max(1, min(16, -(-4 * MALL_BYTES // sb)))
    sets = [first] + [make_batch(wl, device=dev, seed=wl.seed + 1000 * i, mode=args.mode,
                                 table=args.table) for i in range(1, rotate)]

    stream = torch.cuda.Stream()
    probs, outs, wss = [], [], []
    for s in sets:
        p = B.problem_for_batch(s)
        probs.append(p)
        outs.append((torch.empty((rows, wl.H_q, wl.D_v), dtype=torch.bfloat16, device=dev),
                     torch.empty((rows, wl.H_q), dtype=torch.float32, device=dev)))
    ws = B.workspace(probs[0], B.DSA_OP_DECODE_STEP, device=dev)

    def step(i):
        s, p = sets[i % rotate], probs[i % rotate]
        v = s.v if s.v is not None else s.kv
        out, lse = outs[i % rotate]
        B.dsa_decode_step(p, s.qI, s.w, s.kI, s.q, s.kv, v, out, ws, lse=lse, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    launch = "stream"
    graphs = {}
    if args.graph or not args.no_graph_legs:
        # one graph holds `rotate` consecutive steps (one per input set), the
        # way a decode graph holds every layer of a step; a second graph holds
        # the remainder so that exactly `steps` steps are timed
        try:
            for n in sorted({rotate, args.steps % rotate} - {0}):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(n):
                        step(i)
                graphs[n] = g
            with torch.cuda.stream(stream):
                for g in graphs.values():
                    g.replay()
            torch.cuda.synchronize()
            if args.graph:
                launch = f"graph ({rotate} steps per replay)"
        except Exception as e:  # capture unsupported: fall back to stream launches
            print(f"bench.py: graph capture failed ({e}); timing stream launches",
                  file=sys.stderr)
            graphs = {}
    assert B.device_errors(ws) == 0

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        if args.graph and graphs:
            for _ in range(args.steps // rotate):
                graphs[rotate].replay()
            if args.steps % rotate:
                graphs[args.steps % rotate].replay()
        else:
            for i in range(args.steps):
                step(i)
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    assert B.device_errors(ws) == 0
    ms_per_step = 1e3 * gpu_s / args.steps
    value = rows * args.steps / gpu_s

    # ---- per-stage times of the fused step, from HIP events recorded between
    # its kernels on the launch stream; the dominant kernel is the scan
    log(f"headline {name}: {ms_per_step * 1e3:.2f} us per step; stage times")
    st = stage_times(args, sets, probs, outs, ws, stream)
    ib = indexer_bytes(wl, lengths)
    achieved = ib / (st["indexer_us"] * 1e-6) / 1e9
    ab = attention_bytes(wl, lengths)
    _, attn_flops = step_flops(wl, lengths)
    st["attention_gbs"] = round(ab / (st["attention_us"] * 1e-6) / 1e9, 1)
    st["attention_hbm_frac"] = round(st["attention_gbs"] / HBM_PEAK_GBS, 4)
    st["attention_bytes"] = ab
    st["attention_bf16_mfma_frac"] = round(
        attn_flops / (st["attention_us"] * 1e-6) / 1e12 / BF16_PEAK_TFS, 4)
    traffic = recorded_traffic(name)

    result = {
        "metric": "sparse-attn decode tokens/s at 128k ctx, K=2048; % of HBM peak (GB/s)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16 (fp32 accumulate)",
        "data": "synthetic",
        "config": {
            "workload": name, "rows": rows, "context": max(lengths), "K": wl.K,
            "indexer": f"{wl.H_I}x{wl.D_I} e4m3", "attention": f"{wl.H_q} heads {wl.D_qk}/{wl.D_v} bf16"
            + (" latent" if wl.latent else ""), "mode": args.mode or wl.mode,
            "table": args.table or wl.table, "rotation_sets": rotate, "launch": launch,
        },
        "step_gbs": round(sb / (ms_per_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(sb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_bytes": sb,
        "roofline": {
            "bound": "hbm", "kernel": "indexer_scan_kernel (fused step)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "bytes_per_launch": ib, "avg_launch_us": st["indexer_us"],
        },
        "stages": st,
        "wall_s": round(wall, 4),
    }
    if not args.no_scan_leg:
        result["indexer_scores_launch"] = scan_leg(args, wl, lengths, sets, probs, stream)

    result.update(spread_legs(args, graphs, rotate, step, stream, rows))
    if not args.no_mxfp8:
        log("mxfp8 indexer leg")
        result["mxfp8_indexer"] = guarded(mxfp8_leg, args, wl, lengths, stream, rotate_bytes=ib)
    if not args.no_cand:
        log("candidate indexer leg")
        result["candidate_indexer"] = guarded(cand_leg, args, wl, lengths, stream)
    if not args.no_fp8_kv:
        log("fp8 kv leg")
        result["fp8_kv_cache"] = guarded(fp8_kv_leg, args, wl, lengths, stream)
    if not args.no_prolog:
        log("indexer prolog leg")
        result["indexer_prolog"] = guarded(prolog_leg, args, wl, stream)
    legs = [x for x in args.legs.split(",") if x and x != "none" and x != name]
    if legs:
        del sets, probs, outs, graphs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["workloads"] = {x: guarded(workload_leg, args, x, stream) for x in legs}

    if args.copy_calibration:
        n = (args.copy_calibration << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(3):
                torch.neg(src, out=dst)
        torch.cuda.synchronize()
        result["copy_calibration"] = {"kernel": "elementwise neg (float32)",
                                      "read_bytes": 4 * n, "write_bytes": 4 * n, "launches": 3}

    if not args.no_cpu_baseline:
        log("cpu baseline")
        result["cpu_baseline"] = cpu_baseline(first, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def guarded(fn, *a, **kw):
    """A side leg: its result, or the error that stopped it (the headline
    line is still printed)."""
    try:
        return fn(*a, **kw)
    except Exception as e:  # reported in the JSON line, not hidden
        log(f"{fn.__name__} failed: {e!r}")
        return {"error": repr(e)}


def stage_times(args, sets, probs, outs, ws, stream):
    """Average duration of each stage of the fused step over `steps` eager
    launches of dsa_decode_step_timed on the stream, rotating the input
    sets: each kernel's dispatch stamps HIP events with its own start and
    end, so the figures are kernel durations; the gaps between stages are
    reported apart."""
    import torch
    from indexer_top_sparse_score_amd import binding as B
    nset = len(sets)
    names = ("indexer_us", "topk_us", "attention_us", "merge_us")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            for e in evs[i]:
                e.record(stream)  # torch creates its events on first record
        torch.cuda.synchronize()

        def one(i, ev):
            s, p = sets[i % nset], probs[i % nset]
            out, lse = outs[i % nset]
            v = s.v if s.v is not None else s.kv
            B.dsa_decode_step_timed(p, s.qI, s.w, s.kI, s.q, s.kv, v, out, ws, ev, lse=lse,
                                    stream=stream)
        for i in range(args.warmup):
            one(i, evs[i % args.steps])
        torch.cuda.synchronize()
        for i in range(args.steps):
            one(i, evs[i])
    torch.cuda.synchronize()
    assert B.device_errors(ws) == 0
    out = {}
    for k, nm in enumerate(names):
        t = sorted(1e3 * evs[i][2 * k].elapsed_time(evs[i][2 * k + 1]) for i in range(args.steps))
        out[nm] = round(sum(t) / len(t), 3)
        out[nm.replace("_us", "_p50_us")] = round(t[len(t) // 2], 3)
    gaps = [sum(1e3 * evs[i][2 * k + 1].elapsed_time(evs[i][2 * k + 2]) for i in range(args.steps))
            / args.steps for k in range(3)]
    out["gaps_us"] = [round(g, 3) for g in gaps]
    out["sum_us"] = round(sum(out[nm] for nm in names) + sum(gaps), 3)
    out["launch"] = "stream (eager), kernel start/end stamped by the dispatches"
    return out


def scan_leg(args, wl, lengths, sets, probs, stream):
    """The indexer scan launched alone by dsa_indexer_scores over the same
    rotating input sets, timed with HIP events on the stream; its bytes
    include the float32 score rows it writes."""
    import torch
    from indexer_top_sparse_score_amd import binding as B
    nset = len(sets)
    rows = sets[0].rows
    scores = torch.empty((rows, 64 * sets[0].max_blocks), dtype=torch.float32, device="cuda")
    ws_i = B.workspace(probs[0], B.DSA_OP_INDEXER_SCORES, device="cuda")

    def scan(i):
        s = sets[i % nset]
        B.dsa_indexer_scores(probs[i % nset], s.qI, s.w, s.kI, scores, ws_i, stream=stream)

    us = timed_eager(args, scan, stream)
    assert B.device_errors(ws_i) == 0
    ib = indexer_bytes(wl, lengths, scores=True)
    ach = ib / (us * 1e-6) / 1e9
    return {"avg_launch_us": round(us, 3), "bytes_per_launch": ib, "achieved": round(ach, 1),
            "frac": round(ach / HBM_PEAK_GBS, 4)}


def timed_eager(args, fn, stream, steps=None):
    """Average microseconds of fn(i) over `steps` eager launches on the
    stream after the warm-up, with HIP events on that stream."""
    import torch
    steps = steps or args.steps
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            fn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / steps


def workload_leg(args, name, stream):
    """One of the other workload shapes: the fused step over input sets that
    rotate past the Infinity Cache (graph replays of one step per set, as
    the headline), its stage times, tokens/s and HBM fraction; for a
    prefill, also the fraction of the FP8 + bf16 MFMA roofline."""
    import torch
    from indexer_top_sparse_score_amd import binding as B
    from workloads import CONFIGS, make_batch, row_positions
    wl = CONFIGS[name]
    log(f"workload leg {name}")
    dev = torch.device("cuda:0")
    first = make_batch(wl, device=dev, seed=wl.seed, mode=args.mode)
    lengths = [first.lengths[b] if not wl.prefill_rows else p + 1
               for b, p in row_positions(first)]
    rows = first.rows
    sb = step_bytes(wl, lengths)
    fp8, bf16 = step_flops(wl, lengths)
    nset = max(1, min(8, -(-4 * MALL_BYTES // sb)))
    if wl.prefill_rows:
        nset = 1  # compute-bound: nothing to gain from rotation
    # every set has the first one's lengths (ragged shapes: the same mix)
    sets = [first] + [make_batch(wl, device=dev, seed=wl.seed + 1000 * i, mode=args.mode,
                                 lengths=first.lengths) for i in range(1, nset)]
    probs = [B.problem_for_batch(s) for s in sets]
    outs = [(torch.empty((rows, wl.H_q, wl.D_v), dtype=torch.bfloat16, device=dev),
             torch.empty((rows, wl.H_q), dtype=torch.float32, device=dev)) for _ in sets]
    ws = B.workspace(max(probs, key=lambda p: B.dsa_workspace_size(p, B.DSA_OP_DECODE_STEP)),
                     B.DSA_OP_DECODE_STEP, device=dev)

    def step(i):
        s, p = sets[i % nset], probs[i % nset]
        out, lse = outs[i % nset]
        v = s.v if s.v is not None else s.kv
        B.dsa_decode_step(p, s.qI, s.w, s.kI, s.q, s.kv, v, out, ws, lse=lse, stream=stream)

    steps = args.steps if not wl.prefill_rows else max(5, min(args.steps, 20))
    with torch.cuda.stream(stream):
        for i in range(max(1, args.warmup)):
            step(i)
    torch.cuda.synchronize()
    launch = "stream (eager)"
    us = None
    if args.graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(nset):
                    step(i)
            reps = max(1, steps // nset)
            with torch.cuda.stream(stream):
                g.replay()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            us = 1e3 * e0.elapsed_time(e1) / (reps * nset)
            steps = reps * nset
            launch = f"graph ({nset} steps per replay)"
            del g
        except Exception as e:  # capture unsupported: stream launches
            print(f"bench.py: graph capture failed for {name} ({e})", file=sys.stderr)
    if us is None:
        us = timed_eager(args, step, stream, steps)
    assert B.device_errors(ws) == 0
    sargs = argparse.Namespace(**{**vars(args), "steps": min(steps, 20), "warmup": 2})
    st = stage_times(sargs, sets, probs, outs, ws, stream)
    leg = {"rows": rows, "context_max": max(lengths), "rotation_sets": nset, "launch": launch,
           "steps": steps, "step_us": round(us, 3), "tokens_per_s": round(rows / (us * 1e-6), 1),
           "step_bytes": sb, "step_gbs": round(sb / (us * 1e-6) / 1e9, 1),
           "hbm_frac": round(sb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "stages_last_pass": st}
    if not wl.prefill_rows:
        # decode shapes run in one pass of rows: the stages cover the step
        leg["indexer_frac"] = round(indexer_bytes(wl, lengths) / (st["indexer_us"] * 1e-6)
                                    / 1e9 / HBM_PEAK_GBS, 4)
        leg["attention_hbm_frac"] = round(attention_bytes(wl, lengths) / (st["attention_us"]
                                          * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    else:
        ideal_us = 1e6 * (fp8 / (FP8_PEAK_TFS * 1e12) + bf16 / (BF16_PEAK_TFS * 1e12))
        leg.update({"fp8_tflop": round(fp8 / 1e12, 4), "bf16_tflop": round(bf16 / 1e12, 4),
                    "mfma_ideal_us": round(ideal_us, 1),
                    "mfma_roofline_frac": round(ideal_us / us, 4)})
    del sets, probs, outs, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return leg


def mxfp8_leg(args, wl, lengths, stream, rotate_bytes):
    """The same workload with MXFP8 indexer operands (one E8M0 scale per 32
    dims): the indexer scan timed alone, and the fused step, both with HIP
    events on the launch stream over input sets that rotate past the
    Infinity Cache."""
    import torch
    from indexer_top_sparse_score_amd import binding as B
    from workloads import make_batch
    mwl = wl.with_(indexer_fmt="mxfp8")
    dev = torch.device("cuda:0")
    nset = max(1, min(8, -(-4 * MALL_BYTES // rotate_bytes)))
    sets = [make_batch(mwl, device=dev, seed=mwl.seed + 7000 + 1000 * i, mode=args.mode,
                       table=args.table) for i in range(nset)]
    probs = [B.problem_for_batch(s) for s in sets]
    rows = sets[0].rows
    ld = 64 * sets[0].max_blocks
    scores = torch.empty((rows, ld), dtype=torch.float32, device=dev)
    ws_i = B.workspace(probs[0], B.DSA_OP_INDEXER_SCORES, device=dev)
    ws = B.workspace(probs[0], B.DSA_OP_DECODE_STEP, device=dev)
    out = torch.empty((rows, mwl.H_q, mwl.D_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows, mwl.H_q), dtype=torch.float32, device=dev)

    def timed(fn):
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                fn(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.steps):
                fn(i)
            e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / args.steps  # us

    def scan(i):
        s = sets[i % nset]
        B.dsa_indexer_scores(probs[i % nset], s.qI, s.w, s.kI, scores, ws_i, stream=stream)

    def step(i):
        s = sets[i % nset]
        v = s.v if s.v is not None else s.kv
        B.dsa_decode_step(probs[i % nset], s.qI, s.w, s.kI, s.q, s.kv, v, out, ws, lse=lse,
                          stream=stream)

    idx_us = timed(scan)
    step_us = timed(step)
    assert B.device_errors(ws) == 0 and B.device_errors(ws_i) == 0
    ib = indexer_bytes(mwl, lengths, mx=True)
    achieved = ib / (idx_us * 1e-6) / 1e9
    return {"indexer": f"{mwl.H_I}x{mwl.D_I} e4m3 + e8m0/32", "rotation_sets": nset,
            "launch": "stream (eager)", "step_us": round(step_us, 3),
            "tokens_per_s": round(rows / (step_us * 1e-6), 1),
            "indexer_avg_launch_us": round(idx_us, 3), "indexer_bytes_per_launch": ib,
            "indexer_achieved": round(achieved, 1), "indexer_frac": round(achieved / HBM_PEAK_GBS, 4)}


def spread_legs(args, graphs, rotate, step, stream, rows):
    """After the timed region: the spread of the step time (graph replays
    timed one by one with HIP events, per step = replay / steps per replay),
    the same steps in the launch mode that the headline did not time (graph
    replays, or stream launches under --graph 1), and a plain streaming
    read (torch.sum over 1 GiB) as a reference ceiling for HBM reads."""
    import torch
    out = {}
    if graphs:
        n = max(8, args.steps // rotate)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        with torch.cuda.stream(stream):
            for k in range(n):
                evs[2 * k].record(stream)
                graphs[rotate].replay()
                evs[2 * k + 1].record(stream)
        torch.cuda.synchronize()
        per = sorted(1e3 * evs[2 * k].elapsed_time(evs[2 * k + 1]) / rotate for k in range(n))
        pick = lambda q: round(per[min(n - 1, int(q * n))], 3)
        out["step_us_spread"] = {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9),
                                 "replays": n, "steps_per_replay": rotate}
    # the launch mode that the headline did not time
    replay = graphs and not args.graph
    if replay or args.graph:
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                step(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if replay:
                for _ in range(args.steps // rotate):
                    graphs[rotate].replay()
                if args.steps % rotate:
                    graphs[args.steps % rotate].replay()
            else:
                for i in range(args.steps):
                    step(i)
            e1.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / args.steps
        leg = {"step_us": round(us, 3), "tokens_per_s": round(rows / (us * 1e-6), 1)}
        if replay:
            out["graph_replay"] = {**leg, "steps_per_replay": rotate}
        else:
            out["stream_launch"] = leg
    buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.sum(buf)
        e0.record(stream)
        for _ in range(5):
            torch.sum(buf)
        e1.record(stream)
    torch.cuda.synchronize()
    rd = 5 * buf.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    out["read_reference"] = {"kernel": "torch.sum over 1 GiB of float32", "gbs": round(rd, 1)}
    del buf
    return out


def cand_bytes(wl, lengths, n_cand):
    """Algorithmic bytes of one candidate-restricted indexer launch: per row,
    each candidate's key row, list entry and score, at most one block id per
    candidate, the row's queries and weights."""
    tot = 0
    for L in lengths:
        C = min(n_cand, L)
        tot += C * (wl.D_I + 4 + 4) + 4 * min(C, -(-L // 64)) + wl.H_I * wl.D_I + 4 * wl.H_I
    return tot


def fp8_kv_leg(args, wl, lengths, stream):
    """The same workload over an FP8 KV cache (E4M3 latent rows, one float32
    scale per tile of 128 elements): the fused step (stream launches, HIP
    events) and its stage times, over input sets that rotate past the
    Infinity Cache."""
    import torch
    from indexer_top_sparse_score_amd import binding as B
    from workloads import make_batch
    fwl = wl.with_(kv_fmt="fp8")
    dev = torch.device("cuda:0")
    nset = 8
    sets = [make_batch(fwl, device=dev, seed=fwl.seed + 9000 + 1000 * i, mode=args.mode,
                       table=args.table, lengths=lengths) for i in range(nset)]
    probs = [B.problem_for_batch(s) for s in sets]
    rows = sets[0].rows
    ws = B.workspace(probs[0], B.DSA_OP_DECODE_STEP, device=dev)
    outs = [(torch.empty((rows, fwl.H_q, fwl.D_v), dtype=torch.bfloat16, device=dev),
             torch.empty((rows, fwl.H_q), dtype=torch.float32, device=dev)) for _ in range(nset)]

    def step(i):
        s = sets[i % nset]
        out, lse = outs[i % nset]
        B.dsa_decode_step(probs[i % nset], s.qI, s.w, s.kI, s.q, s.kv, s.kv, out, ws, lse=lse,
                          stream=stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    step_us = 1e3 * e0.elapsed_time(e1) / args.steps
    st = stage_times(args, sets, probs, outs, ws, stream)
    assert B.device_errors(ws) == 0
    ab = attention_bytes(fwl, lengths)
    return {"kv_cache": f"e4m3 rows of {fwl.D_qk} + float32 scale per 128", "rotation_sets": nset,
            "launch": "stream (eager)", "step_us": round(step_us, 3),
            "tokens_per_s": round(rows / (step_us * 1e-6), 1),
            "kv_row_bytes": kv_row_bytes(fwl), "attention_bytes": ab,
            "attention_us": st["attention_us"], "merge_us": st["merge_us"],
            "attention_gbs": round(ab / (st["attention_us"] * 1e-6) / 1e9, 1),
            "attention_hbm_frac": round(ab / (st["attention_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "stages": st}


def prolog_leg(args, wl, stream):
    """dsa_indexer_prolog over a 4096-wide input for the headline's rows and
    for 4096 prefill rows: average launch time (HIP events on the launch
    stream, input sets rotating past the Infinity Cache), algorithmic bytes
    (both weight matrices, x, the new keys and every output) and flops."""
    import torch
    from indexer_top_sparse_score_amd import binding as B
    from workloads import PROLOG_D_X, make_batch, make_prolog_inputs, small_workload
    dev = torch.device("cuda:0")
    out = {"D_x": PROLOG_D_X, "indexer": f"{wl.H_I}x{wl.D_I} mxfp8"}
    F = wl.H_I * wl.D_I
    for label, rows in (("decode", wl.rows), ("prefill", 4096)):
        pw = small_workload("prolog", lengths=[64 * (1 + i % 16) for i in range(rows)],
                            H_I=wl.H_I, D_I=wl.D_I, mode="int", indexer_fmt="mxfp8",
                            H_q=wl.H_q, D_qk=wl.D_qk, D_v=wl.D_v, K=wl.K, scale=wl.scale)
        batch = make_batch(pw, device=dev, seed=pw.seed + 11)
        wbytes = 2 * (F + wl.H_I) * PROLOG_D_X
        nset = max(1, min(16, -(-4 * MALL_BYTES // wbytes))) if rows <= 64 else 2
        inps = [make_prolog_inputs(rows, wl.H_I, wl.D_I, D_x=PROLOG_D_X, mode="gauss",
                                   seed=100 + i, device=dev) for i in range(nset)]
        prob = B.problem_for_batch(batch)
        qI = torch.empty((rows, wl.H_I, wl.D_I), dtype=torch.uint8, device=dev)
        qs = torch.empty((rows, wl.H_I, wl.D_I // 32), dtype=torch.uint8, device=dev)
        w = torch.empty((rows, wl.H_I), dtype=torch.float32, device=dev)
        ws = B.workspace(prob, B.DSA_OP_INDEXER_PROLOG, device=dev)

        def run(i):
            inp = inps[i % nset]
            B.dsa_indexer_prolog(prob, inp.x, inp.w_q, inp.w_g, inp.k_new, inp.k_gamma, qI, qs,
                                 w, batch.kI, ws, stream=stream)

        steps = args.steps if rows <= 64 else max(5, args.steps // 5)
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                run(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                run(i)
            e1.record(stream)
        torch.cuda.synchronize()
        assert B.device_errors(ws) == 0
        us = 1e3 * e0.elapsed_time(e1) / steps
        byt = (wbytes + 2 * rows * PROLOG_D_X + 2 * rows * wl.D_I + 2 * wl.D_I
               + rows * (F + F // 32 + 4 * wl.H_I) + rows * (wl.D_I + wl.D_I // 32))
        flops = 2 * rows * (F + wl.H_I) * PROLOG_D_X
        out[label] = {"rows": rows, "rotation_sets": nset, "avg_launch_us": round(us, 3),
                      "bytes": byt, "gbs": round(byt / (us * 1e-6) / 1e9, 1),
                      "hbm_frac": round(byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "tflops": round(flops / (us * 1e-6) / 1e12, 2),
                      "bf16_mfma_frac": round(flops / (us * 1e-6) / 1e12 / 2500.0, 4)}
        del inps, batch
    return out


def cand_leg(args, wl, lengths, stream, n_cand=16384):
    """The same workload with a candidate-restricted indexer (16384 candidate
    positions per row): the indexer timed alone and the fused step (stream
    launches), with HIP events on the launch stream over input sets that
    rotate past the Infinity Cache."""
    import torch
    from indexer_top_sparse_score_amd import binding as B
    from workloads import make_batch
    cwl = wl.with_(n_cand=n_cand)
    dev = torch.device("cuda:0")
    nset = 4  # each set's KV (576 MiB at 4 x 128k) already exceeds the cache
    sets = [make_batch(cwl, device=dev, seed=cwl.seed + 9000 + 1000 * i, mode=args.mode,
                       table=args.table) for i in range(nset)]
    probs = [B.problem_for_batch(s) for s in sets]
    rows = sets[0].rows
    scores = torch.empty((rows, n_cand), dtype=torch.float32, device=dev)
    ws_i = B.workspace(probs[0], B.DSA_OP_INDEXER_SCORES, device=dev)
    ws = B.workspace(probs[0], B.DSA_OP_DECODE_STEP, device=dev)
    out = torch.empty((rows, cwl.H_q, cwl.D_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows, cwl.H_q), dtype=torch.float32, device=dev)

    def timed(fn):
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                fn(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.steps):
                fn(i)
            e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / args.steps  # us

    def scan(i):
        s = sets[i % nset]
        B.dsa_indexer_scores(probs[i % nset], s.qI, s.w, s.kI, scores, ws_i, stream=stream)

    def step(i):
        s = sets[i % nset]
        v = s.v if s.v is not None else s.kv
        B.dsa_decode_step(probs[i % nset], s.qI, s.w, s.kI, s.q, s.kv, v, out, ws, lse=lse,
                          stream=stream)

    idx_us = timed(scan)
    step_us = timed(step)
    assert B.device_errors(ws) == 0 and B.device_errors(ws_i) == 0
    cb = cand_bytes(cwl, lengths, n_cand)
    return {"candidates_per_row": n_cand, "rotation_sets": nset, "launch": "stream (eager)",
            "step_us": round(step_us, 3), "tokens_per_s": round(rows / (step_us * 1e-6), 1),
            "indexer_avg_launch_us": round(idx_us, 3), "indexer_bytes_per_launch": cb,
            "indexer_achieved": round(cb / (idx_us * 1e-6) / 1e9, 1)}


def cpu_baseline(batch, budget_s):
    """The plain C++ oracle, as it stands, on whole rows of the first input
    set: once on one host thread, then on every core this process may run on
    (os.sched_getaffinity), each for about budget_s / 2 seconds of wall time
    (at least one row)."""
    import oracle.cpp
    from workloads import oracle_arrays

    t_copy = time.perf_counter()
    arr = oracle_arrays(batch, rows=list(range(batch.rows)))
    t_copy = time.perf_counter() - t_copy
    oracle.cpp.lib()

    def run(threads, seconds):
        done = 0
        t0 = time.perf_counter()
        while done == 0 or time.perf_counter() - t0 < seconds:
            oracle.cpp.decode_step(
                qI=arr["qI"], w=arr["w"], kI_cache=arr["kI_cache"], q=arr["q"],
                k_cache=arr["k_cache"], v_cache=arr["v_cache"], block_table=arr["block_table"],
                seq_lens=arr["seq_lens"], K=arr["K"], scale=arr["scale"], D_v=arr["D_v"],
                row_seq=arr["row_seq"], row_pos=arr["row_pos"], rows=[done % batch.rows],
                keep_scores=False, qI_scale=arr.get("qI_scale"),
                kI_scale_cache=arr.get("kI_scale_cache"), threads=threads)
            done += 1
        return done, time.perf_counter() - t0

    cores = len(os.sched_getaffinity(0))
    n1, t1 = run(1, budget_s / 2)
    nc, tc = run(cores, budget_s / 2)
    return {"value": round(nc / tc, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"plain C++ oracle (binary64), whole rows of {batch.wl.name} "
                      f"(full history each), cycling over its {batch.rows} rows: {nc} rows in "
                      f"{tc:.1f} s on {cores} threads; host copy {t_copy:.1f} s not timed",
            "single_thread": {"value": round(n1 / t1, 4), "unit": "tokens/s", "cores": 1,
                              "sample": f"{n1} rows in {t1:.1f} s on 1 thread"},
            "affinity_cores": cores, "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
