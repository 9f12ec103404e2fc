#!/usr/bin/env python3
"""Paged decode attention throughput on one MI355X.

A step is one pass of the hot path over one batch, with every input already
resident in HBM:

1. the copy-on-write block copies, when the workload has shared prefixes;
2. the cache write of the tokens the step appends; when those are only each
   decode sequence's newest token, the decode kernel stores them itself
   instead (pa_decode_append; --append on/off overrides);
3. for the mixed continuous-batching workload, the prefill-chunk kernel
   (--overlap on runs it on a second stream beside the decode instead; both
   wait for the cache write);
4. the split-K decode partition kernel, then the rescaling reduce.

Prints one JSON line.  Warm-up runs the W untimed steps and then more, until
--warmup-ms (default 150) of wall time has passed: the GPU lowers its clocks
while the host builds the workload, and the first 20-40 steps after that run
10-20 % slow.  The line records how many warm-up steps ran.

    python bench.py [--steps K] [--warmup W] [--workload c2|c3|c4|c4p|c5]
    python bench.py --study prefix-cache|fragmentation|block-size|batch1|stream-peak

Default workload (c5): the mixed continuous-batching step at 70B-shaped heads,
the largest configuration that fits one GPU.
- 240 decode sequences, lognormal context lengths (median 1024, [64, 8192]),
  plus 16 prefill chunks of 256 queries over contexts U{256..4096}.
- 64 query / 8 KV heads, head_dim 128, bf16 cache in 32-token blocks.
- The step writes the chunks' and the decode tokens' K/V, runs the causal
  prefill chunks, then decodes with the balanced split (--partition P selects
  P-token partitions).
The line carries the decode kernel's HBM roofline (`roofline`), the prefill
kernel's MFMA roofline (`prefill`), and, timed the same way after the mixed
step in the same run, the long-context decode of 8 x 32,768 tokens in its
stated 512-token partitions (`c3_decode`, skipped with --no-extra).

Consecutive steps read different copies of the pools, at least 1 GiB apart
in total, so no step is served from the 256 MB Infinity Cache that the
previous step left warm.

The roofline object covers the decode partition kernel.  Its time comes from
HIP events recorded around that launch alone, on the stream it is launched
on, in every timed step.  Beside it, from a separate pass of the same steps
after the timed region, goes the kernel's time by events that the library
records with the kernel's own dispatch (pa_time_next_partitions:
hipExtLaunchKernel's start and stop events, the clock a kernel trace reports;
such launches cost the step several microseconds, so they stay out of the
timed region).  Its HBM traffic comes from rocprofv3 counters taken on the same command.
`--pmc-summary` turns two counter runs (FETCH_SIZE, then WRITE_SIZE) into the
committed summary that later bench runs read.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA peak, TFLOP/s
METRIC = "paged decode attention: seq-tokens/s and achieved HBM GB/s (% of peak)"
CALIB_BYTES = 1 << 30          # size of the plain copy that calibrates the byte counters
# streaming-read launch shapes timed beside the decode, (workgroups per CU,
# loads per thread, blocked order): the fastest of the stream-peak study
STREAM_SHAPES_BENCH = ((32, 1, 0), (8, 8, 1), (16, 8, 1), (32, 4, 1))

WORKLOAD_TEXT = {
    "c2": "Llama-3-8B-shaped decode: 64 sequences, context U{128..2048}, 32/8 heads, head_dim 128, "
          "bf16 cache, 16-token blocks, pool = need + 10%, one cache write per sequence",
    "c3": "long-context split-K decode: 8 sequences x 32768 tokens, 32/8 heads, head_dim 128, "
          "bf16 cache, 16-token blocks, 512-token partitions, keys x3",
    "c4": "shared-prefix decode with copy-on-write: 32 sequences share a 1016-token prefix "
          "(64 blocks), private suffix U{0..512} + 1 token, 32/8 heads, head_dim 128, bf16",
    "c4p": "shared prompts found by content (automatic prefix caching): 32 requests over 4 prompts "
           "of U{256..1024} tokens + private suffix U{0..512} + 1 token, 8 earlier requests freed, "
           "tight pool (evictions), 32/8 heads, head_dim 128, bf16",
    "c5": "mixed continuous-batching step at 70B-shaped heads: 240 decodes (lognormal context, "
          "median 1024, [64, 8192]) + 16 prefill chunks of 256 queries over context U{256..4096}, "
          "64/8 heads, head_dim 128, bf16, 32-token blocks",
}


# the kernels whose HBM traffic the committed counter summaries give, with
# the sources each is built from
KERNELS = {"decode": ("decode_partition_kernel", ("decode.hip", "pa_internal.h")),
           "prefill": ("prefill_kernel", ("prefill.hip", "pa_internal.h"))}


def kernel_source_hash(kernel="decode"):
    h = hashlib.sha256()
    for name in KERNELS[kernel][1]:
        with open(os.path.join(ROOT, "paged_kv_cache_424_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pmc_path(workload, kernel="decode"):
    stem = "decode_partition" if kernel == "decode" else kernel
    return os.path.join(ROOT, "profiles", f"{stem}_{workload}_pmc.json")


def load_traffic(workload, kernel="decode"):
    """HBM bytes per launch of the kernel from the committed counter summary,
    if it was taken on the current kernel source; else None."""
    path = pmc_path(workload, kernel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return d.get("hbm_bytes_per_launch")


# ---- counter summary ---------------------------------------------------------------------
def _counter_rows(run_dir, counter):
    """(kernel name, value) of every dispatch in a rocprofv3 --pmc CSV output tree."""
    rows = []
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {run_dir}")
    return rows


def _mean(rows, pred):
    vals = [v for name, v in rows if pred(name)]
    if not vals:
        raise SystemExit("no matching dispatch in the counter output")
    return sum(vals) / len(vals), len(vals)


def pmc_summary(args):
    """Write the traffic summary of one kernel (--kernel decode | prefill).

    The calibration kernel is torch's neg over a 1 GiB float32 tensor, which
    reads CALIB_BYTES and writes CALIB_BYTES; each counter is scaled by the
    factor that makes that kernel read exactly its size."""
    fetch = _counter_rows(args.fetch_dir, "FETCH_SIZE")
    write = _counter_rows(args.write_dir, "WRITE_SIZE")
    kname = KERNELS[args.kernel][0]
    is_dec = lambda n: kname in n                               # noqa: E731
    is_cal = lambda n: "neg" in n.lower()                       # noqa: E731
    f_dec, nf = _mean(fetch, is_dec)
    w_dec, nw = _mean(write, is_dec)
    f_cal, _ = _mean(fetch, is_cal)
    w_cal, _ = _mean(write, is_cal)
    ff = CALIB_BYTES / (f_cal * 1024.0)
    wf = CALIB_BYTES / (w_cal * 1024.0)
    d = {
        "workload": args.workload,
        "kernel": kname,
        "kernel_source_hash": kernel_source_hash(args.kernel),
        "dispatches": [nf, nw],
        "fetch_kib_per_launch": f_dec,
        "write_kib_per_launch": w_dec,
        "calibration": f"torch neg over {CALIB_BYTES} B float32 in the same process: "
                       f"FETCH_SIZE {f_cal:.0f} KiB, WRITE_SIZE {w_cal:.0f} KiB",
        "fetch_factor": ff,
        "write_factor": wf,
        "hbm_bytes_per_launch": f_dec * 1024.0 * ff + w_dec * 1024.0 * wf,
        "command": args.command or "",
    }
    with open(pmc_path(args.workload, args.kernel), "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    print(json.dumps(d))


# ---- CPU oracle baseline -----------------------------------------------------------------
def cpu_baseline(w, nseq, min_seconds=6.0, max_reps=400, prefill_chunks=2):
    """The CPU oracle (fp64, as it stands) on a bounded sample of the step.

    Decode: the first nseq sequences, repeated until about min_seconds of CPU
    work.  With prefill chunks (the mixed step), also every row of the first
    `prefill_chunks` chunks, once; the step's CPU time is then estimated as
    the decode time per context token times the step's decode tokens plus the
    prefill time per (query, visible key) pair times the step's pairs.  The
    rate is the step's decode tokens over that time, the GPU line's unit."""
    import numpy as np
    from tests import oracle_run
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:                                  # pragma: no cover
        blas = 1
    cores = len(os.sched_getaffinity(0))
    st = oracle_run.build(w)
    seqs = list(range(min(nseq, len(w.decode_seqs))))
    pairs = None if len(seqs) == len(w.decode_seqs) else [(i, h) for i in seqs for h in range(w.num_q_heads)]
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        out = oracle_run.oracle_decode(w, st, pairs=pairs)
        dt += time.perf_counter() - t0
        reps += 1
    assert np.isfinite(out[seqs]).all()
    toks = sum(w.seq_len(w.decode_seqs[i]) for i in seqs)
    all_toks = sum(w.seq_len(s) for s in w.decode_seqs)
    per_tok = dt / (reps * toks)
    sample = (f"fp64 numpy oracle decode of {len(seqs)} of {len(w.decode_seqs)} sequences "
              f"({toks} context tokens, all {w.num_q_heads} query heads) x {reps}, {dt:.1f} s")
    step_s = per_tok * all_toks
    if w.prefill_seqs:
        stp = st
        qs = np.concatenate([[0], np.cumsum(w.chunk_len)])
        n = min(prefill_chunks, len(w.chunk_len))
        tables, clens = stp.alloc.block_tables(w.prefill_seqs, oracle_run.max_blocks(w))
        rows = [(t, h) for t in range(int(qs[0]), int(qs[n])) for h in range(w.num_q_heads)]
        t0 = time.perf_counter()
        pout = oracle_run.oracle_prefill(w, stp, rows=rows)
        tp = time.perf_counter() - t0
        assert np.isfinite(pout[int(qs[0]):int(qs[n])]).all()
        qk_pairs = lambda cs: sum(C * (int(clens[c]) - C + 1) + C * (C - 1) // 2    # noqa: E731
                                  for c, C in cs)
        done = qk_pairs((c, w.chunk_len[c]) for c in range(n))
        total = qk_pairs(enumerate(w.chunk_len))
        step_s += tp / done * total
        sample += (f"; prefill of every (query, head) row of {n} of {len(w.chunk_len)} chunks "
                   f"({done} of {total} query-key pairs), {tp:.1f} s, scaled to all chunks")
    sample += f"; one Python thread driving BLAS with {blas} threads on {cores} host cpus"
    return {"value": all_toks / step_s, "unit": "seq-tokens/s", "cores": cores, "blas_threads": int(blas),
            "kind": "oracle", "sample": sample}


def prefill_flops(w, clens):
    """4 * D * Hq flops per (query, visible key) pair of the causal chunks."""
    tot = 0
    for C, L in zip(w.chunk_len, clens):
        # query i sits at position L - C + i and sees L - C + i + 1 keys
        tot += C * (L - C + 1) + C * (C - 1) // 2
    return 4 * w.head_dim * w.num_q_heads * tot


DEFAULT_PARTITION = {"c5": 0}          # every other workload: 512 tokens


def attention_loop_ceiling(prefill_tflops, iters=1000, reps=3):
    """TFLOP/s of pa_attention_loop_peak in its three modes (HIP events on the
    current stream); the prefill's rate as a fraction of the full loop's."""
    import torch
    import paged_kv_cache_424_amd as pa
    src = torch.zeros(4 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rates = {}
    for mode in (0, 1, 2):
        pa.pa_attention_loop_peak(src, sink, 20, mode)               # warm-up
        best = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            flops = pa.pa_attention_loop_peak(src, sink, iters, mode)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        rates[mode] = best
    return {"tflops": rates[2], "frac_of_peak": rates[2] / PEAK_BF16_TFLOPS,
            "prefill_over_ceiling": prefill_tflops / rates[2],
            "mfma_and_lds_reads_only_tflops": rates[0], "with_softmax_arithmetic_tflops": rates[1],
            "kernel": "attention_loop_kernel: per 64-key tile and wave 32 MFMA 32x32x16 bf16 with LDS fragment "
                      "reads, 32 exp2, 16 bf16 pair conversions and row-sum steps (each exponential consumed "
                      "four steps later, four row-sum accumulators), 32 KB tile loads per workgroup into "
                      "double-buffered LDS (one load per four MFMAs), 2 workgroups per CU"}


def measure(args, workload):
    """Time one workload's step; returns the bench line's fields (no CPU baseline)."""
    if args.partition is None:
        args = argparse.Namespace(**vars(args))
        args.partition = DEFAULT_PARTITION.get(workload, 512)
    import numpy as np
    import torch
    import paged_kv_cache_424_amd as pa
    import workloads
    from tests import lib_run

    torch.cuda.set_device(0)
    print(f"[bench] workload {workload}: generating inputs", file=sys.stderr, flush=True)
    w = workloads.make(workload)
    st = lib_run.build(w, device="cuda", run_step=True)
    B, Hq, D, H = len(w.decode_seqs), w.num_q_heads, w.head_dim, w.num_kv_heads
    lens = st.lens_host.astype(np.int64)
    tokens = int(lens.sum())
    esz = 2 if w.dtype == "bf16" else 4

    # the step's inputs: the tokens the step appends (the new token of every
    # sequence; shared-prefix: also each private suffix; mixed: also the chunks)
    rows = np.asarray(st.step_rows)
    step_slots = np.asarray(st.step_slots, dtype=np.int64)
    newest = None
    only_newest = len(step_slots) == len(w.decode_seqs) and all(len(sl) == 1 for sl, _ in st.step_writes)
    if args.append == "on" or (args.append == "auto" and only_newest):
        # each decode sequence's newest token (position L - 1) goes in through
        # the decode kernel; the step's other tokens (private suffixes, prefill
        # chunks) through the cache write
        new_slot, new_row = [], []
        for i, s_ in enumerate(w.decode_seqs):
            p = int(st.lens_host[i]) - 1
            new_slot.append(int(st.tables_host[i][p // w.block_size]) * w.block_size + p % w.block_size)
            new_row.append(int(w.tok_rows[s_][p]))
        newest = {"k": lib_run.torch_stored(w.k_tok[new_row], w.dtype).cuda(),
                  "v": lib_run.torch_stored(w.v_tok[new_row], w.dtype).cuda(),
                  "slots": torch.tensor(new_slot, dtype=torch.int64, device="cuda")}
        keep = ~np.isin(step_slots, np.asarray(new_slot, dtype=np.int64))
        rows, step_slots = rows[keep], step_slots[keep]
    k_new = lib_run.torch_stored(w.k_tok[rows], w.dtype).cuda()
    v_new = lib_run.torch_stored(w.v_tok[rows], w.dtype).cuda()
    slots = torch.from_numpy(np.ascontiguousarray(step_slots)).cuda()
    pairs = st.step_pairs

    pre = None
    if w.prefill_seqs:
        ptab, plens = pa.pa_build_block_tables(st.alloc, w.prefill_seqs, st.max_blocks)
        pre = {
            "tables": torch.from_numpy(np.ascontiguousarray(ptab)).cuda(),
            "lens": torch.from_numpy(np.ascontiguousarray(plens)).cuda(),
            "qsl": torch.from_numpy(np.concatenate([[0], np.cumsum(w.chunk_len)]).astype(np.int32)).cuda(),
            "q": lib_run.torch_stored(w.q_pre, w.dtype).cuda(),
            "max_q": max(w.chunk_len),
            "flops": prefill_flops(w, [int(x) for x in plens]),
        }
        pre["out"] = torch.empty(pre["q"].shape, dtype=torch.float32, device="cuda")

    pool_bytes = 2 * pa.pa_cache_pool_bytes(st.desc)
    step_bytes = tokens * 2 * H * D * esz
    copies = max(2, -(-(1 << 30) // max(step_bytes, 1)) + 1)
    pools = [(st.kc, st.vc)] + [(st.kc.clone(), st.vc.clone()) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    print(f"[bench] {B} sequences, {tokens} context tokens, pool {pool_bytes / 1e9:.2f} GB x {copies} copies",
          file=sys.stderr, flush=True)

    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    max_ctx = int(lens.max())
    wsb = pa.pa_decode_workspace_bytes(B, Hq, D, max_ctx, args.partition)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda") if wsb else None

    if args.copy_calibration:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # The mixed step's prefill chunks read the pools the cache write has just
    # filled and nothing the decode writes, so they can run on a second stream
    # (default priority) beside the decode: the decode streams HBM while the
    # prefill keeps the matrix cores busy.  The main stream waits for the
    # second at the end of the step.
    overlap = pre is not None and args.overlap == "on"
    side = torch.cuda.Stream() if overlap else None

    # Events: in the timed steps only around the partition kernel (7, 3) and
    # the prefill kernel (5, 6), so that event records add no gaps elsewhere;
    # a separate pass after the timed region records all of them: 0 start,
    # 1 after copy_blocks, 2 after cache_write, 7 before and 3 after the
    # partition kernel, 4 after the reduce, 5 before and 6 after prefill (on
    # the prefill's stream).
    timed_marks = (7, 3, 5, 6) if pre is not None else (7, 3)

    def step(i, ev=None, marks=timed_marks, dispatch_ev=None, use_side=None):
        use_side = overlap if use_side is None else use_side
        def mark(k):
            if ev is not None and k in marks:
                ev[k].record()
        kc, vc = pools[i % copies]
        mark(0)
        if pairs:
            pa.pa_copy_blocks(kc, vc, st.desc, pairs)
        mark(1)
        if slots.numel():
            pa.pa_cache_write(kc, vc, st.desc, k_new, v_new, slots)
        mark(2)

        def prefill():
            mark(5)
            pa.pa_prefill(pre["out"], pre["q"], kc, vc, st.desc, pre["tables"], pre["lens"], pre["qsl"],
                          pre["max_q"], w.scale)
            mark(6)
        joined = None
        main = torch.cuda.current_stream()
        if pre is not None and use_side:
            side.wait_stream(main)                              # after the cache write
            with torch.cuda.stream(side):
                prefill()
                joined = torch.cuda.Event()
                joined.record()
        # On one stream the prefill runs before the decode: both need only the
        # cache write, and the decode then streams HBM after the compute-bound
        # prefill rather than straight after the cache write (measured on the
        # mixed step: decode 288 vs 291-299 us, step 581 vs 585-594 us).
        if pre is not None and not use_side:
            prefill()
        decode(kc, vc, mark, dispatch_ev)
        if joined is not None:
            main.wait_event(joined)

    def decode(kc, vc, mark, dispatch_ev):
        mark(7)
        if dispatch_ev is not None:
            pa.pa_time_next_partitions(*dispatch_ev)
        if newest is not None:
            pa.pa_decode_append_partitions(out, st.q, newest["k"], newest["v"], newest["slots"], kc, vc,
                                           st.desc, st.tables, st.lens, max_ctx, w.scale, args.partition, ws)
        else:
            pa.pa_decode_partitions(out, st.q, kc, vc, st.desc, st.tables, st.lens, max_ctx, w.scale,
                                    args.partition, ws)
        mark(3)
        pa.pa_decode_reduce(out, st.lens, Hq, D, max_ctx, args.partition, ws)
        mark(4)

    # Warm-up: W steps, and more until --warmup-ms of wall time has passed.
    # The GPU lowers its clocks while the host builds the workload; measured,
    # the first 20-40 steps after a 2 s idle ran 10-20 % slow (prefill 307 ->
    # 258 us, decode 316 -> 280 us) and later steps held steady.  Every
    # warm-up and timed step is the whole step.
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or (time.perf_counter() - t_w) * 1e3 < args.warmup_ms:
        step(n_warm)
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()          # keep the host clock in step with the GPU
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t_w) * 1e3
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(8)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(n_warm + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part_ms = [e[7].elapsed_time(e[3]) for e in evs]
    part_avg_s = float(np.mean(part_ms)) / 1e3

    # the partition kernel's dispatch events (recorded once here so that their
    # HIP events exist, then re-recorded by the kernel launch of each step)
    evd = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]
    for pair in evd:
        for e in pair:
            e.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(n_warm + i, dispatch_ev=evd[i])
    torch.cuda.synchronize()
    dispatch_ms = [e[0].elapsed_time(e[1]) for e in evd]
    assert torch.isfinite(out).all()

    ms_per_step = wall * 1e3 / args.steps

    # the same steps with the prefill on the decode's stream, for comparison
    serial_ms = None
    if overlap:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            step(n_warm + i, use_side=False)
        torch.cuda.synchronize()
        serial_ms = (time.perf_counter() - t1) * 1e3 / args.steps

    # per-kernel times, all events recorded (not part of the timed region)
    evk = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(8)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(n_warm + i, evk[i], marks=(0, 1, 2, 3, 4, 5, 6, 7), use_side=False)
    torch.cuda.synchronize()

    def avg_us(a, b):
        return float(np.mean([e[a].elapsed_time(e[b]) for e in evk])) * 1e3

    # The same step captured once per pool copy as a HIP graph and replayed:
    # the launch gaps between the step's kernels shrink.  Reported beside the
    # eager figures (the timed region above), which carry the kernel's event
    # timing -- events cannot be recorded inside a captured graph here.
    graph_ms = None
    if not args.no_graph:
        graphs = []
        for i in range(copies):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(i)
            graphs.append(gr)
        for i in range(copies):
            graphs[i].replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for i in range(args.steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - tg) * 1e3 / args.steps
        assert torch.isfinite(out).all()
    # algorithmic bytes of one decode: every context token's K and V of every kv
    # head once, the queries, the fp32 outputs, the block ids and lengths
    nblocks = int(np.sum(-(-lens // w.block_size)))
    algo = tokens * 2 * H * D * esz + B * Hq * D * (esz + 4) + 4 * nblocks + 4 * B
    achieved = algo / part_avg_s / 1e9
    res = {
        "metric": METRIC,
        "value": tokens / (ms_per_step / 1e3),
        "unit": "seq-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "warmup_ms": warm_ms,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), bf16 by round-to-nearest-even)",
        "config": {"workload": WORKLOAD_TEXT[workload], "sequences": B,
                   "context_tokens": tokens, "q_heads": Hq, "kv_heads": H, "head_dim": D,
                   "block_size": w.block_size, "partition": args.partition, "pool_copies": copies,
                   "step": ("copy_blocks + " if pairs else "") +
                           ("cache_write + " if slots.numel() else "") +
                           ("prefill + " if pre is not None and not overlap else "") +
                           ("decode_append_partitions" if newest is not None else "decode_partitions") +
                           " + decode_reduce" + (" || prefill (second stream)" if overlap else "")},
        "roofline": {"bound": "hbm", "kernel": "decode_partition_kernel", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": load_traffic(workload), "algorithmic_bytes_per_launch": algo,
                     "avg_launch_us": part_avg_s * 1e6, "median_us": float(np.median(part_ms)) * 1e3,
                     "p10_us": float(np.percentile(part_ms, 10)) * 1e3,
                     "p90_us": float(np.percentile(part_ms, 90)) * 1e3,
                     "timing": "HIP events recorded around the launch call in the timed steps" +
                               (", while the prefill runs on a second stream" if overlap else ""),
                     "avg_launch_us_dispatch_events": float(np.mean(dispatch_ms)) * 1e3,
                     "kernel_source_hash": kernel_source_hash("decode")},
        "decode_gbs_whole_step": algo / (ms_per_step / 1e3) / 1e9,
        "hip_graph_ms_per_step": graph_ms,
        "prefill_on_second_stream": overlap,
        "ms_per_step_one_stream": serial_ms,
        "kernels_us_untimed_pass": {"copy_blocks": avg_us(0, 1) if pairs else None,
                                    "cache_write": avg_us(1, 2) if slots.numel() else None,
                       "decode_partitions": avg_us(7, 3), "decode_reduce": avg_us(3, 4),
                       "prefill": avg_us(5, 6) if pre is not None else None},
    }
    # the practical read rate for the same byte count: a plain streaming read
    # of one contiguous buffer (pa_stream_read), best of a few launch shapes,
    # measured after everything above
    import bench_studies
    sbytes, _, srates = bench_studies.stream_read_rates(algo, 10, shapes=STREAM_SHAPES_BENCH)
    sbest = max(srates, key=lambda k: srates[k]["gbs"])
    res["roofline"]["stream_read_same_bytes"] = {
        "gbs": srates[sbest]["gbs"], "frac_of_peak": srates[sbest]["gbs"] / PEAK_HBM_GBS,
        "bytes": sbytes, "launch_shape": sbest,
        "decode_over_stream": achieved / srates[sbest]["gbs"],
        "kernel": "stream_read_kernel: one contiguous buffer, 16-byte non-temporal loads"}
    if pre is not None:
        pre_ms = [e[5].elapsed_time(e[6]) for e in evs]
        pre_s = float(np.mean(pre_ms)) / 1e3
        tf = pre["flops"] / pre_s / 1e12
        assert torch.isfinite(pre["out"]).all()
        res["prefill"] = {"bound": "mfma", "kernel": "prefill_kernel", "achieved": tf,
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                          "flops_per_launch": pre["flops"], "avg_launch_us": pre_s * 1e6,
                          "median_us": float(np.median(pre_ms)) * 1e3,
                          "p10_us": float(np.percentile(pre_ms, 10)) * 1e3,
                          "p90_us": float(np.percentile(pre_ms, 90)) * 1e3,
                          "timing": "HIP events recorded around the launch call" +
                                    (" on the second stream, while the decode runs" if overlap else ""),
                          "query_tokens": int(sum(w.chunk_len)),
                          "traffic": load_traffic(workload, "prefill"),
                          "kernel_source_hash": kernel_source_hash("prefill")}
        # the practical ceiling of the prefill's inner loop on this chip
        # (pa_attention_loop_peak: the same MFMA, LDS, softmax and tile-load
        # mix per tile, with no paging), best of three launches per mode
        res["prefill"]["loop_ceiling"] = attention_loop_ceiling(tf)
    return res, w


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-ms", type=float, default=150.0,
                    help="after the W warm-up steps, keep running untimed whole steps until this much "
                         "wall time has passed (the GPU lowers its clocks while idle; the first tens of "
                         "steps after the host-side setup run 10-20 %% slow)")
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-extra", action="store_true",
                    help="with the mixed step (c5), skip the long-context decode (c3) that the "
                         "default run times after it")
    ap.add_argument("--partition", type=int, default=None,
                    help="split-K partition in tokens (a multiple of 32), or 0 for the balanced split; "
                         "default: the long-context decode's stated 512-token partitions for c3, the "
                         "balanced split for the mixed step (c5 states no partition size; measured "
                         "faster there), 512 otherwise (measured faster on c2)")
    ap.add_argument("--append", choices=["auto", "on", "off"], default="auto",
                    help="store each decode sequence's newest token inside the decode kernel "
                         "(pa_decode_append) instead of a separate cache write; auto: when the "
                         "step writes no other token (a cache-write launch happens anyway otherwise)")
    ap.add_argument("--overlap", choices=["on", "off"], default="off",
                    help="run the prefill chunks on a second stream, concurrently with the decode "
                         "(both wait for the step's cache write); the per-kernel figures are then "
                         "taken while the two kernels share the chip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra HIP-graph replay measurement of the whole step")
    ap.add_argument("--cpu-seqs", type=int, default=0, help="sequences in the oracle sample (0 = auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB elementwise kernel (scales the HBM byte counters)")
    ap.add_argument("--pmc-summary", action="store_true",
                    help="summarise two rocprofv3 --pmc runs (no GPU work) into profiles/")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--command", help="the profiled command, recorded in the summary")
    ap.add_argument("--kernel", choices=sorted(KERNELS), default="decode",
                    help="with --pmc-summary: the kernel whose counters are summarised")
    ap.add_argument("--study", choices=["prefix-cache", "fragmentation", "block-size", "batch1", "stream-peak"],
                    help="run one of the studies in bench_studies.py instead of the benchmark")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.study:
        import bench_studies
        bench_studies.STUDIES[args.study](args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    res, w = measure(args, args.workload)
    if args.workload == "c5" and not args.no_extra:
        # the long-context decode (8 x 32k tokens), timed the same way after the
        # mixed step: its decode kernel and roofline ride along in this line
        import torch
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        extra_args = argparse.Namespace(**vars(args))
        extra_args.overlap = "off"
        c3, _ = measure(extra_args, "c3")
        res["c3_decode"] = {k: c3[k] for k in ("value", "unit", "ms_per_step", "config", "roofline",
                                                 "decode_gbs_whole_step", "hip_graph_ms_per_step",
                                                 "kernels_us_untimed_pass")}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seqs or len(w.decode_seqs))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
