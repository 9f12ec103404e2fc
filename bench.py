#!/usr/bin/env python3
"""Paged decode attention throughput on one MI355X.

A step is one pass of the decode hot path over one batch: the cache write of
every sequence's new token, then the split-K partition kernel, then the
rescaling reduce (plus the copy-on-write copies for the shared-prefix
workload).  Inputs are resident in HBM before timing starts.  Prints one
JSON line.

    python bench.py [--steps K] [--warmup W] [--workload c3|c2|c4]

Default workload: long-context decode, 8 sequences x 32768 tokens, 32 query /
8 kv heads, head_dim 128, bf16 cache in 16-token blocks, 512-token
partitions, keys scaled x3.  Consecutive steps read different copies of the
pools (at least 1 GiB apart) so that no step is served from the 256 MB
Infinity Cache left warm by the previous one.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak, GB/s
METRIC = "paged decode attention: seq-tokens/s and achieved HBM GB/s (% of peak)"

WORKLOAD_TEXT = {
    "c2": "Llama-3-8B-shaped decode: 64 sequences, context U{128..2048}, 32/8 heads, head_dim 128, "
          "bf16 cache, 16-token blocks, pool = need + 10%, one cache write per sequence",
    "c3": "long-context split-K decode: 8 sequences x 32768 tokens, 32/8 heads, head_dim 128, "
          "bf16 cache, 16-token blocks, 512-token partitions, keys x3",
    "c4": "shared-prefix decode with copy-on-write: 32 sequences share a 1016-token prefix "
          "(64 blocks), private suffix U{0..512} + 1 token, 32/8 heads, head_dim 128, bf16",
}


def kernel_source_hash():
    h = hashlib.sha256()
    for name in ("decode.hip", "pa_internal.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_424_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload, algo_bytes):
    """HBM bytes per partition-kernel launch from the committed counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_partition_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, nseq, min_seconds=10.0, max_reps=5):
    """The CPU oracle (fp64, as it stands) decoding the first nseq sequences of
    the workload, repeated until about min_seconds of CPU work."""
    import numpy as np
    import workloads
    from tests import oracle_run
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:                                  # pragma: no cover
        blas = 1
    sub = workloads.subset(w, w.decode_seqs[:nseq])
    st = oracle_run.build(sub)
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        out = oracle_run.oracle_decode(sub, st)
        dt += time.perf_counter() - t0
        reps += 1
    assert np.isfinite(out).all()
    toks = sum(sub.seq_len(s) for s in sub.decode_seqs)
    return {"value": reps * toks / dt, "unit": "seq-tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": f"fp64 numpy oracle decode of {nseq} of {len(w.decode_seqs)} sequences "
                      f"({toks} context tokens, all {w.num_q_heads} query heads) x {reps}, {dt:.1f} s; "
                      f"one Python thread driving BLAS with {blas} threads, host cpus "
                      f"{len(os.sched_getaffinity(0))}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--partition", type=int, default=512, help="split-K partition (128..512)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=0, help="sequences in the oracle sample (0 = auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device copy (scales the HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import paged_kv_cache_424_amd as pa
    import workloads
    from tests import lib_run

    torch.cuda.set_device(0)
    print(f"[bench] workload {args.workload}: generating inputs", file=sys.stderr, flush=True)
    w = workloads.make(args.workload)
    st = lib_run.build(w, device="cuda", run_step=True)
    B, Hq, D, H = len(w.decode_seqs), w.num_q_heads, w.head_dim, w.num_kv_heads
    lens = st.lens_host.astype(np.int64)
    tokens = int(lens.sum())
    esz = 2 if w.dtype == "bf16" else 4

    # the step's inputs: the tokens the step appends (the new token of every
    # sequence; for the shared-prefix workload also each private suffix)
    rows = np.asarray(st.step_rows)
    k_new = lib_run.torch_stored(w.k_tok[rows], w.dtype).cuda()
    v_new = lib_run.torch_stored(w.v_tok[rows], w.dtype).cuda()
    slots = torch.from_numpy(np.ascontiguousarray(st.step_slots)).cuda()
    pairs = st.step_pairs

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
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(i, ev=None):
        kc, vc = pools[i % copies]
        if pairs:
            pa.pa_copy_blocks(kc, vc, st.desc, pairs)
        pa.pa_cache_write(kc, vc, st.desc, k_new, v_new, slots)
        if ev is not None:
            ev[0].record()
        pa.pa_decode_partitions(out, st.q, kc, vc, st.desc, st.tables, st.lens, max_ctx, w.scale,
                                args.partition, ws)
        if ev is not None:
            ev[1].record()
        pa.pa_decode_reduce(out, st.lens, Hq, D, max_ctx, args.partition, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part_ms = [a.elapsed_time(b) for a, b in evs]
    part_avg_s = float(np.mean(part_ms)) / 1e3
    assert torch.isfinite(out).all()

    ms_per_step = wall * 1e3 / args.steps
    # algorithmic bytes of one decode: every context token's K and V of every kv
    # head once, the queries, the fp32 outputs, the block ids and lengths
    nblocks = int(np.sum(-(-lens // w.block_size)))
    algo = tokens * 2 * H * D * esz + B * Hq * D * (esz + 4) + 4 * nblocks + 4 * B
    achieved = algo / part_avg_s / 1e9
    traffic = load_traffic(args.workload, algo)
    res = {
        "metric": METRIC,
        "value": tokens / (ms_per_step / 1e3),
        "unit": "seq-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), bf16 by round-to-nearest-even)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "sequences": B,
                   "context_tokens": tokens, "q_heads": Hq, "kv_heads": H, "head_dim": D,
                   "block_size": w.block_size, "partition": args.partition, "pool_copies": copies,
                   "step": ("copy_blocks + " if pairs else "") + "cache_write + decode_partitions + decode_reduce"},
        "roofline": {"bound": "hbm", "kernel": "decode_partition_kernel", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": algo,
                     "avg_launch_us": part_avg_s * 1e6,
                     "kernel_source_hash": kernel_source_hash()},
        "decode_gbs_whole_step": algo / (ms_per_step / 1e3) / 1e9,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        nseq = args.cpu_seqs or len(w.decode_seqs)
        res["cpu_baseline"] = cpu_baseline(w, nseq)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
