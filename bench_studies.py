"""Studies beside the benchmark: the pages' tuning knobs and claims, measured
on the library (C ABI through the binding).  Run through bench.py:

    python bench.py --study prefix-cache    # host only
    python bench.py --study fragmentation   # host only
    python bench.py --study block-size      # GPU
    python bench.py --study batch1          # GPU
    python bench.py --study stream-peak     # GPU

Each prints one JSON line per configuration it measures.

prefix-cache: the shared-prompt workload (32 requests over 4 prompts of
    256..1024 tokens, 8 earlier requests freed first) appended through the
    content-addressed call, with and without prefix caching: tokens found
    cached, blocks and slots held, evictions, K/V bytes the cache write skips,
    and host time per call.  [studynote 528] section II (a shared system
    prompt is stored once); [ch.09] closing section.
fragmentation: a saturated request queue served with continuous batching
    under a fixed KV budget, three ways: contiguous regions reserved at the
    maximum length, contiguous regions of each request's exact final length
    (an idealised scheduler that knows it), and the library's paged
    allocator.  Reports, while requests are still waiting, how many run at
    once, how much of the budget holds tokens and the waste inside
    reservations; and the steps needed to serve the whole queue.  [ch.09] "문제: 연속 할당의 단편화" (internal and external
    fragmentation) and "해법: 페이지처럼 나눠 담기"; [velog] "메모리 낭비
    (Internal Fragmentation)"; [studynote 223] section I.  The pages' own
    figures (60-80 % waste, under 4 %) come from traces that are not here:
    the synthetic length mix below is stated, not theirs.
block-size: the Llama-3-8B-shaped decode batch stored with 8, 16, 32, 64 and
    128-token blocks (512-token partitions): partition-kernel time and GB/s
    against the slots left empty in last blocks and the size of the block
    tables.  [studynote 223]
    section IV, checklist item 1; [ch.09] "⚖️ 절충" (small blocks: less
    fragmentation, more table overhead; large blocks the reverse).
stream-peak: a plain streaming read (pa_stream_read: one contiguous buffer,
    16-byte non-temporal loads, grid-stride) of the decode workloads' byte
    counts and of 4 GiB, over a few launch shapes: the practical HBM read rate
    beside the 8 TB/s spec.
batch1: one sequence of 512..32768 tokens, its blocks scattered over the pool
    or laid out in order (identity table), beside 64 sequences of the same
    length: what the indirection and a single sequence cost.  [studynote 223]
    section IV, "안티패턴" (slower than plain code at batch size 1); [velog]
    closing section (table lookup overhead is small).
"""

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

ROTATE_BYTES = 1 << 30      # consecutive launches read pool copies this far apart in total


def _emit(d):
    print(json.dumps(d), flush=True)


# ---- prefix caching ----------------------------------------------------------------------------
def study_prefix_cache(args):
    import paged_kv_cache_424_amd as pa
    import workloads
    w = workloads.make("c4p")
    kv_bytes_tok = 2 * w.num_kv_heads * w.head_dim * 2          # K and V, bf16, one layer
    appended = sum(len(op[2]) for _, op in w.script if op[0] == "append_tokens")
    # token ids as int32 arrays up front, so the timed calls measure the library
    script = [(op[0], op[1], np.asarray(op[2], dtype=np.int32)) if op[0] == "append_tokens" else op
              for _, op in w.script]
    # the ctypes round trip alone, for scale
    h0 = pa.pa_allocator_create(4, 4)
    t0 = time.perf_counter()
    for _ in range(20000):
        pa.pa_num_free(h0)
    call_us = (time.perf_counter() - t0) / 20000 * 1e6
    pa.pa_allocator_destroy(h0)
    for caching in (True, False):
        n_blocks = w.num_blocks if caching else 4 * w.num_blocks
        h = pa.pa_allocator_create(n_blocks, w.block_size, None)
        if caching:
            pa.pa_allocator_enable_prefix_cache(h)
        per_call, sizes = [], []
        try:
            for op in script:
                if op[0] == "create":
                    pa.pa_seq_create(h)
                elif op[0] == "free":
                    pa.pa_seq_free(h, op[1])
                else:
                    t0 = time.perf_counter()
                    pa.pa_seq_append_tokens(h, op[1], op[2])
                    dt = time.perf_counter() - t0
                    per_call.append(dt * 1e6)
                    sizes.append(len(op[2]))
            st = pa.pa_allocator_get_stats(h)
        finally:
            pa.pa_allocator_destroy(h)
        per_call, sizes = np.asarray(per_call), np.asarray(sizes)
        long_calls = sizes > 100
        _emit({
            "study": "prefix_cache", "prefix_caching": caching,
            "workload": w.note, "block_size": w.block_size, "pool_blocks": n_blocks,
            "appended_tokens": appended, "hit_tokens": st["hit_tokens"],
            "hit_rate": st["hit_tokens"] / appended,
            "batch_logical_tokens": st["logical_tokens"], "stored_tokens": st["stored_tokens"],
            "used_blocks": st["used_blocks"], "shared_blocks": st["shared_blocks"],
            "cached_blocks": st["cached_blocks"], "evictions": st["evictions"],
            "kv_bytes_not_written_per_layer": st["hit_tokens"] * kv_bytes_tok,
            "host_us_per_append_call": {"mean": float(np.mean(per_call)),
                                        "p50": float(np.percentile(per_call, 50)),
                                        "p99": float(np.percentile(per_call, 99))},
            "host_ns_per_token_in_calls_over_100_tokens": float(
                per_call[long_calls].sum() * 1e3 / sizes[long_calls].sum()),
            "ctypes_call_us": call_us,
        })


# ---- fragmentation / capacity ----------------------------------------------------------------
class _Arena:
    """A linear region of `size` slots handing out contiguous ranges, first fit."""

    def __init__(self, size):
        self.size = size
        self.free = [(0, size)]          # sorted (start, length)

    def alloc(self, n):
        for i, (s, ln) in enumerate(self.free):
            if ln >= n:
                if ln == n:
                    self.free.pop(i)
                else:
                    self.free[i] = (s + n, ln - n)
                return s
        return None

    def release(self, start, n):
        self.free.append((start, n))
        self.free.sort()
        merged = []
        for s, ln in self.free:
            if merged and merged[-1][0] + merged[-1][1] == s:
                merged[-1] = (merged[-1][0], merged[-1][1] + ln)
            else:
                merged.append((s, ln))
        self.free = merged

    def largest_gap(self):
        return max((ln for _, ln in self.free), default=0)


def _requests(seed, n, max_len):
    """Prompt and output lengths: lognormal (medians 512 and 192 tokens, sigma
    0.8 and 1.0 in natural-log units), clipped so prompt + output <= max_len."""
    rng = np.random.default_rng(seed)
    p = np.clip(np.rint(np.exp(np.log(512) + 0.8 * rng.standard_normal(n))), 16, max_len // 2)
    o = np.clip(np.rint(np.exp(np.log(192) + 1.0 * rng.standard_normal(n))), 1, None)
    o = np.minimum(o, max_len - p)
    return [int(x) for x in p], [int(x) for x in o]


def _simulate_contiguous(prompts, outputs, budget, reserve):
    """reserve(i) slots per request, first fit; every running request adds one
    token per step.  Returns per-step samples and the step count."""
    arena = _Arena(budget)
    queue = list(range(len(prompts)))
    running = {}                         # i -> (start, reserved, held)
    steps = 0
    conc, held_frac, waste_frac, blocked_free = [], [], [], []
    while queue or running:
        while queue:
            i = queue[0]
            r = reserve(i)
            s = arena.alloc(r)
            if s is None:
                free_total = sum(ln for _, ln in arena.free)
                if free_total >= r:
                    blocked_free.append(free_total / budget)   # fits in total, not in one piece
                break
            queue.pop(0)
            running[i] = [s, r, prompts[i]]
        steps += 1
        done = []
        for i, st in running.items():
            st[2] += 1
            if st[2] >= prompts[i] + outputs[i]:
                done.append(i)
        held = sum(st[2] for st in running.values())
        reserved = sum(st[1] for st in running.values())
        if queue:                         # saturated: requests are still waiting
            conc.append(len(running))
            held_frac.append(held / budget)
            waste_frac.append(1.0 - held / reserved if reserved else 0.0)
        for i in done:
            s, r, _ = running.pop(i)
            arena.release(s, r)
    return steps, conc, held_frac, waste_frac, blocked_free


def _simulate_paged(prompts, outputs, budget, bs):
    """The library's allocator: admit while the free blocks cover the prompt
    plus one block per running sequence (room to grow); a sequence that cannot
    get its next block preempts the most recently admitted one, which returns
    to the head of the queue and starts over."""
    import paged_kv_cache_424_amd as pa
    nblocks = budget // bs
    h = pa.pa_allocator_create(nblocks, bs, None)
    queue = list(range(len(prompts)))
    running = {}                         # i -> [seq id, generated]
    order = []                           # admission order of running requests
    steps = preempted = 0
    conc, held_frac, waste_frac = [], [], []
    try:
        while queue or running:
            while queue:
                i = queue[0]
                need = -(-(prompts[i] + 1) // bs) + len(running)
                if pa.pa_num_free(h) < need:
                    break
                queue.pop(0)
                s = pa.pa_seq_create(h)
                pa.pa_seq_append_slots(h, s, prompts[i])
                running[i] = [s, 0]
                order.append(i)
            if not running:
                raise RuntimeError("a request does not fit the budget on its own")
            steps += 1
            done = []
            for i in list(order):
                if i not in running:
                    continue
                s = running[i][0]
                while True:
                    try:
                        pa.pa_seq_append_slots(h, s, 1)
                        break
                    except pa.PAError as e:
                        if e.status != pa.PA_ERR_OUT_OF_BLOCKS:
                            raise
                        victim = order[-1]
                        pa.pa_seq_free(h, running[victim][0])
                        del running[victim]
                        order.pop()
                        queue.insert(0, victim)
                        preempted += 1
                        if victim == i:
                            break
                if i not in running:
                    continue
                running[i][1] += 1
                if running[i][1] >= outputs[i]:
                    done.append(i)
            if queue:                     # saturated: requests are still waiting
                st = pa.pa_allocator_get_stats(h)
                conc.append(len(running))
                held_frac.append(st["stored_tokens"] / budget)
                alloc = st["used_blocks"] * bs
                waste_frac.append(1.0 - st["stored_tokens"] / alloc if alloc else 0.0)
            for i in done:
                pa.pa_seq_free(h, running[i][0])
                del running[i]
                order.remove(i)
    finally:
        pa.pa_allocator_destroy(h)
    return steps, conc, held_frac, waste_frac, preempted


def study_fragmentation(args):
    max_len = 4096
    budget = 64 * max_len                 # 64 maximum-length reservations
    n = 1500
    prompts, outputs = _requests(17, n, max_len)
    total_tokens = sum(outputs)
    common = {"study": "fragmentation", "requests": n, "max_len": max_len, "budget_tokens": budget,
              "lengths": "prompt ~ lognormal(median 512, sigma 0.8) in [16, 2048], output ~ "
                         "lognormal(median 192, sigma 1.0) >= 1, prompt + output <= 4096; all queued at once",
              "mean_prompt": float(np.mean(prompts)), "mean_output": float(np.mean(outputs))}

    def summary(steps, conc, held, waste):
        # averages over the steps where requests were still waiting, after the
        # first tenth of them (the batch filling up); the drain is not sampled
        sl = slice(len(conc) // 10, None)
        return {"steps": steps, "tokens_per_step": total_tokens / steps,
                "mean_running": float(np.mean(conc[sl])), "max_running": int(max(conc)),
                "budget_holding_tokens": float(np.mean(held[sl])),
                "waste_inside_allocations": float(np.mean(waste[sl]))}

    t0 = time.perf_counter()
    r = _simulate_contiguous(prompts, outputs, budget, lambda i: max_len)
    _emit({**common, "policy": "contiguous, maximum length reserved", **summary(*r[:4]),
           "seconds": time.perf_counter() - t0})
    t0 = time.perf_counter()
    r = _simulate_contiguous(prompts, outputs, budget, lambda i: prompts[i] + outputs[i])
    _emit({**common, "policy": "contiguous, exact final length reserved (idealised)", **summary(*r[:4]),
           "admissions_blocked_by_external_fragmentation": len(r[4]),
           "free_share_when_blocked": float(np.mean(r[4])) if r[4] else None,
           "seconds": time.perf_counter() - t0})
    for bs in (16, 128):
        t0 = time.perf_counter()
        r = _simulate_paged(prompts, outputs, budget, bs)
        _emit({**common, "policy": f"paged, {bs}-token blocks (library allocator)", **summary(*r[:4]),
               "preemptions": r[4], "seconds": time.perf_counter() - t0})


# ---- GPU studies ------------------------------------------------------------------------------
def _time_decode(w, st, partition, reps, copies=None):
    """Average microseconds of the partition kernel and of the reduce, with
    consecutive launches reading different pool copies."""
    import torch
    import paged_kv_cache_424_amd as pa
    B, Hq, D = st.q.shape
    lens = st.lens_host.astype(np.int64)
    max_ctx = int(lens.max())
    pool = 2 * pa.pa_cache_pool_bytes(st.desc)
    if copies is None:
        copies = max(2, min(600, -(-ROTATE_BYTES // pool) + 1))
    pools = [(st.kc, st.vc)] + [(st.kc.clone(), st.vc.clone()) for _ in range(copies - 1)]
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    wsb = pa.pa_decode_workspace_bytes(B, Hq, D, max_ctx, partition)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def launch(i, ev=None):
        kc, vc = pools[i % copies]
        if ev:
            ev[0].record()
        pa.pa_decode_partitions(out, st.q, kc, vc, st.desc, st.tables, st.lens, max_ctx, w.scale,
                                partition, ws)
        if ev:
            ev[1].record()
        pa.pa_decode_reduce(out, st.lens, Hq, D, max_ctx, partition, ws)
        if ev:
            ev[2].record()

    for i in range(5):
        launch(i)
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(reps)]
    for i in range(reps):
        launch(5 + i, evs[i])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    part = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
    red = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3
    del pools
    torch.cuda.empty_cache()
    return part, red, copies


def _algo_bytes(w, lens):
    esz = 2 if w.dtype == "bf16" else 4
    B, H, Hq, D = len(lens), w.num_kv_heads, w.num_q_heads, w.head_dim
    nblocks = int(np.sum(-(-lens // w.block_size)))
    return int(lens.sum()) * 2 * H * D * esz + B * Hq * D * (esz + 4) + 4 * nblocks + 4 * B


def study_block_size(args):
    import torch
    import paged_kv_cache_424_amd as pa
    import workloads
    from tests import lib_run
    torch.cuda.set_device(0)
    base = workloads.make("c2")
    for bs in (8, 16, 32, 64, 128):
        w = workloads.relayout(base, block_size=bs, free_seed=77)
        st = lib_run.build(w)
        lens = st.lens_host.astype(np.int64)
        stats = pa.pa_allocator_get_stats(st.alloc)
        part_us, red_us, copies = _time_decode(w, st, 512, args.steps)
        algo = _algo_bytes(w, lens)
        _emit({"study": "block_size", "workload": "c2 decode batch: 64 sequences, context U{128..2048}, "
                                                  "32/8 heads, head_dim 128, bf16",
               "block_size": bs, "partition_us": part_us, "reduce_us": red_us,
               "partition_gbs": algo / (part_us * 1e-6) / 1e9,
               "frac_of_8tbs": algo / (part_us * 1e-6) / 8e12,
               "empty_slots_in_used_blocks": stats["used_blocks"] * bs - stats["stored_tokens"],
               "waste_share": 1 - stats["stored_tokens"] / (stats["used_blocks"] * bs),
               "table_entries": int(np.sum(-(-lens // bs))), "pool_copies": copies,
               "launches": args.steps})
        del st
        torch.cuda.empty_cache()


def study_batch1(args):
    import dataclasses
    import torch
    import workloads
    from tests import lib_run
    torch.cuda.set_device(0)
    for L in (512, 2048, 8192, 32768):
        for B in (1, 64):
            if B * L > 64 * 8192:
                continue
            w = workloads.decode_batch(seed=9, lens=[L] * B, name=f"b{B}")
            for layout in ("scattered", "in order"):
                wl = w if layout == "scattered" else dataclasses.replace(
                    w, free_order=np.arange(w.num_blocks, dtype=np.int32))
                st = lib_run.build(wl)
                lens = st.lens_host.astype(np.int64)
                algo = _algo_bytes(wl, lens)
                for part in (0, 512):
                    part_us, red_us, copies = _time_decode(wl, st, part, args.steps)
                    _emit({"study": "batch1", "sequences": B, "context": L, "blocks": layout,
                           "partition": part, "partition_us": part_us, "reduce_us": red_us,
                           "decode_us": part_us + red_us,
                           "partition_gbs": algo / (part_us * 1e-6) / 1e9,
                           "decode_gbs": algo / ((part_us + red_us) * 1e-6) / 1e9,
                           "pool_copies": copies, "launches": args.steps})
                del st
                torch.cuda.empty_cache()


# launch shapes of the streaming read: (workgroups per CU, loads in flight per
# thread, blocked order)
STREAM_SHAPES = ((4, 4, 0), (16, 8, 0), (32, 1, 0), (64, 1, 0), (4, 8, 1), (4, 16, 1), (8, 4, 1),
                 (8, 8, 1), (8, 16, 1), (16, 4, 1), (16, 8, 1), (32, 4, 1))


def stream_read_rates(nbytes, reps, shapes=STREAM_SHAPES):
    """GB/s of pa_stream_read over nbytes for each launch shape (HIP events
    around each launch; consecutive launches read buffers at least 1 GiB apart
    in total, so no launch is served from the Infinity Cache)."""
    import torch
    import paged_kv_cache_424_amd as pa
    nbytes = max(16, nbytes // 16 * 16)
    copies = 1 if nbytes >= ROTATE_BYTES else -(-ROTATE_BYTES // nbytes) + 1
    bufs = [torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rates = {}
    for bpc, unroll, blocked in shapes:
        for i in range(3):
            pa.pa_stream_read(bufs[i % copies], sink, bpc, unroll, blocked)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i, (e0, e1) in enumerate(evs):
            e0.record()
            pa.pa_stream_read(bufs[(3 + i) % copies], sink, bpc, unroll, blocked)
            e1.record()
        torch.cuda.synchronize()
        us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
        rates[f"{bpc}x{unroll}{'b' if blocked else 's'}"] = {"us": us, "gbs": nbytes / (us * 1e-6) / 1e9}
    del bufs
    torch.cuda.empty_cache()
    return nbytes, copies, rates


def study_stream_peak(args):
    import torch
    torch.cuda.set_device(0)
    # the decode workloads' algorithmic bytes per launch, and a large read
    sizes = {"c2 decode bytes": 302_668_092, "c3 decode bytes": 1_074_004_992, "4 GiB": 4 << 30}
    for name, n in sizes.items():
        nbytes, copies, rates = stream_read_rates(n, args.steps)
        best = max(rates, key=lambda k: rates[k]["gbs"])
        _emit({"study": "stream_peak", "size": name, "bytes": nbytes, "buffers": copies,
               "launches": args.steps, "best_shape": best, "best_gbs": rates[best]["gbs"],
               "best_frac_of_8tbs": rates[best]["gbs"] / 8000.0,
               "shapes": {k: round(v["gbs"], 1) for k, v in rates.items()}})


STUDIES = {"prefix-cache": study_prefix_cache, "fragmentation": study_fragmentation,
           "block-size": study_block_size, "batch1": study_batch1, "stream-peak": study_stream_peak}
