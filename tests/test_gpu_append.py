"""Decode with append (pa_decode_append) against the two-call path it replaces:
pa_cache_write of each sequence's newest token followed by pa_decode.

Both the outputs and the pools must be identical bit for bit: the fused path
stores each newest token inside the decode kernel and reads it back with the
rest of the context.  Also checked: a negative slot stores
nothing (as in pa_cache_write); a valid slot that is not the table's slot of
the newest position is stored there and not read; batches above one launch's 1,024
sequences; both partition modes and both cache dtypes.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_424_amd as pa
import workloads
from tests import lib_run

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _new_tokens(w, st):
    """The step's newest token of every decode sequence: (k_new, v_new, slots)."""
    slots, rows = [], []
    for sl, rw in st.step_writes:
        assert len(sl) == 1, "one new token per sequence"
        slots.append(int(sl[0]))
        rows.append(int(rw[0]))
    assert len(slots) == len(w.decode_seqs)
    k = lib_run.torch_stored(w.k_tok[rows], w.dtype).cuda()
    v = lib_run.torch_stored(w.v_tok[rows], w.dtype).cuda()
    return k, v, torch.tensor(slots, dtype=torch.int64, device="cuda")


def _fused(w, st, part, k_new, v_new, slots):
    B, Hq, D = st.q.shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    wsb = pa.pa_decode_workspace_bytes(B, Hq, D, st.max_ctx, part)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda") if wsb else None
    pa.pa_decode_append(out, st.q, k_new, v_new, slots, st.kc, st.vc, st.desc, st.tables, st.lens,
                        st.max_ctx, w.scale, partition_size=part, workspace=ws)
    torch.cuda.synchronize()
    return out


def _many():
    rng = np.random.default_rng(12)
    lens = rng.integers(1, 80, size=1100)
    lens[rng.choice(1100, size=4, replace=False)] = rng.integers(1500, 2500, size=4)
    return workloads.configs._decode_batch_from(rng, "many", "bf16", lens, 8, 2, 64, 16)


def _many_g16():
    # 1,000 short sequences with 16-head groups at head_dim 128: the balanced
    # split's ranges then hold more pieces than the decode holds back at once
    # (three of 16 x 128), so held-back results are stored both when the
    # buffer fills and at the end of a range, next to the newest-token stores
    rng = np.random.default_rng(13)
    lens = rng.integers(1, 120, size=1000)
    return workloads.configs._decode_batch_from(rng, "many_g16", "bf16", lens, 32, 2, 128, 16)


CASES = [("c1", lambda: workloads.make("c1")), ("c2", lambda: workloads.make("c2", small=True)),
         ("c3", lambda: workloads.make("c3", small=True)), ("many", _many), ("many_g16", _many_g16)]


@pytest.mark.parametrize("part", [512, 0])
@pytest.mark.parametrize("name,make", CASES)
def test_append_equals_write_then_decode(name, make, part):
    _announce(f"decode append {name} partition {part}")
    w = make()
    ref_st = lib_run.build(w)                       # step tokens written by pa_cache_write
    ref = lib_run.decode(w, ref_st, partition_size=part)
    st = lib_run.build(w, run_step=False)           # same tables, step tokens not written
    assert not st.step_pairs
    k_new, v_new, slots = _new_tokens(w, st)
    got = _fused(w, st, part, k_new, v_new, slots)
    assert torch.equal(got, ref)
    for a, b in ((st.kc, ref_st.kc), (st.vc, ref_st.vc)):
        assert np.array_equal(lib_run.pool_bits(a, w.dtype), lib_run.pool_bits(b, w.dtype))


def test_negative_slot_stores_nothing():
    _announce("decode append with negative slots")
    w = workloads.make("c2", small=True)
    st = lib_run.build(w, run_step=False)           # newest slots hold the NaN sentinel
    ref = lib_run.decode(w, st, partition_size=512)
    k_new, v_new, slots = _new_tokens(w, st)
    before_k = lib_run.pool_bits(st.kc, w.dtype).copy()
    before_v = lib_run.pool_bits(st.vc, w.dtype).copy()
    got = _fused(w, st, 512, k_new, v_new, torch.full_like(slots, -1))
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))
    assert torch.isnan(got).all(dim=2).any()        # rows that read the never-written slot
    assert np.array_equal(lib_run.pool_bits(st.kc, w.dtype), before_k)
    assert np.array_equal(lib_run.pool_bits(st.vc, w.dtype), before_v)


def test_append_graph_replays_match_eager():
    # captured in a HIP graph, the fused call (stores included) replays to the
    # eager result every time
    _announce("decode append graph replays")
    w = workloads.make("c2", small=True)
    st = lib_run.build(w, run_step=False)
    k_new, v_new, slots = _new_tokens(w, st)
    eager = _fused(w, st, 512, k_new, v_new, slots)
    B, Hq, D = st.q.shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    wsb = pa.pa_decode_workspace_bytes(B, Hq, D, st.max_ctx, 512)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.pa_decode_append(out, st.q, k_new, v_new, slots, st.kc, st.vc, st.desc, st.tables, st.lens,
                            st.max_ctx, w.scale, partition_size=512, workspace=ws)
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep


@pytest.mark.parametrize("dtype,D,G,bs", [("bf16", 128, 3, 8), ("bf16", 64, 16, 128), ("f32", 64, 5, 32),
                                          ("f32", 128, 1, 256)])
def test_append_shapes(dtype, D, G, bs):
    # other head groups, head sizes, cache dtypes and block sizes; lengths that
    # put the newest token first, last and inside a block and a 32-token chunk
    _announce(f"decode append shapes {dtype} D={D} G={G} bs={bs}")
    lens = [1, 2, bs, bs + 1, 32, 33, 511, 512, 513, 1000]
    w = workloads.decode_batch(seed=G + bs, lens=lens, name="app", Hq=2 * G, Hkv=2, D=D, bs=bs, dtype=dtype)
    ref_st = lib_run.build(w)
    st = lib_run.build(w, run_step=False)
    k_new, v_new, slots = _new_tokens(w, st)
    for part in (512, 0, 32):
        ref = lib_run.decode(w, ref_st, partition_size=part)
        got = _fused(w, st, part, k_new, v_new, slots)
        assert torch.equal(got, ref), part
    for a, b in ((st.kc, ref_st.kc), (st.vc, ref_st.vc)):
        assert np.array_equal(lib_run.pool_bits(a, w.dtype), lib_run.pool_bits(b, w.dtype))


@pytest.mark.parametrize("part", [512, 0])
def test_slot_elsewhere_is_stored_not_read(part):
    # every other sequence's newest token goes to a slot of a block no table
    # holds: pa_cache_write + pa_decode then stores it there and reads the
    # table's slot of the newest position (still the NaN sentinel), so those
    # rows are NaN; the fused call must match that bit for bit
    _announce(f"decode append, slots outside the tables, partition {part}")
    w = workloads.make("c2", small=True)
    ref_st = lib_run.build(w, run_step=False)
    st = lib_run.build(w, run_step=False)
    k_new, v_new, slots = _new_tokens(w, st)
    bs, N = w.block_size, w.num_blocks
    used = set(int(b) for b in st.tables.cpu().numpy().ravel() if b >= 0)
    free = [b for b in range(N) if b not in used]
    assert len(free) * bs >= len(slots) // 2
    moved = slots.clone()
    for i, s_ in enumerate(range(0, len(slots), 2)):
        moved[s_] = free[i // bs] * bs + i % bs
    pa.pa_cache_write(ref_st.kc, ref_st.vc, ref_st.desc, k_new, v_new, moved)
    ref = lib_run.decode(w, ref_st, partition_size=part)
    got = _fused(w, st, part, k_new, v_new, moved)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))
    assert torch.isnan(got[0::2]).all() and not torch.isnan(got[1::2]).any()
    for a, b in ((st.kc, ref_st.kc), (st.vc, ref_st.vc)):
        assert np.array_equal(lib_run.pool_bits(a, w.dtype), lib_run.pool_bits(b, w.dtype))


def test_partition_timing_hook_changes_nothing():
    # pa_time_next_partitions: the next partition pass records the two events
    # with its kernel's dispatch; results are those of an untimed call
    _announce("partition timing hook")
    w = workloads.make("c2", small=True)
    st = lib_run.build(w)
    B, Hq, D = st.q.shape
    wsb = pa.pa_decode_workspace_bytes(B, Hq, D, st.max_ctx, 512)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    outs = []
    for timed in (False, True):
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in ev:
            e.record()
        if timed:
            pa.pa_time_next_partitions(*ev)
        pa.pa_decode_partitions(out, st.q, st.kc, st.vc, st.desc, st.tables, st.lens, st.max_ctx, w.scale,
                                512, ws)
        pa.pa_decode_reduce(out, st.lens, Hq, D, st.max_ctx, 512, ws)
        torch.cuda.synchronize()
        if timed:
            assert ev[0].elapsed_time(ev[1]) > 0
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
