"""Parity at the full workload sizes, in the launch configuration the
benchmark times (512-token partitions, the method's stated partition size),
and with the balanced split as well.

Everything integer is compared whole and bit for bit: block tables, lengths,
the step's slots and copy pairs, and both pools byte for byte (never-written
slots keep their NaN sentinel).  Attention outputs are compared on a sample of
sequences (every head of each) that the oracle computes one by one: the
longest, the shortest and seeded random picks; prefill on a sample of query
rows of every chunk (first, last and random positions).
"""

import numpy as np
import pytest
import torch

import workloads
from tests import lib_run, oracle_run

pytestmark = pytest.mark.gpu

FULL = ["c2", "c3", "c4", "c4a", "c4p", "c5"]
BENCH_PARTITION = 512                  # bench.py's default for every workload
BUDGET = 2e-4                          # bf16 cache, fp32 accumulation


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module", params=FULL)
def full(request):
    name = request.param
    _announce(f"build {name} (full size)")
    w = workloads.make(name)
    st_o = oracle_run.build(w)
    st_l = lib_run.build(w)
    torch.cuda.synchronize()
    yield name, w, st_o, st_l
    del st_l
    torch.cuda.empty_cache()


def _sample_seqs(w, st_l, k=4, seed=0):
    lens = st_l.lens_host
    pick = {int(np.argmax(lens)), int(np.argmin(lens))}
    rng = np.random.default_rng(seed)
    pick.update(int(x) for x in rng.choice(len(lens), size=min(k, len(lens)), replace=False))
    return sorted(pick)


def test_full_tables_slots_pairs_bit_exact(full):
    name, w, st_o, st_l = full
    t_o, l_o = oracle_run.decode_tables(w, st_o)
    assert np.array_equal(np.asarray(t_o, dtype=np.int32), st_l.tables_host)
    assert np.array_equal(np.asarray(l_o, dtype=np.int32), st_l.lens_host)
    assert [tuple(p) for p in st_o.step_pairs] == [tuple(p) for p in st_l.step_pairs]
    assert np.array_equal(np.asarray(st_o.step_slots, dtype=np.int64), st_l.step_slots)


def test_full_pools_bit_exact(full):
    name, w, st_o, st_l = full
    _announce(f"pools {name} (full size)")
    for dev, host in ((st_l.kc, st_o.kpool), (st_l.vc, st_o.vpool)):
        got = lib_run.pool_bits(dev, w.dtype)
        want = host.view(np.uint16 if w.dtype == "bf16" else np.uint32)
        assert got.shape == want.shape
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{bad.size} elements differ, first at {bad[:5]}"


def test_full_decode_sampled(full):
    name, w, st_o, st_l = full
    seqs = _sample_seqs(w, st_l)
    Hq = w.num_q_heads
    pairs = [(s, h) for s in seqs for h in range(Hq)]
    want = oracle_run.oracle_decode(w, st_o, pairs=pairs)[seqs]
    for part in (BENCH_PARTITION, 0):
        _announce(f"decode {name} (full size) partition {part}, sequences {seqs}")
        got = lib_run.decode(w, st_l, partition_size=part).double().cpu().numpy()
        assert np.isfinite(got).all()
        err = np.max(np.abs(got[seqs] - want))
        assert err <= BUDGET, (part, err)


@pytest.mark.parametrize("full", ["c5"], indirect=True)      # the workload with prefill chunks
def test_full_prefill_sampled(full):
    name, w, st_o, st_l = full
    assert w.prefill_seqs
    _announce(f"prefill {name} (full size)")
    qs = np.concatenate([[0], np.cumsum(w.chunk_len)])
    rng = np.random.default_rng(1)
    rows = set()
    for c in range(len(w.chunk_len)):
        q0, q1 = int(qs[c]), int(qs[c + 1])
        for t in {q0, q1 - 1, int(rng.integers(q0, q1))}:
            for h in rng.choice(w.num_q_heads, size=4, replace=False):
                rows.add((t, int(h)))
    rows = sorted(rows)
    want = oracle_run.oracle_prefill(w, st_o, rows=rows)
    got = lib_run.prefill(w, st_l).double().cpu().numpy()
    assert np.isfinite(got).all()
    t_idx = [t for t, _ in rows]
    h_idx = [h for _, h in rows]
    err = np.max(np.abs(got[t_idx, h_idx] - want[t_idx, h_idx]))
    _announce(f"prefill {name} (full size) sampled max err {err:.2e}")
    assert err <= 2e-2
