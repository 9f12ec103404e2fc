"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Bars: block tables, slots, copy-on-write pairs and whole pools (every byte,
the NaN sentinel of never-written slots included) are bit-exact; attention
outputs are within max abs error 1e-5 (fp32 cache) and 2e-2 (bf16 cache,
fp32 accumulation), and additionally within the kernel's own error budget
(2e-6 / 2e-4: fp32 logits and weights, the value pass fed a hi+lo bf16 split
of each weight).  Probes with sharp structure (needles, one-hot and constant
values) catch indexing mistakes that a flat softmax would hide under 2e-2.
"""

import dataclasses

import numpy as np
import pytest
import torch

import workloads
from tests import lib_run, oracle_run

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
BUDGET = {"f32": 2e-6, "bf16": 2e-4}

SMALL = ["c1", "c2", "c3", "c4", "c4a", "c4p", "c5"]


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module", params=SMALL)
def case(request):
    name = request.param
    _announce(f"build {name} (small)")
    w = workloads.make(name, small=True)
    st_o = oracle_run.build(w)
    st_l = lib_run.build(w)
    torch.cuda.synchronize()
    return name, w, st_o, st_l


def test_tables_and_slots_bit_exact(case):
    name, w, st_o, st_l = case
    t_o, l_o = oracle_run.decode_tables(w, st_o)
    assert np.array_equal(np.asarray(t_o, dtype=np.int32), st_l.tables_host)
    assert np.array_equal(np.asarray(l_o, dtype=np.int32), st_l.lens_host)
    assert [tuple(p) for p in st_o.step_pairs] == [tuple(p) for p in st_l.step_pairs]
    assert np.array_equal(np.asarray(st_o.step_slots, dtype=np.int64), st_l.step_slots)


def test_pools_bit_exact(case):
    name, w, st_o, st_l = case
    for dev, host in ((st_l.kc, st_o.kpool), (st_l.vc, st_o.vpool)):
        got = lib_run.pool_bits(dev, w.dtype)
        want = host.view(np.uint16 if w.dtype == "bf16" else np.uint32)
        assert got.shape == want.shape
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{bad.size} elements differ, first at {bad[:5]}"


def test_decode_matches_oracle(case):
    name, w, st_o, st_l = case
    _announce(f"decode {name}")
    want = oracle_run.oracle_decode(w, st_o)
    got = lib_run.decode(w, st_l).double().cpu().numpy()
    err = np.max(np.abs(got - want))
    assert np.isfinite(got).all()
    assert err <= TOL[w.dtype], err
    assert err <= BUDGET[w.dtype], err


@pytest.mark.parametrize("part", [32, 128, 384, 512])
def test_partition_sizes(case, part):
    name, w, st_o, st_l = case
    want = oracle_run.oracle_decode(w, st_o)
    got = lib_run.decode(w, st_l, partition_size=part).double().cpu().numpy()
    assert np.max(np.abs(got - want)) <= BUDGET[w.dtype]


@pytest.mark.parametrize("part", [0, 32])
def test_bf16_output(case, part):
    # both store paths of the output: the balanced split's held-back results
    # and, with 32-token partitions (up to 16 or more pieces a head), the
    # reduce's workgroup per head
    name, w, st_o, st_l = case
    want = oracle_run.oracle_decode(w, st_o)
    got = lib_run.decode(w, st_l, partition_size=part, out_dtype=torch.bfloat16).double().cpu().numpy()
    # rounding the output to bf16 adds at most half an ulp of |out|
    assert np.all(np.abs(got - want) <= BUDGET[w.dtype] + np.abs(want) * 2.0 ** -8)


def test_many_sequences_and_skewed_lengths():
    # more sequences than one launch scans (1024), lengths from 1 to 3000, so
    # balanced ranges cover many whole sequences and cut long ones into pieces
    _announce("decode 1500 sequences")
    rng = np.random.default_rng(11)
    lens = rng.integers(1, 60, size=1500)
    lens[rng.choice(1500, size=6, replace=False)] = rng.integers(2000, 3000, size=6)
    w = workloads.configs._decode_batch_from(rng, "many", "bf16", lens, 8, 2, 64, 16)
    st_o, st_l = oracle_run.build(w), lib_run.build(w)
    want = oracle_run.oracle_decode(w, st_o)
    for part in (0, 64, 512):
        got = lib_run.decode(w, st_l, partition_size=part).double().cpu().numpy()
        assert np.isfinite(got).all()
        assert np.max(np.abs(got - want)) <= BUDGET["bf16"], part


@pytest.mark.parametrize("small", [True, False])
def test_workspace_contents_do_not_matter(small):
    # the workspace is scratch: whatever it holds before a call (and between
    # calls) must not change the result; at full size the balanced split
    # claims dynamic cells through counters kept in the workspace, so random
    # bytes there (any tag, any count) must be recognised as stale
    import paged_kv_cache_424_amd as pa
    w = workloads.make("c2", small=small)
    st = lib_run.build(w)
    B, Hq, D = st.q.shape
    ref = lib_run.decode(w, st)
    wsb = pa.pa_decode_workspace_bytes(B, Hq, D, st.max_ctx, 0)
    rng = np.random.default_rng(7)
    fills = [0, 0xFF, 0x7F] + [torch.from_numpy(rng.integers(0, 256, size=wsb, dtype=np.uint8))]
    for fill in fills:
        if isinstance(fill, int):
            ws = torch.full((wsb,), fill, dtype=torch.uint8, device="cuda")
        else:
            ws = fill.cuda()
        for rep in range(2):
            out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
            pa.pa_decode(out, st.q, st.kc, st.vc, st.desc, st.tables, st.lens, st.max_ctx, w.scale,
                         workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), (str(fill)[:20], rep)


# ---- invariances: bit-identical outputs ----------------------------------------------
def test_relabelled_blocks_bit_identical():
    w = workloads.make("c2", small=True)
    w2 = workloads.relayout(w, free_seed=1234)
    a = lib_run.decode(w, lib_run.build(w))
    st2 = lib_run.build(w2)
    assert not np.array_equal(lib_run.build(w).tables_host, st2.tables_host)
    b = lib_run.decode(w2, st2)
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["c4", "c4a"])
def test_shared_prefix_bit_identical_to_duplicated(name):
    w = workloads.make(name, small=True)
    wd = workloads.relayout(w, duplicate_shared=True)
    st = lib_run.build(w)
    assert len(st.step_pairs) >= len(w.decode_seqs) - 1
    a = lib_run.decode(w, st)
    b = lib_run.decode(wd, lib_run.build(wd))
    assert torch.equal(a, b)


def test_prompt_cache_bit_identical_to_duplicated():
    # requests that found their prompt by content read the blocks another
    # request wrote (some of them freed and evicted meanwhile): the same
    # bits as every request holding private copies
    w = workloads.make("c4p", small=True)
    wd = workloads.relayout(w, duplicate_shared=True)
    st = lib_run.build(w)
    used = st.tables_host[st.tables_host >= 0]
    assert len(np.unique(used)) < used.size           # some blocks are shared
    assert np.any(st.setup_slots < 0)                 # some writes were skipped
    std = lib_run.build(wd)
    for part in (0, 32, 512):
        a = lib_run.decode(w, st, partition_size=part)
        b = lib_run.decode(wd, std, partition_size=part)
        assert torch.equal(a, b), part


@pytest.mark.parametrize("bs", [8, 32, 64, 128])
def test_block_sizes_match_oracle(bs):
    # the Llama-3-8B-shaped batch stored with other block sizes (the sweep's
    # configurations, at parity size)
    _announce(f"decode c2 small, block size {bs}")
    w = workloads.relayout(workloads.make("c2", small=True), block_size=bs, free_seed=77)
    st_o, st_l = oracle_run.build(w), lib_run.build(w)
    t_o, _ = oracle_run.decode_tables(w, st_o)
    assert np.array_equal(np.asarray(t_o, dtype=np.int32), st_l.tables_host)
    want = oracle_run.oracle_decode(w, st_o)
    for part in (0, 512):
        got = lib_run.decode(w, st_l, partition_size=part).double().cpu().numpy()
        assert np.max(np.abs(got - want)) <= BUDGET["bf16"], part


def test_single_sequence_scattered_and_in_order_blocks():
    # one long sequence, blocks scattered over the pool or in order: the same
    # bits, and the oracle's values (every head)
    _announce("decode one sequence of 5000 tokens, two layouts")
    w = workloads.decode_batch(seed=9, lens=[5000], name="b1")
    wi = dataclasses.replace(w, free_order=np.arange(w.num_blocks, dtype=np.int32))
    st_o = oracle_run.build(w)
    want = oracle_run.oracle_decode(w, st_o)
    st_s, st_i = lib_run.build(w), lib_run.build(wi)
    assert not np.array_equal(st_s.tables_host, st_i.tables_host)
    for part in (0, 512):
        a = lib_run.decode(w, st_s, partition_size=part)
        b = lib_run.decode(wi, st_i, partition_size=part)
        assert torch.equal(a, b), part
        assert np.max(np.abs(a.double().cpu().numpy() - want)) <= BUDGET["bf16"], part


@pytest.mark.parametrize("dtype,D,G,bs", [
    ("bf16", 128, 1, 16), ("bf16", 128, 2, 8), ("bf16", 128, 3, 32), ("bf16", 128, 16, 16),
    ("bf16", 64, 4, 16), ("bf16", 64, 8, 64), ("bf16", 64, 5, 8), ("bf16", 128, 12, 128),
    ("f32", 128, 4, 16), ("f32", 64, 2, 32), ("f32", 128, 16, 8), ("f32", 64, 7, 16)])
def test_decode_shapes(dtype, D, G, bs):
    # head groups from 1 to 16 (powers of two or not), both head sizes, both
    # cache dtypes, block sizes 8..128; lengths include 1, exact multiples of
    # a block and of a 32-token chunk, and a ragged tail
    _announce(f"decode shapes {dtype} D={D} G={G} bs={bs}")
    rng = np.random.default_rng(D + 7 * G + bs)
    lens = [1, bs, 32, 96, 511, 512, 513] + [int(x) for x in rng.integers(2, 1500, size=3)]
    w = workloads.decode_batch(seed=D * 100 + G, lens=lens, name="shapes", Hq=2 * G, Hkv=2, D=D,
                               bs=bs, dtype=dtype)
    st_o, st_l = oracle_run.build(w), lib_run.build(w)
    want = oracle_run.oracle_decode(w, st_o)
    for part in (0, 32, 512):
        got = lib_run.decode(w, st_l, partition_size=part).double().cpu().numpy()
        assert np.isfinite(got).all(), part
        assert np.max(np.abs(got - want)) <= BUDGET[dtype], part


@pytest.mark.parametrize("dtype,D,G,Hkv", [("bf16", 128, 16, 2), ("bf16", 128, 8, 8), ("bf16", 64, 16, 4),
                                            ("f32", 128, 4, 8)])
def test_decode_many_pieces_per_range(dtype, D, G, Hkv):
    # ~1000 short sequences: the balanced split's ranges then cover many
    # (sequence, head) pieces each, more than the workgroup holds back at
    # once, so merged results are stored both when the buffer fills and at
    # the end of a range (G = 16 merges in two passes); every row against the
    # oracle, and bit-identical across two calls
    _announce(f"decode many pieces per range {dtype} D={D} G={G} Hkv={Hkv}")
    rng = np.random.default_rng(7 * D + G + Hkv)
    edges = [1, 2, 31, 32, 33, 64, 65]
    lens = [int(x) if rng.random() < 0.7 else int(rng.choice(edges)) for x in rng.integers(1, 120, size=1000)]
    w = workloads.decode_batch(seed=G * 10 + Hkv, lens=lens, name="pieces", Hq=G * Hkv, Hkv=Hkv, D=D, bs=16,
                               dtype=dtype)
    st_o, st_l = oracle_run.build(w), lib_run.build(w)
    want = oracle_run.oracle_decode(w, st_o)
    a = lib_run.decode(w, st_l, partition_size=0)
    b = lib_run.decode(w, st_l, partition_size=0)
    assert torch.equal(a, b)
    got = a.double().cpu().numpy()
    assert np.isfinite(got).all()
    # 4 M outputs of short contexts with an fp32 cache reach 2.02e-6, the edge
    # of the 2e-6 the smaller cases hold (fp32 rounding of the logits); twice
    # that stays 2.5x under the stated 1e-5 and far under any indexing error
    budget = 2 * BUDGET[dtype] if dtype == "f32" else BUDGET[dtype]
    assert np.max(np.abs(got - want)) <= min(budget, TOL[dtype])


@pytest.mark.parametrize("seed", range(16))
def test_decode_random_configs(seed):
    # seeded random configurations: cache dtype, head size, group size (1..16),
    # kv heads, block size (8..256), batch size, a length mix with block and
    # chunk edges, and the partition (balanced, 32-token, or 64..1024 tokens);
    # the plain decode against the oracle, and decode with append bit-identical
    # to write + decode
    import paged_kv_cache_424_amd as pa
    rng = np.random.default_rng(1000 + seed)
    dtype = ["bf16", "f32"][seed % 2]
    D = [64, 128][(seed // 2) % 2]
    G = int(rng.integers(1, 17))
    Hkv = int(rng.integers(1, 5))
    bs = int(2 ** rng.integers(3, 9))
    B = int(rng.integers(1, 24))
    edges = [1, 2, bs, bs + 1, 31, 32, 33, 511, 512, 513]
    lens = [int(x) if rng.random() < 0.6 else int(rng.choice(edges)) for x in rng.integers(1, 1800, size=B)]
    part = int(rng.choice([0, 32, 64, 160, 512, 1024]))
    _announce(f"decode random config {seed}: {dtype} D={D} G={G} Hkv={Hkv} bs={bs} B={B} partition {part}")
    w = workloads.decode_batch(seed=seed, lens=lens, name="rnd", Hq=G * Hkv, Hkv=Hkv, D=D, bs=bs, dtype=dtype)
    st_o, ref_st = oracle_run.build(w), lib_run.build(w)
    want = oracle_run.oracle_decode(w, st_o)
    ref = lib_run.decode(w, ref_st, partition_size=part)
    got = ref.double().cpu().numpy()
    assert np.isfinite(got).all()
    assert np.max(np.abs(got - want)) <= BUDGET[dtype]
    # decode with append: the step's newest tokens stored by the decode kernel
    st = lib_run.build(w, run_step=False)
    slots, rows = [], []
    for sl, rw in st.step_writes:
        slots.append(int(sl[0]))
        rows.append(int(rw[0]))
    k_new = lib_run.torch_stored(w.k_tok[rows], w.dtype).cuda()
    v_new = lib_run.torch_stored(w.v_tok[rows], w.dtype).cuda()
    B_, Hq, _ = st.q.shape
    out = torch.full((B_, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    wsb = pa.pa_decode_workspace_bytes(B_, Hq, D, st.max_ctx, part)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda") if wsb else None
    pa.pa_decode_append(out, st.q, k_new, v_new, torch.tensor(slots, dtype=torch.int64, device="cuda"),
                        st.kc, st.vc, st.desc, st.tables, st.lens, st.max_ctx, w.scale, partition_size=part,
                        workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    for a, b in ((st.kc, ref_st.kc), (st.vc, ref_st.vc)):
        assert np.array_equal(lib_run.pool_bits(a, w.dtype), lib_run.pool_bits(b, w.dtype))


# ---- probes with sharp structure -------------------------------------------------------
def _probe_workload(base, k=None, v=None, q=None):
    return dataclasses.replace(base, k_tok=base.k_tok if k is None else k,
                               v_tok=base.v_tok if v is None else v,
                               q_dec=base.q_dec if q is None else q)


def _bf16(x):
    return workloads.round_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _run_both(w):
    st_o, st_l = oracle_run.build(w), lib_run.build(w)
    return oracle_run.oracle_decode(w, st_o), lib_run.decode(w, st_l).double().cpu().numpy()


@pytest.mark.parametrize("part", [512, 0])
def test_needle_in_every_logical_block(part):
    """Every logical block of every sequence and kv head holds one needle key,
    and across the calls every needle is selected by some query head.

    Block b's needle key is 200 * sign_b * e_{b mod 128} (sign_b = -1 for
    b >= 128), at an offset inside the block that varies with b and the head;
    all other keys are 0.  A query head that looks along +-e_c gives block b's
    needle a logit of 200/sqrt(128) ~ 17.7 and every other key 0 or -17.7, so
    its output is that needle's value row within L * exp(-17.7) ~ 1e-4 of its
    scale ([ch.09] "해법": block j of the table is position range j of the
    contiguous context, whichever physical block holds it).  Needle values are
    small integers that differ between neighbouring blocks in every channel."""
    base = workloads.make("c3", small=True)       # 2 x 3000 tokens: 188 blocks per sequence
    bs, G, D, H = base.block_size, base.group, base.head_dim, base.num_kv_heads
    B, Hq = len(base.decode_seqs), base.num_q_heads
    k = np.zeros(base.k_tok.shape, dtype=np.float32)
    v = np.zeros(base.v_tok.shape, dtype=np.float32)
    nblk = {}
    needle_v = {}
    for si, s in enumerate(base.decode_seqs):
        rows = base.tok_rows[s]
        L = len(rows)
        nb = -(-L // bs)
        assert nb <= 2 * D
        nblk[si] = nb
        for g in range(H):
            for b in range(nb):
                pos = min(b * bs + (5 * b + 3 * g) % bs, L - 1)
                k[rows[pos], g, b % D] = 200.0 if b < D else -200.0
                v[rows[pos], g, :] = ((37 * b + 11 * np.arange(D) + 5 * g + 3 * si) % 64) - 32
                needle_v[(si, g, b)] = v[rows[pos], g, :].astype(np.float64)
    w = _probe_workload(base, k=_bf16(k), v=_bf16(v))
    st_l = lib_run.build(w)
    ncalls = -(-max(nblk.values()) // G)
    seen = set()
    for call in range(ncalls):
        q = np.zeros((B, Hq, D), dtype=np.float32)
        target = {}
        for si in range(B):
            for h in range(Hq):
                b = (call * G + h % G) % nblk[si]
                q[si, h, b % D] = 1.0 if b < D else -1.0
                target[(si, h)] = b
        qd = lib_run.torch_stored(_bf16(q), w.dtype).cuda()
        got = lib_run.decode(w, st_l, partition_size=part, q=qd).double().cpu().numpy()
        for (si, h), b in target.items():
            want = needle_v[(si, h // G, b)]
            err = np.max(np.abs(got[si, h] - want))
            assert err <= 1e-3 * 32, (part, call, si, h, b, err)
            seen.add((si, h // G, b))
    assert seen == set(needle_v)                  # every block of every (sequence, kv head)


def test_constant_values_per_kv_head_and_ones():
    base = workloads.make("c2", small=True)
    v = np.empty(base.v_tok.shape, dtype=np.float32)
    for g in range(base.num_kv_heads):
        v[:, g, :] = g + 1.0
    w = _probe_workload(base, v=_bf16(v))
    _, got = _run_both(w)
    for h in range(base.num_q_heads):
        # the weights sum to one; the hi+lo split keeps each to 2^-18 relative
        c = h // base.group + 1.0
        assert np.max(np.abs(got[:, h, :] / c - 1.0)) <= 1e-5


def test_one_hot_values_give_the_weights():
    base = workloads.make("c1")                    # L <= 48 <= D = 64
    v = np.zeros(base.v_tok.shape, dtype=np.float32)
    for s in base.decode_seqs:
        for pos, row in enumerate(base.tok_rows[s]):
            v[row, :, pos] = 1.0
    w = _probe_workload(base, v=v)
    st_o, st_l = oracle_run.build(w), lib_run.build(w)
    got = lib_run.decode(w, st_l).double().cpu().numpy()
    from oracle import attention
    tables, lens = oracle_run.decode_tables(w, st_o)
    q = attention.stored_to_f64(w.q_dec, w.dtype)
    for i, s in enumerate(w.decode_seqs):
        for h in range(w.num_q_heads):
            wts = attention.decode_weights(q[i, h], st_o.kpool, st_o.vpool, w.dtype, w.num_kv_heads,
                                           w.block_size, w.head_dim, tables[i], lens[i], h // w.group,
                                           w.scale)
            assert np.max(np.abs(got[i, h, :lens[i]] - wts)) <= 1e-6
            assert np.all(got[i, h, lens[i]:] == 0.0)


def test_length_one_returns_v_exactly():
    rng = np.random.default_rng(9)
    w = workloads.configs._decode_batch_from(rng, "len1", "bf16", [1, 1, 2, 1, 513], 32, 8, 128, 16)
    st_l = lib_run.build(w)
    got = lib_run.decode(w, st_l).cpu().numpy()
    for i, s in enumerate(w.decode_seqs):
        if w.seq_len(s) != 1:
            continue
        row = w.tok_rows[s][0]
        vref = (w.v_tok[row].astype(np.uint32) << 16).view(np.float32)   # [Hkv, D]
        for h in range(w.num_q_heads):
            assert np.array_equal(got[i, h], vref[h // w.group])


# ---- edge cases ------------------------------------------------------------------------------
@pytest.mark.parametrize("part", [512, 0])
def test_invalid_rows_give_nan_and_leave_others_alone(part):
    w = workloads.make("c2", small=True)
    st = lib_run.build(w)
    good = lib_run.decode(w, st, partition_size=part)
    lens = st.lens.clone()
    lens[1] = 0                                   # invalid length
    lens[2] = st.max_ctx + 1                      # beyond the declared maximum
    tables = st.tables.clone()
    tables[3, 0] = w.num_blocks                   # out-of-range block id
    tables[4, 1] = -7
    out = lib_run.decode(w, st, lens=lens, tables=tables, partition_size=part)
    for i in (1, 2, 3, 4):
        assert torch.isnan(out[i]).all(), i
    keep = [i for i in range(len(w.decode_seqs)) if i not in (1, 2, 3, 4)]
    if part:
        # fixed partitions: a row's pieces depend on its own length only
        assert torch.equal(out[keep], good[keep])
    else:
        # balanced split: the cut points move with the other rows' lengths,
        # which changes the rounding but not the result
        assert torch.isfinite(out[keep]).all()
        assert torch.max(torch.abs(out[keep] - good[keep])).item() <= BUDGET["bf16"]


def test_empty_batch_is_a_no_op():
    import paged_kv_cache_424_amd as pa
    w = workloads.make("c1")
    st = lib_run.build(w)
    q = st.q[:0]
    out = torch.empty((0, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    pa.pa_decode(out, q, st.kc, st.vc, st.desc, st.tables[:0], st.lens[:0], 1, w.scale)
    pa.pa_cache_write(st.kc, st.vc, st.desc, q[:0, :w.num_kv_heads], q[:0, :w.num_kv_heads],
                      torch.empty(0, dtype=torch.int64, device="cuda"))
    pa.pa_copy_blocks(st.kc, st.vc, st.desc, [])
    torch.cuda.synchronize()


def test_negative_slots_are_padding():
    import paged_kv_cache_424_amd as pa
    w = workloads.make("c1")
    st = lib_run.build(w)
    before_k = lib_run.pool_bits(st.kc, w.dtype).copy()
    k = torch.randn((3, w.num_kv_heads, w.head_dim), device="cuda")
    slots = torch.tensor([-1, -5, -100], dtype=torch.int64, device="cuda")
    pa.pa_cache_write(st.kc, st.vc, st.desc, k, k, slots)
    assert np.array_equal(before_k, lib_run.pool_bits(st.kc, w.dtype))


@pytest.mark.parametrize("dtype,bs,D", [("bf16", 16, 64), ("bf16", 8, 128), ("bf16", 32, 64), ("f32", 16, 64),
                                        ("f32", 8, 128), ("bf16", 12, 64), ("bf16", 16, 48), ("f32", 16, 40)])
def test_cache_write_runs_and_scattered_slots(dtype, bs, D):
    # runs of consecutive slots (aligned, off by one, crossing a block, with
    # padding inside) and scattered slots, on the 16-byte path (head_dim a
    # multiple of 32) and the element path (48, 40); the pools must match the
    # oracle's bit for bit
    import paged_kv_cache_424_amd as pa
    from oracle import cache
    _announce(f"cache_write runs {dtype} bs={bs} D={D}")
    rng = np.random.default_rng(bs + D)
    H, N = 4, 24
    nslots = N * bs
    slots = []
    slots += list(range(0, 8))                       # aligned run
    slots += list(range(3 * bs + 1, 3 * bs + 9))     # off by one
    slots += list(range(5 * bs - 4, 5 * bs + 4))     # crosses a block boundary
    run = list(range(8 * bs, 8 * bs + 8))
    run[3] = -1                                      # padding inside a run
    slots += run
    free = sorted(set(range(nslots)) - set(s for s in slots if s >= 0))
    slots += list(rng.choice(free, size=13, replace=False))   # scattered, ragged tail
    slots = np.asarray(slots, dtype=np.int64)
    T = len(slots)
    x = rng.standard_normal((2, T, H, D), dtype=np.float32)
    fill = workloads.NAN_FILL_BF16 if dtype == "bf16" else workloads.NAN_FILL_F32
    if dtype == "bf16":
        kv = [workloads.round_to_bf16_bits(x[0]), workloads.round_to_bf16_bits(x[1])]
    else:
        kv = [x[0], x[1]]
    kp = cache.new_pool(N, H, bs, D, dtype, fill)
    vp = cache.new_pool(N, H, bs, D, dtype, fill)
    cache.cache_write(kp, vp, H, bs, D, N, kv[0], kv[1], slots)
    desc = pa.cache_desc(N, bs, H, D, dtype)
    n = pa.pa_cache_pool_bytes(desc) // (2 if dtype == "bf16" else 4)
    kc = lib_run.fill_pool(n, dtype, fill, "cuda")
    vc = lib_run.fill_pool(n, dtype, fill, "cuda")
    pa.pa_cache_write(kc, vc, desc, lib_run.torch_stored(kv[0], dtype).cuda(),
                      lib_run.torch_stored(kv[1], dtype).cuda(), torch.from_numpy(slots).cuda())
    for dev, host in ((kc, kp), (vc, vp)):
        got = lib_run.pool_bits(dev, dtype)
        want = host.view(np.uint16 if dtype == "bf16" else np.uint32)
        assert np.array_equal(got, want)


def test_copy_blocks_4096_pairs_bit_exact():
    """A long copy-on-write list (4,096 pairs, more than one launch's batch):
    both pools bit-exact against the oracle's copies, every other block
    untouched."""
    import paged_kv_cache_424_amd as pa
    from oracle import cache
    H, bs, D, N, n = 2, 16, 128, 9000, 4096
    rng = np.random.default_rng(4096)
    blocks = rng.permutation(N)
    src = rng.choice(blocks[:N - n], size=n, replace=True)     # sources may repeat
    dst = blocks[N - n:]                                        # distinct, never a source
    pairs = np.stack([src, dst], axis=1).astype(np.int64)
    _announce(f"copy_blocks {n} pairs, pool {N} blocks")
    kbits = rng.integers(0, 1 << 16, size=N * H * bs * D, dtype=np.uint16)
    vbits = rng.integers(0, 1 << 16, size=N * H * bs * D, dtype=np.uint16)
    desc = pa.cache_desc(N, bs, H, D, "bf16")
    kc = torch.from_numpy(kbits.view(np.int16).copy()).cuda().view(torch.bfloat16)
    vc = torch.from_numpy(vbits.view(np.int16).copy()).cuda().view(torch.bfloat16)
    pa.pa_copy_blocks(kc, vc, desc, pairs)
    torch.cuda.synchronize()
    kw, vw = kbits.copy(), vbits.copy()
    cache.copy_blocks(kw, vw, H, bs, D, N, [tuple(p) for p in pairs.tolist()])
    assert np.array_equal(lib_run.pool_bits(kc, "bf16"), kw)
    assert np.array_equal(lib_run.pool_bits(vc, "bf16"), vw)
