"""Pins of the attention oracle (O2-O4) against things other than itself.

  * brute force: 40-digit decimal arithmetic on the generated logical K/V
    (no pool, no table, no gather) for all of the tiny fp32 workload and for
    random tiny grouped-query cases;
  * a library special case: torch's scaled_dot_product_attention in fp64 on
    the CPU, fed the logical K/V with kv heads repeated per group;
  * properties the pages fix: physical block ids can be anything (relabelling
    changes nothing), a prefix stored once equals a prefix stored per
    sequence, the cache layout is a bijection and a write/read round trip is
    exact, and closed forms (L = 1, identical keys, q = 0, rows sum to 1,
    key shift, linearity in V, a dominant "needle" key, block-size
    invariance, prefill's last query = decode);
  * planted mistakes: each plausible oracle bug (dropped scale, wrong kv head,
    off-by-one offset, transposed read) is planted on the CPU and shown to
    fail a pin.
"""

import decimal
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, cache
from tests import oracle_run


def exact_f64(stored, dtype):
    """Upcast by a route independent of the oracle's own conversion."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).double().numpy()
    t = torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


def brute_force(q, K, V, scale, digits=40):
    """softmax(K q scale) V in decimal arithmetic with `digits` significant digits."""
    with decimal.localcontext() as ctx:
        ctx.prec = digits
        D = decimal.Decimal
        qd = [D(float(x)) for x in q]
        sc = D(float(scale))
        z = [sum(qd[d] * D(float(K[t, d])) for d in range(len(qd))) * sc for t in range(K.shape[0])]
        m = max(z)
        e = [(zt - m).exp() for zt in z]
        tot = sum(e)
        return np.array([float(sum(e[t] * D(float(V[t, d])) for t in range(K.shape[0])) / tot)
                         for d in range(V.shape[1])])


def logical(w, s, g):
    rows = w.tok_rows[s]
    return exact_f64(w.k_tok[rows, g, :], w.dtype), exact_f64(w.v_tok[rows, g, :], w.dtype)


# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def c1():
    w = workloads.make("c1")
    return w, oracle_run.build(w)


def test_c1_brute_force(c1):
    w, st = c1
    out = oracle_run.oracle_decode(w, st)
    q = exact_f64(w.q_dec, w.dtype)
    G = w.group
    for s in w.decode_seqs:
        for h in range(w.num_q_heads):
            K, V = logical(w, s, h // G)
            want = brute_force(q[s, h], K, V, w.scale)
            assert np.max(np.abs(out[s, h] - want)) <= 1e-13


@pytest.mark.parametrize("seed", range(6))
def test_random_tiny_gqa_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    H, G, D, bs = 2, 3, 4, 2
    lens = [int(x) for x in rng.integers(1, 9, size=3)]
    w = workloads.configs._decode_batch_from(rng, "tiny", "f32", lens, H * G, H, D, bs,
                                             num_blocks=16)
    st = oracle_run.build(w)
    out = oracle_run.oracle_decode(w, st)
    q = exact_f64(w.q_dec, "f32")
    for s in w.decode_seqs:
        for h in range(H * G):
            K, V = logical(w, s, h // G)
            assert np.max(np.abs(out[s, h] - brute_force(q[s, h], K, V, w.scale))) <= 1e-13


@pytest.fixture(scope="module")
def c2s():
    w = workloads.make("c2", small=True)
    return w, oracle_run.build(w)


def test_sdpa_cross_check(c2s):
    w, st = c2s
    out = oracle_run.oracle_decode(w, st)
    q = exact_f64(w.q_dec, w.dtype)
    G = w.group
    for s in w.decode_seqs:
        Ks, Vs = zip(*[logical(w, s, g) for g in range(w.num_kv_heads)])
        K = torch.from_numpy(np.stack(Ks)).repeat_interleave(G, dim=0)[None]   # [1, Hq, L, D]
        V = torch.from_numpy(np.stack(Vs)).repeat_interleave(G, dim=0)[None]
        Q = torch.from_numpy(q[s])[None, :, None, :]                             # [1, Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=w.scale)
        assert np.max(np.abs(out[s] - ref[0, :, 0, :].numpy())) <= 1e-12


# --- layout ----------------------------------------------------------------------
def test_layout_is_bijection():
    N, H, bs, D = 3, 2, 4, 8
    b, g, o, d = np.meshgrid(np.arange(N), np.arange(H), np.arange(bs), np.arange(D), indexing="ij")
    for fn in (cache.k_index, cache.v_index):
        idx = fn(H, bs, D, b, g, o, d).ravel()
        assert sorted(idx.tolist()) == list(range(N * H * bs * D))


def test_write_read_round_trip_and_untouched_bytes(c2s):
    w, st = c2s
    tables, lens = oracle_run.decode_tables(w, st)
    fill = np.uint16(w.fill_bits)
    used = np.zeros(st.kpool.shape, dtype=bool)
    H, bs, D = w.num_kv_heads, w.block_size, w.head_dim
    for i, s in enumerate(w.decode_seqs):
        L = lens[i]
        for g in range(H):
            K, V = attention.gather(st.kpool, st.vpool, w.dtype, H, bs, D, tables[i], L, g)
            Kw, Vw = logical(w, s, g)
            assert np.array_equal(K, Kw) and np.array_equal(V, Vw)
        pos = np.arange(L)[:, None, None]
        blk = np.asarray(tables[i])[pos // bs]
        used[cache.k_index(H, bs, D, blk, np.arange(H)[None, :, None], pos % bs,
                           np.arange(D)[None, None, :])] = True
    assert np.all(st.kpool[~used] == fill)       # never-written slots keep the sentinel


def test_copy_blocks_copies_everything_and_only_dst():
    N, H, bs, D = 6, 2, 4, 3
    rng = np.random.default_rng(7)
    k = rng.integers(0, 1 << 16, size=N * H * bs * D, dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=N * H * bs * D, dtype=np.uint16)
    k0, v0 = k.copy(), v.copy()
    cache.copy_blocks(k, v, H, bs, D, N, [(1, 4), (1, 5), (2, 0)])
    tile = H * bs * D
    for src, dst in [(1, 4), (1, 5), (2, 0)]:
        assert np.array_equal(k[dst * tile:(dst + 1) * tile], k0[src * tile:(src + 1) * tile])
        assert np.array_equal(v[dst * tile:(dst + 1) * tile], v0[src * tile:(src + 1) * tile])
    for b in (1, 2, 3):
        assert np.array_equal(k[b * tile:(b + 1) * tile], k0[b * tile:(b + 1) * tile])
    for bad in ([(1, 4), (2, 4)], [(1, 4), (4, 5)], [(0, 6)]):
        with pytest.raises(ValueError):
            cache.copy_blocks(k, v, H, bs, D, N, bad)


# --- properties the pages fix --------------------------------------------------------
def test_block_relabelling_is_bit_identical(c2s):
    w, st = c2s
    out = oracle_run.oracle_decode(w, st)
    w2 = workloads.relayout(w, free_seed=77)
    out2 = oracle_run.oracle_decode(w2, oracle_run.build(w2))
    t1, _ = oracle_run.decode_tables(w, st)
    assert not np.array_equal(np.asarray(t1), np.asarray(oracle_run.decode_tables(w2, oracle_run.build(w2))[0]))
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("name", ["c4", "c4a"])
def test_shared_prefix_equals_duplicated(name):
    w = workloads.make(name, small=True)
    st = oracle_run.build(w)
    shared_blocks = set(st.alloc.tables[0][:60])
    assert all(set(st.alloc.tables[s][:60]) == shared_blocks for s in w.decode_seqs)
    out = oracle_run.oracle_decode(w, st)
    wd = workloads.relayout(w, duplicate_shared=True)
    out_d = oracle_run.oracle_decode(wd, oracle_run.build(wd))
    assert np.array_equal(out, out_d)


def test_block_size_invariance(c2s):
    w, st = c2s
    out = oracle_run.oracle_decode(w, st)
    w32 = workloads.relayout(w, block_size=32)
    assert np.array_equal(out, oracle_run.oracle_decode(w32, oracle_run.build(w32)))


def _single(q, K, V, scale=0.125):
    return attention.attend(q, K, V, scale)


def test_length_one_returns_v_exactly():
    rng = np.random.default_rng(3)
    for _ in range(20):
        q, K, V = rng.standard_normal(8) * 50, rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
        out, w = _single(q, K, V)
        assert np.array_equal(out, V[0]) and w[0] == 1.0


def test_identical_keys_and_zero_query_give_mean_of_v():
    rng = np.random.default_rng(4)
    V = rng.standard_normal((37, 16))
    K = np.tile(rng.standard_normal(16), (37, 1))
    out, w = _single(rng.standard_normal(16), K, V)
    assert np.max(np.abs(out - V.mean(axis=0))) <= 1e-12
    out, _ = _single(np.zeros(16), rng.standard_normal((37, 16)), V)
    assert np.max(np.abs(out - V.mean(axis=0))) <= 1e-12


def test_rows_sum_to_one_and_shift_invariance_and_linearity():
    rng = np.random.default_rng(5)
    for L in (1, 2, 17, 300):
        q, K = rng.standard_normal(32), rng.standard_normal((L, 32)) * 3
        V1, V2 = rng.standard_normal((L, 32)), rng.standard_normal((L, 32))
        out1, w = _single(q, K, V1)
        assert abs(w.sum() - 1.0) <= 1e-12
        t = rng.standard_normal(32)
        assert np.max(np.abs(_single(q, K + t, V1)[0] - out1)) <= 1e-12
        out2, _ = _single(q, K, V2)
        out12, _ = _single(q, K, 2.5 * V1 - 0.75 * V2)
        assert np.max(np.abs(out12 - (2.5 * out1 - 0.75 * out2))) <= 1e-12


def test_needle_key_dominates():
    rng = np.random.default_rng(6)
    L, D, scale = 200, 16, 0.125
    q = rng.standard_normal(D)
    K = rng.standard_normal((L, D)) * 0.1
    j = 123
    K[j] = q / np.dot(q, q) * (40.0 / scale)         # logit of key j is 40
    V = rng.standard_normal((L, D))
    out, _ = attention.attend(q, K, V, scale)
    z = np.array([scale * math.fsum(q * K[t]) for t in range(L)])
    assert z[j] - np.delete(z, j).max() >= 39
    # |out - V_j| = |sum_t w_t (V_t - V_j)| <= sum_{t != j} exp(z_t - z_j) * 2 max|V|
    bound = sum(math.exp(z[t] - z[j]) for t in range(L) if t != j) * 2 * np.abs(V).max()
    assert np.max(np.abs(out - V[j])) <= bound + 1e-15


def test_prefill_last_query_equals_decode():
    w = workloads.make("c5", small=True)
    st = oracle_run.build(w)
    pre = oracle_run.oracle_prefill(w, st)
    tables, lens = st.alloc.block_tables(w.prefill_seqs, oracle_run.max_blocks(w))
    qs = np.concatenate([[0], np.cumsum(w.chunk_len)])
    q = attention.stored_to_f64(w.q_pre, w.dtype)
    for c in range(len(w.prefill_seqs)):
        last = qs[c + 1] - 1
        dec = attention.decode(q[last:last + 1], st.kpool, st.vpool, w.dtype, w.num_kv_heads,
                               w.block_size, w.head_dim, [tables[c]], [lens[c]], w.scale)
        assert np.array_equal(pre[last], dec[0])
    # and a middle query against brute force on the logical data (causal cut)
    c, i, h = 1, 5, 9
    s = w.prefill_seqs[c]
    L, C = lens[c], w.chunk_len[c]
    K, V = logical(w, s, h // w.group)
    P = L - C + i
    want = brute_force(exact_f64(w.q_pre[qs[c] + i, h], w.dtype), K[:P + 1], V[:P + 1], w.scale,
                       digits=30)
    assert np.max(np.abs(pre[qs[c] + i, h] - want)) <= 1e-13


# --- planted mistakes: each must fail a pin ----------------------------------------------
def _c1_error(w, st):
    out = oracle_run.oracle_decode(w, st)
    q = exact_f64(w.q_dec, w.dtype)
    err = 0.0
    for s in w.decode_seqs:
        for h in (0, 5):
            K, V = logical(w, s, h // w.group)
            err = max(err, np.max(np.abs(out[s, h] - brute_force(q[s, h], K, V, w.scale))))
    return err


def test_planted_dropped_scale_is_caught(c1, monkeypatch):
    w, st = c1
    real = attention.attend
    monkeypatch.setattr(attention, "attend", lambda q, K, V, scale: real(q, K, V, 1.0))
    assert _c1_error(w, st) > 1e-3


def test_planted_wrong_offset_is_caught(c1, monkeypatch):
    w, _ = c1
    real = cache.k_index
    # the writer puts each key one slot further on: a plausible off-by-one
    monkeypatch.setattr(attention.cache, "k_index",
                        lambda H, bs, D, b, g, o, d: real(H, bs, D, b, g, (o + 1) % bs, d))
    st = oracle_run.build(w)
    monkeypatch.setattr(attention.cache, "k_index", real)
    assert _c1_error(w, st) > 1e-3


def test_planted_transposed_v_read_is_caught(c1, monkeypatch):
    w, st = c1
    real_k = cache.k_index
    # the reader takes V as if it were laid out like K (token rows, not channel rows)
    monkeypatch.setattr(attention.cache, "v_index", real_k)
    assert _c1_error(w, st) > 1e-3


def test_planted_wrong_kv_head_is_caught(monkeypatch):
    rng = np.random.default_rng(11)
    w = workloads.configs._decode_batch_from(rng, "tiny", "f32", [7, 3], 6, 2, 4, 2, num_blocks=16)
    st = oracle_run.build(w)
    real = attention.gather
    monkeypatch.setattr(attention, "gather",
                        lambda kp, vp, dt, H, bs, D, t, L, head: real(kp, vp, dt, H, bs, D, t, L, (head + 1) % H))
    out = oracle_run.oracle_decode(w, st)
    q = exact_f64(w.q_dec, "f32")
    K, V = logical(w, 0, 0)
    assert np.max(np.abs(out[0, 0] - brute_force(q[0, 0], K, V, w.scale))) > 1e-3
