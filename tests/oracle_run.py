"""Drive the CPU oracle through a workload (test infrastructure).

Builds the oracle's own allocator state, pools, block tables and expected
outputs from a ``workloads.Workload``.  Uses nothing but ``oracle`` and the
workload's seeded inputs.
"""

import numpy as np

from oracle import attention, cache
from oracle.allocator import BlockAllocator, PrefixCachingAllocator


class OracleState:
    pass


def build(w, run_step=True):
    """Run the workload's op script op by op: copy-on-write pairs are copied
    right away, then the append's tokens are written."""
    H, bs, D = w.num_kv_heads, w.block_size, w.head_dim
    a = (PrefixCachingAllocator if w.prefix_cache else BlockAllocator)(w.num_blocks, bs, w.free_order)
    kpool = cache.new_pool(w.num_blocks, H, bs, D, w.dtype, w.fill_bits)
    vpool = cache.new_pool(w.num_blocks, H, bs, D, w.dtype, w.fill_bits)
    st = OracleState()
    st.alloc = a
    st.step_slots = []          # slots written in the step, in script order
    st.step_rows = []           # matching rows of k_tok / v_tok
    st.step_pairs = []          # copy-on-write pairs issued in the step
    st.setup_results = []
    for phase, op in w.script:
        if phase == "step" and not run_step:
            break
        if op[0] == "create":
            res = a.create_seq()
        elif op[0] == "fork":
            res = a.fork(op[1])
        elif op[0] == "cow":
            res = a.cow_block(op[1], op[2])
            if res is not None:
                cache.copy_blocks(kpool, vpool, H, bs, D, w.num_blocks, [res])
                if phase == "step":
                    st.step_pairs.append(res)
        elif op[0] in ("append", "append_tokens"):
            s = op[1]
            n = op[2] if op[0] == "append" else len(op[2])
            start = a.lengths[s]
            res = a.append_slots(s, n) if op[0] == "append" else a.append_tokens(s, op[2])
            slots, cow = res[0], res[1]
            if cow:
                cache.copy_blocks(kpool, vpool, H, bs, D, w.num_blocks, cow)
                if phase == "step":
                    st.step_pairs.extend(cow)
            rows = w.tok_rows[s][start:start + n]
            cache.cache_write(kpool, vpool, H, bs, D, w.num_blocks,
                              w.k_tok[rows], w.v_tok[rows], slots)
            if phase == "step":
                st.step_slots.extend(slots)
                st.step_rows.extend(rows.tolist())
        elif op[0] == "free":
            res = a.free_seq(op[1])
        else:
            raise ValueError(op)
        if phase == "setup":
            st.setup_results.append(res)
    st.kpool, st.vpool = kpool, vpool
    return st


def max_blocks(w):
    return max(-(-len(r) // w.block_size) for r in w.tok_rows.values())


def decode_tables(w, st):
    return st.alloc.block_tables(w.decode_seqs, max_blocks(w))


def oracle_decode(w, st, pairs=None):
    tables, lens = decode_tables(w, st)
    q = attention.stored_to_f64(w.q_dec, w.dtype)
    return attention.decode(q, st.kpool, st.vpool, w.dtype, w.num_kv_heads, w.block_size,
                            w.head_dim, tables, lens, w.scale, pairs=pairs)


def oracle_prefill(w, st, rows=None):
    tables, lens = st.alloc.block_tables(w.prefill_seqs, max_blocks(w))
    qs = np.concatenate([[0], np.cumsum(w.chunk_len)]).astype(np.int64)
    q = attention.stored_to_f64(w.q_pre, w.dtype)
    return attention.prefill(q, st.kpool, st.vpool, w.dtype, w.num_kv_heads, w.block_size,
                             w.head_dim, tables, lens, qs, w.scale, rows=rows)


def logical_kv(w, s, head):
    """A sequence's K/V straight from the generated rows (no pool, no table)."""
    rows = w.tok_rows[s]
    return (attention.stored_to_f64(w.k_tok[rows, head, :], w.dtype),
            attention.stored_to_f64(w.v_tok[rows, head, :], w.dtype))
