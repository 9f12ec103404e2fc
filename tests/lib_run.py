"""Drive the library (C ABI through the binding) through a workload.

Product path only: the library's C++ allocator builds the tables and slots,
its kernels write the cache, copy blocks and decode.  Nothing here touches
``oracle``.
"""

import numpy as np
import torch

import paged_kv_cache_424_amd as pa


def torch_stored(arr, dtype):
    """Workload stored values (uint16 bf16 bits or float32) as a CPU torch tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))


def fill_pool(n_elems, dtype, fill_bits, device):
    if dtype == "bf16":
        t = torch.full((n_elems,), fill_bits - (1 << 16) if fill_bits >= (1 << 15) else fill_bits,
                       dtype=torch.int16, device=device)
        return t.view(torch.bfloat16)
    t = torch.full((n_elems,), fill_bits - (1 << 32) if fill_bits >= (1 << 31) else fill_bits,
                   dtype=torch.int32, device=device)
    return t.view(torch.float32)


class LibState:
    pass


def run_script(w, alloc):
    """Run the op script on the library allocator; return per-phase write lists.

    Setup writes of a content-addressed workload are kept in script order,
    one entry per op: a block freed and later evicted is written again by its
    new owner, and the last write must win."""
    writes = {"setup": [], "step": []}     # (slots, rows)
    pairs = {"setup": [], "step": []}
    if w.prefix_cache:
        pa.pa_allocator_enable_prefix_cache(alloc)
    for phase, op in w.script:
        if op[0] == "create":
            pa.pa_seq_create(alloc)
        elif op[0] == "fork":
            pa.pa_seq_fork(alloc, op[1])
        elif op[0] == "cow":
            pr = pa.pa_seq_cow_block(alloc, op[1], op[2])
            if pr is not None:
                pairs[phase].append(pr)
        elif op[0] == "append":
            s, n = op[1], op[2]
            start = pa.pa_seq_length(alloc, s)
            slots, cow = pa.pa_seq_append_slots(alloc, s, n)
            pairs[phase].extend(cow)
            writes[phase].append((slots, w.tok_rows[s][start:start + n]))
        elif op[0] == "append_tokens":
            s, toks = op[1], op[2]
            start = pa.pa_seq_length(alloc, s)
            slots, cow, _ = pa.pa_seq_append_tokens(alloc, s, toks)
            pairs[phase].extend(cow)
            writes[phase].append((slots, w.tok_rows[s][start:start + len(toks)]))
        elif op[0] == "free":
            pa.pa_seq_free(alloc, op[1])
        else:
            raise ValueError(op)
    return writes, pairs


def _write(st, w, items, device):
    if not items:
        return np.empty(0, dtype=np.int64), np.empty(0, dtype=np.int64)
    slots = np.concatenate([s for s, _ in items]).astype(np.int64)
    rows = np.concatenate([r for _, r in items])
    k = torch_stored(w.k_tok[rows], w.dtype).to(device)
    v = torch_stored(w.v_tok[rows], w.dtype).to(device)
    sl = torch.from_numpy(slots).to(device)
    pa.pa_cache_write(st.kc, st.vc, st.desc, k, v, sl)
    return slots, rows


def build(w, device="cuda", run_step=True):
    """Allocate NaN-filled pools, run setup writes, then the step: copy-on-write
    copies first, then one cache write of every step token."""
    st = LibState()
    st.desc = pa.cache_desc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
    st.alloc = pa.pa_allocator_create(w.num_blocks, w.block_size, w.free_order)
    writes, pairs = run_script(w, st.alloc)
    st.step_pairs = pairs["step"]
    n = pa.pa_cache_pool_bytes(st.desc) // (2 if w.dtype == "bf16" else 4)
    st.kc = fill_pool(n, w.dtype, w.fill_bits, device)
    st.vc = fill_pool(n, w.dtype, w.fill_bits, device)
    # setup: the order of setup copies and writes follows the script's phases
    # (a prefix is written before it is shared, so copies of it see its data)
    if pairs["setup"]:
        raise NotImplementedError("copy-on-write during setup")
    st.setup_slots = (np.concatenate([sl for sl, _ in writes["setup"]]) if writes["setup"]
                      else np.empty(0, dtype=np.int64))
    if w.prefix_cache:
        for item in writes["setup"]:
            _write(st, w, [item], device)
    else:
        _write(st, w, writes["setup"], device)
    st.step_writes = writes["step"]          # (slots, rows) of the step, in script order
    if run_step:
        if st.step_pairs:
            pa.pa_copy_blocks(st.kc, st.vc, st.desc, st.step_pairs)
        st.step_slots, st.step_rows = _write(st, w, writes["step"], device)
    st.max_blocks = max(-(-len(r) // w.block_size) for r in w.tok_rows.values())
    tables, lens = pa.pa_build_block_tables(st.alloc, w.decode_seqs, st.max_blocks)
    st.tables_host, st.lens_host = tables, lens
    st.tables = torch.from_numpy(np.ascontiguousarray(tables)).to(device)
    st.lens = torch.from_numpy(np.ascontiguousarray(lens)).to(device)
    st.q = torch_stored(w.q_dec, w.dtype).to(device) if w.q_dec is not None else None
    st.max_ctx = int(lens.max()) if len(lens) else 1
    return st


def decode(w, st, partition_size=0, out_dtype=torch.float32, max_ctx=None, lens=None, q=None,
           tables=None):
    q = st.q if q is None else q
    lens = st.lens if lens is None else lens
    tables = st.tables if tables is None else tables
    max_ctx = st.max_ctx if max_ctx is None else max_ctx
    B, Hq, D = q.shape
    out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    wsb = pa.pa_decode_workspace_bytes(B, Hq, D, max_ctx, partition_size)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device) if wsb else None
    pa.pa_decode(out, q, st.kc, st.vc, st.desc, tables, lens, max_ctx, w.scale,
                 partition_size=partition_size, workspace=ws)
    return out


def pool_bits(t, dtype):
    """Device pool -> host numpy array of its raw bits (uint16 or uint32)."""
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def prefill(w, st, out_dtype=torch.float32, lens=None, qsl=None, max_query_len=None):
    """Run pa_prefill for the workload's prefill chunks (after build())."""
    dev = st.kc.device
    tables, clens = pa.pa_build_block_tables(st.alloc, w.prefill_seqs, st.max_blocks)
    tab = torch.from_numpy(np.ascontiguousarray(tables)).to(dev)
    lens = torch.from_numpy(np.ascontiguousarray(clens)).to(dev) if lens is None else lens
    if qsl is None:
        qsl = torch.from_numpy(np.concatenate([[0], np.cumsum(w.chunk_len)]).astype(np.int32)).to(dev)
    q = torch_stored(w.q_pre, w.dtype).to(dev)
    out = torch.full((q.shape[0], q.shape[1], q.shape[2]), float("inf"), dtype=out_dtype, device=dev)
    mq = max(w.chunk_len) if max_query_len is None else max_query_len
    pa.pa_prefill(out, q, st.kc, st.vc, st.desc, tab, lens, qsl, mq, w.scale)
    return out
