"""Oracle O4: attention over a paged KV cache, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the method computes.  The pages are explicit that paging changes only
where K and V live, not what attention computes: the speed-up comes from
memory plumbing alone, with no compression or quantisation ([studynote 223]
three-line summary, item 3; section V: the model is not touched), and a
request sees its KV as one logically contiguous sequence even though the
physical blocks are scattered ([studynote 223] section II figure; [ch.09]
"해법: 페이지처럼 나눠 담기").  So the result is ordinary attention over the
gathered context, and that is what is written here:

  1. gather: for positions p = 0..L-1, read block table[p // bs], offset
     p mod bs, from the pool (the layout of ``oracle.cache``), and upcast the
     stored fp32 or bf16 value exactly to fp64;
  2. logits z_p = scale * <q, k_p>;
  3. weights w = exp(z - max z) / sum exp(z - max z);
  4. out = sum_p w_p v_p.

The pages never write the formula; the readings taken:
softmax(q K^T * scale) V with scale given by the caller (1/sqrt(D) in every
workload); query head h reads kv head h // G with G = Hq / Hkv (grouped-query
attention); a decode context length L includes the newly written token; a
prefill chunk's C queries are the last C positions of its context, and query
i (position L - C + i) sees keys 0..L-C+i inclusive.

No online softmax, no partitions, no blocking: one plain pass per (sequence,
head), which is a different algorithm from the kernels'.
"""

import numpy as np

from . import cache


def stored_to_f64(values, dtype):
    """Exact fp64 value of stored fp32 numbers or bf16 bit patterns (uint16)."""
    if dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(values, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def gather(kpool, vpool, dtype, H, bs, D, table, L, head):
    """K and V of one sequence and kv head as contiguous [L, D] fp64 arrays."""
    pos = np.arange(L)[:, None]
    blocks = np.asarray(table, dtype=np.int64)[pos // bs]
    if L and blocks.min() < 0:
        raise ValueError("block table has no entry for a needed position")
    dims = np.arange(D)[None, :]
    kidx = cache.k_index(H, bs, D, blocks, head, pos % bs, dims)
    vidx = cache.v_index(H, bs, D, blocks, head, pos % bs, dims)
    return stored_to_f64(kpool[kidx], dtype), stored_to_f64(vpool[vidx], dtype)


def attend(q, K, V, scale):
    """softmax(K q * scale)^T V for one query vector.  Returns (out, weights)."""
    z = (K @ q) * scale
    z = z - z.max()
    e = np.exp(z)
    w = e / e.sum()
    return w @ V, w


def decode(q, kpool, vpool, dtype, H, bs, D, tables, lens, scale, pairs=None):
    """One query token per sequence.

    q: [B, Hq, D] fp64 (the stored query values, upcast).  Returns
    out [B, Hq, D] fp64.  If `pairs` is a list of (s, h), only those rows are
    computed (the others stay NaN) -- used to spot-check large workloads.
    """
    B, Hq, _ = q.shape
    if Hq % H:
        raise ValueError("query heads must be a multiple of kv heads")
    G = Hq // H
    out = np.full((B, Hq, D), np.nan)
    want = None if pairs is None else set((int(s), int(h)) for s, h in pairs)
    for s in range(B):
        L = int(lens[s])
        if L < 1:
            raise ValueError("context length must be >= 1")
        heads = [h for h in range(Hq) if want is None or (s, h) in want]
        for g in sorted(set(h // G for h in heads)):
            K, V = gather(kpool, vpool, dtype, H, bs, D, tables[s], L, g)
            for h in heads:
                if h // G == g:
                    out[s, h], _ = attend(q[s, h], K, V, scale)
    return out


def decode_weights(q_vec, kpool, vpool, dtype, H, bs, D, table, L, head, scale):
    """The softmax weights of one (sequence, query head) -- for pin checks."""
    K, V = gather(kpool, vpool, dtype, H, bs, D, table, L, head)
    return attend(q_vec, K, V, scale)[1]


def prefill(q, kpool, vpool, dtype, H, bs, D, tables, lens, query_start, scale, rows=None):
    """Causal attention for prefill chunks.

    q: [T, Hq, D] fp64, chunk c owning rows query_start[c]..query_start[c+1]-1.
    Chunk c's context length lens[c] counts the chunk's own tokens, which are
    its last C = query_start[c+1]-query_start[c] positions; query i sits at
    position lens[c] - C + i and sees keys 0..lens[c]-C+i.  Returns out [T, Hq, D]
    (rows not listed in `rows`, a list of (t, h), stay NaN when `rows` is given).
    """
    T, Hq, _ = q.shape
    G = Hq // H
    out = np.full((T, Hq, D), np.nan)
    want = None if rows is None else set((int(t), int(h)) for t, h in rows)
    nchunks = len(query_start) - 1
    for c in range(nchunks):
        q0, q1 = int(query_start[c]), int(query_start[c + 1])
        C = q1 - q0
        L = int(lens[c])
        if C < 0 or L < C:
            raise ValueError("a chunk's context must hold its own queries")
        for g in range(H):
            heads = [h for h in range(g * G, (g + 1) * G)]
            if want is not None and not any((t, h) in want for t in range(q0, q1) for h in heads):
                continue
            K, V = gather(kpool, vpool, dtype, H, bs, D, tables[c], L, g)
            for i in range(C):
                P = L - C + i
                for h in heads:
                    if want is None or (q0 + i, h) in want:
                        out[q0 + i, h], _ = attend(q[q0 + i, h], K[:P + 1], V[:P + 1], scale)
    return out
