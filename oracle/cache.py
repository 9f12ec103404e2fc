"""Oracles O2 and O3: the pool layout, cache write and copy-on-write block copy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix what a slot is -- a token position inside one fixed-size
physical block ([velog] "주요 구성 요소": physical blocks are pages of e.g.
16-64 tokens; [ch.09] "해법": blocks are fixed size) -- but not how the bytes of a
block are arranged.  The arrangement is a design choice of the library; this
module writes that choice out independently, from its statement:

  K pool, element (block b, kv head g, token offset o, channel d) lives at
      (b * H + g) * bs * D + ((d // W) * bs + o) * W + d % W
                                 (groups of W channels, W = 32 when D is a
                                  multiple of 32, else W = D; within a group,
                                  one token row of W channels)
  V pool, the same element lives at
      ((b * H + g) * D + d) * bs + o          (one channel row of bs tokens)

with H kv heads, bs tokens per block and D channels.  One (block, head) tile
is contiguous in both pools.  Pools are flat 1-D numpy arrays holding the
stored values: float32 for fp32 caches, uint16 bit patterns for bf16 caches.

Copy-on-write ([studynote 223] section II, copy-on-write paragraph; [velog]
"메모리 공유 (Copy-on-Write)"): a block that several requests share is copied
to a fresh block before one of them writes into it; every head and every slot
of the block, in both pools, is copied.
"""

import numpy as np


def k_index(H, bs, D, block, head, offset, dim):
    W = 32 if D % 32 == 0 else D
    return (block * H + head) * bs * D + ((dim // W) * bs + offset) * W + dim % W


def v_index(H, bs, D, block, head, offset, dim):
    return ((block * H + head) * D + dim) * bs + offset


def pool_elems(num_blocks, H, bs, D):
    return num_blocks * H * bs * D


def new_pool(num_blocks, H, bs, D, dtype, fill_bits):
    """A pool whose every element holds the bit pattern `fill_bits` (a NaN sentinel)."""
    n = pool_elems(num_blocks, H, bs, D)
    if dtype == "bf16":
        return np.full(n, fill_bits, dtype=np.uint16)
    if dtype == "f32":
        return np.full(n, fill_bits, dtype=np.uint32).view(np.float32)
    raise ValueError(dtype)


def cache_write(kpool, vpool, H, bs, D, num_blocks, k_new, v_new, slots, batch=4096):
    """Store token t's K/V rows (shape [T, H, D]) at cache slot slots[t].

    Negative slots are padding and write nothing.  A slot at or beyond
    num_blocks * bs is an invalid input and raises.  Tokens are handled in
    batches only to bound the size of the index arrays; every element's index
    is the layout formula above, broadcast over (token, head, channel).
    """
    slots = np.asarray(slots, dtype=np.int64)
    T = len(slots)
    assert k_new.shape == (T, H, D) and v_new.shape == (T, H, D)
    if T and slots.max() >= num_blocks * bs:
        raise ValueError("a slot lies outside the pool")
    heads = np.arange(H)[None, :, None]
    dims = np.arange(D)[None, None, :]
    for t0 in range(0, T, batch):
        sl = slots[t0:t0 + batch]
        keep = sl >= 0
        sl = sl[keep]
        block = (sl // bs)[:, None, None]
        offset = (sl % bs)[:, None, None]
        kpool[k_index(H, bs, D, block, heads, offset, dims)] = k_new[t0:t0 + batch][keep]
        vpool[v_index(H, bs, D, block, heads, offset, dims)] = v_new[t0:t0 + batch][keep]


def check_pairs(pairs, num_blocks):
    """Valid copy lists: ids in range, destinations distinct, no destination
    is also a source (the order of copies must not matter)."""
    srcs = [int(s) for s, _ in pairs]
    dsts = [int(d) for _, d in pairs]
    for b in srcs + dsts:
        if not (0 <= b < num_blocks):
            raise ValueError(f"block {b} outside the pool")
    if len(set(dsts)) != len(dsts):
        raise ValueError("destination blocks repeat")
    if set(dsts) & set(srcs):
        raise ValueError("a destination block is also a source")


def copy_blocks(kpool, vpool, H, bs, D, num_blocks, pairs):
    """pool[dst] := pool[src] for each (src, dst), all heads and slots, K and V."""
    check_pairs(pairs, num_blocks)
    for src, dst in pairs:
        for g in range(H):
            for o in range(bs):
                dims = np.arange(D)
                kpool[k_index(H, bs, D, dst, g, o, dims)] = kpool[k_index(H, bs, D, src, g, o, dims)]
                vpool[v_index(H, bs, D, dst, g, o, dims)] = vpool[v_index(H, bs, D, src, g, o, dims)]

