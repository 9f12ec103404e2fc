"""The five workloads, as seeded synthetic inputs.

Recipe: numpy ``default_rng(seed)`` (PCG64), seed =
the workload's number 1..5 unless overridden; values N(0,1) drawn as float32;
bf16 caches and queries are the float32 draws rounded to nearest-even by torch
on the CPU.  Draw order: lengths, then the pool's initial free-block
permutation, then queries, then keys, then values.  A sequence's K/V are drawn
for every position it holds, including the token that the decode step writes
(its last position); a prefill chunk's K/V cover its whole context including
its own tokens.

Each workload carries an allocator op script (create / fork / append / cow)
tagged with the phase it belongs to: "setup" ops build the cache before the
timed step, "step" ops are the appends whose slots the step's cache write
fills.  Both the library's allocator and the oracle's run the same script.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

NAN_FILL_BF16 = 0x7FC1        # quiet NaN, payload 1: marks a never-written bf16 slot
NAN_FILL_F32 = 0x7FC00001     # quiet NaN, payload 1: marks a never-written fp32 slot

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")


def round_to_bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns (round to nearest even, via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normals(rng, shape, dtype, mult=1.0, rows_per_draw=1 << 16):
    """N(0,1) * mult in the stored dtype; drawn in row batches to bound memory."""
    shape = tuple(int(s) for s in shape)
    n0 = shape[0]
    rest = shape[1:]
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for r0 in range(0, n0, rows_per_draw):
        r1 = min(n0, r0 + rows_per_draw)
        x = rng.standard_normal((r1 - r0,) + rest, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        out[r0:r1] = round_to_bf16_bits(x) if dtype == "bf16" else x
    return out


def _ceil_div(a, b):
    return -(-a // b)


@dataclass
class Workload:
    name: str
    dtype: str                  # "f32" or "bf16" (cache and query storage)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray      # int32 [num_blocks], initial free list
    scale: float
    script: list                # [(phase, op)], op as in oracle.allocator.run_script
    # per allocator sequence id: the row of k_tok/v_tok holding each position
    tok_rows: dict
    k_tok: np.ndarray           # [rows, Hkv, D] stored values
    v_tok: np.ndarray
    decode_seqs: list = field(default_factory=list)
    q_dec: np.ndarray = None    # [len(decode_seqs), Hq, D] stored values
    prefill_seqs: list = field(default_factory=list)
    chunk_len: list = field(default_factory=list)   # queries per chunk
    q_pre: np.ndarray = None    # [sum(chunk_len), Hq, D] stored values
    partition_size: int = 512
    prefix_cache: bool = False  # the allocator finds reusable blocks by content
    note: str = ""

    @property
    def fill_bits(self):
        return NAN_FILL_BF16 if self.dtype == "bf16" else NAN_FILL_F32

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    def seq_len(self, s):
        return len(self.tok_rows[s])


def c1_tiny(seed=1):
    """Tiny fp32 decode: lengths {5,17,33,48}, 8/8 heads, D 64, bs 16, pool of 32."""
    rng = np.random.default_rng(seed)
    return _decode_batch_from(rng, "c1", "f32", [5, 17, 33, 48], 8, 8, 64, 16, num_blocks=32,
                              note="tiny paged decode, fp32")


def c2_llama8b(seed=2, batch=64, lo=128, hi=2048):
    """Llama-3-8B-shaped decode: B 64, L ~ U{128..2048}, 32/8 heads, D 128, bs 16."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=batch)
    return _decode_batch_from(rng, "c2", "bf16", lens, 32, 8, 128, 16,
                              note=f"Llama-3-8B-shaped decode, B {batch}, L~U{{{lo}..{hi}}}")


def _decode_batch_from(rng, name, dtype, lens, Hq, Hkv, D, bs, k_mult=1.0, num_blocks=None,
                       partition_size=512, note=""):
    """Independent sequences: context written at setup, one new token per step.

    The pool holds the blocks the sequences need plus 10 % free, unless
    num_blocks is given."""
    lens = [int(x) for x in lens]
    need = sum(_ceil_div(L, bs) for L in lens)
    N = num_blocks if num_blocks is not None else need + _ceil_div(need, 10)
    free_order = rng.permutation(N).astype(np.int32)
    B = len(lens)
    q = _normals(rng, (B, Hq, D), dtype)
    total = sum(lens)
    k = _normals(rng, (total, Hkv, D), dtype, mult=k_mult)
    v = _normals(rng, (total, Hkv, D), dtype)
    script = []
    tok_rows = {}
    row = 0
    for s in range(B):
        script.append(("setup", ("create",)))
        tok_rows[s] = np.arange(row, row + lens[s])
        row += lens[s]
    for s in range(B):
        if lens[s] > 1:
            script.append(("setup", ("append", s, lens[s] - 1)))
    for s in range(B):
        script.append(("step", ("append", s, 1)))
    return Workload(name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=bs, num_blocks=N, free_order=free_order,
                    scale=1.0 / float(np.sqrt(D)), script=script, tok_rows=tok_rows,
                    k_tok=k, v_tok=v, decode_seqs=list(range(B)), q_dec=q,
                    partition_size=partition_size, note=note)


def decode_batch(seed, lens, name="decode", Hq=32, Hkv=8, D=128, bs=16, dtype="bf16"):
    """A plain decode batch of the given context lengths (Llama-3-8B-shaped
    heads by default), drawn as the decode workloads are."""
    rng = np.random.default_rng(seed)
    return _decode_batch_from(rng, name, dtype, list(lens), Hq, Hkv, D, bs,
                              note=f"decode batch of {len(lens)} sequences")


def c3_long(seed=3, batch=8, length=32768):
    """Long-context split-K decode: B 8 x 32768, 32/8 heads, D 128, bs 16, k x3."""
    rng = np.random.default_rng(seed)
    lens = [length] * batch
    return _decode_batch_from(rng, "c3", "bf16", lens, 32, 8, 128, 16, k_mult=3.0,
                              note=f"long-context decode, B {batch} x {length}, k scaled x3")


def c4_shared_prefix(seed=4, batch=32, prefix=1016, suffix_hi=512, privatize_last_shared=False):
    """Shared prefix + copy-on-write: 32 sequences share 64 blocks of a prompt.

    prefix=1016 leaves the last shared block half full, so each sequence's
    first append triggers a real copy-on-write (the last holder writes in
    place).  prefix=1024 fills the 64 blocks exactly; with
    privatize_last_shared=True each sequence then explicitly asks for a private
    copy of logical block 63 before its suffix is written.
    Every sequence then appends its private suffix (U{0..512} tokens) and one
    decode token; all of that happens in the step.
    """
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 32, 8, 128, 16
    suffix = [int(x) for x in rng.integers(0, suffix_hi + 1, size=batch)]
    lens = [prefix + sfx + 1 for sfx in suffix]
    shared_blocks = _ceil_div(prefix, bs)
    private = sum(_ceil_div(L, bs) - (prefix // bs) for L in lens)
    need = shared_blocks + private + batch     # + one copy-on-write block per sequence
    N = need + _ceil_div(need, 10)
    free_order = rng.permutation(N).astype(np.int32)
    q = _normals(rng, (batch, Hq, D), "bf16")
    total = prefix + sum(sfx + 1 for sfx in suffix)
    k = _normals(rng, (total, Hkv, D), "bf16")
    v = _normals(rng, (total, Hkv, D), "bf16")
    script = [("setup", ("create",)), ("setup", ("append", 0, prefix))]
    for _ in range(batch - 1):
        script.append(("setup", ("fork", 0)))
    tok_rows = {}
    row = prefix
    for s in range(batch):
        n_own = suffix[s] + 1
        tok_rows[s] = np.concatenate([np.arange(prefix), np.arange(row, row + n_own)])
        row += n_own
    for s in range(batch):
        if privatize_last_shared:
            script.append(("step", ("cow", s, shared_blocks - 1)))
        script.append(("step", ("append", s, suffix[s] + 1)))
    name = "c4a" if privatize_last_shared else "c4"
    return Workload(name=name, dtype="bf16", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=bs, num_blocks=N, free_order=free_order,
                    scale=1.0 / float(np.sqrt(D)), script=script, tok_rows=tok_rows,
                    k_tok=k, v_tok=v, decode_seqs=list(range(batch)), q_dec=q,
                    note=f"shared {prefix}-token prefix, {batch} sequences, suffix U{{0..{suffix_hi}}}")


def c5_mixed(seed=5, n_decode=240, n_chunks=16, chunk=256, ctx_lo=256, ctx_hi=4096,
             median=1024, sigma=1.0, dec_lo=64, dec_hi=8192):
    """Mixed continuous-batching step at 70B-shaped heads: 64/8 heads, D 128, bs 32.

    n_decode sequences with lognormal context lengths (median 1024, sigma 1 in
    natural-log units, clipped to [64, 8192]) decode one token each; n_chunks
    prefill chunks of `chunk` queries attend causally over contexts
    U{256..4096} that end with the chunk's own tokens.
    """
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 64, 8, 128, 32
    xi = rng.standard_normal(n_decode)
    dlens = [int(x) for x in np.clip(np.rint(np.exp(np.log(median) + sigma * xi)), dec_lo, dec_hi)]
    clens = [int(x) for x in rng.integers(ctx_lo, ctx_hi + 1, size=n_chunks)]
    need = sum(_ceil_div(L, bs) for L in dlens + clens)
    N = need + _ceil_div(need, 10)
    free_order = rng.permutation(N).astype(np.int32)
    q_dec = _normals(rng, (n_decode, Hq, D), "bf16")
    q_pre = _normals(rng, (n_chunks * chunk, Hq, D), "bf16")
    total = sum(dlens) + sum(clens)
    k = _normals(rng, (total, Hkv, D), "bf16")
    v = _normals(rng, (total, Hkv, D), "bf16")
    script = []
    tok_rows = {}
    row = 0
    all_lens = dlens + clens
    for s, L in enumerate(all_lens):
        script.append(("setup", ("create",)))
        tok_rows[s] = np.arange(row, row + L)
        row += L
    for s in range(n_decode):
        if dlens[s] > 1:
            script.append(("setup", ("append", s, dlens[s] - 1)))
    for c in range(n_chunks):
        s = n_decode + c
        if clens[c] > chunk:
            script.append(("setup", ("append", s, clens[c] - chunk)))
    for s in range(n_decode):
        script.append(("step", ("append", s, 1)))
    for c in range(n_chunks):
        script.append(("step", ("append", n_decode + c, chunk)))
    return Workload(name="c5", dtype="bf16", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=bs, num_blocks=N, free_order=free_order,
                    scale=1.0 / float(np.sqrt(D)), script=script, tok_rows=tok_rows,
                    k_tok=k, v_tok=v, decode_seqs=list(range(n_decode)), q_dec=q_dec,
                    prefill_seqs=list(range(n_decode, n_decode + n_chunks)),
                    chunk_len=[chunk] * n_chunks, q_pre=q_pre,
                    note=f"mixed step: {n_decode} decodes + {n_chunks}x{chunk} prefill queries")


def c4_prompt_cache(seed=44, batch=32, n_prompts=4, prompt_lo=256, prompt_hi=1024, suffix_hi=512,
                    n_warm=8, vocab=32000, bs=16, pool_margin=0.10):
    """Shared system prompts found by content (automatic prefix caching), no forks.

    Each of `batch` requests is one of `n_prompts` prompts (lengths
    U{prompt_lo..prompt_hi}) followed by a private suffix of U{0..suffix_hi}
    token ids and one decode token.  Before them, `n_warm` earlier requests of
    the same form run and finish one after another, so the batch finds some
    prompts only among freed blocks and its fresh blocks may evict them.

    Token ids are U{0..vocab-1}, except that prompt i starts with id i, so two
    prompts never coincide by chance.  A token's K/V depends on every token up
    to it: rows of k_tok/v_tok are the nodes of the trie of all requests'
    token lists (numbered in order of first appearance) and are drawn once per
    node, so equal prefixes hold equal K/V.

    Setup: each request is created and appends all its tokens but the last
    through the content-addressed append; warm requests are then freed.  Step:
    every batch request appends its decode token.  The pool holds the blocks
    the batch needs when every prompt is shared, plus `pool_margin`: enough
    for the batch, too few to keep every block the warm requests left, so
    fresh blocks evict cached ones.
    Draw order: prompt lengths and ids, request prompts and suffix lengths,
    suffix ids, the free-block permutation, queries, keys, values.
    """
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = 32, 8, 128
    plen = [int(x) for x in rng.integers(prompt_lo, prompt_hi + 1, size=n_prompts)]
    prompts = []
    for i, L in enumerate(plen):
        ids = rng.integers(0, vocab, size=L)
        ids[0] = i
        prompts.append([int(x) for x in ids])
    n_req = n_warm + batch
    which = [int(x) for x in rng.integers(0, n_prompts, size=n_req)]
    sfx = [int(x) for x in rng.integers(0, suffix_hi + 1, size=n_req)]
    token_ids = {}
    for r in range(n_req):
        own = [int(x) for x in rng.integers(0, vocab, size=sfx[r] + 1)]
        token_ids[r] = prompts[which[r]] + own
    # trie of token lists -> K/V row per node
    node = {}
    tok_rows = {}
    for r in range(n_req):
        parent = -1
        rows = []
        for t in token_ids[r]:
            key = (parent, t)
            if key not in node:
                node[key] = len(node)
            parent = node[key]
            rows.append(parent)
        tok_rows[r] = np.asarray(rows, dtype=np.int64)
    live = list(range(n_warm, n_req))
    # blocks the batch holds: each prompt's full blocks once, the rest per request
    # (equal suffixes could only lower this)
    need = sum(plen[p] // bs for p in sorted({which[r] for r in live}))
    need += sum(_ceil_div(len(token_ids[r]), bs) - plen[which[r]] // bs for r in live)
    N = need + _ceil_div(int(need * pool_margin * 100), 100)
    free_order = rng.permutation(N).astype(np.int32)
    q = _normals(rng, (batch, Hq, D), "bf16")
    k = _normals(rng, (len(node), Hkv, D), "bf16")
    v = _normals(rng, (len(node), Hkv, D), "bf16")
    script = []
    for r in range(n_req):
        script.append(("setup", ("create",)))
        script.append(("setup", ("append_tokens", r, token_ids[r][:-1])))
        if r < n_warm:
            script.append(("setup", ("free", r)))
    for r in live:
        script.append(("step", ("append_tokens", r, token_ids[r][-1:])))
    return Workload(name="c4p", dtype="bf16", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=bs, num_blocks=N, free_order=free_order,
                    scale=1.0 / float(np.sqrt(D)), script=script, tok_rows=tok_rows,
                    k_tok=k, v_tok=v, decode_seqs=live, q_dec=q, prefix_cache=True,
                    note=f"{batch} requests over {n_prompts} prompts U{{{prompt_lo}..{prompt_hi}}} "
                         f"found by content, suffix U{{0..{suffix_hi}}}, {n_warm} earlier requests freed")


def make(name, small=False):
    """Full-size workload by name, or its scaled-down parity variant."""
    if name == "c1":
        return c1_tiny()
    if name == "c2":
        return c2_llama8b(batch=12) if small else c2_llama8b()
    if name == "c3":
        return c3_long(batch=2, length=3000) if small else c3_long()
    if name == "c4":
        return c4_shared_prefix(batch=6, suffix_hi=80) if small else c4_shared_prefix()
    if name == "c4a":
        return (c4_shared_prefix(batch=6, prefix=1024, suffix_hi=80, privatize_last_shared=True)
                if small else c4_shared_prefix(prefix=1024, privatize_last_shared=True))
    if name == "c4p":
        return (c4_prompt_cache(batch=6, n_prompts=2, prompt_lo=20, prompt_hi=90, suffix_hi=40,
                                n_warm=3) if small else c4_prompt_cache())
    if name == "c5":
        return (c5_mixed(n_decode=20, n_chunks=3, chunk=64, ctx_lo=64, ctx_hi=700, dec_hi=2000)
                if small else c5_mixed())
    raise ValueError(name)


def relayout(w, block_size=None, free_seed=None, duplicate_shared=False):
    """The same logical sequences (same K/V rows and queries) in another pool.

    block_size: store them with another block size.  free_seed: start from a
    different free-block permutation, i.e. relabel every physical block.
    duplicate_shared: give every sequence private copies of everything it
    holds (no forks, no copy-on-write), as a fully duplicated layout.
    Scripts keep the same setup/step split: each sequence's last position is
    written in the step; prefill chunks keep their chunk in the step.
    """
    bs = block_size or w.block_size
    seqs = sorted(w.tok_rows)
    if not duplicate_shared and block_size is None:
        script = list(w.script)
    else:
        script = [("setup", ("create",)) for _ in seqs]
        chunk_of = dict(zip(w.prefill_seqs, w.chunk_len))
        for s in seqs:
            L = len(w.tok_rows[s])
            own = chunk_of.get(s, 1)
            if L - own > 0:
                script.append(("setup", ("append", s, L - own)))
        for s in seqs:
            script.append(("step", ("append", s, chunk_of.get(s, 1))))
    if duplicate_shared or block_size is not None:
        need = sum(_ceil_div(len(w.tok_rows[s]), bs) for s in seqs)
        N = need + _ceil_div(need, 10)
    else:
        N = w.num_blocks
    rng = np.random.default_rng(free_seed if free_seed is not None else 1000 + bs)
    free_order = rng.permutation(N).astype(np.int32)
    return Workload(name=w.name + "-relayout", dtype=w.dtype, num_q_heads=w.num_q_heads,
                    num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, block_size=bs,
                    num_blocks=N, free_order=free_order, scale=w.scale, script=script,
                    tok_rows=w.tok_rows, k_tok=w.k_tok, v_tok=w.v_tok,
                    decode_seqs=w.decode_seqs, q_dec=w.q_dec, prefill_seqs=w.prefill_seqs,
                    chunk_len=w.chunk_len, q_pre=w.q_pre, partition_size=w.partition_size,
                    note=w.note + " (relayout)")


def subset(w, seqs):
    """A workload holding only the listed decode sequences (same K/V rows and
    queries), each stored privately in a fresh pool -- a bounded sample of w."""
    seqs = list(seqs)
    idx = [w.decode_seqs.index(s) for s in seqs]
    tok_rows = {i: w.tok_rows[s] for i, s in enumerate(seqs)}
    sub = Workload(name=w.name + "-subset", dtype=w.dtype, num_q_heads=w.num_q_heads,
                   num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, block_size=w.block_size,
                   num_blocks=1, free_order=np.zeros(1, dtype=np.int32), scale=w.scale,
                   script=[], tok_rows=tok_rows, k_tok=w.k_tok, v_tok=w.v_tok,
                   decode_seqs=list(range(len(seqs))), q_dec=w.q_dec[idx],
                   partition_size=w.partition_size, note=w.note + f" (sequences {seqs})")
    return relayout(sub, duplicate_shared=True, free_seed=7)
