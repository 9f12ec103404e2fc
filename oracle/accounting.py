"""Fragmentation and capacity arithmetic -- TEST INFRASTRUCTURE ONLY.

  [velog] "기존 KV 캐시의 문제점": reserving a maximum length of 2048 tokens for
      a request that produces 500 wastes 1548 tokens' worth of memory.
  [studynote 223] section IV, checklist item 1: a 128-token block holding 10
      tokens leaves 118 slots empty; 1-token blocks waste nothing but cost
      table overhead.
  [ch.09] "해법": with paging, internal waste is limited to the last block.
  [studynote 528] section IV, capacity planning: HBM needed = max model
      length x batch x KV bytes (per token).
"""


def contiguous_waste(reserved_tokens, used_tokens):
    """Slots left empty when a request reserves a fixed maximum up front."""
    if used_tokens > reserved_tokens:
        raise ValueError("used more than reserved")
    return reserved_tokens - used_tokens


def paged_waste(length, block_size):
    """Empty slots in a request's blocks: only the last block can have any."""
    blocks = -(-length // block_size)
    return blocks * block_size - length


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, bytes_per_elem):
    """Bytes one token occupies in the cache: a K row and a V row of every kv
    head, in every layer ([studynote 528] section IV: the per-token KV bytes
    of the capacity formula)."""
    return 2 * num_layers * num_kv_heads * head_dim * bytes_per_elem


def capacity_bytes(max_model_len, batch, kv_bytes_per_tok):
    """HBM a contiguous cache reserves for `batch` requests of up to
    max_model_len tokens each ([studynote 528] section IV, capacity planning:
    max-model-len x batch size x KV bytes per token)."""
    return max_model_len * batch * kv_bytes_per_tok
