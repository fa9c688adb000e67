"""Byte accounting for the paged KV cache.

* ``kv_cache_bytes``: the KV memory estimate of "KV cache, PagedAttention"
  (aiwiki.vn), paragraph on the memory formula: two tensors (K and V) times
  layers times tokens times KV heads times head size times bytes per element.
* ``blocks_needed``: a sequence of L tokens holds ceil(L/B) blocks
  ("PagedAttention (vLLM)", troisinh.com, section "Cơ chế Block Table").
* ``decode_algorithmic_bytes``: the bytes one decode (or multi-token) call must
  move at least -- K and V of every valid token once, q, out, the table entries
  in use and the lengths.  Split-K scratch traffic, and the K/V re-read by a
  multi-token call that needs several runs of query tokens, are overhead and are
  not counted.
"""

from __future__ import annotations

import numpy as np


def kv_cache_bytes(layers: int, tokens: int, kv_heads: int, head_size: int,
                   bytes_per_element: int) -> int:
    return 2 * int(layers) * int(tokens) * int(kv_heads) * int(head_size) * int(bytes_per_element)


def blocks_needed(tokens, block_size: int):
    t = np.asarray(tokens, dtype=np.int64)
    return -(-t // int(block_size))


def decode_algorithmic_bytes(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                             block_size: int, elem_bytes: int = 2, unique_tokens=None,
                             query_tokens: int = 1, kv_elem_bytes=None) -> int:
    """Algorithmic bytes of one decode call (``query_tokens`` > 1: one multi-token
    call with that many query rows per sequence, plus its query lengths).
    ``unique_tokens`` replaces the sum of context lengths when sequences share
    physical blocks (count each stored slot once); ``kv_elem_bytes`` is the size of
    one stored K/V element when it differs from q's (1 for fp8 pools)."""
    lens = np.asarray(context_lens, dtype=np.int64)
    S = lens.size
    tokens = int(lens.sum()) if unique_tokens is None else int(unique_tokens)
    kv = tokens * num_kv_heads * head_dim * (kv_elem_bytes or elem_bytes) * 2
    qo = 2 * S * int(query_tokens) * num_q_heads * head_dim * elem_bytes
    tables = int(blocks_needed(lens, block_size).sum()) * 4
    qlens = 4 * S if query_tokens > 1 else 0
    return kv + qo + tables + 4 * S + qlens
