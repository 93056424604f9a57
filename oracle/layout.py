"""The documented block-pool layout, restated for the oracle (test infrastructure only).

A pool (one for K, one for V) is ``[num_layers][num_blocks][num_kv_heads][tile]``
where a tile holds the 16 tokens x head_dim elements of one block and one KV
head.  The 16-token block is the pages' default block size
(blog.mckayzhao.com/?p=56, section "PagedAttention").

Inside a tile, with ``x = 16 // element_bytes`` (elements per 16-byte chunk):

* K tile: offset(t, d) = ((d // x) * 16 + t) * x + d % x
  (head_dim split into 16-byte chunks; for each chunk, the 16 tokens in order)
* V tile: with ``x4 = x // 4``, t = 4*g + j and d = 16*n + c,
  m = n // x4, r = n % x4:
  offset(t, d) = (((m * 4 + g) * 16 + c) * x4 + r) * 4 + j
  (groups of 4 consecutive tokens stored together for each dimension)

This file is written independently of the library source; it follows the
layout as stated in the public header's comments.
"""

import numpy as np

TOKENS_PER_BLOCK = 16


def chunk_elems(dtype: str) -> int:
    return {"f32": 4, "f16": 8, "bf16": 8}[dtype]


def k_offset(t, d, dtype: str):
    x = chunk_elems(dtype)
    t = np.asarray(t, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    return ((d // x) * TOKENS_PER_BLOCK + t) * x + d % x


def v_offset(t, d, dtype: str):
    x4 = chunk_elems(dtype) // 4
    t = np.asarray(t, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    g, j = t // 4, t % 4
    n, c = d // 16, d % 16
    m, r = n // x4, n % x4
    return (((m * 4 + g) * 16 + c) * x4 + r) * 4 + j


def tile_elems(head_dim: int) -> int:
    return TOKENS_PER_BLOCK * head_dim


def supported(dtype: str, head_dim: int) -> bool:
    x = chunk_elems(dtype)
    return head_dim % x == 0 and head_dim % (16 * (x // 4)) == 0
