"""Cache write and block copy on host pool images (oracle; test infrastructure only).

Pool images are numpy arrays of raw element bits with shape
``[num_layers][num_blocks][num_kv_heads][16 * head_dim]`` (see ``layout``).

* ``kv_cache_write``: every processed token appends one K entry and one V
  entry to the cache (devpress.csdn.net/amd/6a408ab810ee7a33f2834f35.html,
  section on prefill, decode and the KV cache, where the cache grows by one
  note per token).  Slot ``s`` means block ``s // 16``, position ``s % 16``
  inside it.  The pages do not say what a slot outside the pool means; here a
  negative slot (a padding token) and one at or past ``num_blocks * 16`` are
  skipped.  Two tokens never share a slot.
* ``copy_blocks``: copy-on-write makes a copy of the shared block and leaves
  the original unchanged (blog.mckayzhao.com/?p=56, section on copy-on-write);
  the copy covers K and V, every KV head and every layer of the pool.  A pair
  naming a block outside the pool is skipped (a reading: the pages do not
  cover it).
"""

import numpy as np

from . import layout


def new_pool(num_layers, num_blocks, num_kv_heads, head_dim, bits_dtype, poison) -> np.ndarray:
    shape = (num_layers, num_blocks, num_kv_heads, layout.tile_elems(head_dim))
    return np.full(shape, poison, dtype=bits_dtype)


def kv_cache_write(k_pool, v_pool, k_new, v_new, slots, dtype, layer=0):
    """Scatter new tokens' K/V bits ([T][Hkv][D]) into the pools at their slots."""
    T, hkv, D = k_new.shape
    slots = np.asarray(slots, dtype=np.int64)
    keep = (slots >= 0) & (slots < k_pool.shape[1] * layout.TOKENS_PER_BLOCK)
    blk = slots[keep] // layout.TOKENS_PER_BLOCK
    pos = slots[keep] % layout.TOKENS_PER_BLOCK
    d = np.arange(D)
    heads = np.arange(hkv)
    # element index inside the tile for every (token, dim)
    koff = layout.k_offset(pos[:, None], d[None, :], dtype)  # [T'][D]
    voff = layout.v_offset(pos[:, None], d[None, :], dtype)
    b3 = blk[:, None, None]
    h3 = heads[None, :, None]
    k_pool[layer, b3, h3, koff[:, None, :]] = k_new[keep]
    v_pool[layer, b3, h3, voff[:, None, :]] = v_new[keep]
    return k_pool, v_pool


def copy_blocks(k_pool, v_pool, pairs):
    """For each (src, dst) in order: block dst := block src, in both pools, all layers."""
    nb = k_pool.shape[1]
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if not (0 <= src < nb and 0 <= dst < nb):
            continue
        k_pool[:, dst] = k_pool[:, src]
        v_pool[:, dst] = v_pool[:, src]
    return k_pool, v_pool
