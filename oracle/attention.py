"""Paged attention, written as its plain definition in fp64 (oracle; test infrastructure only).

The pages make paging a pure rearrangement of storage: the kernel finds each
block through the block table and reads K and V block by block, and the result
is the same as with contiguous storage (blog.mckayzhao.com/?p=56, section
"PagedAttention"; devpress.csdn.net/amd/6a408ab810ee7a33f2834f35.html,
section on the benefits, where answers stay unchanged).  So the oracle

1. gathers every sequence's K and V through its block table into contiguous
   fp64 arrays (ceil(n/16) blocks, the same page's block-count rule), then
2. runs textbook softmax attention.

Readings where the pages are silent:

* ``seq_lens[s]`` counts the tokens in the cache at attention time, including
  the tokens written this step (decode looks at everything before it and the
  cache grows by one entry per token: devpress page, prefill/decode section).
* A sequence contributes ``q_len = qsl[s+1] - qsl[s]`` query rows; row i sits
  at position ``n - q_len + i`` and sees keys 0..n-q_len+i (chunked prefill
  splits a prompt into pieces, blog page, advanced features: this is the only
  reading under which splitting leaves the result unchanged).
* Query head h reads KV head h // (Hq / Hkv).
* The scale is the float32 value passed in, widened exactly to fp64.
* A sequence with seq_len 0 yields zeros.
"""

import numpy as np

from . import layout, numerics


def gather(k_pool, v_pool, table, n, dtype, layer=0):
    """Contiguous K, V of one sequence, fp64 [n][Hkv][D], read block by block via its table."""
    hkv = k_pool.shape[2]
    D = k_pool.shape[3] // layout.TOKENS_PER_BLOCK
    nb = -(-int(n) // layout.TOKENS_PER_BLOCK)
    t = np.arange(int(n))
    blk = np.asarray(table[:nb], dtype=np.int64)[t // layout.TOKENS_PER_BLOCK]
    pos = t % layout.TOKENS_PER_BLOCK
    d = np.arange(D)
    koff = layout.k_offset(pos[:, None], d[None, :], dtype)
    voff = layout.v_offset(pos[:, None], d[None, :], dtype)
    b3 = blk[:, None, None]
    h3 = np.arange(hkv)[None, :, None]
    K = k_pool[layer, b3, h3, koff[:, None, :]]
    V = v_pool[layer, b3, h3, voff[:, None, :]]
    return numerics.to_f64(K, dtype), numerics.to_f64(V, dtype)


def attend(q, K, V, scale, rows=None):
    """Softmax attention of one sequence's query rows over its contiguous K, V.

    q: fp64 [q_len][Hq][D]; K, V: fp64 [n][Hkv][D].  Returns fp64 [len(rows)][Hq][D].
    """
    q_len, hq, D = q.shape
    n, hkv, _ = K.shape
    G = hq // hkv
    rows = range(q_len) if rows is None else rows
    out = np.zeros((len(rows), hq, D), dtype=np.float64)
    s64 = np.float64(scale)
    for r, i in enumerate(rows):
        p = n - q_len + i  # absolute position of this query token
        if p < 0:
            continue
        for g in range(hkv):
            qg = q[i, g * G:(g + 1) * G]  # the G query heads reading KV head g
            s = s64 * (qg @ K[: p + 1, g].T)  # [G][p+1]
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            out[r, g * G:(g + 1) * G] = (w @ V[: p + 1, g]) / w.sum(axis=1, keepdims=True)
    return out


def paged_attention(q_bits, k_pool, v_pool, tables, seq_lens, query_start_loc, scale, dtype,
                    layer=0, seqs=None):
    """Oracle output fp64 [Tq][Hq][D]; rows of sequences not in ``seqs`` are NaN."""
    q = numerics.to_f64(q_bits, dtype)
    out = np.full(q.shape, np.nan, dtype=np.float64)
    S = len(seq_lens)
    for s in (range(S) if seqs is None else seqs):
        a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
        n = int(seq_lens[s])
        if b == a:
            continue
        if n == 0:
            out[a:b] = 0.0
            continue
        K, V = gather(k_pool, v_pool, tables[s], n, dtype, layer)
        out[a:b] = attend(q[a:b], K, V, scale)
    return out


def attention_rows(q_bits_seq, k_pool, v_pool, table, n, scale, dtype, rows, layer=0):
    """Selected query rows of one sequence (for sampled checks at full size)."""
    K, V = gather(k_pool, v_pool, table, n, dtype, layer)
    return attend(numerics.to_f64(q_bits_seq, dtype), K, V, scale, rows=rows)


# ---------------------------------------------------------------------------
# Split of the key range and its merge.  Not used by ``paged_attention``; it
# states the merge rule a split-K kernel relies on, so that a test can check
# the rule against the unsplit definition above.
# ---------------------------------------------------------------------------


def partial_state(qrow, K, V, scale):
    """(m, l, acc) of one query vector over one key range: max logit, sum of
    exp(logit - m), and the exp-weighted sum of V rows."""
    s = np.float64(scale) * (K @ qrow)
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), w @ V


def merge_states(states):
    """Combine partial states of disjoint key ranges: M = max m_p,
    o = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p."""
    M = max(m for m, _, _ in states)
    num = sum(np.exp(m - M) * acc for m, _, acc in states)
    den = sum(np.exp(m - M) * l for m, l, _ in states)
    return num / den
