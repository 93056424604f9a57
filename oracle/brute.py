"""Brute-force attention in pure Python (oracle pin; test infrastructure only).

Works on the *logical* per-sequence arrays (before any scatter into a block
pool): no block table, no NumPy, scalar loops with ``math.exp`` and
``math.fsum``.  Used only on tiny inputs, to check ``oracle.attention``'s
gather, masks and head mapping independently of them.  Element bits are
decoded here with ``struct``, not with the oracle's decoder.
"""

import math
import struct


def decode(bits, dtype):
    """One stored element -> Python float (exact)."""
    b = int(bits)
    if dtype == "f32":
        return struct.unpack("<f", struct.pack("<I", b))[0]
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<H", b))[0]
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", b << 16))[0]
    raise ValueError(dtype)


def to_lists(arr_bits, dtype):
    """Nested lists of floats from a (small) array of element bits."""
    if hasattr(arr_bits, "tolist"):
        arr_bits = arr_bits.tolist()
    if isinstance(arr_bits, list):
        return [to_lists(a, dtype) for a in arr_bits]
    return decode(arr_bits, dtype)


def attention(q, k, v, scale, n_heads_q, n_heads_kv):
    """q: [q_len][Hq][D], k/v: [n][Hkv][D] as lists of floats.

    Row i of the query is token n - q_len + i and sees tokens 0..n-q_len+i.
    """
    q_len, n = len(q), len(k)
    G = n_heads_q // n_heads_kv
    D = len(q[0][0]) if q_len else 0
    out = []
    for i in range(q_len):
        p = n - q_len + i
        row = []
        for h in range(n_heads_q):
            g = h // G
            logits = []
            for t in range(p + 1):
                logits.append(scale * math.fsum(q[i][h][d] * k[t][g][d] for d in range(D)))
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            den = math.fsum(w)
            row.append([math.fsum(w[t] * v[t][g][d] for t in range(p + 1)) / den for d in range(D)])
        out.append(row)
    return out
