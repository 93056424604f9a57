"""A stream of prefix-cached requests whose K/V depend on each token's whole prefix.

Prompts are built from a few 16-token words in random order, so later prompts
recombine blocks of earlier ones, and a small pool keeps evicting cached blocks
(and with them the blocks cached below them).  Every token's K and V come from
``workloads.prefix_kv_bits``: a block that a lookup hands out under a prefix it
was not computed for holds other values, and the request's attention output
moves away from the attention over its own prompt.  The stream is run with any
allocator (the C library or the oracle's model), any cache write and any
attention (the GPU kernels or the oracle's pool image).
"""

import numpy as np

import workloads
from oracle import allocator as oalloc
from oracle import attention as oattn
from oracle import numerics

HQ, HKV, D = 8, 2, 64
SCALE = 1.0 / np.sqrt(D)


def run(seed, alloc, write, attend, n_ops=90, cap=12):
    """Returns (hits per request, worst |attention - oracle over the own prompt|)."""
    rng = np.random.default_rng([446, 104, seed])
    words = [rng.integers(0, 1000, size=16).astype(np.int32) for _ in range(4)]
    live, hits, worst = [], [], 0.0
    for step in range(n_ops):
        if live and rng.random() < 0.35:
            t, nb = live.pop(int(rng.integers(0, len(live))))
            alloc.free_seq(t, nb)
            continue
        n_w = int(rng.integers(1, 5))
        tail = int(rng.integers(0, 12)) * int(rng.integers(0, 2))
        prompt = np.concatenate([words[int(rng.integers(0, 4 if w == 0 else 2))] for w in range(n_w)]
                                + [rng.integers(0, 1000, size=tail).astype(np.int32)]).astype(np.int32)
        t = alloc.new_table(cap)
        hit = alloc.cache_lookup(prompt, t)
        try:
            nb, _, slots, _ = alloc.append_slots(t, hit, hit * 16, len(prompt) - hit * 16)
        except (oalloc.AllocError, RuntimeError):
            alloc.free_seq(t, hit)  # the request cannot start: give its hits back
            continue
        k, v = workloads.prefix_kv_bits(prompt, HKV, D, "bf16")
        if len(slots):
            write(slots, k[hit * 16:], v[hit * 16:])
        alloc.cache_seal(prompt, t, nb)
        q = workloads.normal_bits((446, 104, seed, step), (1, HQ, D), "bf16")
        got = attend(t, nb, len(prompt), q)
        ref = oattn.attend(numerics.to_f64(q, "bf16"), numerics.to_f64(k, "bf16"),
                           numerics.to_f64(v, "bf16"), SCALE)
        worst = max(worst, float(np.abs(got - ref).max()))
        hits.append(hit)
        if rng.random() < 0.5:
            alloc.free_seq(t, nb)
        else:
            live.append((t, nb))
    return hits, worst
