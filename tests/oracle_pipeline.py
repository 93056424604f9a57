"""Runs a workload through the CPU oracle only (tables, pool images, attention)."""

from dataclasses import dataclass

import numpy as np

import workloads
from oracle import allocator as oalloc
from oracle import attention as oattn
from oracle import cache_ops


@dataclass
class OracleRun:
    spec: object
    flow: object
    model: object
    k_pool: np.ndarray
    v_pool: np.ndarray
    tables: np.ndarray
    out: np.ndarray  # fp64 [Tq][Hq][D]


def build_pools(spec, flow, seqs=None):
    """Oracle pool images after every phase of the flow (copies, then writes).

    ``seqs`` restricts the writes to the given sequences' tokens (sampled checks).
    """
    bits = spec.bits_dtype
    poison = workloads.POISON[spec.dtype]
    kp = cache_ops.new_pool(spec.num_layers, spec.num_blocks, spec.num_kv_heads, spec.head_dim, bits, poison)
    vp = cache_ops.new_pool(spec.num_layers, spec.num_blocks, spec.num_kv_heads, spec.head_dim, bits, poison)
    want = None if seqs is None else set(int(s) for s in seqs)
    if spec.shared_prefix and want is not None:
        want.add(0)  # the prefix is written through sequence 0
    for ph in flow.phases:
        cache_ops.copy_blocks(kp, vp, ph.pairs)
        off = 0
        for (s, t0, t1) in ph.src:
            n = t1 - t0
            if n and (want is None or s in want):
                k, v = spec.kv_bits(s, t0, t1)
                cache_ops.kv_cache_write(kp, vp, k, v, ph.slots[off:off + n], spec.dtype)
            off += n
    return kp, vp


def run(spec, seqs=None) -> OracleRun:
    model = oalloc.BlockAllocatorModel(spec.num_blocks, free_order=spec.free_order)
    flow = workloads.run_flow(spec, model)
    kp, vp = build_pools(spec, flow, seqs)
    tables = flow.padded_tables(pad=0)
    q = spec.all_q_bits()
    out = oattn.paged_attention(q, kp, vp, tables, spec.seq_lens, spec.query_start_loc, spec.scale,
                                spec.dtype, seqs=seqs)
    return OracleRun(spec, flow, model, kp, vp, tables, out)
