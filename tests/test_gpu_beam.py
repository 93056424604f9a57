"""Beam search on the GPU against the oracle (blog page, beam search: the
candidates share their beginning; copy-on-write section).

Each request keeps B candidate rows.  Every step the surviving candidates continue
some of the old rows (pkv_seq_reorder), each appends one token, and a row whose
shared last block is partly filled gets a copy of it first (copy_blocks), then
the token's K/V is written (kv_cache_write).  The GPU side runs the C allocator
and the HIP kernels; the oracle side runs the allocator model and the oracle's
cache operations on host pools.  The pools must stay bit-identical and attention
over every candidate must match the oracle.
"""

import numpy as np
import pytest

import workloads
from oracle import allocator as oalloc
from oracle import attention as oattn
from oracle import cache_ops
from oracle import numerics

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,hq,hkv,d,beams,steps", [
    ("bf16", 8, 2, 64, 4, 24), ("f16", 16, 4, 128, 3, 40), ("f32", 4, 4, 64, 5, 18),
])
def test_beam_search_churn_matches_oracle(dtype, hq, hkv, d, beams, steps):
    import torch

    from paged_kv_cache_446_amd import ops
    from paged_kv_cache_446_amd.allocator import BlockAllocator
    from tests import gpu_pipeline as gp

    key = (446, 110, hq, d, beams)
    rng = np.random.default_rng(list(key))
    prompts = [int(x) for x in rng.integers(5, 90, size=3)]
    cap, num_blocks = 16, 3 * beams * 16 + 8
    order = rng.permutation(num_blocks).astype(np.int32)
    ga, oa = BlockAllocator(num_blocks, free_order=order), oalloc.BlockAllocatorModel(num_blocks, free_order=order)
    bits = workloads.DTYPES[dtype][0]
    poison = workloads.POISON[dtype]
    kp_h = cache_ops.new_pool(1, num_blocks, hkv, d, bits, poison)
    vp_h = cache_ops.new_pool(1, num_blocks, hkv, d, bits, poison)
    kp, vp = gp.dev_bits(kp_h.ravel(), dtype), gp.dev_bits(vp_h.ravel(), dtype)
    cache = ops.PagedCache(kp, vp, hkv, d, dtype=dtype)
    gp.log(f"[beam] {dtype} {hq}/{hkv} d{d} beams={beams} steps={steps} prompts={prompts}")

    def write(slots, tag):
        k = workloads.normal_bits(key + tag + (0,), (len(slots), hkv, d), dtype)
        v = workloads.normal_bits(key + tag + (1,), (len(slots), hkv, d), dtype)
        cache_ops.kv_cache_write(kp_h, vp_h, k, v, slots, dtype)
        ops.kv_cache_write(cache, gp.dev_bits(k, dtype), gp.dev_bits(v, dtype),
                           torch.from_numpy(np.asarray(slots, np.int64)).to("cuda:0"))

    def copy(pairs):
        if len(pairs):
            p = np.asarray(pairs, np.int32).reshape(-1, 2)
            cache_ops.copy_blocks(kp_h, vp_h, p)
            ops.copy_blocks(cache, torch.from_numpy(p.copy()).to("cuda:0"))

    # both sides: one table set per request, rows = candidates
    sides = []
    for alloc in (ga, oa):
        reqs = []
        for r, n0 in enumerate(prompts):
            t = np.full((beams, cap), -1, np.int32)
            nb, ln, slots, _ = alloc.append_slots(t[0], 0, 0, n0)
            for b in range(1, beams):
                t[b] = alloc.fork(t[0], nb)
            reqs.append([t, np.full(beams, nb, np.int32), np.full(beams, ln, np.int32), slots])
        sides.append(reqs)
    for r in range(len(prompts)):
        assert np.array_equal(sides[0][r][3], sides[1][r][3])
        write(sides[0][r][3], (r, 100000))  # the prompt's tokens
    n_cow = 0
    for step in range(steps):
        for r in range(len(prompts)):
            parents = rng.integers(0, beams, size=beams).astype(np.int32)
            outs = []
            for alloc, reqs in zip((ga, oa), sides):
                t, nb, ln, _ = reqs[r]
                alloc.reorder(t, nb, ln, parents)
                slots, pairs = [], []
                for b in range(beams):
                    nb[b], ln[b], sl, pr = alloc.append_slots(t[b], int(nb[b]), int(ln[b]), 1)
                    slots += sl.tolist()
                    pairs += pr.tolist()
                outs.append((slots, pairs, t.copy()))
            assert outs[0][0] == outs[1][0] and outs[0][1] == outs[1][1]
            assert np.array_equal(outs[0][2], outs[1][2])
            copy(outs[0][1])  # copy-on-write first, then the new tokens
            write(outs[0][0], (r, step))
            n_cow += len(outs[0][1])
    assert n_cow > 0
    torch.cuda.synchronize()
    assert np.array_equal(gp.host_bits(kp, dtype), kp_h.ravel())
    assert np.array_equal(gp.host_bits(vp, dtype), vp_h.ravel())
    assert ga.num_shared() == oa.num_shared() > 0

    # attention of one query token per candidate over its whole sequence
    tables = np.concatenate([req[0] for req in sides[0]])
    tables = np.where(tables < 0, 0, tables).astype(np.int32)
    seq_lens = np.concatenate([req[2] for req in sides[0]]).astype(np.int64)
    S = len(seq_lens)
    qsl = np.arange(S + 1, dtype=np.int32)
    q = workloads.normal_bits(key + (9,), (S, hq, d), dtype)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ref = oattn.paged_attention(q, kp_h, vp_h, tables, seq_lens, qsl, scale, dtype)
    out = torch.zeros(S * hq * d, dtype=gp._TBITS[dtype], device="cuda:0")
    maxn = int(seq_lens.max())
    ws = torch.empty(ops.workspace_bytes(S, S, maxn, hq, d), dtype=torch.uint8, device="cuda:0")
    for hint in (False, True):
        ops.paged_attention(cache, out, gp.dev_bits(q, dtype), torch.from_numpy(tables).to("cuda:0"),
                            torch.from_numpy(seq_lens.astype(np.int32)).to("cuda:0"),
                            torch.from_numpy(qsl).to("cuda:0"), num_q_heads=hq, max_q_len=1,
                            max_seq_len=maxn, scale=scale, workspace=ws, shared_prefixes=hint)
        torch.cuda.synchronize()
        got = numerics.to_f64(gp.host_bits(out, dtype), dtype).reshape(ref.shape)
        ok, worst = gp.compare(got, ref, dtype)
        gp.log(f"[beam] hint={hint}: {S} rows, {n_cow} copies, worst {worst:.3g}")
        assert ok, worst
