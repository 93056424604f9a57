"""paged_attention at the five workloads' full sizes, as the bench launches it.

The oracle cannot run every row of a full-size batch in seconds, so it runs a
sample of sequences (the shortest, the longest and a spread between, every
chunk of the mixed batch) one by one.  Every row is also checked for
properties that hold at any size: it is finite, it lies inside the range of
the values it averages (softmax weights are a convex combination), and a
second run gives the same bits.
"""

import numpy as np
import pytest

import workloads
from oracle import numerics
from tests import oracle_pipeline as op

pytestmark = pytest.mark.gpu


def _sample(spec, k=8):
    n = spec.seq_lens
    order = np.argsort(n, kind="stable")
    picks = set(int(i) for i in order[np.linspace(0, len(n) - 1, k).astype(int)])
    picks |= set(int(s) for s in np.nonzero(spec.q_lens > 1)[0])  # every prefill chunk
    return sorted(picks)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "c4-9992"])
def test_full_size_sampled_rows_match_oracle(name):
    """c4-9992: the 64 samples share a 9,992-token prefix, so its last block is
    partial and shared; the first private append of each sample copies it."""
    import torch

    from tests import gpu_pipeline as gp

    if name == "c4-9992":
        spec = workloads.scaled_spec("c4", prefix=9992)
    else:
        spec = workloads.named_spec(name)
    gp.log(f"[full] {name}: S={spec.num_seqs} context={int(spec.seq_lens.sum())} "
           f"max_q={int(spec.q_lens.max())} pool={spec.num_blocks}")
    run = gp.prepare(spec)
    if name == "c4-9992":  # every sample copied the shared partial block before its first write
        pairs = np.concatenate([ph.pairs for ph in run.flow.phases if len(ph.pairs)])
        shared_last = 9992 // 16
        assert len(pairs) >= spec.num_seqs - 1
        assert len(set(pairs[:, 0].tolist())) == 1 and len(set(pairs[:, 1].tolist())) == len(pairs)
        # afterwards each sample owns its own copy of that block; one kept the original
        last = [int(t[shared_last]) for t in run.flow.tables]
        assert len(set(last)) == spec.num_seqs and last.count(int(pairs[0, 0])) == 1
    bits = run.out_bits().copy()
    got = numerics.to_f64(bits, spec.dtype).reshape(spec.num_q_tokens, spec.num_q_heads, spec.head_dim)

    # sampled rows against the oracle
    seqs = _sample(spec)
    ref = op.run(spec, seqs=seqs)
    rows = np.concatenate([np.arange(spec.query_start_loc[s], spec.query_start_loc[s + 1]) for s in seqs])
    ok, worst = gp.compare(got[rows], ref.out[rows], spec.dtype)
    gp.log(f"[full] {name}: {len(seqs)} sequences, {len(rows)} rows, worst {worst:.3g}")
    assert ok, f"{name}: worst error {worst}"

    # every row: finite and within the range of the V entries of its KV head (the
    # range over the whole sequence bounds the range over any visible prefix)
    assert np.isfinite(got).all()
    kv_lo, kv_hi = _v_ranges(spec)
    G = spec.group
    qsl = spec.query_start_loc
    for s in range(spec.num_seqs):
        a, b = int(qsl[s]), int(qsl[s + 1])
        lo = np.repeat(kv_lo[s], G, axis=0)[None]  # [1][Hq][D]
        hi = np.repeat(kv_hi[s], G, axis=0)[None]
        tol = 1e-2 if spec.dtype != "f32" else 1e-6
        assert (got[a:b] >= lo - tol).all() and (got[a:b] <= hi + tol).all(), f"{name}: seq {s}"

    # a second call gives the same bits
    gp.attention(run)
    torch.cuda.synchronize()
    assert np.array_equal(bits, run.out_bits())


def _v_ranges(spec):
    """Per sequence, per KV head, per dim: min and max of V over the sequence's tokens."""
    lo = np.empty((spec.num_seqs, spec.num_kv_heads, spec.head_dim))
    hi = np.empty_like(lo)
    for s in range(spec.num_seqs):
        _, v = spec.kv_bits(s)
        vf = numerics.to_f64(v, spec.dtype)
        lo[s], hi[s] = vf.min(axis=0), vf.max(axis=0)
    return lo, hi


def _partition_batch(kind):
    """Decode batches (1 KV head, 4 query heads, head_dim 64, bf16) large enough that the
    plan's estimate picks decode partitions of 2048, 3072 or 4096 tokens (small batches
    keep 1024), with lengths planted on both sides of one and two partitions."""
    if kind == 2048:
        n = np.full(256, 6000, dtype=np.int64)
        n[:6] = [2047, 2048, 2049, 4095, 4096, 4097]
    elif kind == 3072:
        n = np.full(512, 4096, dtype=np.int64)
        n[:6] = [3071, 3072, 3073, 6143, 6144, 6145]
    else:
        rng = np.random.default_rng([446, 102])
        n = np.clip(np.rint(np.exp(rng.uniform(np.log(64), np.log(16384), 1024))), 64, 16384).astype(np.int64)
        n[:6] = [4095, 4096, 4097, 8191, 8192, 8193]
    return workloads.make_spec(f"parts{kind}", (446, 102, kind), "bf16", 4, 1, 64, n - 1, np.ones_like(n))


@pytest.mark.parametrize("kind", [2048, 3072, 4096])
def test_decode_partition_sizes(kind):
    # planted rows (one and two partitions, each +-1 token) and a spread of the
    # others against the oracle; every row finite; a second call gives the same bits
    import torch

    from tests import gpu_pipeline as gp

    spec = _partition_batch(kind)
    gp.log(f"[parts] {kind}: S={spec.num_seqs} context={int(spec.seq_lens.sum())}")
    run = gp.prepare(spec)
    bits = run.out_bits().copy()
    got = numerics.to_f64(bits, spec.dtype).reshape(spec.num_q_tokens, spec.num_q_heads, spec.head_dim)
    seqs = sorted(set(range(6)) | set(_sample(spec, k=6)))
    ref = op.run(spec, seqs=seqs)
    ok, worst = gp.compare(got[seqs], ref.out[seqs], spec.dtype)
    gp.log(f"[parts] {kind}: {len(seqs)} sequences, worst {worst:.3g}")
    assert ok, f"partitions {kind}: worst error {worst}"
    assert np.isfinite(got).all()
    gp.attention(run)
    torch.cuda.synchronize()
    assert np.array_equal(bits, run.out_bits())


@pytest.mark.parametrize("kind", ["one-tile", "two-tile"])
def test_decode_units_beyond_the_grid_cap(kind):
    # A planned decode launch has at most 8 workgroups per resident slot (6,144 for
    # the one-tile kernel at 3 workgroups per CU, 4,096 for the two-tile kernel at 2);
    # here the (item, KV head) units outnumber them, so workgroups take several units
    # one after another.  A few rows past 1024 tokens make the call planned.
    import torch

    from tests import gpu_pipeline as gp

    rng = np.random.default_rng([446, 103, len(kind)])
    if kind == "one-tile":  # 7,000 decode rows x 1 KV head, head_dim 64
        n = rng.integers(1, 40, size=7000, endpoint=True)
        n[rng.choice(7000, size=4, replace=False)] = [1025, 2048, 3000, 4097]
        spec = workloads.make_spec("cap1", (446, 103, 1), "bf16", 4, 1, 64, n - 1, np.ones_like(n))
    else:  # 640 verify rows of 5 tokens x 8 KV heads (20 columns: two tiles)
        n = rng.integers(6, 200, size=640, endpoint=True)
        n[rng.choice(640, size=4, replace=False)] = [1030, 2050, 3000, 4100]
        q = np.full(640, 5, dtype=np.int64)
        spec = workloads.make_spec("cap2", (446, 103, 2), "bf16", 32, 8, 128, n - q, q)
    gp.log(f"[cap] {kind}: S={spec.num_seqs} context={int(spec.seq_lens.sum())}")
    run = gp.prepare(spec)
    bits = run.out_bits().copy()
    got = numerics.to_f64(bits, spec.dtype).reshape(spec.num_q_tokens, spec.num_q_heads, spec.head_dim)
    seqs = sorted(set(int(s) for s in np.argsort(spec.seq_lens)[-4:]) |
                  set(int(s) for s in rng.choice(spec.num_seqs, size=24, replace=False)))
    ref = op.run(spec, seqs=seqs)
    rows = np.concatenate([np.arange(spec.query_start_loc[s], spec.query_start_loc[s + 1]) for s in seqs])
    ok, worst = gp.compare(got[rows], ref.out[rows], spec.dtype)
    gp.log(f"[cap] {kind}: {len(seqs)} sequences, worst {worst:.3g}")
    assert ok, f"{kind}: worst error {worst}"
    assert np.isfinite(got).all()
    gp.attention(run)
    torch.cuda.synchronize()
    assert np.array_equal(bits, run.out_bits())


@pytest.mark.parametrize("hkv", [1, 2, 4, 8])
def test_prefill_list_of_several_rounds_taken_die_by_die(hkv):
    # Prefill lists of at least two rounds of items (two per resident workgroup) are
    # taken die by die, each die's workgroups first taking items d, d + 8, ... and then
    # the other dies' shares; here 512 q-tiles per KV head (32 chunks of 1,024 tokens,
    # 64-token q-tiles at 4 query heads per KV head) plus one chunk over a 40,000-token
    # context, whose q-tiles the plan cuts into pieces.  With fewer than 8 KV heads a
    # die's share mixes heads.  Sampled rows (the long chunk among them) against the
    # oracle, every row finite, a second call the same bits.
    import torch

    from tests import gpu_pipeline as gp

    rng = np.random.default_rng([446, 104, hkv])
    ctx = rng.integers(0, 256, size=33, endpoint=True)
    q = np.full(33, 1024, dtype=np.int64)
    ctx[17], q[17] = 40000, 256
    spec = workloads.make_spec(f"rounds{hkv}", (446, 104, hkv), "bf16", 4 * hkv, hkv, 64, ctx, q)
    gp.log(f"[rounds] Hkv={hkv}: S={spec.num_seqs} query={spec.num_q_tokens} "
           f"context={int(spec.seq_lens.sum())}")
    run = gp.prepare(spec)
    bits = run.out_bits().copy()
    got = numerics.to_f64(bits, spec.dtype).reshape(spec.num_q_tokens, spec.num_q_heads, spec.head_dim)
    seqs = sorted({17, int(np.argmin(spec.seq_lens))} |
                  set(int(s) for s in rng.choice(33, size=3, replace=False)))
    ref = op.run(spec, seqs=seqs)
    rows = np.concatenate([np.arange(spec.query_start_loc[s], spec.query_start_loc[s + 1]) for s in seqs])
    ok, worst = gp.compare(got[rows], ref.out[rows], spec.dtype)
    gp.log(f"[rounds] Hkv={hkv}: {len(seqs)} sequences, {len(rows)} rows, worst {worst:.3g}")
    assert ok, f"Hkv={hkv}: worst error {worst}"
    assert np.isfinite(got).all()
    gp.attention(run)
    torch.cuda.synchronize()
    assert np.array_equal(bits, run.out_bits())
