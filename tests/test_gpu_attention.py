"""paged_attention on the GPU against the fp64 oracle (reduced sizes: several
tiles, ragged tails, split partitions), plus the invariants the pages state."""

import numpy as np
import pytest

import workloads
from oracle import numerics
from tests import oracle_pipeline as op

pytestmark = pytest.mark.gpu


def _gp():
    from tests import gpu_pipeline

    return gpu_pipeline


def _check(spec, label):
    gp = _gp()
    gp.log(f"[attn] {label}: S={spec.num_seqs} max_n={int(spec.seq_lens.max())} "
           f"max_q={int(spec.q_lens.max())} {spec.dtype} Hq={spec.num_q_heads} Hkv={spec.num_kv_heads} D={spec.head_dim}")
    run = gp.prepare(spec)
    ref = op.run(spec)
    got = numerics.to_f64(run.out_bits(), spec.dtype).reshape(ref.out.shape)
    ok, worst = gp.compare(got, ref.out, spec.dtype)
    assert ok, f"{label}: worst error {worst}"
    return run, ref, got


@pytest.mark.parametrize("name,kw", [
    ("c1", {}),
    ("c2", dict(num_seqs=8, max_len=1200, variant=1)),
    ("c3", dict(num_seqs=24, max_len=3000, variant=1)),
    ("c4", dict(num_seqs=6, max_len=60, variant=1, prefix=37)),
    ("c4", dict(num_seqs=6, max_len=60, variant=1, prefix=1024)),
    ("c5", dict(num_seqs=12, max_len=1500, variant=1)),
])
def test_configs_reduced(name, kw):
    _check(workloads.scaled_spec(name, **kw), f"{name}{kw}")


# edge lengths around a block (16 tokens), a wavefront's share of a decode
# partition, and the decode partition itself (1024 tokens) and its multiples
EDGE = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025, 2047, 2048,
        2049, 3073, 8192]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_decode_edge_lengths(dtype):
    n = np.array(EDGE, dtype=np.int64)
    spec = workloads.make_spec(f"edge-{dtype}", (446, 93, len(dtype)), dtype, 8, 2, 64, n - 1,
                               np.ones_like(n))
    _check(spec, f"edge {dtype}")


@pytest.mark.parametrize("dtype,hq,hkv,d", [
    ("bf16", 8, 8, 128), ("bf16", 16, 8, 128), ("bf16", 32, 8, 128), ("bf16", 64, 8, 128),
    ("f16", 8, 1, 64), ("f16", 4, 2, 256), ("bf16", 16, 2, 256), ("f32", 8, 2, 128),
    ("f32", 8, 8, 64),
])
def test_group_sizes_and_head_dims(dtype, hq, hkv, d):
    ctx = np.array([0, 5, 700, 1500, 63, 40], dtype=np.int64)
    q = np.array([1, 1, 1, 1, 9, 33], dtype=np.int64)
    spec = workloads.make_spec(f"g{hq}-{hkv}-{d}", (446, 94, hq, hkv, d), dtype, hq, hkv, d, ctx, q)
    _check(spec, f"{dtype} {hq}/{hkv} d{d}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_chunks_over_empty_context(dtype):
    # first chunks of prompts: row i sees only i + 1 keys, so early rows have outputs
    # of the size of single V rows (the largest errors a 16-bit path makes)
    ctx = np.array([0, 0, 0, 3], dtype=np.int64)
    q = np.array([64, 200, 17, 90], dtype=np.int64)
    spec = workloads.make_spec(f"empty-ctx-{dtype}", (446, 99, len(dtype)), dtype, 32, 8, 128, ctx, q)
    _check(spec, f"chunks over an empty context {dtype}")


def test_chunks_over_long_context():
    # a chunk over a 32768-token context (the mixed batch's upper bound) and a decode
    ctx = np.array([32768, 8191, 100], dtype=np.int64)
    q = np.array([40, 1, 17], dtype=np.int64)
    spec = workloads.make_spec("longchunk", (446, 95), "bf16", 32, 8, 128, ctx, q)
    _check(spec, "long chunk")


def test_zero_length_sequence_yields_zeros():
    import torch

    gp = _gp()
    spec = workloads.make_spec("zero", (446, 96), "bf16", 8, 2, 64, [10, 20], [1, 1])
    run = gp.prepare(spec, run_attention=False)
    run.seq_lens.copy_(torch.tensor([0, 21], dtype=torch.int32, device="cuda:0"))
    run.out.fill_(0x3F80)
    gp.attention(run)
    torch.cuda.synchronize()
    out = numerics.to_f64(run.out_bits(), "bf16").reshape(2, 8, 64)
    assert np.all(out[0] == 0.0) and np.all(out[1] != 1.0)


def test_bitwise_deterministic_and_placement_invariant():
    import torch

    gp = _gp()
    spec = workloads.scaled_spec("c3", num_seqs=16, max_len=2500, variant=2)
    a = gp.prepare(spec)
    first = a.out_bits().copy()
    gp.attention(a)
    torch.cuda.synchronize()
    assert np.array_equal(first, a.out_bits())  # run to run
    other = np.random.default_rng(77).permutation(spec.num_blocks).astype(np.int32)
    b = gp.prepare(spec, free_order=other, table_pad_width=a.tables.shape[1] + 5)
    assert not np.array_equal(a.tables.cpu().numpy(), b.tables.cpu().numpy()[:, :a.tables.shape[1]])
    assert np.array_equal(first, b.out_bits())  # any physical placement


def test_shared_prefix_equals_private_copies_bitwise():
    import torch

    gp = _gp()
    shared = workloads.scaled_spec("c4", num_seqs=6, max_len=50, variant=5, prefix=1024)
    rs = gp.prepare(shared)
    # the same logical tokens, every sequence written into private blocks
    from paged_kv_cache_446_amd import ops
    from paged_kv_cache_446_amd.allocator import BlockAllocator

    nb = int(sum(-(-int(n) // 16) for n in shared.seq_lens)) + 8
    alloc = BlockAllocator(nb)
    S = shared.num_seqs
    tabs = np.zeros((S, rs.tables.shape[1]), np.int32)
    kp = torch.zeros(nb * 8 * 16 * 128, dtype=torch.int16, device="cuda:0")
    vp = torch.zeros_like(kp)
    cache = ops.PagedCache(kp, vp, 8, 128, dtype="bf16")
    for s in range(S):
        t = alloc.new_table(rs.tables.shape[1])
        n = int(shared.seq_lens[s])
        nblk, _, slots, _ = alloc.append_slots(t, 0, 0, n)
        k, v = shared.kv_bits(s)
        ops.kv_cache_write(cache, gp.dev_bits(k, "bf16"), gp.dev_bits(v, "bf16"),
                           torch.from_numpy(slots).to("cuda:0"))
        tabs[s, :nblk] = t[:nblk]
    out = torch.zeros_like(rs.out)
    ops.paged_attention(cache, out, rs.q, torch.from_numpy(tabs).to("cuda:0"), rs.seq_lens, rs.qsl,
                        num_q_heads=32, max_q_len=1, max_seq_len=int(shared.seq_lens.max()),
                        scale=shared.scale, workspace=rs.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(gp.host_bits(out, "bf16"), rs.out_bits())
    assert len(rs.flow.step.pairs) == 3  # even sequences copied the last shared block


# Large chunks take the LDS-tiled prefill kernel (16-bit chunks of more than 32
# (token, head) columns, 16 at head_dim 256): several query tiles per chunk,
# contexts of zero, one block, odd block counts and past a partition, next to
# decode rows and small chunks.
@pytest.mark.parametrize("dtype,hq,hkv,d", [
    ("bf16", 32, 8, 128), ("f16", 32, 8, 128), ("bf16", 8, 8, 128), ("bf16", 16, 8, 64),
    ("f16", 16, 2, 256), ("bf16", 64, 8, 128), ("bf16", 8, 4, 64),
])
def test_prefill_tiled_chunks(dtype, hq, hkv, d):
    ctx = np.array([0, 16, 33, 700, 1500, 3000, 0, 90], dtype=np.int64)
    q = np.array([300, 130, 77, 64, 513, 40, 1, 17], dtype=np.int64)
    spec = workloads.make_spec(f"pf-{hq}-{hkv}-{d}", (446, 97, hq, hkv, d), dtype, hq, hkv, d, ctx, q)
    _check(spec, f"tiled prefill {dtype} {hq}/{hkv} d{d}")


def test_prefill_tiled_deterministic_and_placement_invariant():
    import torch

    gp = _gp()
    ctx = np.array([500, 0, 2000], dtype=np.int64)
    q = np.array([200, 96, 33], dtype=np.int64)
    spec = workloads.make_spec("pf-det", (446, 98), "bf16", 32, 8, 128, ctx, q)
    a = gp.prepare(spec)
    first = a.out_bits().copy()
    gp.attention(a)
    torch.cuda.synchronize()
    assert np.array_equal(first, a.out_bits())
    other = np.random.default_rng(78).permutation(spec.num_blocks).astype(np.int32)
    b = gp.prepare(spec, free_order=other)
    assert np.array_equal(first, b.out_bits())


# Speculative-decoding verification: every sequence appends k+1 = 2..9 tokens
# (blog page, advanced features) and they attend causally to the paged context
# and to each other.  Chunks of up to 32 (token, head) columns take the small
# kernel whose wavefronts split the context's blocks; wider ones the tiled
# kernel (fp32: the per-wavefront kernel).
@pytest.mark.parametrize("dtype,hq,hkv,d", [
    ("bf16", 32, 8, 128), ("f16", 32, 8, 128), ("bf16", 8, 8, 128), ("bf16", 16, 8, 64),
    ("bf16", 64, 8, 128), ("f16", 16, 2, 256), ("bf16", 8, 4, 256), ("f32", 32, 8, 128),
    ("f32", 8, 8, 64),
])
def test_verify_chunks(dtype, hq, hkv, d):
    q = np.arange(16) % 8 + 2  # k+1 = 2..9, twice
    spec = workloads.verify_spec(num_seqs=16, max_len=2600, q_len=q, variant=1, dtype=dtype,
                                 hq=hq, hkv=hkv, d=d)
    _check(spec, f"verify {dtype} {hq}/{hkv} d{d}")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_verify_column_boundaries(G):
    # q_len * G on either side of 16 and 32 columns (one and two column tiles),
    # over contexts of zero, a partial block, exact blocks and several thousand tokens
    cols = [16, 17, 32, 33, 8, 24]
    q = np.array([max(2, -(-c // G)) for c in cols] * 2, dtype=np.int64)
    ctx = np.array([0, 5, 16, 64, 1000, 3001, 47, 2048, 1, 15, 4095, 300], dtype=np.int64)
    spec = workloads.make_spec(f"vb-{G}", (446, 99, G), "bf16", 8 * G, 8, 128, ctx, q)
    _check(spec, f"verify boundaries G={G}")


@pytest.mark.parametrize("q_len,G", [(2, 4), (5, 4), (9, 2), (8, 4), (3, 8)])
def test_verify_partition_starts_inside_the_chunk(q_len, G):
    # the last 1024-token partition of the context begins among the chunk's own
    # tokens, so the chunk's first tokens see nothing of it
    ctx = np.array([1024 - j for j in range(1, q_len)] + [2048 - 1, 3072 - q_len + 1, 4096 - 1],
                   dtype=np.int64)
    q = np.full(len(ctx), q_len, dtype=np.int64)
    spec = workloads.make_spec(f"vp-{q_len}-{G}", (446, 100, q_len, G), "bf16", 8 * G, 8, 128, ctx, q)
    _check(spec, f"verify partition inside chunk q={q_len} G={G}")


def test_verify_long_rows_take_larger_partitions():
    # every row at the longest context: the split rows would not fit the workspace
    # with 1024-token partitions, so the plan doubles them (twice here); a decode
    # row in the same batch keeps 1024-token partitions
    n = np.array([8192, 8192, 8192, 8191, 8192], dtype=np.int64)
    q = np.array([8, 8, 7, 8, 1], dtype=np.int64)
    spec = workloads.make_spec("vlong", (446, 101), "bf16", 32, 8, 128, n - q, q)
    _check(spec, "verify long rows")


def test_verify_full_size_sampled():
    # the verify workload at full size (256 sequences, contexts up to 8192,
    # k+1 = 5): a spread of sequences against the oracle, every row finite
    import torch

    gp = _gp()
    spec = workloads.verify_spec()
    run = gp.prepare(spec)
    got = numerics.to_f64(run.out_bits(), spec.dtype).reshape(spec.num_q_tokens, spec.num_q_heads,
                                                               spec.head_dim)
    order = np.argsort(spec.seq_lens, kind="stable")
    seqs = sorted(set(int(i) for i in order[np.linspace(0, spec.num_seqs - 1, 8).astype(int)]))
    ref = op.run(spec, seqs=seqs)
    rows = np.concatenate([np.arange(spec.query_start_loc[s], spec.query_start_loc[s + 1]) for s in seqs])
    ok, worst = gp.compare(got[rows], ref.out[rows], spec.dtype)
    gp.log(f"[attn] verify full size: {len(seqs)} sequences, worst {worst:.3g}")
    assert ok and np.isfinite(got).all()
    bits = run.out_bits().copy()
    gp.attention(run)
    torch.cuda.synchronize()
    assert np.array_equal(bits, run.out_bits())


# Few long items: the tiled prefill cuts their context into pieces whose partials
# a merge kernel combines.  A chunk of 100-300 tokens over 5,000-20,000 cached
# tokens (a prompt's later chunk, or the new tokens after a prefix-cache hit),
# alone or beside decode rows, with piece boundaries before, inside and after
# the chunk's own tokens.
@pytest.mark.parametrize("dtype,hq,hkv,d", [
    ("bf16", 32, 8, 128), ("f16", 32, 8, 128), ("bf16", 8, 8, 128), ("bf16", 16, 2, 256),
    ("bf16", 64, 8, 64),
])
def test_prefill_split_long_context(dtype, hq, hkv, d):
    ctx = np.array([20000, 7, 5000, 12345], dtype=np.int64)
    q = np.array([300, 1, 129, 100], dtype=np.int64)
    spec = workloads.make_spec(f"pfs-{hq}-{hkv}-{d}", (446, 103, hq, hkv, d), dtype, hq, hkv, d, ctx, q)
    _check(spec, f"split prefill {dtype} {hq}/{hkv} d{d}")


def test_prefill_split_deterministic_and_placement_invariant():
    import torch

    gp = _gp()
    ctx = np.array([9000, 3000], dtype=np.int64)
    q = np.array([256, 64], dtype=np.int64)
    spec = workloads.make_spec("pfs-det", (446, 104), "bf16", 32, 8, 128, ctx, q)
    a = gp.prepare(spec)
    first = a.out_bits().copy()
    for _ in range(3):
        gp.attention(a)
        torch.cuda.synchronize()
        assert np.array_equal(first, a.out_bits())
    other = np.random.default_rng(79).permutation(spec.num_blocks).astype(np.int32)
    b = gp.prepare(spec, free_order=other)
    assert np.array_equal(first, b.out_bits())


@pytest.mark.parametrize("name,kw", [
    ("c4", dict(num_seqs=12, max_len=300, variant=6, prefix=2500)),
    ("c3", dict(num_seqs=24, max_len=3000, variant=6)),
    ("c5", dict(num_seqs=12, max_len=1500, variant=6)),
])
def test_shared_prefix_hint_changes_no_bits(name, kw):
    # batches whose plan keeps 1024-token partitions either way: the hint only
    # reorders the work (rows that share blocks read them together)
    import torch

    gp = _gp()
    spec = workloads.scaled_spec(name, **kw)
    run = gp.prepare(spec, run_attention=False)
    gp.attention(run, shared_prefixes=False)
    torch.cuda.synchronize()
    plain = run.out_bits().copy()
    gp.attention(run, shared_prefixes=True)
    torch.cuda.synchronize()
    assert np.array_equal(plain, run.out_bits())
    if name == "c4":
        assert run.alloc.num_shared() > 0


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f16", 8, 1, 64), ("f32", 8, 8, 64),
                                            ("bf16", 16, 2, 256), ("f16", 16, 8, 128)])
def test_shared_prefix_order_changes_no_bits_across_shapes(dtype, hq, hkv, d):
    # The shared-prefix order lists partitions partition-major and deals units
    # head-major; sequence order lists them row by row.  Both run the same
    # per-partition arithmetic and the same merge.
    import torch

    gp = _gp()
    n = np.array([1, 1023, 1024, 1025, 2049, 3073, 64, 17, 2048, 5], dtype=np.int64)
    spec = workloads.make_spec(f"orders-{dtype}", (446, 98, hq, hkv, d), dtype, hq, hkv, d, n - 1,
                               np.ones_like(n))
    run = gp.prepare(spec, run_attention=False)
    gp.attention(run, shared_prefixes=False)
    torch.cuda.synchronize()
    plain = run.out_bits().copy()
    gp.attention(run, shared_prefixes=True)
    torch.cuda.synchronize()
    assert np.array_equal(plain, run.out_bits())


@pytest.mark.parametrize("rows", [257, 1024, 1025])
def test_decode_row_counts_around_the_plan_thread_limit(rows):
    # The plan kernel's 1024 threads hold one row each up to 1024 rows, two past
    # that.  Short rows plus a few that span several 1024-token partitions.  The
    # rows of a few tokens give outputs up to |o| ~ 3.6, where bf16 keeps only
    # 2^-7 relative: the weights must enter P.V with more than bf16's 8 bits.
    rng = np.random.default_rng([446, 97, rows])
    n = rng.integers(1, 40, size=rows, endpoint=True)
    n[rng.choice(rows, size=5, replace=False)] = [1025, 2048, 2049, 3000, 1500]
    spec = workloads.make_spec(f"rows{rows}", (446, 97, rows), "bf16", 8, 2, 64, n - 1, np.ones_like(n))
    _check(spec, f"{rows} rows")


def _contiguous_pool(spec, gp):
    """Every sequence's tokens in one run of consecutive blocks (sequence order)."""
    import torch

    from oracle import cache_ops
    from paged_kv_cache_446_amd import ops

    nb = -(-spec.seq_lens // 16)
    first = np.concatenate([[0], np.cumsum(nb)[:-1]]).astype(np.int32)
    num_blocks = int(nb.sum()) + 3
    bits = spec.bits_dtype
    poison = workloads.POISON[spec.dtype]
    kp_h = cache_ops.new_pool(1, num_blocks, spec.num_kv_heads, spec.head_dim, bits, poison)
    vp_h = cache_ops.new_pool(1, num_blocks, spec.num_kv_heads, spec.head_dim, bits, poison)
    kp = gp.dev_bits(kp_h.ravel(), spec.dtype)
    vp = gp.dev_bits(vp_h.ravel(), spec.dtype)
    cache = ops.PagedCache(kp, vp, spec.num_kv_heads, spec.head_dim, dtype=spec.dtype)
    width = int(nb.max())
    tables = np.zeros((spec.num_seqs, width), np.int32)
    for s in range(spec.num_seqs):
        n = int(spec.seq_lens[s])
        tables[s, :nb[s]] = first[s] + np.arange(nb[s])
        t = np.arange(n)
        slots = (first[s] + t // 16).astype(np.int64) * 16 + t % 16
        k, v = spec.kv_bits(s)
        cache_ops.kv_cache_write(kp_h, vp_h, k, v, slots, spec.dtype)
        ops.kv_cache_write(cache, gp.dev_bits(k, spec.dtype), gp.dev_bits(v, spec.dtype),
                           torch.from_numpy(slots).to("cuda:0"))
    return cache, kp_h, vp_h, tables, first


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f16", 40, 40, 128), ("f32", 8, 2, 64)])
def test_contiguous_baseline_equals_paged_bitwise(dtype, hq, hkv, d):
    import torch

    from oracle import attention as oattn
    from paged_kv_cache_446_amd import ops

    gp = _gp()
    n = np.array([1, 15, 16, 17, 1023, 1024, 1025, 3000, 64, 200], dtype=np.int64)
    spec = workloads.make_spec(f"contig-{dtype}", (446, 99, hq, hkv, d), dtype, hq, hkv, d, n - 1,
                               np.ones_like(n))
    gp.log(f"[contig] {dtype} {hq}/{hkv} d{d}")
    cache, kp_h, vp_h, tables, first = _contiguous_pool(spec, gp)
    q = gp.dev_bits(spec.all_q_bits(), dtype)
    sl = torch.from_numpy(spec.seq_lens.astype(np.int32)).to("cuda:0")
    qsl = torch.from_numpy(spec.query_start_loc).to("cuda:0")
    maxn = int(spec.seq_lens.max())
    ws = torch.empty(ops.workspace_bytes(spec.num_seqs, spec.num_q_tokens, maxn, hq, d),
                     dtype=torch.uint8, device="cuda:0")
    out_p = torch.zeros_like(q)
    out_c = torch.full_like(q, 7)
    ops.paged_attention(cache, out_p, q, torch.from_numpy(tables).to("cuda:0"), sl, qsl,
                        num_q_heads=hq, max_q_len=1, max_seq_len=maxn, scale=spec.scale,
                        workspace=ws)
    ops.contiguous_attention(cache, out_c, q, torch.from_numpy(first).to("cuda:0"), sl, qsl,
                             num_q_heads=hq, max_seq_len=maxn, scale=spec.scale, workspace=ws)
    torch.cuda.synchronize()
    bp, bc = gp.host_bits(out_p, dtype), gp.host_bits(out_c, dtype)
    assert np.array_equal(bp, bc)
    ref = oattn.paged_attention(spec.all_q_bits(), kp_h, vp_h, tables, spec.seq_lens,
                                spec.query_start_loc, spec.scale, dtype)
    ok, worst = gp.compare(numerics.to_f64(bc, dtype).reshape(ref.shape), ref, dtype)
    assert ok, worst


def test_contiguous_baseline_leaves_chunk_rows_unwritten():
    # the table-free baseline takes decode rows only: rows of short chunks keep
    # whatever the output held, decode rows equal the paged kernel's bitwise
    import torch

    from paged_kv_cache_446_amd import ops

    gp = _gp()
    ctx = np.array([1500, 40, 2100, 7, 999], dtype=np.int64)
    q_lens = np.array([1, 3, 1, 2, 1], dtype=np.int64)
    spec = workloads.make_spec("contig-mixed", (446, 102), "bf16", 8, 2, 64, ctx, q_lens)
    cache, kp_h, vp_h, tables, first = _contiguous_pool(spec, gp)
    q = gp.dev_bits(spec.all_q_bits(), "bf16")
    sl = torch.from_numpy(spec.seq_lens.astype(np.int32)).to("cuda:0")
    qsl = torch.from_numpy(spec.query_start_loc).to("cuda:0")
    maxn = int(spec.seq_lens.max())
    ws = torch.empty(ops.workspace_bytes(spec.num_seqs, spec.num_q_tokens, maxn, 8, 64),
                     dtype=torch.uint8, device="cuda:0")
    out_p = torch.zeros_like(q)
    out_c = torch.full_like(q, 7)
    ops.paged_attention(cache, out_p, q, torch.from_numpy(tables).to("cuda:0"), sl, qsl,
                        num_q_heads=8, max_q_len=3, max_seq_len=maxn, scale=spec.scale, workspace=ws)
    ops.contiguous_attention(cache, out_c, q, torch.from_numpy(first).to("cuda:0"), sl, qsl,
                             num_q_heads=8, max_seq_len=maxn, scale=spec.scale, workspace=ws)
    torch.cuda.synchronize()
    bp = gp.host_bits(out_p, "bf16").reshape(spec.num_q_tokens, -1)
    bc = gp.host_bits(out_c, "bf16").reshape(spec.num_q_tokens, -1)
    qsl_h = spec.query_start_loc
    for s_ in range(spec.num_seqs):
        rows = slice(int(qsl_h[s_]), int(qsl_h[s_ + 1]))
        if q_lens[s_] == 1:
            assert np.array_equal(bp[rows], bc[rows])
        else:
            assert (bc[rows] == 7).all()


@pytest.mark.parametrize("prefix,tail_a,tail_b,q_b", [(1000, 37, 50, 1), (10000, 5, 256, 256), (40, 0, 9, 9)])
def test_prefix_cache_reuse_gives_the_same_attention(prefix, tail_a, tail_b, q_b):
    """Request B repeats request A's prompt: it takes A's cached blocks, writes only
    its own tokens, and attends exactly as over its whole prompt."""
    import torch

    from oracle import attention as oattn
    from paged_kv_cache_446_amd import ops
    from paged_kv_cache_446_amd.allocator import BlockAllocator

    gp = _gp()
    gp.log(f"[prefix-cache] prefix {prefix} tails {tail_a}/{tail_b} q_b {q_b}")
    nA, nB = prefix + tail_a, prefix + tail_b
    # sequence 0 = request A, sequence 1 = request B; both start with the shared prefix K/V
    spec = workloads.make_spec("pcache", (446, 101, prefix), "bf16", 32, 8, 128,
                               [nA, nB - q_b], [0, q_b], shared_prefix=prefix)
    rng = np.random.default_rng(prefix)
    tok_prefix = rng.integers(0, 32000, size=prefix).astype(np.int32)
    tok_a = np.concatenate([tok_prefix, rng.integers(0, 32000, size=tail_a).astype(np.int32)])
    tok_b = np.concatenate([tok_prefix, rng.integers(0, 32000, size=tail_b).astype(np.int32)])
    nblocks = 2 * (-(-nB // 16)) + 8
    alloc = BlockAllocator(nblocks, free_order=np.random.default_rng(3).permutation(nblocks).astype(np.int32))
    kp = torch.zeros(nblocks * 8 * 16 * 128, dtype=torch.int16, device="cuda:0")
    vp = torch.zeros_like(kp)
    cache = ops.PagedCache(kp, vp, 8, 128, dtype="bf16")
    cap = -(-nB // 16) + 1

    def write(seq, t0, t1, slots):
        k, v = spec.kv_bits(seq, t0, t1)
        ops.kv_cache_write(cache, gp.dev_bits(k, "bf16"), gp.dev_bits(v, "bf16"),
                           torch.from_numpy(np.ascontiguousarray(slots)).to("cuda:0"))

    # request A: nothing cached yet
    ta = alloc.new_table(cap)
    assert alloc.cache_lookup(tok_a, ta) == 0
    nb_a, _, slots_a, _ = alloc.append_slots(ta, 0, 0, nA)
    write(0, 0, nA, slots_a)
    alloc.cache_seal(tok_a, ta, nb_a)
    alloc.free_seq(ta, nb_a)  # A finishes; its full blocks stay cached
    # request B: the cached full blocks of the shared prompt, then its own tokens
    tb = alloc.new_table(cap)
    hit = alloc.cache_lookup(tok_b, tb)
    assert hit == prefix // 16
    nb_b, _, slots_b, _ = alloc.append_slots(tb, hit, hit * 16, nB - hit * 16)
    write(1, hit * 16, nB, slots_b)
    alloc.cache_seal(tok_b, tb, nb_b)
    torch.cuda.synchronize()

    q = gp.dev_bits(spec.q_bits(1), "bf16")
    out = torch.zeros_like(q)
    ws = torch.empty(ops.workspace_bytes(1, q_b, nB, 32, 128), dtype=torch.uint8, device="cuda:0")
    ops.paged_attention(cache, out, q, torch.from_numpy(tb[None, :nb_b].copy()).to("cuda:0"),
                        torch.tensor([nB], dtype=torch.int32, device="cuda:0"),
                        torch.tensor([0, q_b], dtype=torch.int32, device="cuda:0"),
                        num_q_heads=32, max_q_len=q_b, max_seq_len=nB, scale=spec.scale, workspace=ws)
    torch.cuda.synchronize()
    K, V = (numerics.to_f64(x, "bf16") for x in spec.kv_bits(1))
    ref = oattn.attend(numerics.to_f64(spec.q_bits(1), "bf16"), K, V, spec.scale)
    got = numerics.to_f64(gp.host_bits(out, "bf16"), "bf16").reshape(ref.shape)
    ok, worst = gp.compare(got, ref, "bf16")
    assert ok, worst


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefix_cache_stream_attends_over_its_own_prefix(seed):
    """Recombined prompts on a small evicting pool, every token's K/V derived from its
    whole prefix: each request's attention, from the C allocator's blocks, the cache
    write and the attention kernels, matches the oracle over the request's own prompt.
    A hit on a block computed under another prefix would move the output far outside
    rounding (the same stream on the CPU catches a planted stale-child hit)."""
    import torch

    from paged_kv_cache_446_amd import ops
    from paged_kv_cache_446_amd.allocator import BlockAllocator
    from tests import prefix_stream as ps

    gp = _gp()
    gp.log(f"[prefix-stream] seed {seed}")
    blocks = 14
    order = np.random.default_rng(seed + 7).permutation(blocks).astype(np.int32)
    alloc = BlockAllocator(blocks, free_order=order)
    kp = torch.zeros(blocks * ps.HKV * 16 * ps.D, dtype=torch.int16, device="cuda:0")
    vp = torch.zeros_like(kp)
    cache = ops.PagedCache(kp, vp, ps.HKV, ps.D, dtype="bf16")
    ws = torch.empty(ops.workspace_bytes(1, 1, 16 * 12, ps.HQ, ps.D), dtype=torch.uint8, device="cuda:0")

    def write(slots, k, v):
        ops.kv_cache_write(cache, gp.dev_bits(k, "bf16"), gp.dev_bits(v, "bf16"),
                           torch.from_numpy(np.ascontiguousarray(slots)).to("cuda:0"))

    def attend(t, nb, n, q):
        qd = gp.dev_bits(q, "bf16")
        out = torch.zeros_like(qd)
        ops.paged_attention(cache, out, qd, torch.from_numpy(t[None, :nb].copy()).to("cuda:0"),
                            torch.tensor([n], dtype=torch.int32, device="cuda:0"),
                            torch.tensor([0, 1], dtype=torch.int32, device="cuda:0"),
                            num_q_heads=ps.HQ, max_q_len=1, max_seq_len=n, scale=ps.SCALE,
                            workspace=ws, shared_prefixes=alloc.num_shared() > 0)
        torch.cuda.synchronize()
        return numerics.to_f64(gp.host_bits(out, "bf16"), "bf16").reshape(q.shape)

    hits, worst = ps.run(seed, alloc, write, attend)
    gp.log(f"[prefix-stream] seed {seed}: {len(hits)} requests, {sum(h > 0 for h in hits)} with hits, "
           f"worst {worst:.3g}")
    assert sum(h > 0 for h in hits) > 10 and max(hits) >= 2
    assert worst <= 1e-2


@pytest.mark.parametrize("name,kw", [("c1", {}), ("c5", dict(num_seqs=12, max_len=1500, variant=3)),
                                     ("c4", dict(num_seqs=6, max_len=60, variant=3, prefix=37))])
def test_step_captured_in_a_graph_replays_like_eager(name, kw):
    """One step (copy-on-write copies, cache write, attention) captured in a HIP graph:
    every replay, with eager work between replays, gives the eager bits."""
    import torch

    from paged_kv_cache_446_amd import ops

    gp = _gp()
    spec = workloads.scaled_spec(name, **kw)
    gp.log(f"[graph] {name} {kw}")
    run = gp.prepare(spec, run_attention=False)
    stp = run.flow.step
    ks, vs = workloads.step_kv_bits(spec)
    k_step, v_step = gp.dev_bits(ks, spec.dtype), gp.dev_bits(vs, spec.dtype)
    slots = torch.from_numpy(stp.slots).to("cuda:0")
    pairs = torch.from_numpy(stp.pairs.copy()).to("cuda:0") if len(stp.pairs) else None
    kp0, vp0 = run.cache.k_pool.clone(), run.cache.v_pool.clone()

    def step(out):
        if pairs is not None:
            ops.copy_blocks(run.cache, pairs)
        ops.kv_cache_write(run.cache, k_step, v_step, slots)
        gp.attention(run, out=out)

    eager = torch.zeros_like(run.out)
    step(eager)
    torch.cuda.synchronize()
    ref = gp.host_bits(eager, spec.dtype).copy()
    kp1, vp1 = run.cache.k_pool.clone(), run.cache.v_pool.clone()

    out = torch.zeros_like(run.out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(out)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step(out)
    torch.cuda.synchronize()
    for r in range(4):
        run.cache.k_pool.copy_(kp0)  # eager work between replays: reset the pools
        run.cache.v_pool.copy_(vp0)
        out.fill_(0x7F7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gp.host_bits(out, spec.dtype), ref), f"replay {r}"
        assert torch.equal(run.cache.k_pool, kp1) and torch.equal(run.cache.v_pool, vp1)
