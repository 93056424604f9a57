"""kv_cache_write and copy_blocks on the GPU: bit-exact against the oracle's pool images."""

import numpy as np
import pytest

import workloads
from oracle import allocator as oalloc
from oracle import cache_ops
from tests import oracle_pipeline as op

pytestmark = pytest.mark.gpu


def _gp():
    from tests import gpu_pipeline

    return gpu_pipeline


@pytest.mark.parametrize("name,kw", [
    ("c1", {}),
    ("c2", dict(num_seqs=6, max_len=400, variant=1)),
    ("c3", dict(num_seqs=12, max_len=1500, variant=1)),
    ("c4", dict(num_seqs=5, max_len=30, variant=1, prefix=37)),
    ("c4", dict(num_seqs=5, max_len=30, variant=1, prefix=64)),
    ("c5", dict(num_seqs=10, max_len=700, variant=1)),
])
def test_pool_after_writes_and_copies_is_bit_exact(name, kw):
    gp = _gp()
    spec = workloads.scaled_spec(name, **kw)
    gp.log(f"[cache] {name} {kw}")
    run = gp.prepare(spec, run_attention=False)
    ref = op.run(spec)
    kg, vg = run.pool_bits()
    assert np.array_equal(kg, ref.k_pool.ravel())
    assert np.array_equal(vg, ref.v_pool.ravel())


@pytest.mark.parametrize("dtype,hkv,d,layers", [("bf16", 8, 128, 2), ("f16", 4, 64, 1),
                                                 ("f32", 2, 64, 3), ("bf16", 2, 256, 1)])
def test_write_with_skipped_slots_and_layers(dtype, hkv, d, layers):
    import torch

    from paged_kv_cache_446_amd import ops

    gp = _gp()
    gp.log(f"[write] {dtype} hkv={hkv} d={d} layers={layers}")
    rng = np.random.default_rng(11)
    nb = 9
    bits = workloads.DTYPES[dtype][0]
    poison = workloads.POISON[dtype]
    kp = cache_ops.new_pool(layers, nb, hkv, d, bits, poison)
    vp = cache_ops.new_pool(layers, nb, hkv, d, bits, poison)
    kdev = gp.dev_bits(kp.ravel(), dtype)
    vdev = gp.dev_bits(vp.ravel(), dtype)
    cache = ops.PagedCache(kdev, vdev, hkv, d, dtype=dtype, num_layers=layers)
    for layer in range(layers):
        T = 37
        slots = rng.choice(nb * 16, size=T, replace=False).astype(np.int64)
        slots[::5] = -1  # skipped tokens
        top = (1 << 16) if bits == np.uint16 else (1 << 31)
        k = rng.integers(0, top, size=(T, hkv, d)).astype(bits)
        v = rng.integers(0, top, size=(T, hkv, d)).astype(bits)
        cache_ops.kv_cache_write(kp, vp, k, v, slots, dtype, layer=layer)
        ops.kv_cache_write(cache, gp.dev_bits(k, dtype), gp.dev_bits(v, dtype),
                           torch.from_numpy(slots).to("cuda:0"), layer=layer)
    torch.cuda.synchronize()
    assert np.array_equal(gp.host_bits(kdev, dtype), kp.ravel())
    assert np.array_equal(gp.host_bits(vdev, dtype), vp.ravel())
    # copy-on-write pairs across every layer
    pairs = np.array([[0, 5], [3, 7], [8, 1]], dtype=np.int32)
    cache_ops.copy_blocks(kp, vp, pairs)
    ops.copy_blocks(cache, torch.from_numpy(pairs).to("cuda:0"))
    ops.copy_blocks(cache, torch.zeros((0, 2), dtype=torch.int32, device="cuda:0"))  # no-op
    torch.cuda.synchronize()
    assert np.array_equal(gp.host_bits(kdev, dtype), kp.ravel())
    assert np.array_equal(gp.host_bits(vdev, dtype), vp.ravel())


def test_copy_on_write_leaves_source_untouched_on_gpu():
    import torch

    gp = _gp()
    gp.log("[cow] shared partial block")
    spec = workloads.scaled_spec("c4", num_seqs=4, max_len=12, variant=4, prefix=37)
    run = gp.prepare(spec, run_attention=False)
    pairs = np.concatenate([ph.pairs for ph in run.flow.phases])
    assert len(pairs)
    m = oalloc.BlockAllocatorModel(spec.num_blocks, free_order=spec.free_order)
    flow = workloads.run_flow(spec, m)
    # pool right after the prefix phase (before any copy or tail write)
    only_prefix = workloads.Flow(flow.tables, flow.nblk, flow.phases[:1])
    kp0, _ = op.build_pools(spec, only_prefix)
    kg, _ = run.pool_bits()
    kg = kg.reshape(kp0.shape)
    src = int(pairs[0, 0])
    pre = kp0[:, src] != workloads.POISON["bf16"]
    assert pre.any() and np.array_equal(kg[:, src][pre], kp0[:, src][pre])
    torch.cuda.synchronize()


def _run_slots(rng, nb, kind):
    """Slot maps made of runs of consecutive slots (prefill chunks) of every start and
    length inside a block, single tokens between them, and slots the write skips."""
    pool = nb * 16
    if kind == "runs":
        starts = rng.permutation(nb)[: nb - 1] * 16
        out = []
        for s in starts:
            pos = int(rng.integers(0, 16))
            L = int(rng.integers(1, 17 - pos))
            out.extend(range(s + pos, s + pos + L))
        return np.array(out, np.int64)
    if kind == "across":  # one long run through several blocks, then a ragged tail
        b = rng.permutation(nb)[:4]
        out = list(range(b[0] * 16 + 3, b[0] * 16 + 16)) + list(range(b[1] * 16, b[1] * 16 + 16))
        out += list(range(b[2] * 16, b[2] * 16 + 7)) + [int(b[3]) * 16 + 9]
        return np.array(out, np.int64)
    # "skips": runs broken by slots outside the pool
    s = int(rng.integers(0, nb)) * 16
    return np.array([s, s + 1, -1, s + 2, s + 3, s + 4, s + 5, pool, s + 6, s + 7, pool + 8,
                     s + 8, s + 9, s + 10, s + 11, s + 12, s + 13, s + 14, s + 15], np.int64)


@pytest.mark.parametrize("kind", ["runs", "across", "skips"])
@pytest.mark.parametrize("dtype,hkv,d,aligned", [("bf16", 8, 128, True), ("bf16", 8, 128, False),
                                                 ("f16", 2, 64, True), ("f32", 4, 128, True),
                                                 ("f32", 8, 256, True), ("bf16", 1, 256, False)])
def test_write_runs_bit_exact(kind, dtype, hkv, d, aligned):
    """Runs of consecutive slots (groups of four written as whole K lines and V
    chunks) next to ragged ends and single tokens written element by element, in
    chunks whose other tokens were written before; v_new also off 16-byte alignment."""
    import torch

    from paged_kv_cache_446_amd import ops

    gp = _gp()
    gp.log(f"[runs] {kind} {dtype} hkv={hkv} d={d} aligned={aligned}")
    rng = np.random.default_rng(abs(hash((kind, dtype, hkv, d, aligned))) % (1 << 31))
    nb, layers = 12, 2
    bits = workloads.DTYPES[dtype][0]
    top = (1 << 16) if bits == np.uint16 else (1 << 31)
    kp = rng.integers(0, top, size=(layers, nb, hkv, 16 * d)).astype(bits)  # old contents
    vp = rng.integers(0, top, size=(layers, nb, hkv, 16 * d)).astype(bits)
    kdev = gp.dev_bits(kp.ravel(), dtype)
    vdev = gp.dev_bits(vp.ravel(), dtype)
    cache = ops.PagedCache(kdev, vdev, hkv, d, dtype=dtype, num_layers=layers)
    for layer in range(layers):
        for _ in range(2):  # the second call fills in around the first one's tokens
            slots = _run_slots(rng, nb, kind)
            T = len(slots)
            k = rng.integers(0, top, size=(T, hkv, d)).astype(bits)
            v = rng.integers(0, top, size=(T, hkv, d)).astype(bits)
            keep = np.ones(T, bool)
            seen = set()
            for i, s in enumerate(slots):  # a slot once per call
                keep[i] = int(s) not in seen or s < 0 or s >= nb * 16
                seen.add(int(s))
            slots[~keep] = -1
            cache_ops.kv_cache_write(kp, vp, k, v, slots, dtype, layer=layer)
            vd = gp.dev_bits(v, dtype)
            if not aligned:  # same values one element past a 16-byte boundary
                buf = torch.empty(vd.numel() + 8, dtype=vd.dtype, device="cuda:0")
                buf[1:1 + vd.numel()] = vd.view(-1)
                vd = buf[1:1 + vd.numel()]
            ops.kv_cache_write(cache, gp.dev_bits(k, dtype), vd,
                               torch.from_numpy(slots).to("cuda:0"), layer=layer)
    torch.cuda.synchronize()
    assert np.array_equal(gp.host_bits(kdev, dtype), kp.ravel())
    assert np.array_equal(gp.host_bits(vdev, dtype), vp.ravel())


def test_copy_blocks_skips_pairs_outside_the_pool():
    import torch

    from paged_kv_cache_446_amd import ops

    gp = _gp()
    gp.log("[copy] pairs outside the pool")
    rng = np.random.default_rng(5)
    nb = 6
    kp = rng.integers(0, 1 << 16, size=(2, nb, 2, 16 * 64)).astype(np.uint16)
    vp = rng.integers(0, 1 << 16, size=(2, nb, 2, 16 * 64)).astype(np.uint16)
    kdev, vdev = gp.dev_bits(kp.ravel(), "bf16"), gp.dev_bits(vp.ravel(), "bf16")
    cache = ops.PagedCache(kdev, vdev, 2, 64, dtype="bf16", num_layers=2)
    pairs = np.array([[1, 4], [0, nb], [-1, 2], [nb + 3, 0], [2, -7], [3, 5]], np.int32)
    cache_ops.copy_blocks(kp, vp, pairs)
    ops.copy_blocks(cache, torch.from_numpy(pairs).to("cuda:0"))
    torch.cuda.synchronize()
    assert np.array_equal(gp.host_bits(kdev, "bf16"), kp.ravel())
    assert np.array_equal(gp.host_bits(vdev, "bf16"), vp.ravel())


def test_debug_checks_stop_bad_metadata_before_launch():
    """With the binding's debug checks on, metadata that breaks a rule raises on the host
    and nothing is launched (the pools keep their bytes); valid metadata goes through."""
    import torch

    from paged_kv_cache_446_amd import checks, ops

    gp = _gp()
    gp.log("[debug] host checks before launch")
    kdev = torch.zeros(2 * 4 * 16 * 64, dtype=torch.int16, device="cuda:0")
    vdev = torch.zeros_like(kdev)
    cache = ops.PagedCache(kdev, vdev, 2, 64, dtype="bf16")
    k = torch.ones((3, 2, 64), dtype=torch.int16, device="cuda:0")
    old = ops.DEBUG
    ops.DEBUG = True
    try:
        for bad in ([1, 2, 1], [0, 5, 64]):  # a shared slot; a slot past the 4-block pool
            with pytest.raises(checks.MetadataError):
                ops.kv_cache_write(cache, k, k, torch.tensor(bad, dtype=torch.int64, device="cuda:0"))
        with pytest.raises(checks.MetadataError):
            ops.copy_blocks(cache, torch.tensor([[0, 1], [2, 1]], dtype=torch.int32, device="cuda:0"))
        torch.cuda.synchronize()
        assert int(kdev.abs().sum()) == 0 and int(vdev.abs().sum()) == 0
        ops.kv_cache_write(cache, k, k, torch.tensor([0, 1, 17], dtype=torch.int64, device="cuda:0"))
        torch.cuda.synchronize()
        assert int((kdev != 0).sum()) == 3 * 2 * 64
    finally:
        ops.DEBUG = old
