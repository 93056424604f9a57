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
