"""Pins of the oracle's allocator model and cache operations (runs on CPU).

P5  the pages' allocator rules and worked examples (tests/golden/pages_examples.json)
P6  cache write / block copy: hand-computed layout offsets, round trip,
    poison preservation, copy-on-write leaves the source untouched
"""

import json
import math
import os

import numpy as np
import pytest

import workloads
from oracle import allocator as oalloc
from oracle import attention as oattn
from oracle import cache_ops, layout, numerics
from tests import oracle_pipeline as op

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pages():
    with open(os.path.join(GOLDEN, "pages_examples.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# P5: allocator rules
# ---------------------------------------------------------------------------


def test_p5_block_count_and_tail_waste_rule():
    g = _pages()["block_rule"]
    bs, most = g["block_size"], g["max_tail_waste"]
    for n in range(1, 100001):
        b = oalloc.blocks_for_tokens(n)
        assert b == math.ceil(n / bs)
        assert 0 <= b * bs - n <= most
    assert oalloc.blocks_for_tokens(0) == 0


def test_p5_c1_block_usage():
    spec = workloads.named_spec("c1")
    run = op.run(spec)
    assert list(run.flow.nblk) == [1, 2, 3, 4]
    assert [oalloc.BlockAllocatorModel.tail_waste(int(n)) for n in spec.seq_lens] == [15, 15, 15, 14]
    assert run.model.num_free() == 32 - 10


def test_p5_naive_reservation_example():
    g = _pages()["naive_reservation"]
    assert g["reserved"] - g["used"] == g["wasted"]
    b = oalloc.blocks_for_tokens(g["used"])
    assert b == 4 and b * 16 - g["used"] == 14


def test_p5_prefill_then_decode_growth():
    g = _pages()["prefill_then_decode"]
    m = oalloc.BlockAllocatorModel(8)
    t = m.new_table(4)
    nb, sl, slots, _ = m.append_slots(t, 0, 0, g["prompt_tokens"])
    assert sl == g["after_prefill"] and len(slots) == g["prompt_tokens"]
    for d, expect in enumerate(g["after_decode_steps"], start=1):
        nb, sl, slots, _ = m.append_slots(t, nb, sl, 1)
        assert sl == expect and len(slots) == 1
        assert nb == math.ceil((g["prompt_tokens"] + d) / 16)


def test_p5_pool_diagram_reproduced():
    g = _pages()["pool_diagram"]
    names = g["pool"]
    m = oalloc.BlockAllocatorModel(len(names))  # B1..B9 = blocks 0..8, in order
    tabs = {r: m.new_table(4) for r in "ABCD"}
    st = {r: (0, 0) for r in "ABCD"}

    def grow(r, n):
        nb, sl, _, _ = m.append_slots(tabs[r], st[r][0], st[r][1], n)
        st[r] = (nb, sl)

    # interleaved on-demand growth; request D finishes early
    grow("A", 16); grow("B", 16); grow("B", 16); grow("A", 16)
    grow("C", 5); grow("D", 3); grow("A", 16)
    m.free_seq(tabs["D"], st["D"][0])
    for r, want in g["tables"].items():
        got = [names[b] for b in tabs[r][: st[r][0]]]
        assert got == want
    assert sorted(names[b] for b in m.free) == sorted(g["free"])


def test_p5_sharing_diagram_reproduced():
    g = _pages()["sharing_diagram"]
    names = ["B%d" % i for i in range(1, 10)]
    idx = {n: i for i, n in enumerate(names)}
    order = [idx[n] for n in ["B1", "B2", "B5", "B6", "B7", "B3", "B4", "B8", "B9"]]
    m = oalloc.BlockAllocatorModel(9, free_order=order)
    a = m.new_table(4)
    nb, sl, _, _ = m.append_slots(a, 0, 0, 32)  # shared beginning fills B1, B2
    b = m.fork(a, nb)
    c = m.fork(a, nb)
    out = {}
    for r, t in (("A", a), ("B", b), ("C", c)):
        m.append_slots(t, nb, sl, 1)
        out[r] = names[t[2]]
        assert [names[x] for x in t[:2]] == g["shared"]
    assert out == g["private"]
    assert m.refcount(idx["B1"]) == 3 and m.refcount(idx["B2"]) == 3
    for r in "ABC":
        assert m.refcount(idx[g["private"][r]]) == 1


def test_p5_finish_returns_every_block():
    spec = workloads.scaled_spec("c4", num_seqs=6, max_len=40, variant=2, prefix=37)
    run = op.run(spec)
    m = run.model
    for s, t in enumerate(run.flow.tables):
        m.free_seq(t, int(run.flow.nblk[s]))
    assert m.num_free() == spec.num_blocks and all(r == 0 for r in m.ref)


def test_p5_parent_free_keeps_child_alive():
    m = oalloc.BlockAllocatorModel(8)
    a = m.new_table(4)
    nb, sl, _, _ = m.append_slots(a, 0, 0, 20)
    b = m.fork(a, nb)
    m.free_seq(a, nb)
    assert m.num_free() == 6 and all(m.refcount(int(x)) == 1 for x in b[:nb])


def test_p5_out_of_blocks_rolls_back():
    m = oalloc.BlockAllocatorModel(3)
    t = m.new_table(8)
    nb, sl, _, _ = m.append_slots(t, 0, 0, 20)
    before = (t.copy(), list(m.ref), list(m.free))
    with pytest.raises(oalloc.OutOfBlocks):
        m.append_slots(t, nb, sl, 40)
    assert np.array_equal(t, before[0]) and m.ref == before[1] and list(m.free) == before[2]
    # copy-on-write with an empty pool
    u = m.fork(t, nb)
    m.alloc()  # take the last free block: the pool is now empty
    before = (u.copy(), list(m.ref))
    with pytest.raises(oalloc.OutOfBlocks):
        m.append_slots(u, nb, sl, 1)  # needs a copy of the shared partial block
    assert np.array_equal(u, before[0]) and m.ref == before[1]


def test_p5_refcount_and_argument_errors():
    m = oalloc.BlockAllocatorModel(4)
    b = m.alloc()
    m.decref(b)
    with pytest.raises(oalloc.RefcountError):
        m.decref(b)
    with pytest.raises(oalloc.RefcountError):
        m.incref(b)
    with pytest.raises(oalloc.InvalidArgument):
        m.incref(7)
    t = m.new_table(2)
    with pytest.raises(oalloc.InvalidArgument):
        m.append_slots(t, 0, 0, 40)  # table too small
    with pytest.raises(oalloc.InvalidArgument):
        m.append_slots(t, 1, 0, 1)  # nblk inconsistent with seq_len
    nb, sl, _, _ = m.append_slots(t, 0, 0, 3)
    m.decref(int(t[0]))  # drop the sequence's only reference behind its back
    with pytest.raises(oalloc.RefcountError):
        m.free_seq(t, nb)


def test_p5_free_seq_undoes_on_error():
    m = oalloc.BlockAllocatorModel(6)
    t = m.new_table(4)
    nb, _, _, _ = m.append_slots(t, 0, 0, 40)  # 3 blocks
    m.decref(int(t[2]))  # the third entry is now free
    before = (list(m.ref), list(m.free))
    with pytest.raises(oalloc.RefcountError):
        m.free_seq(t, nb)
    assert m.ref == before[0] and list(m.free) == before[1]


@pytest.mark.parametrize("name", ["c2", "c3", "c5"])
def test_p5_waste_below_four_percent(name):
    spec = workloads.named_spec(name)
    n = spec.seq_lens
    used = n.sum()
    slots = sum(oalloc.blocks_for_tokens(int(x)) * 16 for x in n)
    frac = (slots - used) / slots
    assert frac < _pages()["waste_after_paging"]["max_fraction"]


def test_llama13b_reading_of_the_garbled_block_size():
    g = _pages()["llama13b_kv"]
    per_token = 2 * g["layers"] * g["hidden"] * g["bytes_per_elem"]
    assert per_token == 819200
    assert per_token * 2048 / 1e9 <= g["request_gb_upper"]
    assert per_token * 16 // 1024 == g["block_kib_all_layers"]


# ---------------------------------------------------------------------------
# P6: layout, cache write, block copy
# ---------------------------------------------------------------------------


def test_p6_layout_hand_offsets():
    with open(os.path.join(GOLDEN, "layout_offsets.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 16
    for dtype, D, ten, t, d, off in rows:
        fn = layout.k_offset if ten == "K" else layout.v_offset
        assert int(fn(int(t), int(d), dtype)) == int(off), (dtype, D, ten, t, d)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64), ("f32", 64), ("f32", 128), ("bf16", 256)])
def test_p6_layout_is_a_bijection(dtype, D):
    t, d = np.meshgrid(np.arange(16), np.arange(D), indexing="ij")
    for fn in (layout.k_offset, layout.v_offset):
        off = np.sort(fn(t, d, dtype).ravel())
        assert np.array_equal(off, np.arange(16 * D))


def test_p6_write_then_gather_round_trip_and_poison():
    spec = workloads.make_spec("rt", (446, 92), "bf16", 4, 2, 64, [30, 0, 47], [3, 16, 1])
    run = op.run(spec)
    for s in range(spec.num_seqs):
        k, v = spec.kv_bits(s)
        K, V = oattn.gather(run.k_pool, run.v_pool, run.tables[s], int(spec.seq_lens[s]), "bf16")
        assert np.array_equal(K, numerics.to_f64(k, "bf16"))
        assert np.array_equal(V, numerics.to_f64(v, "bf16"))
    written = int(spec.seq_lens.sum()) * 2 * 64
    poison = workloads.POISON["bf16"]
    assert int((run.k_pool != poison).sum()) == written
    assert int((run.v_pool != poison).sum()) == written


def test_p6_negative_slot_is_skipped():
    kp = cache_ops.new_pool(1, 2, 1, 32, np.uint16, 0x7FC0)
    vp = kp.copy()
    k = np.full((2, 1, 32), 0x3F80, np.uint16)
    cache_ops.kv_cache_write(kp, vp, k, k, np.array([-1, 17]), "bf16")
    assert int((kp != 0x7FC0).sum()) == 32 and int((kp[0, 1] == 0x3F80).sum()) == 32


def test_p6_slot_past_the_pool_and_foreign_pairs_are_skipped():
    kp = cache_ops.new_pool(1, 2, 1, 32, np.uint16, 0x7FC0)
    vp = kp.copy()
    k = np.full((3, 1, 32), 0x3F80, np.uint16)
    cache_ops.kv_cache_write(kp, vp, k, k, np.array([32, 1 << 40, 5]), "bf16")
    assert int((kp != 0x7FC0).sum()) == 32 and int((vp[0, 0] == 0x3F80).sum()) == 32
    k0, v0 = kp.copy(), vp.copy()
    cache_ops.copy_blocks(kp, vp, np.array([[0, 2], [-1, 1], [5, 1], [0, -3]], np.int32))
    assert np.array_equal(kp, k0) and np.array_equal(vp, v0)


def test_p6_copy_blocks_leaves_source_and_others():
    rng = np.random.default_rng(3)
    kp = rng.integers(0, 1 << 16, size=(2, 6, 2, 16 * 32), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(2, 6, 2, 16 * 32), dtype=np.uint16)
    k0, v0 = kp.copy(), vp.copy()
    cache_ops.copy_blocks(kp, vp, np.array([[1, 4], [2, 0]], np.int32))
    for L in range(2):  # every layer is copied
        assert np.array_equal(kp[L, 4], k0[L, 1]) and np.array_equal(vp[L, 0], v0[L, 2])
    for b in (1, 2, 3, 5):
        assert np.array_equal(kp[:, b], k0[:, b]) and np.array_equal(vp[:, b], v0[:, b])


def test_p6_copy_on_write_leaves_original_block_unchanged():
    rng = np.random.default_rng(9)
    m = oalloc.BlockAllocatorModel(8)
    kp = cache_ops.new_pool(1, 8, 2, 32, np.uint16, 0x7FC0)
    vp = kp.copy()
    a = m.new_table(4)
    nb, sl, slots, _ = m.append_slots(a, 0, 0, 20)  # one full block, one holding 4 tokens
    ka = rng.integers(0, 0x7F00, size=(20, 2, 32), dtype=np.uint16)
    va = rng.integers(0, 0x7F00, size=(20, 2, 32), dtype=np.uint16)
    cache_ops.kv_cache_write(kp, vp, ka, va, slots, "bf16")
    shared = int(a[1])
    k_before, v_before = kp[:, shared].copy(), vp[:, shared].copy()
    b = m.fork(a, nb)
    _, _, bslots, pairs = m.append_slots(b, nb, sl, 1)  # B modifies the shared last block
    assert pairs.tolist() == [[shared, int(b[1])]] and int(b[1]) != shared
    kb = rng.integers(0, 0x7F00, size=(1, 2, 32), dtype=np.uint16)
    cache_ops.copy_blocks(kp, vp, pairs)
    cache_ops.kv_cache_write(kp, vp, kb, kb, bslots, "bf16")
    assert np.array_equal(kp[:, shared], k_before) and np.array_equal(vp[:, shared], v_before)
    KA, _ = oattn.gather(kp, vp, a, 20, "bf16")
    KB, _ = oattn.gather(kp, vp, b, 21, "bf16")
    assert np.array_equal(KA, numerics.to_f64(ka, "bf16"))
    assert np.array_equal(KB[:20], KA) and np.array_equal(KB[20], numerics.to_f64(kb[0], "bf16"))
    assert m.refcount(shared) == 1 and m.refcount(int(b[1])) == 1
