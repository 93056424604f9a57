"""The seeded workload generators against the recipe the benchmarks are quoted on:
dtypes, head counts, head_dim, batch sizes and the length ranges of every named
configuration, and that the same seed gives the same inputs.  The generators hold
no attention arithmetic; these checks keep the inputs the parity tests and the
bench use equal to the stated shapes."""

import math

import numpy as np
import pytest

import workloads
from oracle import numerics


def _shape(spec):
    return spec.dtype, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.num_seqs


def test_tiny_decode():
    s = workloads.named_spec("c1")
    assert _shape(s) == ("f32", 4, 4, 64, 4)
    assert s.seq_lens.tolist() == [1, 17, 33, 50] and (s.q_lens == 1).all()
    assert s.num_blocks == 32


def test_llama13b_decode_layer():
    s = workloads.named_spec("c2")
    assert _shape(s) == ("f16", 40, 40, 128, 64)
    assert (s.q_lens == 1).all()
    assert s.seq_lens.min() >= 128 and s.seq_lens.max() <= 2048


def test_llama3_8b_gqa_decode_lengths_are_log_uniform():
    s = workloads.named_spec("c3")
    assert _shape(s) == ("bf16", 32, 8, 128, 256)
    assert (s.q_lens == 1).all()
    n = s.seq_lens
    assert n.min() >= 64 and n.max() <= 8192
    # log-uniform on [64, 8192]: about half below the geometric middle, and the
    # log-lengths spread evenly over the seven octaves
    assert 0.4 < np.mean(n < math.sqrt(64 * 8192)) < 0.6
    octave = np.floor(np.log2(n / 64)).clip(0, 6)
    counts = np.bincount(octave.astype(int), minlength=7)
    assert counts.min() >= 20, counts


def test_shared_prefix_sampling():
    s = workloads.named_spec("c4")
    assert _shape(s) == ("bf16", 32, 8, 128, 64)
    assert s.shared_prefix == 10000
    tails = s.seq_lens - 10000 - 1  # the step's new token follows the private tail
    assert tails.min() >= 0 and tails.max() <= 256
    nine = workloads.scaled_spec("c4", prefix=9992)
    assert nine.shared_prefix == 9992 and nine.num_seqs == 64


def test_mixed_prefill_and_decode_batch():
    s = workloads.named_spec("c5")
    assert _shape(s) == ("bf16", 32, 8, 128, 144)
    chunk = s.q_lens > 1
    assert chunk.sum() == 16
    q, ctx = s.q_lens[chunk], s.seq_lens[chunk] - s.q_lens[chunk]
    assert q.min() >= 16 and q.max() <= 512 and ctx.min() >= 0 and ctx.max() <= 32768
    dec = s.seq_lens[~chunk]
    assert dec.min() >= 64 and dec.max() <= 8192
    # chunks and decodes are shuffled together, not listed in two runs
    runs = np.count_nonzero(np.diff(chunk.astype(int)))
    assert runs > 2


def test_speculative_verify_batch():
    s = workloads.named_spec("verify")
    assert _shape(s) == ("bf16", 32, 8, 128, 256)
    assert (s.q_lens == 5).all()
    n = s.seq_lens - s.q_lens + 1  # the drawn length before the step's last four drafts
    assert n.min() >= 64 and n.max() <= 8192


@pytest.mark.parametrize("name", ["c2", "c3", "c5", "verify"])
def test_same_seed_same_inputs(name):
    a, b = workloads.named_spec(name), workloads.named_spec(name)
    assert np.array_equal(a.seq_lens, b.seq_lens) and np.array_equal(a.q_lens, b.q_lens)
    assert np.array_equal(a.free_order, b.free_order)
    s = int(np.argmin(a.seq_lens))
    ka, va = a.kv_bits(s)
    kb, vb = b.kv_bits(s)
    assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    assert np.array_equal(a.q_bits(s), b.q_bits(s))


def test_values_are_standard_normal_rounded_to_the_storage_type():
    s = workloads.named_spec("c2")
    k, v = s.kv_bits(int(np.argmax(s.seq_lens)))
    x = numerics.to_f64(np.concatenate([k.ravel(), v.ravel()]), s.dtype)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1.0) < 0.02
    # every value is representable in fp16: rounding again changes nothing
    assert np.array_equal(x.astype(np.float16).astype(np.float64), x)


def test_block_placement_is_a_permutation_of_the_pool():
    for name in ("c1", "c3", "c5"):
        s = workloads.named_spec(name)
        assert np.array_equal(np.sort(s.free_order), np.arange(s.num_blocks))
