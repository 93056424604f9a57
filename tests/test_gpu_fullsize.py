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


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_full_size_sampled_rows_match_oracle(name):
    import torch

    from tests import gpu_pipeline as gp

    spec = workloads.named_spec(name)
    gp.log(f"[full] {name}: S={spec.num_seqs} context={int(spec.seq_lens.sum())} "
           f"max_q={int(spec.q_lens.max())} pool={spec.num_blocks}")
    run = gp.prepare(spec)
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
