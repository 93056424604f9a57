"""Host-side parts of bench.py, on the CPU: the algorithmic figures its roofline
divides by, the gate that ties the measured-traffic figure to the kernel sources it
was taken on, and the one-GPU limit.  Expected values are counted element by
element or pair by pair here, not taken from bench.py's formulas."""

import hashlib
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _spec(dtype="bf16", hq=8, hkv=2, d=16):
    # three decodes and two chunks (one over an empty context), lengths off the block edges
    ctx = np.array([1, 15, 40, 0, 33])
    q = np.array([1, 1, 1, 7, 18])
    return workloads.make_spec("bench-host", (446, 900), dtype, hq, hkv, d, ctx, q)


def test_algorithmic_bytes_count_each_kv_element_once_per_kv_head():
    spec = _spec()
    e = 2
    kv = 0
    for s in range(spec.num_seqs):
        for _t in range(int(spec.seq_lens[s])):
            for _h in range(spec.num_kv_heads):
                kv += 2 * spec.head_dim * e  # one K row and one V row
    qo = 0
    for _tok in range(spec.num_q_tokens):
        for _h in range(spec.num_q_heads):
            qo += 2 * spec.head_dim * e  # one Q row read, one output row written
    table = 4 * sum(len(range(0, int(n), 16)) for n in spec.seq_lens)  # one entry per block
    got_kv, got_all = bench.algorithmic_bytes(spec)
    assert got_kv == kv
    assert got_all == kv + qo + table


def test_unique_bytes_count_a_shared_block_once():
    spec = _spec()
    nb = [len(range(0, int(n), 16)) for n in spec.seq_lens]
    tables = np.full((spec.num_seqs, max(nb) + 1), -1, dtype=np.int32)
    nxt = 100
    for s in range(spec.num_seqs):
        for j in range(nb[s]):
            tables[s, j] = 7 if j == 0 else nxt  # every sequence's first block is block 7
            nxt += 0 if j == 0 else 1
    distinct = {int(tables[s, j]) for s in range(spec.num_seqs) for j in range(nb[s])}
    kv = len(distinct) * spec.num_kv_heads * 16 * spec.head_dim * 2 * 2
    qo = spec.num_q_tokens * spec.num_q_heads * spec.head_dim * 2 * 2
    assert bench.unique_bytes(spec, tables) == kv + qo + 4 * sum(nb)


def test_prefill_flops_count_visible_pairs():
    spec = _spec()
    rows = np.array([3, 4])
    pairs = 0
    for s in rows:
        q_len, n = int(spec.q_lens[s]), int(spec.seq_lens[s])
        for i in range(q_len):  # query token i of the chunk sits at position n - q_len + i
            for t in range(n):
                pairs += t <= n - q_len + i
    assert bench.prefill_flops(spec, rows) == pairs * spec.num_q_heads * 4 * spec.head_dim


def _copy_tree_for_traffic(dst):
    os.makedirs(os.path.join(dst, "profiles"))
    os.makedirs(os.path.join(dst, "paged_kv_cache_446_amd", "csrc"))
    prof = "paged_attention_decode_llama3-8b-gqa_b256_pmc.md"
    shutil.copy(os.path.join(ROOT, "profiles", prof), os.path.join(dst, "profiles", prof))
    for f in ("attention.hip", "attn_common.h", "pkv_device.h"):
        shutil.copy(os.path.join(ROOT, "paged_kv_cache_446_amd", "csrc", f),
                    os.path.join(dst, "paged_kv_cache_446_amd", "csrc", f))


def test_measured_traffic_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    _copy_tree_for_traffic(str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    prof = (tmp_path / "profiles" / "paged_attention_decode_llama3-8b-gqa_b256_pmc.md").read_text()
    h = hashlib.sha256()
    for f in ("attention.hip", "attn_common.h", "pkv_device.h"):
        h.update((tmp_path / "paged_kv_cache_446_amd" / "csrc" / f).read_bytes())
    recorded = prof.split("kernel_sources_sha256: ")[1].split()[0]
    bytes_line = int(prof.split("traffic_bytes_per_launch: ")[1].split()[0])
    if recorded == h.hexdigest():
        assert bench.measured_traffic() == bytes_line
    else:  # sources changed since the counters were taken: the figure is withheld
        assert bench.measured_traffic() is None
    # any change to a kernel source withholds it
    src = tmp_path / "paged_kv_cache_446_amd" / "csrc" / "attn_common.h"
    src.write_bytes(src.read_bytes() + b"\n")
    assert bench.measured_traffic() is None
    # as does a summary without the machine-readable lines
    (tmp_path / "profiles" / "paged_attention_decode_llama3-8b-gqa_b256_pmc.md").write_text("none")
    assert bench.measured_traffic() is None


def test_committed_traffic_matches_the_committed_kernel_sources():
    # the committed summary was taken on the committed decode kernel sources
    assert bench.measured_traffic() is not None


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu_before_touching_a_device(argv, env):
    e = dict(os.environ)
    e.update(env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
