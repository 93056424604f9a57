#!/usr/bin/env python3
"""Paged decode attention throughput on one MI355X (gfx950).

One step = one pass of the hot path over one batch: the step's copy-on-write
block copies (if the workload has any), kv_cache_write of the step's new
tokens, and paged_attention over every sequence.  The host block allocator ran
before the timed region (its per-step cost is timed separately and reported
as ``host_alloc_us``); inputs are resident in HBM when timing starts.

Default workload: Llama-3-8B-shaped GQA decode (256 sequences, contexts
log-uniform in [64, 8192], 32 query / 8 KV heads, head_dim 128, bf16,
16-token blocks placed by a seeded permutation of a 2x pool).

Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix peak, published

WORKLOAD_NAMES = {
    "c1": "tiny paged decode: 4 seqs (1,17,33,50), 4 heads MHA, head_dim 64, fp32",
    "c2": "LLaMA-13B-shaped decode layer: 64 seqs, context U[128,2048], 40/40 heads, head_dim 128, fp16",
    "c3": "Llama-3-8B-shaped GQA decode: 256 seqs, context log-uniform [64,8192], 32q/8kv heads, head_dim 128, bf16",
    "c4": "shared-prefix parallel sampling: 64 seqs share a 10000-token prefix + U[0,256] private tails, CoW, 32q/8kv, bf16",
    "c5": "mixed chunked-prefill + decode: 16 chunks q U[16,512] over context U[0,32768] + 128 decodes U[64,8192], 32q/8kv, bf16",
    "verify": "speculative-decoding verify: 256 seqs, context log-uniform [64,8192], k+1=5 query tokens each, 32q/8kv heads, head_dim 128, bf16",
    "beam": "beam search: 64 requests x 4 candidates, prompts U[512,4096], each step a reorder + 1 token per candidate (copy-on-write of shared last blocks), 32q/8kv heads, head_dim 128, bf16",
    "prefix-cache": "repeated 10000-token prompt + 256 new tokens (second request), 32q/8kv heads, head_dim 128, bf16",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def unique_bytes(spec, tables):
    """K/V bytes of the distinct physical blocks the batch reads (each shared block once),
    plus Q, the output and the table entries: what HBM must deliver at the least."""
    e = spec.elem_bytes
    nb = -(-spec.seq_lens.astype(np.int64) // 16)
    blocks = np.unique(np.concatenate([tables[s, :nb[s]] for s in range(spec.num_seqs)]))
    kv = int(blocks.size) * spec.num_kv_heads * 16 * spec.head_dim * 2 * e
    qo = spec.num_q_tokens * spec.num_q_heads * spec.head_dim * e * 2
    return kv + qo + int(nb.sum()) * 4


def algorithmic_bytes(spec):
    """Bytes the method must move per paged_attention call (each KV element once
    per KV-head group, plus Q, the output and the block-table entries)."""
    e = spec.elem_bytes
    n = spec.seq_lens.astype(np.int64)
    kv = int(n.sum()) * spec.num_kv_heads * spec.head_dim * 2 * e
    qo = spec.num_q_tokens * spec.num_q_heads * spec.head_dim * e * 2
    table = int((-(-n // 16)).sum()) * 4
    return kv, kv + qo + table


def prefill_flops(spec, rows):
    """Matrix FLOPs the method must do for the chunks of ``rows``: per query head, 2 D for
    the score and 2 D for the weighted V of every visible (query token, key) pair; row i
    of a chunk over ctx cached tokens sees ctx + i + 1 keys (masked pairs not counted)."""
    q = spec.q_lens[rows].astype(np.int64)
    ctx = spec.seq_lens[rows].astype(np.int64) - q
    return int((4 * spec.num_q_heads * spec.head_dim * (q * ctx + q * (q + 1) // 2)).sum())


class ContiguousPlacer:
    """Storage without paging, for the paging-overhead comparison: every sequence
    gets one run of consecutive blocks sized for its final length, in sequence
    order.  Offers the allocator calls a workload flow issues; no sharing."""

    def __init__(self, final_lens):
        self.nb = -(-np.asarray(final_lens, dtype=np.int64) // 16)
        self.first = np.concatenate([[0], np.cumsum(self.nb)[:-1]]).astype(np.int32)
        self._next = 0

    def new_table(self, cap):
        s = self._next
        self._next += 1
        t = np.full(cap, -1, dtype=np.int32)
        t[: self.nb[s]] = self.first[s] + np.arange(self.nb[s])
        return t

    def append_slots(self, table, nblk, seq_len, n_new):
        pos = np.arange(seq_len, seq_len + n_new, dtype=np.int64)
        slots = table[pos // 16].astype(np.int64) * 16 + pos % 16
        return int(-(-(seq_len + n_new) // 16)), seq_len + n_new, slots, np.zeros((0, 2), np.int32)

    def fork(self, table, nblk):
        raise ValueError("contiguous placement has no shared blocks")

    make_writable = fork


def measured_traffic():
    """HBM bytes per paged_attention launch from the committed counter summary,
    or None if the kernel sources changed since the counters were taken."""
    import hashlib
    import re

    prof = os.path.join(ROOT, "profiles", "paged_attention_decode_llama3-8b-gqa_b256_pmc.md")
    csrc = os.path.join(ROOT, "paged_kv_cache_446_amd", "csrc")
    try:
        txt = open(prof).read()
        h = hashlib.sha256()
        for f in ("attention.hip", "attn_common.h", "pkv_device.h"):
            h.update(open(os.path.join(csrc, f), "rb").read())
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch: (\d+)", txt)
    k = re.search(r"kernel_sources_sha256: ([0-9a-f]{64})", txt)
    if not m or not k or k.group(1) != h.hexdigest():
        return None
    return int(m.group(1))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, out_bits, target_s, one_thread=True):
    """The oracle (as it stands) on a bounded sample of the same workload, on every
    core this process may use (BLAS threads set to that count), and on one thread."""
    import threadpoolctl

    from oracle import allocator as oalloc
    from oracle import attention as oattn
    from oracle import numerics
    from tests import oracle_pipeline as op
    import workloads

    S = spec.num_seqs
    sample = list(range(0, S, 8)) if S >= 64 else list(range(S))
    model = oalloc.BlockAllocatorModel(spec.num_blocks, free_order=spec.free_order)
    flow = workloads.run_flow(spec, model)
    log(f"cpu baseline: building oracle pools for {len(sample)} sampled sequences")
    kp, vp = op.build_pools(spec, flow, seqs=sample)
    tables = flow.padded_tables(pad=0)
    q = spec.all_q_bits()
    qsl = spec.query_start_loc
    cores = len(os.sched_getaffinity(0))

    def timed(threads, budget_s):
        reps, elapsed, ref = 0, 0.0, None
        with threadpoolctl.threadpool_limits(limits=threads):
            while elapsed < budget_s and reps < 50:
                t0 = time.perf_counter()
                ref = oattn.paged_attention(q, kp, vp, tables, spec.seq_lens, qsl, spec.scale,
                                            spec.dtype, seqs=sample)
                elapsed += time.perf_counter() - t0
                reps += 1
        return reps, elapsed, ref

    reps, elapsed, ref = timed(cores, target_s)
    kv_sample = int(spec.seq_lens[sample].sum()) * spec.num_kv_heads * spec.head_dim * 2 * spec.elem_bytes
    tok_sample = int(sum(qsl[s + 1] - qsl[s] for s in sample))
    # parity of the GPU rows of the sample against the oracle
    got = numerics.to_f64(out_bits, spec.dtype).reshape(ref.shape)
    rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in sample])
    assert len(rows) > 0 and not np.isnan(ref[rows]).any()
    diff = np.abs(got[rows] - ref[rows])
    if spec.dtype == "f32":
        worst = float((diff.max(axis=-1) / np.abs(ref[rows]).max(axis=-1)).max())
        ok = worst <= 1e-5
    else:
        worst = float(diff.max())
        ok = worst <= 1e-2
    base = {
        "value": round(kv_sample * reps / elapsed / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(tok_sample * reps / elapsed, 2),
        "cores": cores,
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": f"{len(sample)} of {S} sequences{' (every 8th)' if S >= 64 else ''}, "
                  f"{int(spec.seq_lens[sample].sum())} context tokens, "
                  f"{reps} pass(es) in {elapsed:.1f} s, fp64 NumPy, BLAS threads = {cores} "
                  f"(the cores of os.sched_getaffinity)",
    }
    if one_thread:
        reps1, elapsed1, _ = timed(1, target_s / 2)
        base["one_thread"] = {"value": round(kv_sample * reps1 / elapsed1 / 1e9, 4), "unit": "GB/s",
                              "tokens_per_s": round(tok_sample * reps1 / elapsed1, 2),
                              "sample": f"the same sample, {reps1} pass(es) in {elapsed1:.1f} s"}
    parity = {"rows": int(len(rows)), "worst": worst, "ok": bool(ok),
              "tolerance": "1e-5 row-relative" if spec.dtype == "f32" else "1e-2 absolute"}
    return base, parity


def bench_prefix_cache(args):
    """A repeated ~10,000-token prompt (the pages' prefix-caching example) with 256
    new tokens, one attention layer: the second request's cache write + prefill
    attention with its prefix served from the cache, and without the cache."""
    import torch

    import workloads
    from paged_kv_cache_446_amd import ops
    from paged_kv_cache_446_amd.allocator import BlockAllocator
    from tests.gpu_pipeline import dev_bits

    dev = "cuda:0"
    P, tail, hq, hkv, D = 10000, 256, 32, 8, 128
    n = P + tail
    spec = workloads.make_spec("prefix-cache", (446, 60), "bf16", hq, hkv, D, [n - tail, 0], [tail, n],
                               shared_prefix=P)
    rng = np.random.default_rng([446, 61])
    prompt = rng.integers(0, 32000, size=P).astype(np.int32)
    tokens = np.concatenate([prompt, rng.integers(0, 32000, size=tail).astype(np.int32)])
    nblocks = 4 * (-(-n // 16))
    alloc = BlockAllocator(nblocks, free_order=np.random.default_rng([446, 62]).permutation(nblocks)
                           .astype(np.int32))
    kp = torch.zeros(nblocks * hkv * 16 * D, dtype=torch.int16, device=dev)
    vp = torch.zeros_like(kp)
    cache = ops.PagedCache(kp, vp, hkv, D, dtype="bf16")
    cap = -(-n // 16) + 1
    # the first request: its prompt written and sealed, then finished
    t1 = alloc.new_table(cap)
    nb1, _, s1, _ = alloc.append_slots(t1, 0, 0, P)
    k, v = spec.kv_bits(1, 0, P)
    ops.kv_cache_write(cache, dev_bits(k, "bf16"), dev_bits(v, "bf16"), torch.from_numpy(s1).to(dev))
    alloc.cache_seal(prompt, t1, nb1)
    alloc.free_seq(t1, nb1)
    # the second request, served from the cache (host time measured)
    t0 = time.perf_counter()
    t2 = alloc.new_table(cap)
    hit = alloc.cache_lookup(tokens, t2)
    nb2, _, s2, _ = alloc.append_slots(t2, hit, hit * 16, n - hit * 16)
    lookup_us = (time.perf_counter() - t0) * 1e6
    # and without the cache: the whole prompt in fresh blocks
    t3 = alloc.new_table(cap)
    nb3, _, s3, _ = alloc.append_slots(t3, 0, 0, n)
    kc, vc = spec.kv_bits(1, hit * 16, n)
    kf, vf = spec.kv_bits(1, 0, n)
    q_all = spec.q_bits(1)  # [n][Hq][D]: the uncached prefill queries every prompt token
    modes = {
        "cached": dict(k=dev_bits(kc, "bf16"), v=dev_bits(vc, "bf16"), slots=torch.from_numpy(s2).to(dev),
                       table=torch.from_numpy(t2[None, :nb2].copy()).to(dev), q=dev_bits(q_all[n - (n - hit * 16):], "bf16")),
        "uncached": dict(k=dev_bits(kf, "bf16"), v=dev_bits(vf, "bf16"), slots=torch.from_numpy(s3).to(dev),
                         table=torch.from_numpy(t3[None, :nb3].copy()).to(dev), q=dev_bits(q_all, "bf16")),
    }
    seq_lens = torch.tensor([n], dtype=torch.int32, device=dev)
    res = {}
    for name, m in modes.items():
        qn = m["q"].shape[0]
        qsl = torch.tensor([0, qn], dtype=torch.int32, device=dev)
        out = torch.zeros_like(m["q"])
        ws = torch.empty(ops.workspace_bytes(1, qn, n, hq, D), dtype=torch.uint8, device=dev)

        def step():
            ops.kv_cache_write(cache, m["k"], m["v"], m["slots"])
            ops.paged_attention(cache, out, m["q"], m["table"], seq_lens, qsl, num_q_heads=hq,
                                max_q_len=qn, max_seq_len=n, scale=spec.scale, workspace=ws)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            step()
        b.record()
        torch.cuda.synchronize()
        res[name] = dict(ms=a.elapsed_time(b) / args.steps, query_tokens=qn)
        log(f"{name}: {qn} query tokens over {n} keys: {res[name]['ms']:.3f} ms")
    print(json.dumps({
        "metric": "second request of a repeated 10,000-token prompt: cache write + prefill attention "
                  "(one layer), prefix cache on vs off",
        "value": round(res["cached"]["ms"], 4), "unit": "ms", "higher_is_better": False,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
        "without_cache_ms": round(res["uncached"]["ms"], 4),
        "speedup": round(res["uncached"]["ms"] / res["cached"]["ms"], 2),
        "cached_blocks": hit, "host_lookup_and_append_us": round(lookup_us, 1),
        "config": {"workload": WORKLOAD_NAMES["prefix-cache"], "num_q_heads": hq, "num_kv_heads": hkv,
                   "head_dim": D, "block_size": 16},
    }), flush=True)


def bench_beam(args):
    """Beam search churn (blog page, beam search; copy-on-write section): every step
    the candidates of each request continue random parents (pkv_seq_reorder), each
    appends one token (copy-on-write of a shared, partly filled last block), then
    copy_blocks + kv_cache_write + paged_attention run over all candidates.  value =
    median host time of the reorder + appends + median GPU time of the three calls."""
    import torch

    import workloads
    from paged_kv_cache_446_amd import ops
    from paged_kv_cache_446_amd.allocator import BlockAllocator
    from tests.gpu_pipeline import dev_bits

    dev = "cuda:0"
    R, B, hq, hkv, D = 64, 4, 32, 8, 128
    steps_total = args.warmup + args.steps
    rng = np.random.default_rng([446, 70])
    prompts = rng.integers(512, 4096, size=R, endpoint=True)
    cap = int(-(-(prompts.max() + steps_total + 1) // 16)) + 1
    num_blocks = int(2 * (-(-prompts // 16)).sum() + 2 * R * B * (-(-steps_total // 16) + 2))
    alloc = BlockAllocator(num_blocks, free_order=rng.permutation(num_blocks).astype(np.int32))
    kp = torch.zeros(num_blocks * hkv * 16 * D, dtype=torch.int16, device=dev)
    vp = torch.zeros_like(kp)
    cache = ops.PagedCache(kp, vp, hkv, D, dtype="bf16")
    tables = np.full((R * B, cap), -1, np.int32)
    nblk = np.zeros(R * B, np.int32)
    lens = np.zeros(R * B, np.int32)
    for r in range(R):  # the prompt once, its candidates forks of it
        t = tables[r * B:(r + 1) * B]
        nb, ln, slots, _ = alloc.append_slots(t[0], 0, 0, int(prompts[r]))
        for b in range(1, B):
            t[b] = alloc.fork(t[0], nb)
        nblk[r * B:(r + 1) * B], lens[r * B:(r + 1) * B] = nb, ln
        k = workloads.normal_bits((446, 71, r, 0), (len(slots), hkv, D), "bf16")
        v = workloads.normal_bits((446, 71, r, 1), (len(slots), hkv, D), "bf16")
        ops.kv_cache_write(cache, dev_bits(k, "bf16"), dev_bits(v, "bf16"), torch.from_numpy(slots).to(dev))
    S = R * B
    k_new = dev_bits(workloads.normal_bits((446, 72, 0), (S, hkv, D), "bf16"), "bf16")
    v_new = dev_bits(workloads.normal_bits((446, 72, 1), (S, hkv, D), "bf16"), "bf16")
    q = dev_bits(workloads.normal_bits((446, 72, 2), (S, hq, D), "bf16"), "bf16")
    out = torch.zeros_like(q)
    qsl = torch.arange(S + 1, dtype=torch.int32, device=dev)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    max_n = int(lens.max()) + steps_total + 1
    ws = torch.empty(ops.workspace_bytes(S, S, max_n, hq, D), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    host_us, pairs_n, gpu_ms, copy_ms, attn_ms = [], [], [], [], []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for it in range(steps_total):
        t0 = time.perf_counter()
        # each candidate continues one of its own request's candidates (parents are row
        # numbers of the whole batch: one native call reorders every request)
        parents = (rng.integers(0, B, size=(R, B)) + (np.arange(R) * B)[:, None]).astype(np.int32)
        alloc.reorder(tables, nblk, lens, parents.ravel())
        slots, pairs = alloc.batch_append_slots(tables, nblk, lens, np.ones(S, np.int32))
        dt = (time.perf_counter() - t0) * 1e6
        d_slots = torch.from_numpy(slots).to(dev)
        d_pairs = torch.from_numpy(pairs.copy()).to(dev) if len(pairs) else None
        d_tables = torch.from_numpy(np.where(tables < 0, 0, tables)).to(dev)
        d_lens = torch.from_numpy(lens.copy()).to(dev)
        torch.cuda.synchronize()  # the step's uploads are done
        # a short spin keeps the GPU busy while the host queues the step, so the
        # events time the kernels, not the host's launch latency
        torch.cuda._sleep(500_000)
        ev[0].record()
        if d_pairs is not None:
            ops.copy_blocks(cache, d_pairs)
        ev[1].record()
        ops.kv_cache_write(cache, k_new, v_new, d_slots)
        ev[2].record()
        ops.paged_attention(cache, out, q, d_tables, d_lens, qsl, num_q_heads=hq, max_q_len=1,
                            max_seq_len=max_n, scale=scale, workspace=ws,
                            shared_prefixes=alloc.num_shared() > 0)
        ev[3].record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            host_us.append(dt)
            pairs_n.append(len(pairs))
            gpu_ms.append(ev[0].elapsed_time(ev[3]))
            copy_ms.append(ev[0].elapsed_time(ev[1]))
            attn_ms.append(ev[2].elapsed_time(ev[3]))
    gpu_ms, copy_ms, attn_ms, host_med = (np.median(x) for x in (gpu_ms, copy_ms, attn_ms, host_us))
    step_ms = float(gpu_ms) + float(host_med) / 1e3
    log(f"{args.steps} steps: host {host_med:.0f} us, GPU {gpu_ms * 1e3:.0f} us (medians: "
        f"copy_blocks {copy_ms * 1e3:.1f} us for {np.mean(pairs_n):.0f} pairs, attention "
        f"{attn_ms * 1e3:.0f} us), shared blocks {alloc.num_shared()}")
    pair_bytes = 2 * hkv * 16 * D * 2 * 2  # K and V of a block, read and written
    print(json.dumps({
        "metric": "beam search step: host reorder + append, then copy_blocks + kv_cache_write + "
                  "paged_attention (one layer)",
        "value": round(step_ms, 4), "unit": "ms", "higher_is_better": False, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
        "host_us": round(float(host_med), 1), "gpu_us": round(float(gpu_ms) * 1e3, 1),
        "cow_pairs_per_step": round(float(np.mean(pairs_n)), 1),
        "copy_blocks_us": round(float(copy_ms) * 1e3, 2),
        "copy_blocks_GBps": round(float(np.mean(pairs_n)) * pair_bytes / (float(copy_ms) * 1e-3) / 1e9, 1),
        "attention_us": round(float(attn_ms) * 1e3, 1),
        "shared_blocks": alloc.num_shared(),
        "config": {"workload": WORKLOAD_NAMES["beam"], "requests": R, "beams": B, "num_q_heads": hq,
                   "num_kv_heads": hkv, "head_dim": D, "block_size": 16},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--num-seqs", type=int, default=None,
                    help="decode workloads c2/c3 only: a batch of this many rows drawn from the "
                         "same length distribution (its own seed stream); default: the "
                         "workload's own batch")
    ap.add_argument("--prefix-len", type=int, default=None,
                    help="c4 only: shared prefix length (default 10000, a whole number of blocks: "
                         "the step copies the last shared block explicitly; 9992 leaves that "
                         "block partial, so the first private append copies it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--placement", default="random", choices=["random", "contiguous"],
                    help="random: blocks from a seeded permutation of the pool (paged); "
                         "contiguous: each sequence in one run of consecutive blocks")
    ap.add_argument("--kernel", default="paged", choices=["paged", "contiguous"],
                    help="contiguous: the table-free baseline (needs --placement contiguous)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (a kernel of known size for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.kernel == "contiguous" and args.placement != "contiguous":
        ap.error("--kernel contiguous needs --placement contiguous")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this path runs on a single MI355X with no sharding "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads
    from paged_kv_cache_446_amd import ops
    from paged_kv_cache_446_amd.allocator import BlockAllocator
    from tests.gpu_pipeline import dev_bits, host_bits

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.config == "prefix-cache":
        return bench_prefix_cache(args)
    if args.config == "beam":
        return bench_beam(args)
    dev = "cuda:0"
    if args.num_seqs is not None:
        if args.config not in ("c2", "c3") or args.num_seqs < 1:
            raise SystemExit("--num-seqs applies to the decode workloads c2 and c3 (>= 1 rows)")
        spec = workloads.scaled_spec(args.config, num_seqs=args.num_seqs, variant=11)
    elif args.prefix_len is not None:
        if args.config != "c4" or not 1 <= args.prefix_len <= 65536:
            raise SystemExit("--prefix-len applies to c4 (1 .. 65536 tokens)")
        spec = workloads.scaled_spec("c4", prefix=args.prefix_len)
    else:
        spec = workloads.named_spec(args.config)
    log(f"workload {args.config}: S={spec.num_seqs} context tokens={int(spec.seq_lens.sum())} "
        f"pool blocks={spec.num_blocks}")

    # ---- host allocator (a1): timed on its own ----------------------------
    if args.placement == "contiguous":
        if spec.shared_prefix:
            raise SystemExit("contiguous placement: this workload shares blocks")
        placer = ContiguousPlacer(spec.seq_lens)
        flow = workloads.run_flow(spec, placer)
    else:
        alloc = BlockAllocator(spec.num_blocks, free_order=spec.free_order)
        flow = workloads.run_flow(spec, alloc)
    # per-step host cost: one batched append of the step's tokens on a copy of the state
    probe = BlockAllocator(spec.num_blocks, free_order=spec.free_order)
    pflow_tables = np.stack([t.copy() for t in workloads.run_flow(spec, probe).tables])
    S = spec.num_seqs
    nblk = np.array([-(-int(c) // 16) for c in spec.seq_lens], dtype=np.int32)
    lens = spec.seq_lens.astype(np.int32).copy()
    t0 = time.perf_counter()
    probe.batch_append_slots(pflow_tables, nblk, lens, np.ones(S, np.int32))
    host_alloc_us = (time.perf_counter() - t0) * 1e6

    # ---- device state -------------------------------------------------------
    elems = spec.num_layers * spec.num_blocks * spec.num_kv_heads * 16 * spec.head_dim
    tdt = torch.int16 if spec.elem_bytes == 2 else torch.int32
    poison = np.array([workloads.POISON[spec.dtype]], dtype=workloads.DTYPES[spec.dtype][0]).view(
        np.int16 if spec.elem_bytes == 2 else np.int32)[0]
    kp = torch.full((elems,), int(poison), dtype=tdt, device=dev)
    vp = torch.full((elems,), int(poison), dtype=tdt, device=dev)
    cache = ops.PagedCache(kp, vp, spec.num_kv_heads, spec.head_dim, dtype=spec.dtype)
    t0 = time.perf_counter()
    for ph in flow.setup:
        if len(ph.pairs):
            ops.copy_blocks(cache, torch.from_numpy(ph.pairs.copy()).to(dev))
        for slots, k, v in workloads.iter_phase_chunks(spec, ph, max_tokens=1 << 15):
            ops.kv_cache_write(cache, dev_bits(k, spec.dtype), dev_bits(v, spec.dtype),
                               torch.from_numpy(slots).to(dev))
    torch.cuda.synchronize()
    log(f"cached context written in {time.perf_counter() - t0:.1f} s")
    stp = flow.step
    step_pairs = torch.from_numpy(stp.pairs.copy()).to(dev) if len(stp.pairs) else None
    step_slots = torch.from_numpy(stp.slots).to(dev)
    ks, vs = workloads.step_kv_bits(spec)
    k_step, v_step = dev_bits(ks, spec.dtype), dev_bits(vs, spec.dtype)
    tables = torch.from_numpy(flow.padded_tables(pad=0)).to(dev)
    seq_lens = torch.from_numpy(spec.seq_lens.astype(np.int32)).to(dev)
    qsl = torch.from_numpy(spec.query_start_loc).to(dev)
    q = dev_bits(spec.all_q_bits(), spec.dtype)
    out = torch.zeros_like(q)
    max_q, max_n = int(spec.q_lens.max()), int(spec.seq_lens.max())
    ws = torch.empty(ops.workspace_bytes(S, spec.num_q_tokens, max_n, spec.num_q_heads, spec.head_dim),
                     dtype=torch.uint8, device=dev)

    if args.kernel == "contiguous":
        first_block = torch.from_numpy(placer.first).to(dev)

        def attention():
            ops.contiguous_attention(cache, out, q, first_block, seq_lens, qsl,
                                     num_q_heads=spec.num_q_heads, max_seq_len=max_n,
                                     scale=spec.scale, workspace=ws)
    else:
        # the allocator knows whether some block has several users: then the rows are
        # read so that sharers read shared blocks together
        shared = args.placement == "random" and alloc.num_shared() > 0

        def attention():
            ops.paged_attention(cache, out, q, tables, seq_lens, qsl, num_q_heads=spec.num_q_heads,
                                max_q_len=max_q, max_seq_len=max_n, scale=spec.scale,
                                workspace=ws, shared_prefixes=shared)

    def step(ev_a=None, ev_b=None):
        if step_pairs is not None:
            ops.copy_blocks(cache, step_pairs)
        ops.kv_cache_write(cache, k_step, v_step, step_slots)
        if ev_a is not None:
            ev_a.record()
        attention()
        if ev_b is not None:
            ev_b.record()

    if args.pmc_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("pmc calibration: copied 268435456 bytes")
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record()
    for i in range(K):
        step(ev_a[i], ev_b[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = start.elapsed_time(end) / K
    attn_ms = [a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]
    attn_avg = float(np.mean(attn_ms))
    log(f"{K} steps: {ms_step * 1e3:.1f} us/step (GPU events), wall {wall / K * 1e6:.1f} us/step, "
        f"attention {attn_avg * 1e3:.1f} us (min {min(attn_ms) * 1e3:.1f})")

    graph_ms = None
    if args.graph:
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            step()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=gs):
                step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record()
        for _ in range(K):
            g.replay()
        gb.record()
        torch.cuda.synchronize()
        graph_ms = ga.elapsed_time(gb) / K
        log(f"graph replay: {graph_ms * 1e3:.1f} us/step (eager {ms_step * 1e3:.1f})")

    # cold cache: a 512 MiB write between reps (outside the events) evicts the
    # 256 MB last-level cache, so attention reads its K/V from HBM
    evict = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(min(K, 20)):
        evict.fill_(i & 255)
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record()
        attention()
        eb.record()
        cold.append((ea, eb))
    torch.cuda.synchronize()
    cold_ms = float(np.median([a.elapsed_time(b) for a, b in cold]))
    del evict
    # the practical read rate: one plain stream over 4 GiB (calibration kernel)
    buf = torch.ones(4 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    for _ in range(3):
        ops.calib_stream_read(buf, sink)
    sr = []
    for _ in range(10):
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record()
        ops.calib_stream_read(buf, sink)
        eb.record()
        sr.append((ea, eb))
    torch.cuda.synchronize()
    stream_gbs = buf.numel() / (float(np.median([a.elapsed_time(b) for a, b in sr])) * 1e-3) / 1e9
    del buf, sink
    log(f"cold-cache attention {cold_ms * 1e3:.1f} us (warm {attn_avg * 1e3:.1f}); "
        f"stream read {stream_gbs:.0f} GB/s")

    # chunks past 32 (token, head) columns per KV head take the tiled prefill kernel, which
    # is bound by MFMA, not HBM: timed alone over the same cache, for its own roofline
    prefill = None
    pf_rows = np.nonzero(spec.q_lens * spec.group > 32)[0]
    if len(pf_rows) and args.kernel == "paged" and spec.dtype != "f32":
        sel = torch.from_numpy(pf_rows.astype(np.int64)).to(dev)
        pq_lens = spec.q_lens[pf_rows].astype(np.int64)
        q_rows = np.concatenate([np.arange(spec.query_start_loc[s], spec.query_start_loc[s + 1])
                                 for s in pf_rows])
        p_tables = tables.index_select(0, sel).contiguous()
        p_lens = seq_lens.index_select(0, sel).contiguous()
        p_qsl = torch.from_numpy(np.concatenate([[0], np.cumsum(pq_lens)]).astype(np.int32)).to(dev)
        p_q = q.view(spec.num_q_tokens, -1).index_select(0, torch.from_numpy(q_rows).to(dev)).contiguous()
        p_out = torch.zeros_like(p_q)
        p_max_n = int(spec.seq_lens[pf_rows].max())
        p_ws = torch.empty(ops.workspace_bytes(len(pf_rows), len(q_rows), p_max_n, spec.num_q_heads,
                                               spec.head_dim), dtype=torch.uint8, device=dev)

        def prefill_call():
            ops.paged_attention(cache, p_out, p_q, p_tables, p_lens, p_qsl,
                                num_q_heads=spec.num_q_heads, max_q_len=int(pq_lens.max()),
                                max_seq_len=p_max_n, scale=spec.scale, workspace=p_ws)

        for _ in range(args.warmup):
            prefill_call()
        pev = []
        for _ in range(K):
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ea.record()
            prefill_call()
            eb.record()
            pev.append((ea, eb))
        torch.cuda.synchronize()
        pf_ms = float(np.mean([a.elapsed_time(b) for a, b in pev]))
        flops = prefill_flops(spec, pf_rows)
        tflops = flops / (pf_ms * 1e-3) / 1e12
        prefill = {
            "kernel": "paged_attention over the batch's prefill chunks alone (prefill plan + "
                      "tiled prefill kernel + merge)",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": round(pf_ms * 1e3, 2),
            "chunks": int(len(pf_rows)),
        }
        log(f"prefill chunks alone: {pf_ms * 1e3:.1f} us, {tflops:.0f} TFLOP/s")

    kv_bytes, attn_bytes = algorithmic_bytes(spec)
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = attn_bytes / (attn_avg * 1e-3) / 1e9
    result = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) + tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) K/V/Q, seeded block placement)",
        "config": {
            "workload": WORKLOAD_NAMES[args.config] + (
                "" if args.num_seqs is None else
                f" (batch of {args.num_seqs} rows from the same length distribution)") + (
                "" if args.prefix_len is None else f" (shared prefix of {args.prefix_len} tokens)"),
            "num_seqs": S,
            "query_tokens": spec.num_q_tokens,
            "context_tokens": int(spec.seq_lens.sum()),
            "num_q_heads": spec.num_q_heads,
            "num_kv_heads": spec.num_kv_heads,
            "head_dim": spec.head_dim,
            "block_size": 16,
            "pool_blocks": spec.num_blocks,
            "step": "copy_blocks (CoW pairs, if any) + kv_cache_write + paged_attention",
            "placement": args.placement,
            "kernel": args.kernel,
            "shared_prefix_hint": bool(args.kernel == "paged" and args.placement == "random"
                                       and alloc.num_shared() > 0),
        },
        "tokens_per_s": round(spec.num_q_tokens / (ms_step * 1e-3), 1),
        "context_tokens_per_s": round(int(spec.seq_lens.sum()) / (ms_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "host_alloc_us": round(host_alloc_us, 1),
        "graph_ms_per_step": round(graph_ms, 5) if graph_ms is not None else None,
        "roofline": {
            "kernel": ("contiguous_attention" if args.kernel == "contiguous" else "paged_attention") +
                      " (plan + partitioned decode kernel + partition merge)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic() if (args.config, args.placement, args.kernel,
                                               args.num_seqs) == ("c3", "random", "paged", None)
            else None,
            "algorithmic_bytes_per_launch": attn_bytes,
            "avg_launch_us": round(attn_avg * 1e3, 2),
            # a plain 4 GiB read stream on the same GPU: the practical read rate
            "stream_read_GBps": round(stream_gbs, 1),
            "frac_of_stream_read": round(achieved / stream_gbs, 4),
            # the same call after a 512 MiB write evicted the last-level cache
            "cold_cache_us": round(cold_ms * 1e3, 2),
            "cold_cache_GBps": round(attn_bytes / (cold_ms * 1e-3) / 1e9, 2),
        },
    }
    if prefill is not None and prefill["avg_launch_us"] > 0.5 * result["roofline"]["avg_launch_us"]:
        # the prefill kernel dominates the call: the roofline is its MFMA one; the whole
        # call's HBM figures stay beside it
        result["roofline_call_hbm"] = result["roofline"]
        result["roofline"] = prefill
    elif prefill is not None:
        result["roofline_prefill"] = prefill
    if args.placement == "random" and alloc.num_shared() > 0:
        # rows share blocks: the algorithmic bytes count a shared block once per row that
        # reads it; the distinct blocks are what HBM must deliver
        ub = unique_bytes(spec, tables.cpu().numpy())
        result["roofline"]["unique_bytes_per_launch"] = ub
        result["roofline"]["unique_GBps"] = round(ub / (attn_avg * 1e-3) / 1e9, 2)
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        # a one-thread time too for the decode workloads (every row one query token)
        base, parity = cpu_baseline(spec, host_bits(out, spec.dtype), args.cpu_seconds,
                                    one_thread=bool((spec.q_lens == 1).all()))
        result["cpu_baseline"] = base
        result["parity_sample"] = parity
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
