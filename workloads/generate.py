"""Seeded workload descriptions for the five paged-attention configurations.

The five configurations come from the pages' workloads: 16-token blocks
(blog.mckayzhao.com/?p=56, section "PagedAttention"), the LLaMA-13B shape
(same page, section "KV Cache"), a ~10,000-token shared prefix (same page,
section on advanced features, prefix caching) and a mixed chunked-prefill plus
decode batch described as one {request_id: num_tokens} dict (same page,
section "V1").

Random streams (numpy PCG64 through ``default_rng``):

* ``rng(seed_key)``                 lengths, then the block placement permutation
* ``rng(seed_key + (1, s))``        private K then V of sequence ``s`` (fp32 N(0,1))
* ``rng(seed_key + (2, s))``        Q of sequence ``s``
* ``rng(seed_key + (3,))``          K then V of the shared prefix (shared-prefix workload)

Values are drawn in fp32 and rounded to the storage dtype with round to
nearest even; a workload hands out raw bit patterns (uint32 for fp32, uint16
for fp16/bf16), so both consumers see the same bits.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Iterator, List, Optional, Tuple

import numpy as np

# element storage: numpy container for the raw bits, bytes per element
DTYPES = {"f32": (np.uint32, 4), "f16": (np.uint16, 2), "bf16": (np.uint16, 2)}
# quiet-NaN bit patterns used to pre-fill pools (stale slots must never leak)
POISON = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}

BLOCK_SIZE = 16
CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")


def _to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 samples -> raw bits of ``dtype`` (round to nearest even; finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return u.astype(np.uint16)
    raise ValueError(dtype)


def normal_bits(key, shape, dtype: str) -> np.ndarray:
    """Seeded fp32 N(0,1) values of `shape`, as raw bits of `dtype` (rng(key))."""
    rng = np.random.default_rng(list(key))
    return _to_bits(rng.standard_normal(shape, dtype=np.float32), dtype)


def prefix_kv_bits(tokens, num_kv_heads: int, head_dim: int, dtype: str):
    """K and V bits [n][Hkv][D] of a prompt whose token t's entries depend on the whole
    prefix tokens[0..t]: each token's N(0,1) draw is seeded by a running 64-bit BLAKE2b
    digest of the token ids so far.  Two prompts get equal entries at a position exactly
    when their prefixes up to it are equal, so a block reused under another prefix holds
    different values."""
    import hashlib

    h = hashlib.blake2b(digest_size=8)
    k = np.empty((len(tokens), num_kv_heads, head_dim), np.float32)
    v = np.empty_like(k)
    for t, tok in enumerate(np.asarray(tokens, dtype=np.int64)):
        h.update(int(tok).to_bytes(8, "little", signed=True))
        rng = np.random.default_rng(int.from_bytes(h.copy().digest(), "little"))
        kv = rng.standard_normal((2, num_kv_heads, head_dim), dtype=np.float32)
        k[t], v[t] = kv[0], kv[1]
    return _to_bits(k, dtype), _to_bits(v, dtype)


@dataclass
class Spec:
    """One batch: per-sequence cached context and tokens appended this step."""

    name: str
    seed_key: Tuple[int, ...]
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    ctx_lens: np.ndarray  # int64 [S]: tokens already cached before this step
    q_lens: np.ndarray  # int64 [S]: tokens appended (and queried) this step
    num_blocks: int
    free_order: np.ndarray  # int32 [num_blocks]: placement permutation
    shared_prefix: int = 0  # leading context tokens shared by every sequence
    explicit_cow_block: int = -1  # logical block the even sequences make private
    num_layers: int = 1
    _prefix_cache: Optional[Tuple[np.ndarray, np.ndarray]] = field(default=None, repr=False)

    # ---- shape helpers -------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def seq_lens(self) -> np.ndarray:
        return (self.ctx_lens + self.q_lens).astype(np.int64)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return DTYPES[self.dtype][1]

    @property
    def bits_dtype(self):
        return DTYPES[self.dtype][0]

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(head_dim), as the float32 value both sides use."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def query_start_loc(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def num_q_tokens(self) -> int:
        return int(self.q_lens.sum())

    # ---- random data -----------------------------------------------------
    def _normal(self, key, shape) -> np.ndarray:
        rng = np.random.default_rng(list(self.seed_key) + list(key))
        return rng.standard_normal(shape, dtype=np.float32)

    def _prefix(self) -> Tuple[np.ndarray, np.ndarray]:
        if self._prefix_cache is None:
            rng = np.random.default_rng(list(self.seed_key) + [3])
            shp = (self.shared_prefix, self.num_kv_heads, self.head_dim)
            k = _to_bits(rng.standard_normal(shp, dtype=np.float32), self.dtype)
            v = _to_bits(rng.standard_normal(shp, dtype=np.float32), self.dtype)
            self._prefix_cache = (k, v)
        return self._prefix_cache

    def kv_bits(self, s: int, t0: int = 0, t1: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Logical K and V bits of sequence ``s`` for tokens [t0, t1): [t][Hkv][D]."""
        n = int(self.seq_lens[s])
        t1 = n if t1 is None else t1
        p = self.shared_prefix
        shp = (n - p, self.num_kv_heads, self.head_dim)
        parts_k, parts_v = [], []
        if t0 < p:
            pk, pv = self._prefix()
            parts_k.append(pk[t0:min(t1, p)])
            parts_v.append(pv[t0:min(t1, p)])
        if t1 > p:
            rng = np.random.default_rng(list(self.seed_key) + [1, s])
            k = rng.standard_normal(shp, dtype=np.float32)
            v = rng.standard_normal(shp, dtype=np.float32)
            a, b = max(t0, p) - p, t1 - p
            parts_k.append(_to_bits(k[a:b], self.dtype))
            parts_v.append(_to_bits(v[a:b], self.dtype))
        return np.concatenate(parts_k), np.concatenate(parts_v)

    def q_bits(self, s: int) -> np.ndarray:
        """Q bits of sequence ``s``: [q_len][Hq][D]."""
        shp = (int(self.q_lens[s]), self.num_q_heads, self.head_dim)
        return _to_bits(self._normal((2, s), shp), self.dtype)

    def all_q_bits(self) -> np.ndarray:
        return np.concatenate([self.q_bits(s) for s in range(self.num_seqs)])


def _blocks(n) -> np.ndarray:
    return -(-np.asarray(n, dtype=np.int64) // BLOCK_SIZE)


def make_spec(name, seed_key, dtype, hq, hkv, d, ctx, q, *, num_blocks=None,
              shared_prefix=0, explicit_cow_block=-1, rng=None) -> Spec:
    """Build a Spec; the pool is twice the blocks needed, placed by a seeded permutation."""
    ctx = np.asarray(ctx, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    rng = rng if rng is not None else np.random.default_rng(list(seed_key))
    if num_blocks is None:
        n = ctx + q
        if shared_prefix:
            # one copy of the prefix, the private tail of each sequence, and one
            # copied block per sequence for copy-on-write
            need = int(_blocks(shared_prefix)) + int(_blocks(n - shared_prefix).sum()) + len(n)
        else:
            need = int(_blocks(n).sum())
        num_blocks = max(2 * need, 1)
    free_order = rng.permutation(num_blocks).astype(np.int32)
    return Spec(name=name, seed_key=tuple(seed_key), dtype=dtype, num_q_heads=hq,
                num_kv_heads=hkv, head_dim=d, ctx_lens=ctx, q_lens=q,
                num_blocks=num_blocks, free_order=free_order,
                shared_prefix=shared_prefix, explicit_cow_block=explicit_cow_block)


def _log_uniform(rng, lo, hi, size) -> np.ndarray:
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def named_spec(name: str) -> Spec:
    """The five full-size configurations, or the verify workload."""
    if name == "verify":
        return verify_spec()
    return scaled_spec(name)


def verify_spec(num_seqs: Optional[int] = None, max_len: Optional[int] = None, q_len: int = 5,
                variant: int = 0, dtype: str = "bf16", hq: int = 32, hkv: int = 8,
                d: int = 128) -> Spec:
    """Speculative-decoding verification (blog page, advanced features): every
    sequence appends ``q_len`` = k+1 tokens (the last accepted token and k
    drafted ones) in one pass, over the Llama-3-8B-shaped GQA decode batch's
    contexts (log-uniform in [64, 8192]).  ``q_len`` may be a scalar or one
    length per sequence."""
    key = (446, 6) if variant == 0 else (446, 6, 7, variant)
    rng = np.random.default_rng(list(key))
    S = num_seqs or 256
    hi = min(8192, max_len or 8192)
    n = _log_uniform(rng, min(64, hi), hi, S)
    q = np.broadcast_to(np.asarray(q_len, dtype=np.int64), (S,)).copy()
    return make_spec("verify", key, dtype, hq, hkv, d, n - 1, q, rng=rng)


def scaled_spec(name: str, num_seqs: Optional[int] = None, max_len: Optional[int] = None,
                variant: int = 0, prefix: Optional[int] = None) -> Spec:
    """A configuration, optionally shrunk (fewer sequences, shorter contexts).

    ``variant`` > 0 selects an independent seed stream for the shrunk copies.
    """
    cid = CONFIG_NAMES.index(name) + 1
    key = (446, cid) if variant == 0 else (446, cid, 7, variant)
    rng = np.random.default_rng(list(key))
    if name == "c1":
        n = np.array([1, 17, 33, 50], dtype=np.int64)
        return make_spec("c1", key, "f32", 4, 4, 64, n - 1, np.ones_like(n),
                         num_blocks=32, rng=rng)
    if name == "c2":
        S = num_seqs or 64
        hi = min(2048, max_len or 2048)
        n = rng.integers(min(128, hi), hi, size=S, endpoint=True)
        return make_spec("c2", key, "f16", 40, 40, 128, n - 1, np.ones_like(n), rng=rng)
    if name == "c3":
        S = num_seqs or 256
        hi = min(8192, max_len or 8192)
        n = _log_uniform(rng, min(64, hi), hi, S)
        return make_spec("c3", key, "bf16", 32, 8, 128, n - 1, np.ones_like(n), rng=rng)
    if name == "c4":
        S = num_seqs or 64
        P = 10000 if prefix is None else prefix
        hi = min(256, max_len or 256)
        tails = rng.integers(0, hi, size=S, endpoint=True)
        cow = (P // BLOCK_SIZE) - 1 if P % BLOCK_SIZE == 0 else -1
        return make_spec("c4", key, "bf16", 32, 8, 128, P + tails, np.ones_like(tails),
                         shared_prefix=P, explicit_cow_block=cow, rng=rng)
    if name == "c5":
        nc = 16 if num_seqs is None else max(1, num_seqs // 9)
        nd = 128 if num_seqs is None else max(1, num_seqs - nc)
        qhi = 512 if max_len is None else min(512, max(16, max_len // 4))
        chi = 32768 if max_len is None else min(32768, max_len)
        dhi = 8192 if max_len is None else min(8192, max_len)
        cq = rng.integers(16, qhi, size=nc, endpoint=True)
        cc = rng.integers(0, chi, size=nc, endpoint=True)
        dn = rng.integers(min(64, dhi), dhi, size=nd, endpoint=True)
        ctx = np.concatenate([cc, dn - 1])
        q = np.concatenate([cq, np.ones_like(dn)])
        order = rng.permutation(nc + nd)  # the batch dict mixes both kinds
        return make_spec("c5", key, "bf16", 32, 8, 128, ctx[order], q[order], rng=rng)
    raise ValueError(name)


# ---------------------------------------------------------------------------
# Operation sequence ("flow") a workload issues against a block allocator.
# Works with any object that offers the allocator interface:
#   new_table() -> int32 array, append_slots(table, nblk, seq_len, n_new)
#   -> (nblk, seq_len, slots, pairs), fork(table, nblk) -> table,
#   make_writable(table, nblk, j) -> pairs.
# ---------------------------------------------------------------------------


@dataclass
class Phase:
    """One batch of cache updates: copy ``pairs`` first, then write the tokens
    of ``src`` (segments (seq, t0, t1), in order) to ``slots``."""

    pairs: np.ndarray  # int32 [k][2] copy-on-write (src, dst)
    slots: np.ndarray  # int64 [T]
    src: List[Tuple[int, int, int]]

    @property
    def num_tokens(self) -> int:
        return int(self.slots.shape[0])


@dataclass
class Flow:
    tables: List[np.ndarray]  # int32 per-sequence block tables (capacity-sized)
    nblk: np.ndarray  # int32 [S]
    phases: List[Phase]  # setup phases, then the step as the last phase

    @property
    def setup(self) -> List[Phase]:
        return self.phases[:-1]

    @property
    def step(self) -> Phase:
        return self.phases[-1]

    def padded_tables(self, pad: int = 0, width: Optional[int] = None) -> np.ndarray:
        w = width or max(1, int(self.nblk.max()))
        out = np.full((len(self.tables), w), pad, dtype=np.int32)
        for s, t in enumerate(self.tables):
            out[s, : self.nblk[s]] = t[: self.nblk[s]]
        return out


def _cat_slots(parts) -> np.ndarray:
    return np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)


def _cat_pairs(parts) -> np.ndarray:
    parts = [p for p in parts if len(p)]
    return np.concatenate(parts).astype(np.int32).reshape(-1, 2) if parts else np.zeros((0, 2), np.int32)


def run_flow(spec: Spec, alloc) -> Flow:
    """Issue the workload's allocator operations in a fixed order.

    Setup: every sequence's cached context is appended (sequence-major,
    logical order); with a shared prefix, sequence 0 appends the prefix in a
    phase of its own and every other sequence is forked from it before the
    private tails are appended.
    Step: even sequences make ``explicit_cow_block`` private (if set), then
    every sequence appends its ``q_len`` new tokens.  All copies of a phase
    precede its writes.
    """
    S = spec.num_seqs
    n_final = spec.seq_lens
    cap = int(_blocks(n_final.max())) + 1
    tables = [alloc.new_table(cap) for _ in range(S)]
    nblk = np.zeros(S, np.int32)
    slen = np.zeros(S, np.int64)
    phases = []
    P = spec.shared_prefix
    if P:
        nb, sl, sl_out, pr = alloc.append_slots(tables[0], 0, 0, P)
        nblk[0], slen[0] = nb, sl
        phases.append(Phase(_cat_pairs([pr]), _cat_slots([sl_out]), [(0, 0, P)]))
        for s in range(1, S):
            tables[s] = alloc.fork(tables[0], int(nblk[0]))
            nblk[s], slen[s] = nblk[0], slen[0]
    slots, src, pairs = [], [], []
    for s in range(S):
        c = int(spec.ctx_lens[s])
        if c > slen[s]:
            nb, sl, sl_out, pr = alloc.append_slots(tables[s], int(nblk[s]), int(slen[s]), c - int(slen[s]))
            slots.append(sl_out)
            src.append((s, int(slen[s]), c))
            pairs.append(pr)
            nblk[s], slen[s] = nb, sl
    phases.append(Phase(_cat_pairs(pairs), _cat_slots(slots), src))
    slots, src, pairs = [], [], []
    if spec.explicit_cow_block >= 0:
        for s in range(0, S, 2):
            pairs.append(alloc.make_writable(tables[s], int(nblk[s]), spec.explicit_cow_block))
    for s in range(S):
        q = int(spec.q_lens[s])
        nb, sl, sl_out, pr = alloc.append_slots(tables[s], int(nblk[s]), int(slen[s]), q)
        slots.append(sl_out)
        src.append((s, int(slen[s]), int(slen[s]) + q))
        pairs.append(pr)
        nblk[s], slen[s] = nb, sl
    phases.append(Phase(_cat_pairs(pairs), _cat_slots(slots), src))
    return Flow(tables=tables, nblk=nblk, phases=phases)


def iter_phase_chunks(spec: Spec, phase: Phase, max_tokens: int = 1 << 16) -> Iterator[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """Yield (slots, K bits, V bits) of a phase's writes in bounded chunks."""
    off = 0
    ks, vs, n = [], [], 0
    for (s, t0, t1) in phase.src:
        if t1 <= t0:
            continue
        k, v = spec.kv_bits(s, t0, t1)
        ks.append(k)
        vs.append(v)
        n += t1 - t0
        if n >= max_tokens:
            yield phase.slots[off:off + n], np.concatenate(ks), np.concatenate(vs)
            off += n
            ks, vs, n = [], [], 0
    if n:
        yield phase.slots[off:off + n], np.concatenate(ks), np.concatenate(vs)


def step_kv_bits(spec: Spec) -> Tuple[np.ndarray, np.ndarray]:
    """K and V bits of this step's new tokens, in query order: [T_new][Hkv][D]."""
    ks, vs = [], []
    for s in range(spec.num_seqs):
        k, v = spec.kv_bits(s, int(spec.ctx_lens[s]), int(spec.seq_lens[s]))
        ks.append(k)
        vs.append(v)
    return np.concatenate(ks), np.concatenate(vs)
