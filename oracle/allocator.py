"""Reference model of the host block allocator (oracle; test infrastructure only).

Rules from the pages:

* The KV cache memory is a pool of equal blocks; any free block can serve any
  request, adjacency is not needed; a request receives a new block when its
  last block is full (devpress.csdn.net/amd/6a408ab810ee7a33f2834f35.html,
  section "PagedAttention: core idea", walk-through steps one and two).
* N tokens occupy ceil(N / 16) blocks, so at most 15 slots are wasted, all in
  the last block (blog.mckayzhao.com/?p=56, section "PagedAttention").
* Blocks carry reference counts; several sequences may point at one block; a
  sequence about to modify a shared block copies it and modifies the copy
  (blog page, section on copy-on-write; devpress page, section on sharing).
* A finished request returns all its blocks to the free pool (devpress page,
  core-idea walk-through, "afterwards").

Policies the pages leave open, fixed here and in the library alike:

* The free pool is a FIFO queue, seeded with ``free_order``: allocation takes
  the front, a block whose count drops to zero goes to the back.
* ``append_slots`` is all-or-nothing.  When the first new token lands in a
  partially filled last block whose count is above one, that block is copied
  first (the copy is allocated before any new block); new blocks follow in
  logical order.  Slot = block * 16 + position.
* ``free_seq`` decrements in logical order; on an error it undoes what it did.
"""

import collections

import numpy as np

BLOCK_SIZE = 16


class AllocError(Exception):
    code = "error"


class OutOfBlocks(AllocError):
    code = "out_of_blocks"


class RefcountError(AllocError):
    code = "refcount"


class InvalidArgument(AllocError):
    code = "invalid_argument"


def blocks_for_tokens(n: int, block_size: int = BLOCK_SIZE) -> int:
    """ceil(n / block_size): the pages' block-count rule."""
    if n < 0 or block_size <= 0:
        raise InvalidArgument("negative token count")
    return -(-n // block_size)


class BlockAllocatorModel:
    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, free_order=None):
        if num_blocks <= 0 or block_size != BLOCK_SIZE:
            raise InvalidArgument("bad pool")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArgument("free_order must be a permutation")
        self.num_blocks = num_blocks
        self.ref = [0] * num_blocks
        self.free = collections.deque(order)

    # ---- single blocks ---------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, b: int) -> int:
        self._check_id(b)
        return self.ref[b]

    def _check_id(self, b):
        if not (0 <= b < self.num_blocks):
            raise InvalidArgument("block id out of range")

    def alloc(self) -> int:
        if not self.free:
            raise OutOfBlocks()
        b = self._take_front()
        self.ref[b] = 1
        return b

    def incref(self, b: int):
        self._check_id(b)
        if self.ref[b] <= 0:
            raise RefcountError("incref of a free block")
        self.ref[b] += 1

    def decref(self, b: int):
        self._check_id(b)
        if self.ref[b] <= 0:
            raise RefcountError("decref of a free block")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    # ---- sequences ---------------------------------------------------------
    def new_table(self, cap: int) -> np.ndarray:
        return np.full(cap, -1, dtype=np.int32)

    def append_slots(self, table, nblk: int, seq_len: int, n_new: int):
        cap = len(table)
        if n_new < 0 or seq_len < 0 or nblk != blocks_for_tokens(seq_len):
            raise InvalidArgument("inconsistent sequence state")
        need_blocks = blocks_for_tokens(seq_len + n_new)
        if need_blocks > cap:
            raise InvalidArgument("block table too small")
        if nblk > 0:  # the one existing entry an append reads: its last block
            self._check_id(int(table[nblk - 1]))
            if self.ref[int(table[nblk - 1])] <= 0:
                raise RefcountError("the last block is free")
        cow = n_new > 0 and seq_len % BLOCK_SIZE != 0 and self.ref[int(table[nblk - 1])] > 1
        if need_blocks - nblk + int(cow) > len(self.free):
            raise OutOfBlocks()
        pairs = []
        if cow:
            src = int(table[nblk - 1])
            dst = self.alloc()
            self.decref(src)
            table[nblk - 1] = dst
            pairs.append((src, dst))
        for j in range(nblk, need_blocks):
            table[j] = self.alloc()
        pos = np.arange(seq_len, seq_len + n_new, dtype=np.int64)
        slots = table[pos // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + pos % BLOCK_SIZE
        return need_blocks, seq_len + n_new, slots, np.array(pairs, dtype=np.int32).reshape(-1, 2)

    def make_writable(self, table, nblk: int, j: int):
        """Copy-on-write of logical block j ahead of a modification."""
        if not (0 <= j < nblk):
            raise InvalidArgument("logical block out of range")
        src = int(table[j])
        self._check_id(src)
        if self.ref[src] <= 0:
            raise RefcountError("table holds a free block")
        if self.ref[src] == 1:
            return np.zeros((0, 2), dtype=np.int32)
        if not self.free:
            raise OutOfBlocks()
        dst = self.alloc()
        self.decref(src)
        table[j] = dst
        return np.array([[src, dst]], dtype=np.int32)

    def fork(self, table, nblk: int):
        """A child sequence pointing at the same blocks (each count + 1)."""
        for j in range(nblk):
            self._check_id(int(table[j]))
            if self.ref[int(table[j])] <= 0:
                raise RefcountError("table holds a free block")
        for j in range(nblk):
            self.ref[int(table[j])] += 1
        child = np.array(table, dtype=np.int32, copy=True)
        child[nblk:] = -1
        return child

    def reorder(self, tables, nblk, seq_lens, parents):
        """Beam reorder (blog page, beam search: candidates share their beginning): new
        row i continues old row parents[i].  Every parent block gains one user per
        child (child order), then every old row's blocks lose one (row order).  In
        place on tables [R][cap], nblk [R], seq_lens [R]."""
        R, cap = tables.shape
        for r in range(R):
            nb, ln, par = int(nblk[r]), int(seq_lens[r]), int(parents[r])
            if nb < 0 or nb > cap or ln < 0 or nb != -(-ln // BLOCK_SIZE):
                raise InvalidArgument("row lengths")
            if not (0 <= par < R):
                raise InvalidArgument("parent out of range")
            for j in range(nb):
                self._check_id(int(tables[r, j]))
                if self.ref[int(tables[r, j])] <= 0:
                    raise RefcountError("table holds a free block")
        for i in range(R):
            p = int(parents[i])
            for j in range(int(nblk[p])):
                self.ref[int(tables[p, j])] += 1
        for r in range(R):
            for j in range(int(nblk[r])):
                self.decref(int(tables[r, j]))
        old_t, old_n, old_l = tables.copy(), nblk.copy(), seq_lens.copy()
        for i in range(R):
            p = int(parents[i])
            tables[i] = old_t[p]
            nblk[i] = old_n[p]
            seq_lens[i] = old_l[p]

    def free_seq(self, table, nblk: int):
        done = []
        try:
            for j in range(nblk):
                self.decref(int(table[j]))
                done.append(int(table[j]))
        except AllocError:
            for b in reversed(done):  # undo, newest first
                if self.ref[b] == 0:
                    assert self.free[-1] == b
                    self.free.pop()
                self.ref[b] += 1
            raise

    # ---- prefix cache -------------------------------------------------------
    # A request whose prompt starts with an earlier request's tokens reuses the K/V
    # blocks computed for them (blog.mckayzhao.com/?p=56, advanced features and V1
    # sections: automatic prefix caching; devpress page, sharing section).  The K/V
    # of a token depend on every token before it, so a full block caches the K/V of
    # one exact prefix: logical block j of a prompt is keyed by the tuple of ALL of
    # the prompt's tokens 0 .. 16(j+1)-1.  Cached blocks stay findable after their
    # count drops to zero; the free queue hands out the block released longest ago
    # first, and a cached block taken that way leaves the cache together with every
    # cached key that extends its key (a lookup walks a prompt's blocks from the
    # first one and stops at the first miss, so what is cached below an evicted
    # block is dropped with it: the plainest policy, which the pages leave open).

    def _cache(self):
        if not hasattr(self, "key_of"):
            self.key_of = {}   # block -> key (full prefix tuple)
            self.block_of = {}  # key -> block
        return self.key_of, self.block_of

    def _take_front(self) -> int:
        b = self.free.popleft()
        if b in self._cache()[0]:
            self._evict(b)
        return b

    def _evict(self, b):
        """Drop cached block b and every cached key that extends its key."""
        key_of, block_of = self._cache()
        gone = key_of[b]
        for key in [k for k in block_of if k[:len(gone)] == gone]:
            del key_of[block_of.pop(key)]

    @staticmethod
    def _prefix_key(tokens, table, j):
        """Key of logical block j of a prompt: all of its tokens up to that block's end."""
        return tuple(tokens[:(j + 1) * BLOCK_SIZE])

    def cache_lookup(self, tokens, table) -> int:
        key_of, block_of = self._cache()
        tokens = [int(t) for t in tokens]
        n = min(len(tokens) // BLOCK_SIZE, len(table))
        j = 0
        while j < n:
            b = block_of.get(self._prefix_key(tokens, table, j))
            if b is None:
                break
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            table[j] = b
            j += 1
        return j

    def cache_seal(self, tokens, table, nblk: int):
        key_of, block_of = self._cache()
        tokens = [int(t) for t in tokens]
        n = min(len(tokens) // BLOCK_SIZE, nblk)
        keys = [self._prefix_key(tokens, table, j) for j in range(n)]
        for j in range(n):
            b = int(table[j])
            self._check_id(b)
            if self.ref[b] <= 0:
                raise RefcountError("table holds a free block")
            if b in key_of and key_of[b] != keys[j]:
                raise InvalidArgument("a cached block must keep its contents")
        for j in range(n):
            b = int(table[j])
            if b in key_of or keys[j] in block_of:
                continue
            key_of[b] = keys[j]
            block_of[keys[j]] = b

    def num_cached(self) -> int:
        return len(self._cache()[0])

    def num_shared(self) -> int:
        """Blocks that several sequences use (devpress page, how memory is shared):
        a reference count of two or more."""
        return sum(1 for r in self.ref if r >= 2)

    # ---- statistics ---------------------------------------------------------
    @staticmethod
    def tail_waste(n: int) -> int:
        """Unused slots in the last block of an n-token sequence."""
        return blocks_for_tokens(n) * BLOCK_SIZE - n
