"""Python handle over the C block allocator of libpkv (marshalling only)."""

import ctypes

import numpy as np

from . import _lib

_lib.load()

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _p32(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_i32p)


def _p64(a: np.ndarray):
    assert a.dtype == np.int64 and a.flags.c_contiguous
    return a.ctypes.data_as(_i64p)


def blocks_for_tokens(n: int, block_size: int = 16) -> int:
    return int(_lib.load().pkv_blocks_for_tokens(int(n), int(block_size)))


class BlockAllocator:
    """Reference-counted block pool (pkv_ba_*); tables are numpy int32 arrays."""

    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        self._lib = _lib.load()
        h = ctypes.c_void_p()
        fo = None
        if free_order is not None:
            self._free_order = np.ascontiguousarray(free_order, dtype=np.int32)
            fo = _p32(self._free_order)
        _lib.check(self._lib.pkv_ba_create(int(num_blocks), int(block_size), fo, ctypes.byref(h)),
                   "pkv_ba_create")
        self._h = h
        self.num_blocks = int(num_blocks)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pkv_ba_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    # ---- single blocks -----------------------------------------------------
    def alloc(self) -> int:
        b = ctypes.c_int32()
        _lib.check(self._lib.pkv_ba_alloc(self._h, ctypes.byref(b)), "pkv_ba_alloc")
        return b.value

    def incref(self, b: int):
        _lib.check(self._lib.pkv_ba_incref(self._h, int(b)), "pkv_ba_incref")

    def decref(self, b: int):
        _lib.check(self._lib.pkv_ba_decref(self._h, int(b)), "pkv_ba_decref")

    def refcount(self, b: int) -> int:
        c = ctypes.c_int32()
        _lib.check(self._lib.pkv_ba_refcount(self._h, int(b), ctypes.byref(c)), "pkv_ba_refcount")
        return c.value

    def num_free(self) -> int:
        return int(self._lib.pkv_ba_num_free(self._h))

    # ---- sequences -----------------------------------------------------------
    def new_table(self, cap: int) -> np.ndarray:
        return np.full(int(cap), -1, dtype=np.int32)

    def append_slots(self, table: np.ndarray, nblk: int, seq_len: int, n_new: int):
        nb = ctypes.c_int32(int(nblk))
        sl = ctypes.c_int32(int(seq_len))
        slots = np.empty(max(int(n_new), 1), dtype=np.int64)
        pair = np.zeros(2, dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _lib.check(self._lib.pkv_seq_append_slots(self._h, _p32(table), len(table), ctypes.byref(nb),
                                                  ctypes.byref(sl), int(n_new), _p64(slots),
                                                  _p32(pair), ctypes.byref(ncow)),
                   "pkv_seq_append_slots")
        return nb.value, sl.value, slots[: int(n_new)], pair[: 2 * ncow.value].reshape(-1, 2)

    def batch_append_slots(self, tables: np.ndarray, nblk: np.ndarray, seq_lens: np.ndarray,
                           n_new: np.ndarray):
        """tables int32 [S][cap], nblk/seq_lens int32 [S] (updated in place), n_new int32 [S]."""
        S, cap = tables.shape
        slots = np.empty(max(int(n_new.sum()), 1), dtype=np.int64)
        pairs = np.zeros((max(S, 1), 2), dtype=np.int32)
        ncow, ndone = ctypes.c_int32(0), ctypes.c_int32(0)
        rc = self._lib.pkv_batch_append_slots(self._h, _p32(tables), cap, _p32(nblk), _p32(seq_lens),
                                              _p32(n_new), S, _p64(slots), _p32(pairs),
                                              ctypes.byref(ncow), ctypes.byref(ndone))
        _lib.check(rc, f"pkv_batch_append_slots (done {ndone.value})")
        return slots[: int(n_new.sum())], pairs[: ncow.value]

    def make_writable(self, table: np.ndarray, nblk: int, j: int):
        pair = np.zeros(2, dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _lib.check(self._lib.pkv_seq_make_writable(self._h, _p32(table), int(nblk), int(j), _p32(pair),
                                                   ctypes.byref(ncow)), "pkv_seq_make_writable")
        return pair[: 2 * ncow.value].reshape(-1, 2)

    def fork(self, table: np.ndarray, nblk: int) -> np.ndarray:
        child = np.full(len(table), -1, dtype=np.int32)
        _lib.check(self._lib.pkv_seq_fork(self._h, _p32(table), int(nblk), _p32(child)), "pkv_seq_fork")
        return child

    def reorder(self, tables: np.ndarray, nblk: np.ndarray, seq_lens: np.ndarray, parents: np.ndarray):
        """Beam reorder: new row i continues old row parents[i] (tables int32 [R][cap],
        nblk/seq_lens int32 [R], updated in place)."""
        R, cap = tables.shape
        work = np.empty(max(R * cap, 1), dtype=np.int32)
        par = np.ascontiguousarray(parents, dtype=np.int32)
        _lib.check(self._lib.pkv_seq_reorder(self._h, _p32(tables), cap, _p32(nblk), _p32(seq_lens), R,
                                             _p32(par), _p32(work)), "pkv_seq_reorder")

    def free_seq(self, table: np.ndarray, nblk: int):
        _lib.check(self._lib.pkv_seq_free(self._h, _p32(table), int(nblk)), "pkv_seq_free")

    # ---- prefix cache ------------------------------------------------------------
    def cache_lookup(self, tokens: np.ndarray, table: np.ndarray) -> int:
        """Take the cached full blocks that start this prompt; returns how many."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        nb = ctypes.c_int32(0)
        _lib.check(self._lib.pkv_seq_cache_lookup(self._h, _p32(tokens) if len(tokens) else None,
                                                  len(tokens), _p32(table), len(table),
                                                  ctypes.byref(nb)), "pkv_seq_cache_lookup")
        return nb.value

    def cache_seal(self, tokens: np.ndarray, table: np.ndarray, nblk: int):
        """Register the sequence's full blocks (their K/V written) in the cache."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        _lib.check(self._lib.pkv_seq_cache_seal(self._h, _p32(tokens) if len(tokens) else None,
                                                len(tokens), _p32(table), int(nblk)),
                   "pkv_seq_cache_seal")

    def num_cached(self) -> int:
        return int(self._lib.pkv_ba_num_cached(self._h))

    def num_shared(self) -> int:
        """Blocks with a reference count of two or more."""
        return int(self._lib.pkv_ba_num_shared(self._h))


def prefix_hash(parent: int, tokens16) -> int:
    t = np.ascontiguousarray(tokens16, dtype=np.int32)
    assert t.shape == (16,)
    return int(_lib.load().pkv_prefix_hash(ctypes.c_uint64(parent), _p32(t)))
